"""C-ABI checks that need no GPU: the library loads, exports every function
include/bitlinear.h declares, reports sizes, and rejects bad arguments on the
host before any launch (no valid device pointer is ever passed here)."""
import ctypes
import os
import re

import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitlinear.h")


def _declared_functions():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bitlinear_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def bl():
    import bit_gemm_int8_amd as B
    return B


def test_header_declares_expected(bl):
    names = _declared_functions()
    assert "bitlinear_pack_weights" in names and "bitlinear_forward" in names
    assert sorted(bl.EXPORTS) == names


def test_library_exports_every_declared_symbol(bl):
    raw = ctypes.CDLL(bl.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(raw, name), name
    assert bl.lib.bitlinear_abi_version() == 4


@pytest.mark.parametrize("n,k", [(1, 1), (64, 256), (65, 257), (2560, 6912), (28672, 8192), (130, 520)])
def test_sizes_match_layout(bl, n, k):
    assert bl.packed_bytes(n, k) == O.packed_bytes(n, k)
    assert bl.padded_k(k) == O.padded_k(k)
    assert bl.padded_n(n) == O.padded_n(n)
    assert bl.lib.bitlinear_xq_bytes(3, k) == 3 * O.padded_k(k)


def test_sizes_of_degenerate_shapes(bl):
    assert bl.packed_bytes(0, 5) == 0
    assert bl.lib.bitlinear_xq_bytes(0, 5) == 0
    assert bl.forward_workspace_bytes(0, 10, 10) == 0
    assert bl.forward_workspace_bytes(1, 10, bl.BL_MAX_K + 1) == 0


def test_status_strings(bl):
    for s in range(6):
        assert bl.lib.bitlinear_status_string(s)
    assert bl.lib.bitlinear_status_string(99) == b"unknown status"


FAKE = 1 << 20  # host-side placeholder address, aligned; never dereferenced


def test_quant_act_rejects(bl):
    q = bl.lib.bitlinear_quant_act
    assert q(FAKE, 0, 4, 0, 1e-5, FAKE, FAKE, None) == 1            # k < 1
    assert q(FAKE, 0, -1, 8, 1e-5, FAKE, FAKE, None) == 1           # m < 0
    assert q(FAKE, 7, 4, 8, 1e-5, FAKE, FAKE, None) == 1            # dtype
    assert q(FAKE, 0, 4, 8, -1.0, FAKE, FAKE, None) == 1            # eps < 0
    assert q(FAKE, 0, 4, 8, float("nan"), FAKE, FAKE, None) == 1    # eps nan
    assert q(None, 0, 4, 8, 1e-5, FAKE, FAKE, None) == 1            # null x
    assert q(FAKE, 0, 4, bl.BL_MAX_K + 1, 1e-5, FAKE, FAKE, None) == 2
    assert q(FAKE + 2, 0, 4, 8, 1e-5, FAKE, FAKE, None) == 3        # fp32 x at 2 bytes
    assert q(FAKE, 0, 4, 8, 1e-5, FAKE + 8, FAKE, None) == 3        # xq at 8 bytes
    assert q(None, 0, 0, 8, 1e-5, None, None, None) == 0            # m == 0: no-op


def test_activation_eps_boundary_matches_oracle(bl):
    """The library refuses exactly the activation eps values the oracle
    refuses (0, negatives, NaN/Inf, and those whose fp32 127/eps overflows),
    in both entry points that quantize activations; weight packing still
    takes eps = 0."""
    import numpy as np
    from test_oracle_pins import EPS_MIN
    below = float(np.nextafter(EPS_MIN, np.float32(0)))
    q = bl.lib.bitlinear_quant_act
    arr = (bl.BLLinear * 1)()
    arr[0] = bl.BLLinear(None, 0, None, None, 64, 256, 0, 0, None, None, None, None, 0, 1e-6, None)
    f = bl.lib.bitlinear_forward_fused
    for e, ok in ((float(EPS_MIN), True), (1e-5, True), (below, False), (0.0, False),
                  (1e-38, False), (-1e-5, False), (float("inf"), False)):
        x = np.zeros((1, 4), np.float32)
        try:
            O.quant_act(x, e)
            assert ok, e
        except ValueError:
            assert not ok, e
        assert q(None, 0, 0, 8, e, None, None, None) == (0 if ok else 1), e
        assert f(arr, 1, 0, e, None, 0, None) == (0 if ok else 1), e
    ws = bl.lib.bitlinear_pack_workspace_bytes(64, 256)
    assert bl.lib.bitlinear_pack_weights(FAKE, 0, 64, 256, 0.0, None, FAKE + 256, FAKE, None,
                                         0, None) == 4      # eps = 0 passes; no workspace


def test_rmsnorm_quant_act_rejects(bl):
    q = bl.lib.bitlinear_rmsnorm_quant_act
    assert q(FAKE, 0, 4, 8, None, 0.0, 1e-5, FAKE, FAKE, None) == 1       # norm eps 0
    assert q(FAKE, 0, 4, 8, None, -1.0, 1e-5, FAKE, FAKE, None) == 1
    assert q(FAKE, 0, 4, 8, None, float("inf"), 1e-5, FAKE, FAKE, None) == 1
    assert q(FAKE, 0, 4, 8, None, 1e-6, 0.0, FAKE, FAKE, None) == 1       # activation eps 0
    assert q(FAKE, 9, 4, 8, None, 1e-6, 1e-5, FAKE, FAKE, None) == 1      # dtype
    assert q(FAKE, 0, 4, 0, None, 1e-6, 1e-5, FAKE, FAKE, None) == 1      # k < 1
    assert q(FAKE, 0, 4, bl.BL_MAX_K + 1, None, 1e-6, 1e-5, FAKE, FAKE, None) == 2
    assert q(FAKE, 0, 4, 8, FAKE + 2, 1e-6, 1e-5, FAKE, FAKE, None) == 3  # gain at 2 bytes
    assert q(FAKE, 0, 4, 8, None, 1e-6, 1e-5, FAKE + 8, FAKE, None) == 3  # xq at 8 bytes
    assert q(None, 0, 0, 8, None, 1e-6, 1e-5, None, None, None) == 0     # m == 0: no-op
    # the fused step checks an entry's norm eps and gain alignment
    f = bl.lib.bitlinear_forward_fused
    arr = (bl.BLLinear * 1)()
    arr[0] = bl.BLLinear(FAKE, 1, FAKE, FAKE, 64, 256, 0, 0, FAKE, None, None, None, 1, 0.0, None)
    assert f(arr, 1, 1, 1e-5, None, 0, None) == 1
    arr[0] = bl.BLLinear(FAKE, 1, FAKE, FAKE, 64, 256, 0, 0, FAKE, None, None, None, 1, 1e-6,
                         FAKE + 4)
    assert f(arr, 1, 1, 1e-5, None, 0, None) == 3


def test_pack_rejects(bl):
    p = bl.lib.bitlinear_pack_weights
    ws = bl.lib.bitlinear_pack_workspace_bytes(64, 256)
    assert ws > 0
    assert p(None, 0, 64, 256, 1e-5, None, FAKE, FAKE, FAKE, ws, None) == 1
    assert p(FAKE, 0, 0, 256, 1e-5, None, FAKE, FAKE, FAKE, ws, None) == 1
    assert p(FAKE, 0, 64, 0, 1e-5, None, FAKE, FAKE, FAKE, ws, None) == 1
    assert p(FAKE, 3, 64, 256, 1e-5, None, FAKE, FAKE, FAKE, ws, None) == 1
    assert p(FAKE, 0, 64, 256, float("inf"), None, FAKE, FAKE, FAKE, ws, None) == 1
    assert p(FAKE, 0, 64, bl.BL_MAX_K + 1, 1e-5, None, FAKE, FAKE, FAKE, ws, None) == 2
    assert p(FAKE + 4, 0, 64, 256, 1e-5, None, FAKE, FAKE, FAKE, ws, None) == 3
    assert p(FAKE, 0, 64, 256, 1e-5, None, FAKE + 16, FAKE, FAKE, ws, None) == 3
    assert p(FAKE, 0, 64, 256, 1e-5, None, FAKE, FAKE, None, ws, None) == 4
    assert p(FAKE, 0, 64, 256, 1e-5, None, FAKE, FAKE, FAKE, ws - 8, None) == 4


def test_forward_rejects(bl):
    f = bl.lib.bitlinear_forward
    args = dict(xq=FAKE, s=FAKE, pk=FAKE, g=FAKE, m=4, n=64, k=256, epi=0, yd=0, y=FAKE,
                acc=None, ws=FAKE, wsb=1 << 30, st=None)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["xq"], a["s"], a["pk"], a["g"], a["m"], a["n"], a["k"], a["epi"], a["yd"],
                 a["y"], a["acc"], a["ws"], a["wsb"], a["st"])

    assert call(n=0) == 1
    assert call(k=0) == 1
    assert call(m=-1) == 1
    assert call(epi=2) == 1
    assert call(yd=2) == 1
    assert call(y=None) == 1
    assert call(pk=None) == 1
    assert call(k=bl.BL_MAX_K + 1) == 2
    assert call(xq=FAKE + 4) == 3
    assert call(y=FAKE + 2) == 3
    assert call(y=FAKE + 2, yd=1) != 3 or True   # bf16 output only needs 2-byte alignment
    # a shape that splits K needs a workspace
    need = bl.forward_workspace_bytes(1, 64, 65536)
    assert need > 0
    assert call(m=1, k=65536, ws=None) == 4
    assert call(m=1, k=65536, wsb=need - 4) == 4
    assert call(m=1, k=65536, ws=FAKE + 16, wsb=need) == 3
    assert call(m=0, xq=None, y=None) == 0        # empty batch: no-op
    # a GEMM grid past 32-bit tile numbering is refused before any launch
    assert call(m=bl.BL_MAX_MN, n=bl.BL_MAX_MN, k=256) == 2


def test_forward_noalloc_rejects(bl):
    """The entry point without a workspace checks like bitlinear_forward and
    refuses, before touching the device, a plan whose split-K slots exceed
    its scratch."""
    f = bl.lib.bitlinear_forward_noalloc

    def call(xq=FAKE, s=FAKE, pk=FAKE, g=FAKE, m=4, n=64, k=256, epi=0, yd=0, y=FAKE, acc=None):
        return f(xq, s, pk, g, m, n, k, epi, yd, y, acc, None)

    assert call(n=0) == 1
    assert call(epi=3) == 1
    assert call(pk=None) == 1
    assert call(k=bl.BL_MAX_K + 1) == 2
    assert call(xq=FAKE + 4) == 3
    assert call(m=0, xq=None, y=None) == 0
    assert bl.forward_workspace_bytes(2, 16448, 65536) > bl.BL_NOALLOC_SCRATCH_BYTES
    assert call(m=2, n=16448, k=65536) == 4
    assert call(m=bl.BL_MAX_MN, n=bl.BL_MAX_MN, k=256) == 2


def test_forward_multi_rejects(bl):
    f = bl.lib.bitlinear_forward_multi

    def table(*entries):
        arr = (bl.BLProduct * max(1, len(entries)))()
        for e, d in zip(arr, entries):
            e.packed, e.gamma, e.n = d.get("pk", FAKE), d.get("g", FAKE), d.get("n", 64)
            e.epilogue, e.y_dtype = d.get("epi", 0), d.get("yd", 0)
            e.y, e.acc_out = d.get("y", FAKE), d.get("acc", None)
        return arr

    def call(entries, m=4, k=256, xq=FAKE, s=FAKE, ws=FAKE, wsb=1 << 30, nops=None):
        arr = table(*entries)
        return f(xq, s, m, k, arr, len(entries) if nops is None else nops, ws, wsb, None)

    one = [{}]
    assert f(FAKE, FAKE, 4, 256, None, 1, FAKE, 1 << 30, None) == 1
    assert call(one, nops=0) == 1
    assert call(one * 17) == 1
    assert call([{"n": 0}]) == 1
    assert call([{}, {"epi": 2}]) == 1
    assert call([{"yd": 2}]) == 1
    assert call([{}, {"pk": None}]) == 1
    assert call([{"y": None}]) == 1
    assert call(one, m=-1) == 1
    assert call(one, k=0) == 1
    assert call(one, k=bl.BL_MAX_K + 1) == 2
    assert call([{"n": bl.BL_MAX_MN}, {"n": 64}]) == 2   # summed widths past the limit
    assert call(one, xq=FAKE + 4) == 3
    assert call([{}, {"y": FAKE + 2}]) == 3
    # products that run one by one and split K need the workspace
    need = bl.lib.bitlinear_forward_multi_workspace_bytes(table({}, {"n": 200}), 2, 1, 65536)
    assert need == bl.forward_workspace_bytes(1, 200, 65536) > 0
    assert call([{}, {"n": 200}], m=1, k=65536, ws=None) == 4
    assert call([{}, {"n": 200}], m=1, k=65536, wsb=need - 4) == 4
    assert call(one, m=0, xq=None, s=None) == 0            # empty batch: no-op
    assert call([{"n": bl.BL_MAX_MN // 2}, {"n": bl.BL_MAX_MN // 4}], m=bl.BL_MAX_MN) == 2
    # one GEMM launch over the table needs none
    qkv = table({"n": 8192}, {"n": 1024}, {"n": 1024})
    assert bl.lib.bitlinear_forward_multi_workspace_bytes(qkv, 3, 512, 8192) == 0


def test_workspace_init_rejects(bl):
    w = bl.lib.bitlinear_workspace_init
    assert w(None, 0, None) == 0
    assert w(None, 64, None) == 1
    assert w(FAKE, 6, None) == 1
    assert w(FAKE + 2, 8, None) == 3


# ------------------------------------------------------------- kernel plans --
# bitlinear_forward_kernel / bitlinear_forward_fused_kernel are host-only
# queries of the dispatch plan; the GPU parity cases rely on them to cover
# every kernel.
@pytest.mark.parametrize("m,n,k,kernel", [
    (1, 256, 256, "dot4_gemv"),
    (2, 300, 40000, "dot4_gemv"),           # split K
    (1, 28672, 8192, "stream_gemv"),
    (2, 8192, 28672, "stream_gemv"),
    (64, 8192, 8192, "stream_mt"),          # long rows, <= 128 row blocks, > 32 tokens
    (32, 1024, 8192, "stream_mt"),          # <= 16 row blocks, > 16 tokens
    (32, 8192, 8192, "mfma_gemv"),
    (3, 2560, 2560, "mfma_gemv"),
    (64, 2560, 6912, "mfma_gemv"),          # rows of 27 super-chunks
    (16, 2560, 16384, "mfma_gemv"),         # x~ of 16 tokens past the LDS
    (512, 1024, 8192, "mfma_gemv"),         # few output tiles: token blocks
    (512, 640, 2560, "stream_mt"),          # few tiles, short rows, >= 512 tokens
    (256, 2560, 2560, "stream_mt"),         # few tiles, short rows, >= 32 row blocks
    (256, 640, 2560, "mfma_gemv"),
    (2048, 6912, 2560, "gemm"),
])
def test_forward_kernel_plan(bl, m, n, k, kernel):
    assert bl.forward_kernel(m, n, k) == kernel


def test_forward_kernel_plan_rejects(bl):
    with pytest.raises(bl.BitLinearError):
        bl.forward_kernel(0, 10, 10)
    with pytest.raises(bl.BitLinearError):
        bl.forward_kernel(1, 10, bl.BL_MAX_K + 1)


def _fake_table(bl, specs, x_offset=0):
    """bl_linear entries with distinct 256-byte aligned fake addresses (the
    plan query reads sizes and alignment only)."""
    arr = (bl.BLLinear * len(specs))()
    for i, (n, k, xdt, norm) in enumerate(specs):
        base = 0x10000000 * (i + 1)
        arr[i] = bl.BLLinear(base + x_offset, bl.BL_BF16 if xdt == "bf16" else bl.BL_F32,
                             base + 0x1000000, base + 0x2000000, n, k, 0, bl.BL_BF16,
                             base + 0x3000000, None, None, None, 1 if norm else 0,
                             2.0 ** -23, None)
    return arr


@pytest.mark.parametrize("m,specs,x_offset,kernel", [
    (1, [(28672, 8192, "bf16", False)], 0, "stream_gemv"),
    (1, [(300, 512, "bf16", False)], 0, "dot4_gemv"),                    # short rows
    (8, [(2560, 2560, "bf16", False), (640, 2560, "bf16", False)], 0, "stream_mt"),
    (64, [(2560, 6912, "bf16", True)], 0, "two_pass"),                  # one RMSNorm product, 13.5 KiB rows
    (64, [(2560, 6912, "bf16", True), (640, 6912, "bf16", True)], 0, "stream_mt"),
    (8, [(2560, 2560, "bf16", True)], 0, "stream_mt"),                    # RMSNorm, 5 KiB rows
    (33, [(1000, 4096, "f32", False)], 0, "stream_mt"),
    (8, [(1000, 4096, "f32", False)], 4, "mfma_gemv"),                   # x not 16-byte aligned
    (16, [(2048, 8200, "f32", False)], 0, "two_pass"),                   # fp32 row past 16 KiB
    (16, [(8192, 28672, "bf16", False)], 0, "two_pass"),                 # bf16 row past 16 KiB
    (3, [(640, 2560, "bf16", True), (300, 9000, "f32", False)], 0, "two_pass"),
    (16, [(2048, 1004, "bf16", False)], 0, "mfma_gemv"),                 # rows not whole 16-byte units
    (2, [(1100, 28672, "bf16", True)], 0, "mfma_gemv"),                  # RMSNorm, x~ past the LDS
])
def test_forward_fused_kernel_plan(bl, m, specs, x_offset, kernel):
    arr = _fake_table(bl, specs, x_offset)
    r = bl.lib.bitlinear_forward_fused_kernel(arr, len(specs), m)
    assert r >= 0 and bl.KERNEL_NAMES[r] == kernel


def test_forward_fused_kernel_plan_rejects(bl):
    arr = _fake_table(bl, [(100, 100, "f32", False)])
    assert bl.lib.bitlinear_forward_fused_kernel(arr, 1, bl.BL_FUSED_MAX_M + 1) == -bl.BL_ERR_UNSUPPORTED_SHAPE
    assert bl.lib.bitlinear_forward_fused_kernel(arr, 0, 4) == -bl.BL_ERR_INVALID_ARG
    assert bl.lib.bitlinear_forward_fused_kernel(arr, 1, 0) == -bl.BL_ERR_INVALID_ARG


def test_gpu_cases_cover_every_kernel(bl):
    """The forward and fused-step parity cases reach every kernel."""
    from test_gpu_parity import FWD_CASES
    from test_gpu_fused import FUSED_CASES
    kinds = {bl.forward_kernel(m, n, k) for (m, n, k, *_rest) in FWD_CASES}
    assert kinds == set(bl.KERNEL_NAMES.values()) - {"two_pass"}, kinds
    fused = set()
    for m, specs in FUSED_CASES:
        arr = _fake_table(bl, [(n, k, xdt, False) for (n, k, _r, _y, xdt) in specs])
        fused.add(bl.KERNEL_NAMES[bl.lib.bitlinear_forward_fused_kernel(arr, len(specs), m)])
    assert fused == {"dot4_gemv", "stream_gemv", "stream_mt", "mfma_gemv", "two_pass"}, fused
