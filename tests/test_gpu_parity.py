"""GPU parity of every step of the pass against the CPU oracle, called
through the C ABI (via the thin binding).  Integers and bytes are compared bit
for bit; outputs within 1e-5 (fp32) / 1e-2 (bf16) relative, zeros exact."""
import numpy as np
import pytest

import oracle as O
from datagen import random_case
from gpu_util import (assert_y_close, dev, gamma_agrees, host, log, x_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_gemm_int8_amd as B
    return B


# ------------------------------------------------------------ activations --
# rows held in registers (1 to 16 16-byte vectors per thread), rows read
# twice (longer, or not a whole number of 16-byte vectors)
QA_CASES = [(1, 1, "f32"), (1, 7, "bf16"), (3, 256, "f32"), (4, 272, "bf16"), (5, 1000, "f32"),
            (9, 2560, "bf16"), (2, 6912, "bf16"), (64, 300, "f32"), (33, 8, "bf16"),
            (1, 28672, "bf16"), (130, 520, "f32"), (3, 16000, "bf16"), (2, 16384, "f32"),
            (2, 40000, "bf16"), (3, 20000, "f32"), (4, 1001, "f32")]


@pytest.mark.parametrize("m,k,xdt", QA_CASES)
def test_quant_act(B, m, k, xdt):
    log(f"quant_act m={m} k={k} {xdt}")
    _, x = random_case(1000 + m * 7 + k, m, 1, k, x_kind="t3")
    if m > 2:
        x[1] = 0.0                                  # all-zero token
        x[2] = 0.0
        x[2, k // 2] = -3.0                         # single nonzero
    xd, xo = x_device(x, xdt)
    xq, s = B.quant_act(xd)
    xq, s = host(xq), host(s)
    oq, os_ = O.quant_act(xo)
    np.testing.assert_array_equal(s, os_)
    np.testing.assert_array_equal(xq[:, :k], oq)
    assert np.all(xq[:, k:] == 0)
    assert xq.shape[1] == O.padded_k(k)


def test_quant_act_ties(B):
    # x*s lands exactly on k + 0.5 for many elements (beta = 127 -> s = 1)
    x = np.array([[127.0, 2.5, -3.5, 0.5, -0.5, 1.5, 126.5, -126.5] * 32], np.float32)
    xq, s = B.quant_act(dev(x))
    oq, os_ = O.quant_act(x)
    np.testing.assert_array_equal(host(xq)[:, :256], oq)
    np.testing.assert_array_equal(host(s), os_)


def test_quant_act_worked_example(B):
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))["activations"]
    xq, s = B.quant_act(dev(np.array(g["x"], np.float32)))
    np.testing.assert_array_equal(host(xq)[:, :4], np.array(g["xq"], np.int8))
    np.testing.assert_array_equal(host(s), np.array(g["s"], np.float32))


@pytest.mark.parametrize("m", [1, 2, 5, 20])
def test_zero_tokens_at_smallest_eps(B, m):
    """All-zero tokens with the smallest activation eps the ABI accepts:
    s = fp32(127 / eps) is the largest finite fp32 and x~ = 0, y = 0 exactly,
    through bitlinear_quant_act + forward and through the fused step (dot4 at
    1-2 tokens, the matrix cores from 3)."""
    import torch
    from test_oracle_pins import EPS_MIN
    n, k = 192, 1000
    w, x = random_case(4400 + m, m, n, k, x_kind="t3")
    x[0] = 0.0
    if m > 2:
        x[m // 2] = 0.0
    xd, xo = x_device(x, "bf16")
    packed, gamma = B.pack_weights(dev(w))
    g = host(gamma)[0]
    r = O.forward(xo, w, gamma=g, act_eps=EPS_MIN, y_dtype="f32")
    assert r["s"][0] == np.float32(3.4028235e38) and not r["xq"][0].any()
    xq, s = B.quant_act(xd, eps=float(EPS_MIN))
    np.testing.assert_array_equal(host(s), r["s"])
    np.testing.assert_array_equal(host(xq)[:, :k], r["xq"])
    y, acc = B.forward(xq, s, packed, gamma, n, k, acc_out=True)
    np.testing.assert_array_equal(host(acc), r["acc"])
    assert_y_close(host(y), r["y"], "f32", f"zero tokens m={m}")
    assert not host(y)[0].any()
    ops = [dict(x=xd, packed=packed, gamma=gamma, n=n, k=k,
                y=torch.empty((m, n), dtype=torch.float32, device="cuda"),
                acc_out=torch.empty((m, n), dtype=torch.int32, device="cuda"),
                xq_out=torch.full((m, O.padded_k(k)), 99, dtype=torch.int8, device="cuda"),
                scale_out=torch.empty(m, dtype=torch.float32, device="cuda"))]
    B.forward_fused(ops, eps=float(EPS_MIN))
    o = ops[0]
    np.testing.assert_array_equal(host(o["scale_out"]), r["s"])
    np.testing.assert_array_equal(host(o["xq_out"])[:, :k], r["xq"])
    np.testing.assert_array_equal(host(o["acc_out"]), r["acc"])
    assert_y_close(host(o["y"]), r["y"], "f32", f"fused zero tokens m={m}")
    assert not host(o["y"])[0].any()


def test_quant_act_unaligned_pointer(B):
    import torch
    _, x = random_case(5, 3, 1, 100)
    big = dev(np.concatenate([np.zeros(1, np.float32), x.ravel()]))
    xv = big[1:].view(3, 100)                        # 4-byte aligned, not 16
    xq, s = B.quant_act(xv)
    oq, os_ = O.quant_act(x)
    np.testing.assert_array_equal(host(xq)[:, :100], oq)
    np.testing.assert_array_equal(host(s), os_)


# ---------------------------------------------------------------- packing --
PACK_CASES = [(1, 1), (3, 5), (64, 256), (65, 257), (130, 520), (256, 256), (640, 2560),
              (100, 1000), (7, 4097)]


@pytest.mark.parametrize("n,k", PACK_CASES)
def test_pack_gamma_in(B, n, k):
    log(f"pack gamma_in n={n} k={k}")
    w, _ = random_case(2000 + n + k, 1, n, k)
    g = O.absmean_gamma(w)
    packed, gout = B.pack_weights(dev(w), gamma_in=dev(np.array([g], np.float32)))
    ref = O.pack_ternary(O.ternary_codes(w, g))
    np.testing.assert_array_equal(host(packed)[:ref.size], ref)
    assert host(gout)[0] == g


@pytest.mark.parametrize("n,k", PACK_CASES)
def test_pack_gamma_device(B, n, k):
    log(f"pack n={n} k={k}")
    w, _ = random_case(3000 + n + k, 1, n, k)
    packed, gout = B.pack_weights(dev(w))
    g = host(gout)[0]
    assert gamma_agrees(g, w)
    ref = O.pack_ternary(O.ternary_codes(w, np.float32(g)))
    np.testing.assert_array_equal(host(packed), ref)


def test_pack_bf16_weights(B):
    from datagen import to_bf16_bits, bf16_bits_to_f32
    from gpu_util import dev_bf16
    w, _ = random_case(77, 1, 200, 600)
    bits = to_bf16_bits(w)
    wf = bf16_bits_to_f32(bits)
    packed, gout = B.pack_weights(dev_bf16(bits))
    assert gamma_agrees(host(gout)[0], wf)
    np.testing.assert_array_equal(host(packed), O.pack_ternary(O.ternary_codes(wf, host(gout)[0])))


def test_pack_threshold_neighbours(B):
    # weights at and next to every decision point |w|/d = 0.5, 1.5 for a
    # given gamma; eps as on the pages.
    gamma = np.float32(0.015625)
    eps = np.float32(1e-5)
    d = np.float32(gamma + eps)
    pts = []
    for base in (np.float32(d * np.float32(0.5)), np.float32(d * np.float32(1.5)), d / 2, d):
        v = np.float32(base)
        for _ in range(6):
            v = np.nextafter(v, np.float32(-np.inf))
        for _ in range(13):
            pts += [v, -v]
            v = np.nextafter(v, np.float32(np.inf))
    w = np.array(pts, np.float32)
    w = np.resize(w, (4, 256)).astype(np.float32)
    codes = O.ternary_codes(w, gamma, eps)
    assert (codes == 0).any() and (codes != 0).any()
    packed, _ = B.pack_weights(dev(w), eps=float(eps), gamma_in=dev(np.array([gamma], np.float32)))
    np.testing.assert_array_equal(host(packed), O.pack_ternary(codes))


def test_pack_degenerate(B):
    w = np.zeros((70, 300), np.float32)
    packed, g = B.pack_weights(dev(w))
    assert host(g)[0] == 0 and not host(packed).any()
    packed, g = B.pack_weights(dev(w), eps=0.0)
    assert not host(packed).any()
    # the two-readings example: divisor gamma + eps
    w = np.array([[0.4375, -0.4375, 1.0, -1.375]], np.float32)
    packed, g = B.pack_weights(dev(w), eps=0.1875)
    assert host(g)[0] == np.float32(0.8125)
    np.testing.assert_array_equal(O.unpack_ternary(host(packed), 1, 4), [[0, 0, 1, -1]])


# ---------------------------------------------------------------- forward --
FWD_CASES = [
    # m, n, k, relu2, y dtype, x dtype
    # dot4 GEMV (1 and 2 tokens)
    (1, 1, 1, False, "f32", "f32"),
    (1, 256, 256, False, "f32", "f32"),
    (1, 100, 272, True, "bf16", "bf16"),
    (2, 640, 2560, False, "bf16", "bf16"),
    (1, 64, 8192, False, "f32", "bf16"),
    (1, 200, 16384, True, "bf16", "bf16"),
    (1, 20000, 512, False, "bf16", "bf16"),
    (2, 300, 40000, True, "f32", "bf16"),        # split K
    (2, 16448, 4100, True, "bf16", "bf16"),      # >= 256 row blocks: 64-row groups, 4 waves, ragged K
    (40, 1000, 3000, True, "f32", "bf16"),       # 33-64 tokens, <= 64 row blocks: 32-token blocks, the 2nd partial
    (64, 4160, 6400, False, "bf16", "f32"),      # 64 tokens, 65 row blocks, long rows: 64-token blocks, 4 slices
    # streaming matrix-core GEMV (1-2 tokens, >= 1024 rows, x~ within the LDS)
    (1, 1024, 3072, False, "bf16", "bf16"),      # 64 sub-blocks, one per workgroup
    (1, 5000, 12345, True, "f32", "bf16"),       # ragged N and K
    (2, 1030, 2056, False, "bf16", "f32"),       # ragged, 9 super-chunks at two tokens
    (1, 16448, 4100, True, "bf16", "bf16"),      # 1028 sub-blocks over 256 workgroups
    (2, 1088, 32000, False, "f32", "bf16"),      # x~ of two tokens fills the LDS
    (1, 3000, 28672, False, "bf16", "bf16"),     # 16 waves x 3 units in flight
    # 3 to 64 tokens: the multi-token streaming GEMV where x~ of a 16-token
    # block fits the LDS (most of the rows below), else the windowed MFMA
    # GEMV (rows of >= 16384 inputs); the kernel plan tests list which
    # windowed MFMA GEMV, 3 to 16 tokens: 2 row groups x 4 slices
    (3, 130, 520, True, "f32", "f32"),           # 3 super-chunks: an empty slice
    (4, 300, 1000, False, "f32", "bf16"),
    (5, 200, 600, False, "f32", "f32"),
    (16, 256, 512, True, "bf16", "bf16"),
    (12, 1000, 3000, True, "f32", "bf16"),       # ragged row block, vector stores
    (7, 1001, 2560, False, "bf16", "f32"),       # odd N: element stores
    # ... 8 slices (few long rows)
    (4, 100, 30000, False, "f32", "f32"),
    (3, 130, 40000, False, "bf16", "bf16"),
    (4, 70, 65536, False, "f32", "bf16"),
    (8, 2560, 16384, False, "bf16", "bf16"),
    (16, 2048, 8192, True, "bf16", "bf16"),
    # ... wide row groups (>= 256 row blocks), whole K per wave
    (10, 16448, 768, False, "f32", "bf16"),      # 257 blocks: idle groups
    (9, 16450, 1024, True, "bf16", "bf16"),      # odd N: element stores
    (8, 16384, 9000, False, "bf16", "bf16"),     # ragged K
    # ... 17 to 32 tokens (2 token groups)
    (17, 300, 1000, False, "f32", "bf16"),
    (32, 640, 2560, False, "bf16", "bf16"),
    (24, 16448, 1000, True, "bf16", "bf16"),     # wide row groups
    # ... 33 to 64 tokens (4 token groups)
    (33, 100, 257, True, "f32", "f32"),
    (64, 512, 2560, False, "bf16", "bf16"),
    (48, 2000, 7000, True, "bf16", "f32"),       # long rows: 4 K-slices
    (40, 6000, 2000, False, "f32", "bf16"),      # short rows, many blocks: 2 K-slices
    (50, 16400, 700, False, "f32", "bf16"),      # wide row groups
    (64, 16385, 512, True, "bf16", "f32"),       # wide, odd N
    # ... more than 64 tokens with few output tiles: token blocks of 64
    (65, 129, 300, False, "f32", "f32"),         # a last block of 1 token
    (130, 320, 1024, True, "bf16", "bf16"),
    (129, 260, 5000, True, "f32", "bf16"),
    (256, 384, 768, False, "f32", "bf16"),
    (200, 1001, 700, False, "bf16", "f32"),      # odd N: element stores
    (200, 6000, 512, True, "bf16", "bf16"),      # short rows, many blocks
    # multi-token streaming GEMV (long rows of few row blocks past 16-32
    # tokens; x~ of a 16-token block within the LDS): row ranges x blocks
    (33, 2560, 8200, False, "bf16", "bf16"),     # 3 blocks, the last of 1 token; 80 row ranges
    (64, 1030, 8192, False, "f32", "bf16"),      # 128 KiB of x~; N % 4 != 0: element stores
    (20, 100, 8000, True, "bf16", "f32"),        # one row range per sub-block, 2 blocks
    (40, 130, 8100, False, "f32", "bf16"),       # 12 row ranges: not a multiple of 8
    (48, 8192, 9000, True, "bf16", "bf16"),      # x~ staging past 8 units per thread
    (17, 1000, 8192, False, "bf16", "bf16"),     # a last block of 1 token, 64 row ranges
    # ... and larger batches with few output tiles on short rows
    (512, 2560, 2560, True, "bf16", "bf16"),     # 32 token blocks x 8 row ranges
    (1000, 640, 3000, False, "f32", "bf16"),     # a last block of 8 tokens; 4 row ranges (not grouped)
    (300, 2100, 1000, False, "bf16", "f32"),     # 19 token blocks, 8 row ranges (XCD-grouped)
    # wide-wave MFMA GEMM (more than 64 tokens, >= 128 tiles)
    (1000, 6100, 300, True, "bf16", "bf16"),     # 64 x 512 tiles, ragged M, N, K
    (1024, 6144, 512, False, "f32", "bf16"),     # 64 x 512, vector stores
    (256, 8192, 768, False, "bf16", "f32"),      # 64 x 256
    (1100, 9001, 300, True, "bf16", "bf16"),     # 64 x 256, ragged M, odd N
    (1536, 10240, 300, True, "bf16", "bf16"),    # 128 x 512 tiles
    (2000, 2560, 320, False, "bf16", "bf16"),    # 96 x 256 tiles, ragged M
    (1000, 6200, 300, True, "bf16", "bf16"),     # whole-line bf16 rows, a column-tail wave
    (1500, 4104, 520, False, "bf16", "f32"),     # whole lines, 8-column tail
]


def _forward_case(B, m, n, k, relu2, ydt, xdt, seed):
    import torch
    w, x = random_case(seed, m, n, k, x_kind="t3")
    if m > 3:
        x[3] = 0.0
    xd, xo = x_device(x, xdt)
    packed, gamma = B.pack_weights(dev(w))
    xq, s = B.quant_act(xd)
    y, acc = B.forward(xq, s, packed, gamma, n, k, relu2=relu2,
                       out_dtype=torch.bfloat16 if ydt == "bf16" else torch.float32, acc_out=True)
    g = host(gamma)[0]
    assert gamma_agrees(g, w)
    r = O.forward(xo, w, relu2=relu2, y_dtype=ydt, gamma=g)
    np.testing.assert_array_equal(host(acc), r["acc"])
    assert_y_close(host(y), r["y"], ydt, f"m={m} n={n} k={k}")


@pytest.mark.parametrize("m,n,k,relu2,ydt,xdt", FWD_CASES)
def test_forward(B, m, n, k, relu2, ydt, xdt):
    log(f"forward m={m} n={n} k={k} relu2={relu2} y={ydt} x={xdt}")
    _forward_case(B, m, n, k, relu2, ydt, xdt, seed=m * 1000003 + n * 101 + k)


def test_forward_worked_example(B):
    import json, os
    import torch
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))
    w = np.array(gold["weights_basic"]["w"], np.float32)
    x = np.array(gold["activations"]["x"], np.float32)
    f = gold["forward"]
    packed, gamma = B.pack_weights(dev(w))
    xq, s = B.quant_act(dev(x))
    y, acc = B.forward(xq, s, packed, gamma, 2, 4, acc_out=True)
    np.testing.assert_array_equal(host(acc), f["acc"])
    np.testing.assert_array_equal(host(y), np.array(f["y_f32"], np.float32))
    y2 = B.forward(xq, s, packed, gamma, 2, 4, relu2=True)
    np.testing.assert_array_equal(host(y2), np.array(f["y_relu2_f32"], np.float32))
    yb = B.forward(xq, s, packed, gamma, 2, 4, out_dtype=torch.bfloat16)
    np.testing.assert_array_equal(O.bf16_bits_to_f32(host(yb)), np.array(f["y_bf16"], np.float32))


def test_forward_extreme_accumulator(B):
    # every code +1 or -1 against full-scale activations: |acc| = 127*K
    import torch
    k = 8192
    w = np.ones((64, k), np.float32)
    w[1::2] *= -1
    x = np.full((3, k), 5.0, np.float32)
    x[1] *= -1
    packed, gamma = B.pack_weights(dev(w))
    xq, s = B.quant_act(dev(x))
    _, acc = B.forward(xq, s, packed, gamma, 64, k, acc_out=True)
    a = host(acc)
    assert a[0, 0] == 127 * k and a[0, 1] == -127 * k and a[1, 0] == -127 * k
    xq5, s5 = B.quant_act(dev(np.tile(x, (3, 1))))
    _, acc5 = B.forward(xq5, s5, packed, gamma, 64, k, acc_out=True)
    assert host(acc5)[0, 0] == 127 * k and host(acc5)[4, 0] == -127 * k


def test_forward_deterministic_and_workspace_clean(B):
    import torch
    # rows too long for the streaming kernel's LDS (157 super-chunks at two
    # tokens): the dot4 GEMV splits K over workgroups
    w, x = random_case(9, 2, 2560, 40000)
    packed, gamma = B.pack_weights(dev(w))
    xq, s = B.quant_act(dev(x))
    ws = B.Workspace()
    outs = [host(B.forward(xq, s, packed, gamma, 2560, 40000, workspace=ws)) for _ in range(3)]
    assert B.forward_workspace_bytes(2, 2560, 40000) > 0
    np.testing.assert_array_equal(outs[0], outs[1])
    np.testing.assert_array_equal(outs[0], outs[2])
    torch.cuda.synchronize()
    assert not host(ws.buf).any(), "workspace not left zero-filled"
    r = O.forward(x, w, gamma=host(gamma)[0])
    from gpu_util import assert_y_close
    assert_y_close(outs[2], r["y"], "f32")


def test_workspace_shared_across_paths(B):
    # split-K GEMV calls of different shapes, with calls that use no
    # workspace between them, share one workspace; every call must find it
    # zero-filled and leave it so.
    import torch
    ws = B.Workspace()
    cases = [(1, 64, 16384), (2, 300, 40000), (70, 129, 5000), (2, 64, 16384), (1, 200, 16384),
             (8, 256, 8192), (1, 64, 16384)]
    for (m, n, k) in cases:
        assert (B.forward_workspace_bytes(m, n, k) > 0) == (m <= 2), (m, n, k)
        w, x = random_case(m * 7 + n + k, m, n, k, x_kind="t3")
        packed, gamma = B.pack_weights(dev(w))
        xq, s = B.quant_act(dev(x))
        y, acc = B.forward(xq, s, packed, gamma, n, k, workspace=ws, acc_out=True)
        r = O.forward(x, w, gamma=host(gamma)[0])
        np.testing.assert_array_equal(host(acc), r["acc"], err_msg=str((m, n, k)))
        torch.cuda.synchronize()
        assert not host(ws.buf).any(), f"workspace not clean after {(m, n, k)}"


def test_forward_no_write_past_output(B):
    import torch
    for (m, n, k) in [(1, 100, 300), (20, 70, 300), (130, 200, 512)]:
        w, x = random_case(m + n, m, n, k)
        packed, gamma = B.pack_weights(dev(w))
        xq, s = B.quant_act(dev(x))
        buf = torch.full((m * n + 4096,), -7.0, dtype=torch.float32, device="cuda")
        y = buf[: m * n].view(m, n)
        B.forward(xq, s, packed, gamma, n, k, y=y)
        assert torch.all(buf[m * n:] == -7.0).item()
        r = O.forward(x, w, gamma=host(gamma)[0])
        assert_y_close(host(y), r["y"], "f32")


def test_gemm_bf16_lines_stay_inside_output(B):
    # bf16 rows leave the GEMM as whole 16-byte pieces; nothing past the
    # output (ragged M and N) may change
    import torch
    for (m, n, k) in [(1000, 6200, 300), (1100, 8192, 256)]:
        w, x = random_case(m + n + 1, m, n, k, x_kind="t3")
        packed, gamma = B.pack_weights(dev(w))
        xq, s = B.quant_act(dev(x))
        buf = torch.full((m * n + 8192,), -7.0, dtype=torch.bfloat16, device="cuda")
        y = buf[: m * n].view(m, n)
        B.forward(xq, s, packed, gamma, n, k, y=y, relu2=True)
        assert torch.all(buf[m * n:] == -7.0).item()
        r = O.forward(x, w, relu2=True, y_dtype="bf16", gamma=host(gamma)[0])
        assert_y_close(host(y), r["y"], "bf16", f"m={m} n={n}")


MULTI_CASES = [
    # m, k, [(n, relu2, y dtype)]
    (1024, 512, [(4096, True, "bf16"), (1000, False, "f32"), (640, False, "bf16")]),   # one GEMM
    (300, 1000, [(130, True, "bf16"), (2560, False, "bf16"), (6000, True, "f32")]),   # ragged
    (1024, 256, [(512, i % 2 == 1, "bf16" if i % 3 else "f32") for i in range(16)]),  # 16 entries
    (3, 2560, [(2560, False, "bf16"), (640, False, "bf16"), (640, False, "bf16")]),   # one by one
    (1, 16384, [(200, False, "f32"), (64, True, "bf16")]),                           # split K
]


@pytest.mark.parametrize("m,k,specs", MULTI_CASES)
def test_forward_multi_matches_forward(B, m, k, specs):
    # the same numbers as one bitlinear_forward per entry, bit for bit
    import torch
    log(f"forward_multi m={m} k={k} entries={len(specs)}")
    _, x = random_case(m * 7 + k, m, 1, k, x_kind="t3")
    xq, s = B.quant_act(x_device(x, "bf16")[0])
    ops, refs = [], []
    for i, (n, relu2, ydt) in enumerate(specs):
        w, _ = random_case(1000 + 31 * i + n, 1, n, k)
        packed, gamma = B.pack_weights(dev(w))
        dt = torch.bfloat16 if ydt == "bf16" else torch.float32
        ops.append(dict(packed=packed, gamma=gamma, n=n, relu2=relu2,
                        y=torch.empty((m, n), dtype=dt, device="cuda"),
                        acc_out=torch.empty((m, n), dtype=torch.int32, device="cuda")))
        refs.append(B.forward(xq, s, packed, gamma, n, k, relu2=relu2, out_dtype=dt,
                              acc_out=True))
    B.forward_multi(xq, s, k, ops)
    for i, (o, (y, acc)) in enumerate(zip(ops, refs)):
        np.testing.assert_array_equal(host(o["acc_out"]), host(acc), err_msg=f"acc of entry {i}")
        np.testing.assert_array_equal(host(o["y"].view(torch.int16 if o["y"].dtype == torch.bfloat16
                                                       else torch.int32)),
                                      host(y.view(torch.int16 if y.dtype == torch.bfloat16
                                                  else torch.int32)), err_msg=f"y of entry {i}")


def test_forward_multi_against_oracle(B):
    # a table that runs as one GEMM launch, checked against the oracle
    m, k = 520, 300
    specs = [(3000, True, "bf16"), (136, False, "f32"), (4100, False, "bf16")]
    assert B.lib.bitlinear_forward_multi_workspace_bytes(
        (B.BLProduct * 3)(*[B.BLProduct(n=n) for (n, _, _) in specs]), 3, m, k) == 0
    _, x = random_case(77, m, 1, k, x_kind="t3")
    xd, xo = x_device(x, "f32")
    xq, s = B.quant_act(xd)
    import torch
    ops, ws = [], []
    for i, (n, relu2, ydt) in enumerate(specs):
        w, _ = random_case(500 + i, 1, n, k)
        packed, gamma = B.pack_weights(dev(w))
        dt = torch.bfloat16 if ydt == "bf16" else torch.float32
        ops.append(dict(packed=packed, gamma=gamma, n=n, relu2=relu2,
                        y=torch.empty((m, n), dtype=dt, device="cuda"),
                        acc_out=torch.empty((m, n), dtype=torch.int32, device="cuda")))
        ws.append(w)
    B.forward_multi(xq, s, k, ops)
    for i, (o, w, (n, relu2, ydt)) in enumerate(zip(ops, ws, specs)):
        g = host(o["gamma"])[0]
        r = O.forward(xo, w, relu2=relu2, y_dtype=ydt, gamma=g)
        np.testing.assert_array_equal(host(o["acc_out"]), r["acc"], err_msg=f"entry {i}")
        assert_y_close(host(o["y"]), r["y"], ydt, f"entry {i}")


def test_forward_empty_batch(B):
    import torch
    w, _ = random_case(1, 1, 64, 256)
    packed, gamma = B.pack_weights(dev(w))
    xq = torch.empty((0, 256), dtype=torch.int8, device="cuda")
    s = torch.empty(0, dtype=torch.float32, device="cuda")
    y = B.forward(xq, s, packed, gamma, 64, 256)
    assert y.shape == (0, 64)


def test_graph_replays_match_eager(B):
    # captured launches (a split-K GEMV with its workspace, a fused decode
    # step, a GEMM table) replayed several times, with eager work between
    # the replays, give the eager bits every time
    import torch
    w1, x1 = random_case(11, 1, 300, 40000)            # dot4 GEMV, split K
    p1, g1 = B.pack_weights(dev(w1))
    xq1, s1 = B.quant_act(dev(x1))
    w2, x2 = random_case(12, 1, 640, 2560, x_kind="t3")
    p2, g2 = B.pack_weights(dev(w2))
    x2d = x_device(x2, "bf16")[0]
    _, x3 = random_case(13, 600, 1, 512, x_kind="t3")
    xq3, s3 = B.quant_act(dev(x3))
    mats3 = [B.pack_weights(dev(random_case(14 + i, 1, n, 512)[0])) for i, n in
             enumerate((4096, 640, 1000))]
    ws = B.Workspace()
    y1 = torch.empty((1, 300), dtype=torch.float32, device="cuda")
    y2 = torch.empty((1, 640), dtype=torch.bfloat16, device="cuda")
    y3 = [torch.empty((600, n), dtype=torch.bfloat16, device="cuda") for n in (4096, 640, 1000)]
    step = B.FusedStep([dict(x=x2d, packed=p2, gamma=g2, n=640, k=2560, y=y2)], workspace=ws)
    ops3 = [dict(packed=p, gamma=g, n=n, y=y, relu2=(i == 0))
            for i, ((p, g), n, y) in enumerate(zip(mats3, (4096, 640, 1000), y3))]

    def work():
        B.forward(xq1, s1, p1, g1, 300, 40000, y=y1, workspace=ws)
        step()
        B.forward_multi(xq3, s3, 512, ops3, workspace=ws)

    work()
    torch.cuda.synchronize()
    ref = [t.clone() for t in [y1, y2] + y3]
    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        work()                                         # warm on the capture stream
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        work()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in [y1, y2] + y3:
            t.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip([y1, y2] + y3, ref)):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)), \
                f"replay {rep}, output {i}"
        work()                                         # eager work between replays
        torch.cuda.synchronize()
    assert not host(ws.buf).any(), "workspace not left zero-filled"


def test_graph_replays_match_eager_batched(B):
    # the batched-decode kernels under graph capture: a fused step on the
    # multi-token streaming kernel (8 tokens, shared input), a plain product
    # on it (48 tokens, long rows), one on the windowed MFMA GEMV (16
    # tokens) and a two-pass fused step (4 tokens, rows of 9000 bf16, shared
    # input: quantization, two products and the scratch fill in the graph),
    # replayed with eager work between the replays, against the eager bits
    # and the oracle; the workspace stays zero-filled
    import torch
    assert B.forward_kernel(48, 1030, 8192) == "stream_mt"
    assert B.forward_kernel(16, 2560, 2560) == "mfma_gemv"
    mats = {name: random_case(20 + i, 1, n, k)[0] for i, (name, n, k) in
            enumerate((("q", 2560, 2560), ("k", 640, 2560), ("mt", 1030, 8192), ("win", 2560, 2560),
                       ("tp1", 300, 9000), ("tp2", 200, 9000)))}
    packed = {nm: B.pack_weights(dev(w)) for nm, w in mats.items()}
    _, x8 = random_case(30, 8, 1, 2560, x_kind="t3")
    x8d = x_device(x8, "bf16")[0]
    _, x48 = random_case(31, 48, 1, 8192, x_kind="t3")
    xq48, s48 = B.quant_act(dev(x48))
    _, x16 = random_case(32, 16, 1, 2560, x_kind="t3")
    xq16, s16 = B.quant_act(dev(x16))
    _, x4 = random_case(33, 4, 1, 9000, x_kind="t3")
    x4d, x4o = x_device(x4, "bf16")
    ys = {"q": torch.empty((8, 2560), dtype=torch.bfloat16, device="cuda"),
          "k": torch.empty((8, 640), dtype=torch.bfloat16, device="cuda"),
          "mt": torch.empty((48, 1030), dtype=torch.float32, device="cuda"),
          "win": torch.empty((16, 2560), dtype=torch.bfloat16, device="cuda"),
          "tp1": torch.empty((4, 300), dtype=torch.bfloat16, device="cuda"),
          "tp2": torch.empty((4, 200), dtype=torch.float32, device="cuda")}
    ws = B.Workspace()
    step = B.FusedStep([dict(x=x8d, packed=packed[nm][0], gamma=packed[nm][1], n=n, k=2560,
                             y=ys[nm], relu2=(nm == "k")) for nm, n in (("q", 2560), ("k", 640))],
                       workspace=ws)
    assert step.kernel() == "stream_mt"
    step2 = B.FusedStep([dict(x=x4d, packed=packed[nm][0], gamma=packed[nm][1], n=n, k=9000,
                              y=ys[nm], relu2=(nm == "tp2")) for nm, n in (("tp1", 300), ("tp2", 200))],
                        workspace=ws)
    assert step2.kernel() == "two_pass" and step2.nbytes > 0

    def work():
        step()
        step2()
        B.forward(xq48, s48, packed["mt"][0], packed["mt"][1], 1030, 8192, y=ys["mt"], workspace=ws)
        B.forward(xq16, s16, packed["win"][0], packed["win"][1], 2560, 2560, relu2=True,
                  y=ys["win"], workspace=ws)

    work()
    torch.cuda.synchronize()
    ref = {nm: t.clone() for nm, t in ys.items()}
    # the eager results against the oracle
    x8o = x_device(x8, "bf16")[1]                      # the bf16 values x8d holds
    for nm, xo, relu2, ydt in (("q", x8o, False, "bf16"), ("k", x8o, True, "bf16"),
                               ("mt", x48, False, "f32"), ("win", x16, True, "bf16"),
                               ("tp1", x4o, False, "bf16"), ("tp2", x4o, True, "f32")):
        g = host(packed[nm][1])[0]
        r = O.forward(xo, mats[nm], relu2=relu2, y_dtype=ydt, gamma=g)
        assert_y_close(host(ref[nm]), r["y"], ydt, f"eager {nm}")
    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        work()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=stream):
        work()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in ys.values():
            t.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        for nm, t in ys.items():
            a, b = (t.view(torch.int16), ref[nm].view(torch.int16)) if t.dtype == torch.bfloat16 \
                else (t.view(torch.int32), ref[nm].view(torch.int32))
            assert torch.equal(a, b), f"replay {rep}, {nm}"
        assert not host(ws.buf).any(), f"replay {rep}: workspace left non-zero"
        work()
        torch.cuda.synchronize()
