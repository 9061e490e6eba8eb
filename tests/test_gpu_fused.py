"""GPU parity of the fused decode step (bitlinear_forward_fused): activation
quantization in the kernel prologue plus the GEMV for several matrices in one
launch, against the CPU oracle and against the unfused entry points."""
import numpy as np
import pytest

import oracle as O
from datagen import random_case
from gpu_util import assert_y_close, dev, gamma_agrees, host, log, x_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_gemm_int8_amd as B
    return B


def _entries(B, specs, m, seed, shared_x=False):
    """specs: list of (n, k, relu2, ydt, xdt).  Returns (ops, refs)."""
    import torch
    ops, refs = [], []
    xs = {}
    for i, (n, k, relu2, ydt, xdt) in enumerate(specs):
        w, x = random_case(seed + 97 * i, m, n, k, x_kind="t3")
        key = (k, xdt)
        if shared_x and key in xs:
            xd, xo = xs[key]
        else:
            if m > 2:
                x[1] = 0.0
            xd, xo = x_device(x, xdt)
            xs[key] = (xd, xo)
        packed, gamma = B.pack_weights(dev(w))
        y = torch.empty((m, n), dtype=torch.bfloat16 if ydt == "bf16" else torch.float32,
                        device="cuda")
        ops.append(dict(x=xd, packed=packed, gamma=gamma, n=n, k=k, y=y, relu2=relu2,
                        acc_out=torch.empty((m, n), dtype=torch.int32, device="cuda"),
                        xq_out=torch.full((m, O.padded_k(k)), 99, dtype=torch.int8, device="cuda"),
                        scale_out=torch.empty(m, dtype=torch.float32, device="cuda")))
        refs.append((w, xo, relu2, ydt))
    return ops, refs


def _check(B, ops, refs):
    for i, (o, (w, xo, relu2, ydt)) in enumerate(zip(ops, refs)):
        g = host(o["gamma"])[0]
        assert gamma_agrees(g, w)
        r = O.forward(xo, w, relu2=relu2, y_dtype=ydt, gamma=g)
        k = o["k"]
        xq = host(o["xq_out"])
        np.testing.assert_array_equal(xq[:, :k], r["xq"], err_msg=f"x~ of entry {i}")
        assert np.all(xq[:, k:] == 0)
        np.testing.assert_array_equal(host(o["scale_out"]), r["s"])
        np.testing.assert_array_equal(host(o["acc_out"]), r["acc"], err_msg=f"acc of entry {i}")
        assert_y_close(host(o["y"]), r["y"], ydt, f"entry {i}")


FUSED_CASES = [
    (1, [(256, 256, False, "f32", "f32")]),
    (1, [(100, 272, True, "bf16", "bf16"), (640, 2560, False, "bf16", "bf16"),
         (70, 1000, False, "f32", "f32")]),
    (2, [(300, 1000, False, "f32", "bf16"), (64, 8192, True, "bf16", "bf16")]),
    (3, [(130, 522, False, "f32", "f32"), (200, 16384, False, "bf16", "bf16")]),   # K % 4 != 0
    (4, [(129, 300, True, "f32", "bf16"), (64, 30000, False, "bf16", "f32"),
         (1000, 777, False, "bf16", "bf16")]),
    (1, [(64, 256, False, "f32", "f32")] * 16),
    (1, [(100, 20000, True, "bf16", "bf16")]),                                     # long row, split K, 16-row groups
    (1, [(2560, 2560, False, "bf16", "bf16"), (6912, 2560, True, "bf16", "bf16"),
         (2560, 6912, False, "bf16", "bf16")]),                                     # 64-row groups
    # the streaming matrix-core kernel: fp32 activations, ragged N, entries of
    # one workgroup, two tokens
    (1, [(1000, 4096, False, "f32", "f32"), (70, 2048, True, "bf16", "f32")]),
    (2, [(2000, 3000, True, "bf16", "f32"), (1040, 8192, False, "f32", "f32")]),
    (2, [(8192, 8192, False, "bf16", "bf16"), (1024, 8192, False, "bf16", "bf16"),
         (1024, 8192, False, "bf16", "bf16")]),
    (2, [(1040, 28672, False, "bf16", "bf16"), (300, 4096, True, "bf16", "bf16")]),  # 16 waves: rows past 8 waves' registers
    # 3 to 16 tokens: int8 matrix cores
    (8, [(2560, 2560, False, "bf16", "bf16"), (640, 2560, False, "bf16", "bf16"),
         (6912, 2560, True, "bf16", "bf16")]),                                        # all bf16
    (16, [(300, 1000, True, "f32", "bf16"), (64, 8200, False, "bf16", "bf16")]),    # K % 16 != 0
    (12, [(500, 777, False, "bf16", "f32"), (129, 300, True, "f32", "bf16")]),     # odd K, mixed x
    (5, [(16400, 512, False, "bf16", "bf16")]),                                    # >= 256 row blocks
    (9, [(64, 64, False, "f32", "f32"), (65, 320, True, "bf16", "bf16")]),         # empty K-slices
    (16, [(64, 256, False, "f32", "f32")] * 16),
    # 17 to 64 tokens: token blocks of 16
    (17, [(300, 1000, True, "f32", "bf16"), (64, 8200, False, "bf16", "bf16")]),    # a block of 1
    (40, [(2560, 2560, False, "bf16", "bf16"), (640, 2560, False, "bf16", "bf16")]),
    (64, [(500, 777, False, "bf16", "f32"), (16400, 512, True, "bf16", "bf16")]),  # >= 256 row blocks
    # the multi-token streaming kernel (rows of whole aligned 16-byte units,
    # one activation dtype, a row within 16 units per lane)
    (64, [(2560, 6912, False, "bf16", "bf16")]),                                   # 14 units per lane
    (33, [(1000, 4096, True, "f32", "f32"), (70, 2048, False, "bf16", "f32")]),    # fp32 x, 16 units
    (3, [(64, 256, False, "f32", "bf16")] * 3),
    (50, [(2560, 2560, False, "bf16", "bf16"), (640, 2560, False, "bf16", "bf16"),
          (640, 2560, True, "bf16", "bf16")]),                                      # a block of 2
]


@pytest.mark.parametrize("m,specs", FUSED_CASES)
def test_fused_vs_oracle(B, m, specs):
    log(f"fused m={m} entries={len(specs)}")
    ops, refs = _entries(B, specs, m, seed=m * 31 + len(specs))
    B.forward_fused(ops)
    _check(B, ops, refs)


def test_fused_shared_inputs_and_unfused_agree(B):
    import torch
    m = 1
    specs = [(2560, 2560, False, "bf16", "bf16"), (640, 2560, False, "bf16", "bf16"),
             (640, 2560, False, "bf16", "bf16"), (6912, 2560, True, "bf16", "bf16")]
    ops, refs = _entries(B, specs, m, seed=5, shared_x=True)
    ws = B.Workspace()
    B.forward_fused(ops, workspace=ws)
    _check(B, ops, refs)
    for o in ops:
        xq, s = B.quant_act(o["x"])
        y = B.forward(xq, s, o["packed"], o["gamma"], o["n"], o["k"], relu2=o["relu2"],
                      out_dtype=o["y"].dtype)
        assert torch.equal(y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32),
                           o["y"].view(torch.int16) if y.dtype == torch.bfloat16 else o["y"].view(torch.int32))
    torch.cuda.synchronize()
    assert ws.buf is None or not host(ws.buf).any()


@pytest.mark.parametrize("m", [1, 8])
def test_fused_c2_decode_set(B, m):
    """The decode set at 2B-class shapes, full size, one launch (1 token: the
    dot4 kernel; 8 tokens: the matrix cores)."""
    import torch
    import datagen
    wl = datagen.WORKLOADS["c2"]
    ops, refs = [], []
    xin = {}
    for g in wl.groups():
        bits, _ = datagen.activations(wl, g, m)
        from gpu_util import dev_bf16
        xin[g] = (dev_bf16(bits), datagen.bf16_bits_to_f32(bits))
    for name, (n, k, relu2, grp) in wl.matrices.items():
        w = datagen.workload_weights(wl, name)
        packed, gamma = B.pack_weights(dev(w))
        ops.append(dict(x=xin[grp][0], packed=packed, gamma=gamma, n=n, k=k, relu2=relu2,
                        y=torch.empty((m, n), dtype=torch.bfloat16, device="cuda"),
                        acc_out=torch.empty((m, n), dtype=torch.int32, device="cuda"),
                        xq_out=torch.empty((m, O.padded_k(k)), dtype=torch.int8, device="cuda"),
                        scale_out=torch.empty(m, dtype=torch.float32, device="cuda")))
        refs.append((w, xin[grp][1], relu2, "bf16"))
    step = B.FusedStep(ops)
    for _ in range(3):                      # repeated calls reuse the workspace
        step()
    _check(B, ops, refs)


def _extreme_rows(m, k, seed):
    """bf16 bit patterns [m, k] of t3 activations with rows whose magnitudes
    test the fused prologue's absmax: above 2^121 (past what fp16 orders:
    the exact path), exactly 2^121 (fp16's infinity pattern), all in fp16's
    denormal range (below 2^-119, with a max above the smallest eps), signed
    zeros, and a negative max in the last unit of the row."""
    from datagen import to_bf16_bits
    rng = np.random.default_rng(seed)
    _, x = random_case(seed, m, 1, k, x_kind="t3")
    bits = to_bf16_bits(x)
    kinds = ["above", "tiny", "at", "above_neg", "zeros", "last"]
    for i in range(m):
        kind = kinds[i % len(kinds)] if i < 2 * len(kinds) else "plain"
        j = int(rng.integers(0, k))
        if kind == "above":
            bits[i, j] = 0x7C01
        elif kind == "at":
            bits[i, j] = 0xFC00                         # -2^121
        elif kind == "above_neg":
            bits[i, j] = 0xFC80                         # -2^122
        elif kind == "tiny":
            bits[i] = rng.integers(0, 1 << 16, k).astype(np.uint16) & 0x83FF
            bits[i, j] = 0x03F0                         # ~1.4e-36, above the smallest eps
        elif kind == "zeros":
            bits[i] = np.where(rng.integers(0, 2, k) == 1, 0x8000, 0x0000).astype(np.uint16)
            bits[i, j] = 0xBF80                         # -1
        elif kind == "last":
            bits[i, k - 1] = 0xC2F0                     # -120, in the row's last unit
    return bits


@pytest.mark.parametrize("xdt", ["bf16", "f32"])
@pytest.mark.parametrize("m", [1, 2, 5, 16, 40])
def test_fused_absmax_extremes(B, m, xdt):
    """The fused prologue's absmax (fp16 maximum of bf16 pairs with its
    exact fallback, fp32 max3 of magnitudes) against the oracle on extreme
    rows, at 1-2 tokens (streaming kernel) and 3-64 (multi-token kernel),
    with the smallest activation eps the ABI accepts."""
    import torch
    from datagen import bf16_bits_to_f32
    from test_oracle_pins import EPS_MIN
    n, k = 1040, 1024
    bits = _extreme_rows(m, k, 7100 + m)
    xo = bf16_bits_to_f32(bits)
    xd = dev(bits.view(np.int16)).view(torch.bfloat16) if xdt == "bf16" else dev(xo)
    w, _ = random_case(7200 + m, 1, n, k)
    packed, gamma = B.pack_weights(dev(w))
    g = host(gamma)[0]
    ops = [dict(x=xd, packed=packed, gamma=gamma, n=n, k=k,
                y=torch.empty((m, n), dtype=torch.float32, device="cuda"),
                acc_out=torch.empty((m, n), dtype=torch.int32, device="cuda"),
                xq_out=torch.full((m, O.padded_k(k)), 99, dtype=torch.int8, device="cuda"),
                scale_out=torch.empty(m, dtype=torch.float32, device="cuda"))]
    step = B.FusedStep(ops, eps=float(EPS_MIN))
    log(f"absmax extremes m={m} x={xdt} kernel={step.kernel()}")
    step()
    r = O.forward(xo, w, gamma=g, act_eps=EPS_MIN, y_dtype="f32")
    o = ops[0]
    np.testing.assert_array_equal(host(o["scale_out"]), r["s"])
    np.testing.assert_array_equal(host(o["xq_out"])[:, :k], r["xq"])
    np.testing.assert_array_equal(host(o["acc_out"]), r["acc"])
    assert_y_close(host(o["y"]), r["y"], "f32", f"extremes m={m} {xdt}")


@pytest.mark.parametrize("m", [3, 16, 64])
def test_two_pass_shared_inputs_and_workspace(B, m):
    """Tables with an activation row of more than 16 KiB at 3 or more tokens
    (the two-pass plan): entries that share an input and ask for no x~ read
    one quantization from the workspace scratch, an entry with xq_out and
    scale_out gets its own, RMSNorm entries with a gain run the normalizing
    quantization.  Every output against the oracle; the workspace is all
    zeros after the step, and a split-K forward that reuses it stays exact."""
    import torch
    from test_gpu_norm import check_norm_quant
    k1, k2 = 9000, 5000
    _, x1 = random_case(8100 + m, m, 1, k1, x_kind="t3")
    x1[m // 2] = 0.0
    _, x2 = random_case(8200 + m, m, 1, k2, x_kind="t3")
    x1d, x1o = x_device(x1, "bf16")
    x2d, x2o = x_device(x2, "f32")
    gain = (np.random.default_rng(m).random(k2, dtype=np.float32) + 0.5).astype(np.float32)
    gd = dev(gain)
    neps = 2.0 ** -23
    # (input, n, relu2, y dtype, outputs asked for)
    specs = [(1, 700, False, "bf16", False), (1, 130, True, "f32", False),
             (1, 2100, False, "bf16", False), (2, 640, False, "f32", True),
             (1, 300, True, "bf16", True), (2, 96, False, "bf16", False)]
    ops, ws_w = [], []
    for i, (src, n, relu2, ydt, outs) in enumerate(specs):
        k = k1 if src == 1 else k2
        w, _ = random_case(8300 + 31 * i + m, 1, n, k)
        packed, gamma = B.pack_weights(dev(w))
        o = dict(x=x1d if src == 1 else x2d, packed=packed, gamma=gamma, n=n, k=k, relu2=relu2,
                 y=torch.empty((m, n), dtype=torch.bfloat16 if ydt == "bf16" else torch.float32,
                               device="cuda"),
                 acc_out=torch.empty((m, n), dtype=torch.int32, device="cuda"))
        if src == 2:
            o.update(rmsnorm=True, norm_weight=gd, norm_eps=neps)
        if outs:
            o.update(xq_out=torch.full((m, O.padded_k(k)), 99, dtype=torch.int8, device="cuda"),
                     scale_out=torch.empty(m, dtype=torch.float32, device="cuda"))
        ops.append(o)
        ws_w.append(w)
    ws = B.Workspace()
    step = B.FusedStep(ops, workspace=ws)
    assert step.kernel() == "two_pass" and step.nbytes > 0
    log(f"two-pass m={m} workspace={step.nbytes}")
    for rep in range(2):
        step()
        torch.cuda.synchronize()
        assert not host(ws.buf[:step.nbytes]).any(), "workspace left non-zero"
        # the RMSNorm input: its own outputs (entry 3) against the oracle
        xq3, s3 = host(ops[3]["xq_out"]), host(ops[3]["scale_out"])
        check_norm_quant(x2o, gain, neps, xq3, s3, f"two-pass m={m} norm")
        r1 = O.forward(x1o, ws_w[4], gamma=host(ops[4]["gamma"])[0])
        np.testing.assert_array_equal(host(ops[4]["xq_out"])[:, :k1], r1["xq"])
        np.testing.assert_array_equal(host(ops[4]["scale_out"]), r1["s"])
        for i, (src, n, relu2, ydt, outs) in enumerate(specs):
            g = host(ops[i]["gamma"])[0]
            assert gamma_agrees(g, ws_w[i])
            codes = O.ternary_codes(ws_w[i], g)
            xq = r1["xq"] if src == 1 else xq3[:, :k2]
            sv = r1["s"] if src == 1 else s3
            acc = O.contract(xq, codes)
            np.testing.assert_array_equal(host(ops[i]["acc_out"]), acc, err_msg=f"entry {i}")
            yo = O.round_output(O.dequant(acc, g, sv, relu2), ydt)
            assert_y_close(host(ops[i]["y"]), yo, ydt, f"two-pass m={m} entry {i} rep {rep}")
    # the same workspace then serves a split-K product
    n5, k5 = 200, 20000
    assert B.forward_workspace_bytes(1, n5, k5) > 0
    w5, x5 = random_case(8400 + m, 1, n5, k5, x_kind="t3")
    packed5, gamma5 = B.pack_weights(dev(w5))
    xq5, s5 = B.quant_act(dev(x5))
    y5, acc5 = B.forward(xq5, s5, packed5, gamma5, n5, k5, acc_out=True, workspace=ws)
    r5 = O.forward(x5, w5, gamma=host(gamma5)[0])
    np.testing.assert_array_equal(host(acc5), r5["acc"])


def test_fused_rejects(B):
    import torch
    m = B.BL_FUSED_MAX_M + 1
    x = torch.zeros((m, 256), dtype=torch.float32, device="cuda")
    packed, gamma = B.pack_weights(torch.zeros((64, 256), dtype=torch.float32, device="cuda"))
    y = torch.empty((m, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(B.BitLinearError) as e:
        B.forward_fused([dict(x=x, packed=packed, gamma=gamma, n=64, k=256, y=y)])
    assert e.value.status == 2        # m above the limit
