"""GPU parity of the RMSNorm ahead of the activation quantization (the
BitLinear listing of "BitNet b1.58 2B4T Guide", section "End-to-End
Implementation: Building a Native BitLinear Layer": nn.RMSNorm before
quantize_activations_int8), through bitlinear_rmsnorm_quant_act and through
the fused decode step (streaming kernel at 1-2 tokens, matrix-core kernel at
3-64 tokens and for tables the streaming kernel does not take).

x~ and s are compared bit for bit with the oracle.  The device sums x^2 in
fp64 in its own fixed order; the oracle takes the exactly rounded sum.  The
two give the same fp32 mean square unless the exact mean lies within the
fp64 summation error (at most 2 K 2^-53 relative for positive terms) of an
fp32 rounding boundary; for such a token either neighbour is a correct
result, and the test accepts the oracle's outputs for either."""
import math

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


def ms_candidates(xo):
    """Per token: the oracle's fp32 mean square, and the other fp32 value a
    correct fp64 summation may round to (None when the rounding is robust)."""
    k = xo.shape[1]
    base, other = [], []
    for row in np.asarray(xo, np.float32):
        d = row.astype(np.float64)
        s = math.fsum((d * d).tolist())
        ms = np.float32(s / k)
        rel = 4.0 * k * 2.0 ** -53
        alts = {np.float32(s * (1 - rel) / k), np.float32(s * (1 + rel) / k)} - {ms}
        base.append(ms)
        other.append(alts.pop() if alts else None)
    return np.array(base, np.float32), other


def check_norm_quant(xo, gain, norm_eps, xq, s, where):
    """x~ [m, >= k] and s [m] from the device against the oracle."""
    k = xo.shape[1]
    ms, other = ms_candidates(xo)
    oq, os_ = O.quant_act(O.rmsnorm(xo, gain, norm_eps, ms))
    for i in range(xo.shape[0]):
        ok = np.array_equal(xq[i, :k], oq[i]) and s[i] == os_[i]
        if not ok and other[i] is not None:
            ms2 = ms.copy()
            ms2[i] = other[i]
            aq, as_ = O.quant_act(O.rmsnorm(xo[i:i + 1], gain, norm_eps, ms2[i:i + 1]))
            ok = np.array_equal(xq[i, :k], aq[0]) and s[i] == as_[0]
        assert ok, f"{where}: token {i} x~/s differ from the oracle"
        assert not xq[i, k:].any(), f"{where}: padding of token {i}"
    return oq, os_


@pytest.mark.parametrize("m,k,xdt,with_gain", [(3, 2560, "bf16", True), (16, 28672, "bf16", True),
                                              (5, 4096, "f32", False), (2, 6912, "bf16", False),
                                              (4, 16384, "f32", True)])
def test_rmsnorm_register_and_loop_kernels_agree(B, m, k, xdt, with_gain):
    """bitlinear_rmsnorm_quant_act holds 16-byte aligned rows in registers and
    loops over the others; both add the squares in the same order, so the
    same rows give the same bits whether x sits at a 16-byte boundary or 4
    bytes past one."""
    import torch
    _, x = random_case(9300 + m, m, 1, k, x_kind="t3")
    x[:, ::61] *= np.float32(500.0)
    xd, _ = x_device(x, xdt)
    esz = 2 if xdt == "bf16" else 4
    shift = 4 // esz
    buf = torch.empty(m * k + 16, dtype=xd.dtype, device="cuda")
    xs = buf[shift:shift + m * k].view(m, k)
    xs.copy_(xd)
    assert xd.data_ptr() % 16 == 0 and xs.data_ptr() % 16 == 4
    gd = dev(np.linspace(0.25, 2.0, k, dtype=np.float32)) if with_gain else None
    q1, s1 = B.rmsnorm_quant_act(xd, gd, norm_eps=1e-6)
    q2, s2 = B.rmsnorm_quant_act(xs, gd, norm_eps=1e-6)
    assert torch.equal(q1, q2)
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32))
    check_norm_quant(x_device(x, xdt)[1], None if gd is None else host(gd), np.float32(1e-6),
                     host(q1), host(s1), f"register kernel m={m} k={k}")


NQ_CASES = [
    # m, k, x dtype, gain, norm eps
    (1, 8, "bf16", True, 2.0 ** -23),
    (3, 256, "f32", False, 2.0 ** -23),
    (4, 1000, "bf16", True, 1e-5),
    (2, 1001, "f32", True, 1e-6),           # odd K: element loads
    (7, 6912, "bf16", True, 2.0 ** -23),
    (2, 28672, "bf16", False, 2.0 ** -23),
    (64, 2560, "bf16", True, 1e-2),
    (1, 40000, "f32", True, 2.0 ** -23),
]


@pytest.mark.parametrize("m,k,xdt,with_gain,neps", NQ_CASES)
def test_rmsnorm_quant_act(B, m, k, xdt, with_gain, neps):
    log(f"rmsnorm_quant m={m} k={k} {xdt} gain={with_gain} eps={neps}")
    _, x = random_case(7000 + m + k, m, 1, k, x_kind="t3")
    if m > 2:
        x[1] = 0.0                                   # zero token: y = 0, x~ = 0
        x[2] *= 1e-20                                # tiny token: eps dominates its mean square
    gain = (np.random.default_rng(k).standard_normal(k) * 0.5 + 1.0).astype(np.float32) \
        if with_gain else None
    xd, xo = x_device(x, xdt)
    xq, s = B.rmsnorm_quant_act(xd, None if gain is None else dev(gain), norm_eps=neps)
    check_norm_quant(xo, gain, np.float32(neps), host(xq), host(s), f"m={m} k={k}")


def _fused_norm_case(B, m, specs, seed, shared=False):
    """specs: (n, k, relu2, x dtype, gain, rmsnorm).  One fused launch; every
    entry's x~, s, acc and y against the oracle."""
    import torch
    ops, refs, xs = [], [], {}
    for i, (n, k, relu2, xdt, with_gain, norm) in enumerate(specs):
        w, x = random_case(seed + 31 * i, m, n, k, x_kind="t3")
        if shared and (k, xdt) in xs:
            xd, xo = xs[(k, xdt)]
        else:
            if m > 2:
                x[1] = 0.0
            xd, xo = x_device(x, xdt)
            xs[(k, xdt)] = (xd, xo)
        gain = (np.random.default_rng(seed + i).standard_normal(k) * 0.4 + 1.0).astype(np.float32) \
            if with_gain else None
        packed, gamma = B.pack_weights(dev(w))
        ops.append(dict(x=xd, packed=packed, gamma=gamma, n=n, k=k, relu2=relu2,
                        y=torch.empty((m, n), dtype=torch.bfloat16, device="cuda"),
                        acc_out=torch.empty((m, n), dtype=torch.int32, device="cuda"),
                        xq_out=torch.full((m, O.padded_k(k)), 99, dtype=torch.int8, device="cuda"),
                        scale_out=torch.empty(m, dtype=torch.float32, device="cuda"),
                        rmsnorm=norm, norm_weight=None if gain is None else dev(gain),
                        norm_eps=1e-6 if with_gain else 2.0 ** -23))
        refs.append((w, xo, gain, norm))
    B.forward_fused(ops)
    for i, (o, (w, xo, gain, norm)) in enumerate(zip(ops, refs)):
        g = host(o["gamma"])[0]
        assert gamma_agrees(g, w)
        where = f"m={m} entry {i}"
        xq, s = host(o["xq_out"]), host(o["scale_out"])
        if norm:
            oq, os_ = check_norm_quant(xo, gain, np.float32(o["norm_eps"]), xq, s, where)
            # with the device's own (checked) x~ and s the product is exact
            oq, os_ = xq[:, :o["k"]], s
        else:
            oq, os_ = O.quant_act(xo)
            np.testing.assert_array_equal(xq[:, :o["k"]], oq, err_msg=where)
            np.testing.assert_array_equal(s, os_, err_msg=where)
        codes = O.ternary_codes(w, g)
        acc = O.contract(oq, codes)
        np.testing.assert_array_equal(host(o["acc_out"]), acc, err_msg=where)
        assert_y_close(host(o["y"]), O.round_output(O.dequant(acc, g, os_, o["relu2"]), "bf16"),
                       "bf16", where)


FUSED_NORM_CASES = [
    # streaming kernel (1-2 tokens)
    (1, [(2560, 2560, False, "bf16", True, True), (640, 2560, False, "bf16", True, True),
         (640, 2560, False, "bf16", True, True)], True),      # q/k/v sharing x and the gain
    (1, [(8192, 28672, False, "bf16", True, True)]),          # long rows, 16 waves
    (1, [(1024, 4096, True, "f32", False, True), (300, 2048, False, "f32", True, False)]),
    (2, [(2000, 3000, True, "bf16", True, True), (64, 256, False, "bf16", False, True)]),
    (1, [(64, 256, False, "bf16", True, True)]),              # short rows: still streaming
    # the fused windowed matrix-core kernel
    (2, [(1100, 28672, False, "bf16", True, True)]),          # 2 tokens, rows past its registers
    (1, [(300, 1001, False, "f32", True, True)]),             # odd K: element loads
    (5, [(2560, 2560, False, "bf16", True, True), (500, 777, True, "f32", True, True)]),
    (16, [(6912, 2560, True, "bf16", False, True), (2560, 6912, False, "bf16", True, True)]),
    (40, [(1000, 3000, True, "bf16", True, True), (64, 8200, False, "bf16", True, False)]),
    # the multi-token streaming kernel (one dtype, whole aligned units)
    (8, [(2560, 2560, False, "bf16", True, True), (640, 2560, False, "bf16", True, True),
         (640, 2560, False, "bf16", True, True)], True),
    (33, [(3000, 4096, False, "f32", True, True), (640, 2048, True, "f32", False, True)]),
    (64, [(2560, 6912, False, "bf16", True, True), (300, 512, True, "bf16", False, False)]),
]


@pytest.mark.parametrize("case", FUSED_NORM_CASES, ids=lambda c: f"m{c[0]}-{len(c[1])}e")
def test_fused_rmsnorm(B, case):
    m, specs = case[0], case[1]
    shared = len(case) > 2 and case[2]
    log(f"fused rmsnorm m={m} {specs}")
    _fused_norm_case(B, m, specs, seed=8000 + m * 7 + len(specs), shared=shared)


@pytest.mark.parametrize("m,k,xdt,nent,kernel", [
    (1, 4096, "bf16", 1, "stream_gemv"), (8, 4096, "bf16", 1, "stream_mt"),
    (20, 8192, "bf16", 2, "stream_mt"),            # rows of 16 units per lane
    (40, 4096, "f32", 2, "stream_mt"), (3, 2560, "bf16", 1, "stream_mt"),
    (16, 6912, "bf16", 1, "two_pass")])
def test_rmsnorm_fused_equals_two_step(B, m, k, xdt, nent, kernel):
    """The fused step with RMSNorm gives the same bits as
    bitlinear_rmsnorm_quant_act followed by bitlinear_forward: x~, s, the
    accumulator and y.  From 3 tokens the fused kernel sums the squares in
    the standalone kernel's order, so this holds for every token, also one
    whose mean square sits at an fp32 rounding boundary; rows with outlier
    channels spread the squares over many binades."""
    import torch
    n = 3000
    w, x = random_case(8100 + m, m, n, k, x_kind="t3")
    x[:, ::97] *= np.float32(300.0)
    x[m // 2, :] *= np.float32(1e-3)
    gain = np.linspace(0.5, 1.5, k, dtype=np.float32)
    xd, _ = x_device(x, xdt)
    gd = dev(gain)
    packed, gamma = B.pack_weights(dev(w))
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    acc = torch.empty((m, n), dtype=torch.int32, device="cuda")
    xq1 = torch.full((m, O.padded_k(k)), 99, dtype=torch.int8, device="cuda")
    s1 = torch.empty(m, dtype=torch.float32, device="cuda")
    ops = [dict(x=xd, packed=packed, gamma=gamma, n=n, k=k, y=y, acc_out=acc, xq_out=xq1,
                scale_out=s1, rmsnorm=True, norm_weight=gd, norm_eps=1e-5)]
    if nent == 2:                                     # a second product on the same rows
        ops.append(dict(x=xd, packed=packed, gamma=gamma, n=640, k=k,
                        y=torch.empty((m, 640), dtype=torch.bfloat16, device="cuda"),
                        rmsnorm=True, norm_weight=gd, norm_eps=1e-5))
    step = B.FusedStep(ops)
    log(f"fused rmsnorm vs two-step m={m} k={k} {xdt} entries={nent} kernel={step.kernel()}")
    assert step.kernel() == kernel
    step()
    xq, s = B.rmsnorm_quant_act(xd, gd, norm_eps=1e-5)
    y2, acc2 = B.forward(xq, s, packed, gamma, n, k, out_dtype=torch.bfloat16, acc_out=True)
    assert torch.equal(xq1, xq), m
    assert torch.equal(s1.view(torch.int32), s.view(torch.int32)), m
    assert torch.equal(acc, acc2), m
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), m


@pytest.mark.parametrize("rmsnorm", [True, False])
def test_bitlinear_module_page_harness_shapes(B, rmsnorm):
    """BitLinearW158A8(128, 256) on x [4, 16, 128] -> [4, 16, 256], the shapes
    of the page's validation harness ("Functional Validation Harness"): 64
    tokens through one fused launch, and 130 tokens through the quant +
    forward path, every output against the oracle."""
    import torch
    w, _ = random_case(8200, 1, 256, 128)
    layer = B.BitLinearW158A8(128, 256, rmsnorm=rmsnorm).load_weight(dev(w))
    g = host(layer.gamma)[0]
    assert gamma_agrees(g, w)
    codes = O.ternary_codes(w, g)
    for shape in ((4, 16, 128), (2, 65, 128)):
        _, x = random_case(8201 + shape[1], int(np.prod(shape[:-1])), 1, 128, x_kind="t3")
        xd = dev(x.reshape(shape))
        y = layer(xd)
        assert tuple(y.shape) == shape[:-1] + (256,) and y.dtype == torch.float32
        yg = host(y).reshape(-1, 256)

        def ref_of(ms):
            xn = O.rmsnorm(x, None, np.float32(B.NORM_EPS_DEFAULT), ms) if rmsnorm else x
            oq, os_ = O.quant_act(xn)
            return O.round_output(O.dequant(O.contract(oq, codes), g, os_), "f32")
        ms, other = ms_candidates(x)
        ref = ref_of(ms)
        for i, alt in enumerate(other):            # either rounding of an ambiguous mean square
            if rmsnorm and alt is not None:
                ms2 = ms.copy()
                ms2[i] = alt
                r2 = ref_of(ms2)
                if np.all(np.abs(yg[i] - r2[i]) <= 1e-5 * np.abs(r2[i])):
                    ref[i] = r2[i]
        assert_y_close(yg, ref, "f32", f"module {shape}")


@pytest.mark.parametrize("k,n,relu2,m,kernel", [
    (2560, 6912, True, 1, "stream_gemv"), (2560, 6912, True, 8, "stream_mt"),
    (6912, 2560, False, 16, "two_pass"), (6912, 2560, False, 80, None),
    (2560, 6912, True, 72, None)])
def test_bitlinear_module_2b_shapes(B, k, n, relu2, m, kernel):
    """BitLinearW158A8 at the 2B-class up and down shapes with an RMSNorm
    gain, bf16 activations and fp32 outputs: one token (streaming kernel),
    8 tokens (multi-token kernel), the down product at 16 tokens (two-pass
    plan), and past 64 tokens (bitlinear_rmsnorm_quant_act, then
    bitlinear_forward); every output against the oracle."""
    import torch
    from datagen import bf16_bits_to_f32, to_bf16_bits
    w, x = random_case(8600 + m, m, n, k, x_kind="t3")
    bits = to_bf16_bits(x)
    xo = bf16_bits_to_f32(bits)
    layer = B.BitLinearW158A8(k, n, relu2=relu2, out_dtype=torch.float32).load_weight(dev(w))
    gain = np.linspace(0.5, 1.5, k, dtype=np.float32)
    layer.norm_weight = dev(gain)
    if kernel is not None:
        probe = B.FusedStep([dict(x=dev(bits.view(np.int16)).view(torch.bfloat16),
                                  packed=layer.packed, gamma=layer.gamma, n=n, k=k,
                                  y=torch.empty((m, n), dtype=torch.float32, device="cuda"),
                                  rmsnorm=True, norm_weight=layer.norm_weight)])
        assert probe.kernel() == kernel
    y = layer(dev(bits.view(np.int16)).view(torch.bfloat16))
    assert tuple(y.shape) == (m, n) and y.dtype == torch.float32
    yg = host(y)
    g = host(layer.gamma)[0]
    assert gamma_agrees(g, w)
    codes = O.ternary_codes(w, g)

    def ref_of(ms):
        oq, os_ = O.quant_act(O.rmsnorm(xo, gain, np.float32(B.NORM_EPS_DEFAULT), ms))
        return O.round_output(O.dequant(O.contract(oq, codes), g, os_, relu2), "f32")
    ms, other = ms_candidates(xo)
    ref = ref_of(ms)
    for i, alt in enumerate(other):                # either rounding of an ambiguous mean square
        if alt is not None:
            ms2 = ms.copy()
            ms2[i] = alt
            r2 = ref_of(ms2)
            if np.all(np.abs(yg[i] - r2[i]) <= 1e-5 * np.abs(r2[i])):
                ref[i] = r2[i]
    log(f"module k={k} n={n} m={m}")
    assert_y_close(yg, ref, "f32", f"module {k}->{n} m={m}")

