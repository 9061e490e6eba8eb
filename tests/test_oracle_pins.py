"""Pins of the CPU oracle to facts outside itself (no GPU needed).

Each test checks the oracle against something it does not compute itself:
hand-worked examples (tests/golden/worked_examples.json), closed forms,
brute force on tiny inputs, library routines with known semantics, and
invariants the equations imply.  A plausible slip in the oracle (dropped eps,
wrong tie rule, swapped operand, wrong bit position in the packing, wrong
order of rescale) fails at least one of them."""
import json
import math
import os

import numpy as np
import pytest

import oracle as O
from datagen import random_case, gaussian_weights

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


@pytest.fixture(scope="module")
def gold():
    with open(GOLDEN) as f:
        return json.load(f)


def f32(a):
    return np.asarray(a, dtype=np.float32)


# ----------------------------------------------------------------- weights --
@pytest.mark.parametrize("case", ["weights_basic", "weights_eps_placement", "weights_ties"])
def test_weights_worked(gold, case):
    g = gold[case]
    w = f32(g["w"])
    gamma = O.absmean_gamma(w)
    assert gamma == np.float32(g["gamma"])
    codes = O.ternary_codes(w, gamma, np.float32(g["eps"]))
    np.testing.assert_array_equal(codes, np.array(g["codes"], dtype=np.int8))
    if "codes_if_divisor_max" in g:
        alt = O.ternary_codes(w, gamma, np.float32(g["eps"]), divisor="max")
        np.testing.assert_array_equal(alt, np.array(g["codes_if_divisor_max"], dtype=np.int8))


def test_gamma_matches_exact_sum():
    # math.fsum returns the correctly rounded sum; the oracle's fp64 sum must
    # round to the same fp32 gamma.
    for seed in range(5):
        w, _ = random_case(100 + seed, 1, 300, 257)
        exact = math.fsum(abs(float(v)) for v in w.ravel()) / w.size
        assert O.absmean_gamma(w) == np.float32(exact)


def test_gamma_closed_forms():
    assert O.absmean_gamma(np.full((3, 5), -0.375, np.float32)) == np.float32(0.375)
    # mean of |k/64| for k = -32..31 over 64 entries = (32*33/2 + 31*32/2)/64/64
    w = (np.arange(-32, 32, dtype=np.float32) / 64).reshape(4, 16)
    assert O.absmean_gamma(w) == np.float32((528 + 496) / 64 / 64)


def test_gamma_expectation_gaussian():
    # E|W| = sigma*sqrt(2/pi) for W ~ N(0, sigma^2)
    w = gaussian_weights(7, "q", 2560, 2560)
    g = float(O.absmean_gamma(w))
    mean = 0.02 * math.sqrt(2 / math.pi)
    sd = 0.02 * math.sqrt(1 - 2 / math.pi) / math.sqrt(w.size)
    assert abs(g - mean) < 6 * sd


def test_zero_fraction_closed_form():
    # a weight is zero iff |W| < gamma/2; with gamma -> sigma*sqrt(2/pi) the
    # fraction is erf(1/(2*sqrt(pi))) = 0.3101, and +1 / -1 split the rest.
    w = gaussian_weights(2, "q", 2560, 2560)
    codes = O.ternary_codes(w, O.absmean_gamma(w))
    n = codes.size
    p0 = math.erf(1 / (2 * math.sqrt(math.pi)))
    bound = 5 * math.sqrt(p0 * (1 - p0) / n) + 0.002
    assert abs((codes == 0).mean() - p0) < bound
    pp = (1 - p0) / 2
    assert abs((codes == 1).mean() - pp) < bound
    assert abs((codes == -1).mean() - pp) < bound
    assert abs(p0 - 0.31006) < 1e-4


def test_codes_are_ternary_and_odd():
    w, _ = random_case(3, 1, 70, 333, w_sigma=1.0)
    g = O.absmean_gamma(w)
    c = O.ternary_codes(w, g)
    assert set(np.unique(c)) <= {-1, 0, 1}
    np.testing.assert_array_equal(O.ternary_codes(-w, g), -c)


def test_codes_power_of_two_scaling():
    w, _ = random_case(4, 1, 64, 256)
    c0 = O.ternary_codes(w, O.absmean_gamma(w), eps=0.0)
    for j in (-3, 5):
        ws = w * np.float32(2.0 ** j)
        assert O.absmean_gamma(ws) == O.absmean_gamma(w) * np.float32(2.0 ** j)
        np.testing.assert_array_equal(O.ternary_codes(ws, O.absmean_gamma(ws), eps=0.0), c0)


def test_codes_boundary_is_half():
    # fp32(W/d) > 0.5 is the exact condition for a nonzero code; probe fp32
    # neighbours of d/2 with d = 1 (eps = 0, gamma = 1).
    d = np.float32(1.0)
    half = np.float32(0.5)
    above = np.nextafter(half, np.float32(1))
    below = np.nextafter(half, np.float32(0))
    w = f32([[half, above, below, -above, -half, np.float32(1.5), np.float32(2.5)]])
    c = O.ternary_codes(w, d, eps=0.0)
    np.testing.assert_array_equal(c, [[0, 1, 0, -1, 0, 1, 1]])


def test_all_zero_weights():
    w = np.zeros((3, 7), np.float32)
    g = O.absmean_gamma(w)
    assert g == 0
    np.testing.assert_array_equal(O.ternary_codes(w, g), 0)
    np.testing.assert_array_equal(O.ternary_codes(w, g, eps=0.0), 0)


# ------------------------------------------------------------- activations --
def test_activations_worked(gold):
    g = gold["activations"]
    xq, s = O.quant_act(f32(g["x"]), np.float32(g["eps"]))
    np.testing.assert_array_equal(xq, np.array(g["xq"], dtype=np.int8))
    np.testing.assert_array_equal(s, f32(g["s"]))


def test_activation_invariants():
    _, x = random_case(5, 33, 4, 1000, x_kind="t3")
    x[3] = 0.0
    x[4, :] = 0.0
    x[4, 17] = -5e-4
    xq, s = O.quant_act(x)
    assert xq.min() >= -127 and xq.max() <= 127
    beta = np.abs(x).max(axis=1)
    for m in range(x.shape[0]):
        if beta[m] >= O.EPS_DEFAULT:
            j = int(np.argmax(np.abs(x[m])))
            assert abs(int(xq[m, j])) == 127
        # sign preserved or zeroed
        assert np.all((np.sign(xq[m]) == np.sign(x[m])) | (xq[m] == 0))
        order = np.argsort(x[m], kind="stable")
        assert np.all(np.diff(xq[m][order].astype(np.int32)) >= 0)
    np.testing.assert_array_equal(xq[3], 0)
    np.testing.assert_array_equal(O.quant_act(-x)[0], -xq)


def smallest_act_eps():
    """The smallest fp32 e with fp32(127 / e) finite, by bisection over the
    positive fp32 bit patterns (their order is the order of the values)."""
    lo, hi = 1, int(np.float32(1.0).view(np.uint32))      # 127/lo overflows, 127/hi does not
    with np.errstate(over="ignore", divide="ignore"):
        while hi - lo > 1:
            mid = (lo + hi) // 2
            e = np.uint32(mid).view(np.float32)
            if np.isfinite(np.float32(127.0) / e):
                hi = mid
            else:
                lo = mid
    return np.uint32(hi).view(np.float32)


EPS_MIN = smallest_act_eps()


def test_activation_eps_rule():
    # 127 / eps must be a finite fp32 (the listing clamps beta at a positive
    # eps); eps = 0 would make an all-zero token 0 * inf = NaN
    assert EPS_MIN == np.float32(3.7321948e-37)
    x = np.zeros((2, 5), np.float32)
    x[1, 2] = -0.75
    below = np.nextafter(EPS_MIN, np.float32(0))
    for bad in (0.0, -1e-5, below, float("nan"), float("inf"), 1e-38):
        with pytest.raises(ValueError):
            O.quant_act(x, bad)
    xq, s = O.quant_act(x, EPS_MIN)
    np.testing.assert_array_equal(xq, [[0] * 5, [0, 0, -127, 0, 0]])
    assert s[0] == np.float32(3.4028235e38) and np.isfinite(s[0])     # 127 / EPS_MIN
    assert s[1] == np.float32(127) / np.float32(0.75)
    xq, s = O.quant_act(x, np.float32(1e-5))
    assert s[0] == np.float32(12700000.0) and not xq[0].any()


def test_activation_power_of_two_scaling():
    _, x = random_case(6, 5, 4, 300)
    xq, s = O.quant_act(x, eps=EPS_MIN)
    for j in (-4, 6):
        xq2, s2 = O.quant_act(x * np.float32(2.0 ** j), eps=EPS_MIN)
        np.testing.assert_array_equal(xq2, xq)
        np.testing.assert_array_equal(s2, s / np.float32(2.0 ** j))


def test_activation_single_nonzero_and_k1(gold):
    g = gold["k_equals_1"]
    xq, s = O.quant_act(f32(g["x"]))
    np.testing.assert_array_equal(xq, g["xq"])
    for v in (3.0, -0.01, 1e-3, 77.7):
        x = np.zeros((1, 9), np.float32)
        x[0, 4] = v
        assert O.quant_act(x)[0][0, 4] == (127 if v > 0 else -127)


# ------------------------------------------------------------- contraction --
def test_contraction_brute_force():
    rng = np.random.default_rng(11)
    for (m, n, k) in [(1, 1, 1), (3, 5, 7), (4, 9, 64), (2, 3, 300)]:
        xq = rng.integers(-127, 128, size=(m, k)).astype(np.int8)
        codes = rng.integers(-1, 2, size=(n, k)).astype(np.int8)
        ref = np.zeros((m, n), dtype=np.int64)
        for i in range(m):
            for j in range(n):
                t = 0
                for kk in range(k):
                    t += int(xq[i, kk]) * int(codes[j, kk])
                ref[i, j] = t
        np.testing.assert_array_equal(O.contract(xq, codes), ref)
        np.testing.assert_array_equal(O.contract_addsub(xq, codes), ref)


def test_contraction_extremes():
    # |acc| reaches 127*K when every code matches the sign of a full-scale x~
    k = 28672
    xq = np.full((2, k), 127, np.int8)
    xq[1] = -127
    codes = np.ones((3, k), np.int8)
    codes[1] = -1
    codes[2] = 0
    acc = O.contract(xq, codes)
    np.testing.assert_array_equal(acc, [[127 * k, -127 * k, 0], [-127 * k, 127 * k, 0]])


def test_forward_worked(gold):
    gw, ga, gf = gold["weights_basic"], gold["activations"], gold["forward"]
    w = f32(gw["w"])
    r = O.forward(f32(ga["x"]), w, eps=np.float32(1e-5), y_dtype="f32")
    np.testing.assert_array_equal(r["acc"], gf["acc"])
    np.testing.assert_array_equal(r["y"], f32(gf["y_f32"]))
    r2 = O.forward(f32(ga["x"]), w, eps=np.float32(1e-5), relu2=True, y_dtype="f32")
    np.testing.assert_array_equal(r2["y"], f32(gf["y_relu2_f32"]))
    rb = O.forward(f32(ga["x"]), w, eps=np.float32(1e-5), y_dtype="bf16")
    np.testing.assert_array_equal(O.bf16_bits_to_f32(rb["y"]), f32(gf["y_bf16"]))


def test_forward_k1(gold):
    g = gold["k_equals_1"]
    r = O.forward(f32(g["x"]), f32(g["w"]), eps=np.float32(g["eps"]))
    np.testing.assert_array_equal(r["codes"], g["codes"])
    np.testing.assert_array_equal(r["acc"], g["acc"])
    assert r["y64"][0, 0] == -2.0 * float(np.float32(0.3))


def test_dequant_matches_page_form():
    # the page rescales by beta*gamma/Q_b; the oracle divides by s = 127/beta.
    # They differ only by the fp32 rounding of s (relative 2^-24 each way).
    w, x = random_case(12, 8, 40, 512, x_kind="t3")
    r = O.forward(x, w)
    beta = np.maximum(np.abs(x).max(axis=1), O.EPS_DEFAULT).astype(np.float64)
    page = r["acc"].astype(np.float64) * beta[:, None] * float(r["gamma"]) / 127.0
    nz = page != 0
    rel = np.abs(r["y64"][nz] - page[nz]) / np.abs(page[nz])
    assert rel.max() <= 2.0 ** -23
    np.testing.assert_array_equal(r["y64"][~nz], 0.0)


def test_dequant_scaling_law():
    w, x = random_case(13, 3, 16, 256)
    base = O.forward(x, w, eps=0.0, act_eps=EPS_MIN)["y64"]
    sc = O.forward(x * np.float32(4.0), w * np.float32(0.125), eps=0.0, act_eps=EPS_MIN)["y64"]
    np.testing.assert_array_equal(sc, base * 0.5)


def test_relu2():
    acc = np.array([[5, -5, 0, 127]], np.int32)
    y = O.dequant(acc, np.float32(0.5), f32([2.0]), relu2=True)
    np.testing.assert_array_equal(y, [[1.5625, 0.0, 0.0, (127 * 0.25) ** 2]])


def test_bf16_rounding_against_torch():
    import torch
    rng = np.random.default_rng(3)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 1000,
        np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x3F80FFFF, 0x7F7FFFFF, 0x00000001],
                 dtype=np.uint32).view(np.float32),
        f32([0.0, -0.0, 1.0, -2.5]),
    ]).astype(np.float32)
    ours = O.f32_to_bf16_bits(vals)
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    # ties go to even: 1.00390625 -> 1.0, 1.01171875 -> 1.015625
    assert O.f32_to_bf16_bits(np.array([0x3F808000], np.uint32).view(np.float32))[0] == 0x3F80
    assert O.f32_to_bf16_bits(np.array([0x3F818000], np.uint32).view(np.float32))[0] == 0x3F82


# ----------------------------------------------------------------- packing --
def test_pack_word_bits(gold):
    g = gold["pack_word_bits"]
    codes = np.array([g["codes_row0"]], dtype=np.int8)
    words = O.pack_ternary(codes).view(np.uint32)
    assert words.size == g["total_words"]
    assert words[0] == int(g["word0"], 16)
    assert np.all(words[1:] == 0)


def test_pack_word_index(gold):
    g = gold["pack_word_index"]
    n, k = g["n"], g["k"]
    for e in g["entries"]:
        codes = np.zeros((n, k), np.int8)
        codes[e["n"], e["k"]] = e["code"]
        words = O.pack_ternary(codes).view(np.uint32)
        assert words.size == g["total_words"]
        nz = np.nonzero(words)[0]
        assert list(nz) == [e["word"]]
        assert words[e["word"]] == int(e["value"], 16)
        assert O.packed_word_index(e["n"], e["k"], n, k)[0] == e["word"]


@pytest.mark.parametrize("shape", [(1, 1), (64, 256), (65, 257), (130, 520), (7, 1000)])
def test_pack_roundtrip(shape):
    rng = np.random.default_rng(sum(shape))
    codes = rng.integers(-1, 2, size=shape).astype(np.int8)
    packed = O.pack_ternary(codes)
    assert packed.nbytes == O.packed_bytes(*shape)
    np.testing.assert_array_equal(O.unpack_ternary(packed, *shape), codes)
    # padding holds zero codes; 0b10 never appears
    npad, kpad = O.padded_n(shape[0]), O.padded_k(shape[1])
    full = O.unpack_ternary(packed, npad, kpad)
    assert np.all(full[shape[0]:, :] == 0) and np.all(full[:, shape[1]:] == 0)
    words = packed.view(np.uint32)
    for sh in range(0, 32, 2):
        assert not np.any(((words >> np.uint32(sh)) & np.uint32(3)) == 2)


def test_pack_rejects_non_ternary():
    with pytest.raises(ValueError):
        O.pack_ternary(np.array([[2]], np.int8))


# ----------------------------------------------------------------- RMSNorm --
def _f32_nearest(fr):
    """The fp32 nearest to the rational fr, ties to even, by exact comparison
    with the midpoints of the fp32 neighbours (no float rounding involved)."""
    from fractions import Fraction
    c = np.float32(float(fr))
    lo = c if Fraction(float(c)) <= fr else np.nextafter(c, np.float32(-np.inf))
    hi = np.nextafter(lo, np.float32(np.inf))
    mid = (Fraction(float(lo)) + Fraction(float(hi))) / 2
    if fr < mid:
        return lo
    if fr > mid:
        return hi
    return lo if (int(np.asarray(lo).view(np.uint32)) & 1) == 0 else hi


def test_rmsnorm_worked_example():
    # x = [3, 4]: mean of squares 12.5; with eps = 2^-23 (below half an ulp
    # of 12.5) v = 12.5, r = 1/sqrt(12.5) = sqrt(2)/5, y = (3 r, 4 r) * w
    from decimal import Decimal, getcontext
    from fractions import Fraction
    getcontext().prec = 60
    r_exact = Fraction(Decimal(2).sqrt() / Decimal(5))
    r32 = _f32_nearest(r_exact)
    x = f32([[3.0, 4.0]])
    w = f32([2.0, 0.5])
    y = O.rmsnorm(x, w)
    assert O.mean_square(x[0]) == np.float32(12.5)
    exp = [_f32_nearest(Fraction(float(_f32_nearest(3 * Fraction(float(r32))))) * 2),
           _f32_nearest(Fraction(float(_f32_nearest(4 * Fraction(float(r32))))) / 2)]
    np.testing.assert_array_equal(y[0], f32(exp))


def test_rmsnorm_mean_square_is_exact():
    # squares spanning 120 binades: the correctly rounded sum, then / K
    from fractions import Fraction
    rng = np.random.default_rng(21)
    for k in (1, 7, 1000):
        row = (rng.standard_normal(k) * 2.0 ** rng.integers(-60, 60, k)).astype(np.float32)
        exact = sum(Fraction(float(v)) ** 2 for v in row)
        assert O.mean_square(row) == np.float32(float(exact) / k)


def test_rmsnorm_against_torch():
    # torch's nn.RMSNorm (CPU, fp32) computes the same formula with its own
    # reduction order and rsqrt: agreement to a few ulp pins the formula
    # (mean rather than sum, eps inside the root, the gain, no bias)
    import torch
    _, x = random_case(31, 6, 1, 3000, x_kind="t3")
    x[2] *= 1e-3
    x[3, :17] *= 100.0
    w = (np.random.default_rng(3).standard_normal(3000) * 0.3 + 1.0).astype(np.float32)
    for eps in (2.0 ** -23, 1e-5, 1e-2):
        norm = torch.nn.RMSNorm(3000, eps=eps)
        with torch.no_grad():
            norm.weight.copy_(torch.from_numpy(w))
            yt = norm(torch.from_numpy(x)).numpy()
        yo = O.rmsnorm(x, w, np.float32(eps))
        np.testing.assert_allclose(yo, yt, rtol=4e-6, atol=0)


def test_rmsnorm_closed_forms():
    k = 64
    # zero row -> 0; constant row c -> sign(c) * w; one nonzero x_j -> sqrt(K) sign(x_j) w_j
    w = (np.arange(k, dtype=np.float32) / 16 + 0.5).astype(np.float32)
    x = np.zeros((4, k), np.float32)
    x[1] = 3.0
    x[2] = -0.125
    x[3, 9] = -7.0
    y = O.rmsnorm(x, w, np.float32(1e-30))
    assert not y[0].any()
    np.testing.assert_allclose(y[1], w, rtol=2.5e-7)
    np.testing.assert_allclose(y[2], -w, rtol=2.5e-7)
    assert not np.delete(y[3], 9).any()
    np.testing.assert_allclose(y[3, 9], -8.0 * w[9], rtol=2.5e-7)   # sqrt(64) = 8
    # K = 1: x / |x|
    np.testing.assert_array_equal(O.rmsnorm(f32([[-5.0], [0.25]]), None, np.float32(1e-30)),
                                  f32([[-1.0], [1.0]]))


def test_rmsnorm_power_of_two_scaling():
    # eps far below the mean square: scaling x by 2^j leaves y unchanged bit for bit
    _, x = random_case(32, 5, 1, 700, x_kind="t3")
    w = np.linspace(0.5, 2.0, 700, dtype=np.float32)
    y = O.rmsnorm(x, w, np.float32(1e-30))
    for j in (-6, 9):
        np.testing.assert_array_equal(O.rmsnorm(x * np.float32(2.0 ** j), w, np.float32(1e-30)), y)


def test_rmsnorm_then_quant():
    # every nonzero token reaches |x~| = 127 at the largest |y|; the listing's
    # order (norm, then quant) inside forward
    _, x = random_case(33, 4, 1, 500, x_kind="t3")
    x[1] = 0.0
    w = np.linspace(0.1, 3.0, 500, dtype=np.float32)
    yn = O.rmsnorm(x, w)
    xq, s = O.quant_act(yn)
    for m in (0, 2, 3):
        assert np.abs(xq[m]).max() == 127
        assert int(np.argmax(np.abs(yn[m]))) in np.flatnonzero(np.abs(xq[m]) == 127)
    assert not xq[1].any()
    wt, _ = random_case(34, 1, 8, 500)
    r = O.forward(x, wt, norm=True, norm_weight=w)
    np.testing.assert_array_equal(r["xq"], xq)
    np.testing.assert_array_equal(r["s"], s)


def test_rmsnorm_rejects_bad_eps():
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        with pytest.raises(ValueError):
            O.rmsnorm(np.ones((1, 4), np.float32), None, bad)


# ------------------------------------------------------ page-code cross-check --
def _listing_weight_quant(w):
    """What the page's WeightQuantFunction.forward computes, in CPU torch
    (fp32): gamma = mean|W| clamped below at 1e-5, codes = clamp(round(W /
    gamma), -1, 1).  Returns (codes, gamma)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(w, np.float32))
    g = t.abs().mean().clamp(min=1e-5)
    return torch.clamp(torch.round(t / g), -1, 1).to(torch.int8).numpy(), np.float32(g.item())


def _listing_act_quant(x):
    """What the page's quantize_activations_int8 computes, in CPU torch
    (fp32): beta = max|x| over the last dimension clamped below at 1e-5,
    x~ = clamp(round(x * (127 / beta)), -128, 127)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32))
    beta = t.abs().amax(dim=-1, keepdim=True).clamp(min=1e-5)
    q = torch.clamp(torch.round(t * (127.0 / beta)), -128, 127)
    return q.to(torch.int8).numpy(), beta[:, 0].numpy()


def test_page_code_cross_check():
    """The page's listing, run with CPU torch, against the oracle in its
    max(gamma, eps) divisor mode: codes identical given the same gamma (the
    only freedom is torch.mean's fp32 reduction order, which moves gamma by
    a few ulp); x~ identical, and 127/beta equal to the oracle's s."""
    for seed, (n, k) in enumerate([(64, 256), (256, 2560), (640, 2560), (70, 1001)]):
        w, x = random_case(900 + seed, 6, n, k, x_kind="t3")
        x[2] = 0.0
        codes_t, g_t = _listing_weight_quant(w)
        g_o = O.absmean_gamma(w)
        assert abs(float(g_t) - float(g_o)) <= 4 * float(np.spacing(g_o))
        np.testing.assert_array_equal(codes_t, O.ternary_codes(w, g_t, divisor="max"))
        # the readings part only on weights within a hair of a 0.5 boundary
        diff = O.ternary_codes(w, g_o) != codes_t
        assert diff.mean() < 1e-3
        xq_t, beta_t = _listing_act_quant(x)
        xq_o, s_o = O.quant_act(x)
        np.testing.assert_array_equal(xq_t, xq_o)
        np.testing.assert_array_equal((np.float32(127.0) / beta_t).astype(np.float32), s_o)
        # the listing's rescale beta*gamma/127 against the oracle's gamma/s
        acc = O.contract(xq_o, codes_t)
        y_t = acc.astype(np.float32) * ((beta_t * g_t) / np.float32(127.0))[:, None]
        y_o = O.dequant(acc, g_t, s_o)
        np.testing.assert_allclose(y_t, y_o, rtol=1e-6, atol=0)
