"""Seeded random shapes through bitlinear_forward and the fused decode step,
every result against the oracle: sizes drawn across the plans' boundaries
(tokens 1-300, ragged N and K, fp32 and bf16 activations and outputs, ReLU^2
or not), so that each kernel meets shapes no hand-picked case names.  Integers
bit for bit; y within the rounding of the rescale."""
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


def _draw(rng, fused, long_rows=False):
    """(m, n, k, relu2, y dtype, x dtype) with m*n*k kept small enough for the
    oracle's contraction; ``long_rows`` draws 33-64 tokens on rows of more
    than 8192 weights and few row blocks (the multi-token streaming plan)."""
    while long_rows:
        m, n, k = int(rng.choice([33, 48, 64])), int(rng.integers(1, 600)), int(rng.integers(8193, 12000))
        if m * n * k <= 3.5e8:
            return (m, n, k, bool(rng.integers(0, 2)), str(rng.choice(["f32", "bf16"])),
                    str(rng.choice(["f32", "bf16"])))
    while True:
        m = int(rng.choice([1, 2, 3, 5, 8, 15, 16, 17, 31, 33, 48, 64] +
                           ([] if fused else [65, 100, 129, 200, 300])))
        n = int(rng.integers(1, 3000))
        k = int(rng.integers(1, 9000))
        if m * n * k <= 1.5e8:
            break
    return (m, n, k, bool(rng.integers(0, 2)), str(rng.choice(["f32", "bf16"])),
            str(rng.choice(["f32", "bf16"])))


CASES = ([(seed, False, False) for seed in range(40)] + [(seed, True, False) for seed in range(40, 70)]
         + [(seed, False, True) for seed in range(70, 76)] + [(seed, True, True) for seed in range(76, 82)])


@pytest.mark.parametrize("seed,fused,long_rows", CASES, ids=lambda v: str(v))
def test_random_shape(B, seed, fused, long_rows):
    import torch
    rng = np.random.default_rng(seed)
    m, n, k, relu2, ydt, xdt = _draw(rng, fused, long_rows)
    kernel = None
    w, x = random_case(50000 + seed, m, n, k, x_kind="t3")
    if m > 3:
        x[m // 2] = 0.0
    xd, xo = x_device(x, xdt)
    packed, gamma = B.pack_weights(dev(w))
    g = host(gamma)[0]
    assert gamma_agrees(g, w)
    ty = torch.bfloat16 if ydt == "bf16" else torch.float32
    if fused:
        y = torch.empty((m, n), dtype=ty, device="cuda")
        acc = torch.empty((m, n), dtype=torch.int32, device="cuda")
        xq = torch.full((m, O.padded_k(k)), 99, dtype=torch.int8, device="cuda")
        s = torch.empty(m, dtype=torch.float32, device="cuda")
        step = B.FusedStep([dict(x=xd, packed=packed, gamma=gamma, n=n, k=k, y=y, relu2=relu2,
                                 acc_out=acc, xq_out=xq, scale_out=s)])
        kernel = step.kernel()
        step()
    else:
        kernel = B.forward_kernel(m, n, k)
        xq, s = B.quant_act(xd)
        y, acc = B.forward(xq, s, packed, gamma, n, k, relu2=relu2, out_dtype=ty, acc_out=True)
    log(f"random seed={seed} fused={fused} m={m} n={n} k={k} relu2={relu2} y={ydt} x={xdt} "
        f"kernel={kernel}")
    r = O.forward(xo, w, relu2=relu2, y_dtype=ydt, gamma=g)
    xqh = host(xq)
    np.testing.assert_array_equal(xqh[:, :k], r["xq"])
    assert not xqh[:, k:].any()
    np.testing.assert_array_equal(host(s), r["s"])
    np.testing.assert_array_equal(host(acc), r["acc"])
    assert_y_close(host(y), r["y"], ydt, f"seed {seed}")
