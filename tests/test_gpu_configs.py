"""Parity at the workloads' full sizes through quant_act + forward: every
output of the 256x256 layer, the 2B-class decode set, the 2B-class stack's
matrices at 1/8/32/64 tokens and the 2048-token prefill.  The 100B-class layer
and the benchmark's fused launch configurations are in test_gpu_full.py."""
import numpy as np
import pytest

import datagen
import oracle as O
from gpu_util import assert_y_close, dev, dev_bf16, gamma_agrees, host, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_gemm_int8_amd as B
    return B


def _x(wl, group, m):
    """(device activations, fp32 values the oracle sees)."""
    if wl.x_dtype == "bf16":
        bits, _ = datagen.activations(wl, group, m)
        return dev_bf16(bits), datagen.bf16_bits_to_f32(bits)
    x = datagen.activations_f32(wl, group, m)
    return dev(x), x


def _run_full(B, wl, name, m, w=None):
    import torch
    n, k, relu2, group = wl.matrices[name]
    w = datagen.workload_weights(wl, name) if w is None else w
    xd, xo = _x(wl, group, m)
    packed, gamma = B.pack_weights(dev(w))
    xq, s = B.quant_act(xd)
    ydt = torch.bfloat16 if wl.y_dtype == "bf16" else torch.float32
    y, acc = B.forward(xq, s, packed, gamma, n, k, relu2=relu2, out_dtype=ydt, acc_out=True)
    g = host(gamma)[0]
    assert gamma_agrees(g, w)
    return w, xo, g, packed, host(xq), host(s), host(acc), host(y), relu2


def test_c1_full(B):
    wl = datagen.WORKLOADS["c1"]
    log("c1")
    w, xo, g, packed, xq, s, acc, y, relu2 = _run_full(B, wl, "w", 4)
    r = O.forward(xo, w, gamma=g, y_dtype="f32")
    np.testing.assert_array_equal(host(packed), O.pack_ternary(r["codes"]))
    np.testing.assert_array_equal(xq[:, :256], r["xq"])
    np.testing.assert_array_equal(s, r["s"])
    np.testing.assert_array_equal(acc, r["acc"])
    assert_y_close(y, r["y"], "f32", "c1")


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "up", "down"])
def test_c2_full(B, name):
    wl = datagen.WORKLOADS["c2"]
    log(f"c2 {name}")
    w, xo, g, packed, xq, s, acc, y, relu2 = _run_full(B, wl, name, 1)
    r = O.forward(xo, w, gamma=g, relu2=relu2, y_dtype="bf16")
    np.testing.assert_array_equal(host(packed), O.pack_ternary(r["codes"]))
    np.testing.assert_array_equal(xq[:, :w.shape[1]], r["xq"])
    np.testing.assert_array_equal(acc, r["acc"])
    assert_y_close(y, r["y"], "bf16", f"c2 {name}")


@pytest.mark.parametrize("m", [1, 8, 32, 64])
@pytest.mark.parametrize("name", ["q", "k", "v", "o", "up", "down"])
def test_c3_batches(B, m, name):
    wl = datagen.WORKLOADS["c3"]
    log(f"c3 {name} m={m}")
    w, xo, g, packed, xq, s, acc, y, relu2 = _run_full(B, wl, name, m)
    r = O.forward(xo, w, gamma=g, relu2=relu2, y_dtype="bf16")
    np.testing.assert_array_equal(acc, r["acc"])
    assert_y_close(y, r["y"], "bf16", f"c3 {name} m={m}")


@pytest.mark.parametrize("name", ["up", "down"])
def test_c4_full(B, name):
    wl = datagen.WORKLOADS["c4"]
    log(f"c4 {name}")
    w, xo, g, packed, xq, s, acc, y, relu2 = _run_full(B, wl, name, 2048)
    codes = O.ternary_codes(w, g)
    oq, os_ = O.quant_act(xo)
    np.testing.assert_array_equal(xq[:, :w.shape[1]], oq)
    np.testing.assert_array_equal(s, os_)
    racc = O.contract(oq, codes)
    np.testing.assert_array_equal(acc, racc)
    assert_y_close(y, O.round_output(O.dequant(racc, g, os_, relu2), "bf16"), "bf16", f"c4 {name}")
