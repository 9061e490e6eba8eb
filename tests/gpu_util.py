"""Helpers for the GPU parity tests: move seeded numpy inputs to the device,
call the library through its binding, bring results back, and compare with
the oracle at the tolerances the pass states (bit-exact integers; 1e-5
relative for fp32 outputs, 1e-2 relative for bf16 outputs, exact zeros)."""
import sys

import numpy as np

import oracle as O

TOL = {"f32": 1e-5, "bf16": 1e-2}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def x_device(x_f32, x_dtype):
    """fp32 numpy activations -> device tensor of the given dtype, and the
    fp32 values the oracle must see (bf16 rounding is part of the input)."""
    from datagen import to_bf16_bits, bf16_bits_to_f32
    if x_dtype == "bf16":
        bits = to_bf16_bits(x_f32)
        return dev_bf16(bits), bf16_bits_to_f32(bits)
    return dev(x_f32), np.asarray(x_f32, np.float32)


def y_as_f32(y, y_dtype):
    return O.bf16_bits_to_f32(y) if y_dtype == "bf16" else np.asarray(y, np.float32)


def assert_y_close(y_gpu, y_ora, y_dtype, where=""):
    """Elementwise |y_gpu - y_ora| <= tol * |y_ora|; y_ora == 0 must be exact."""
    g = y_as_f32(y_gpu, y_dtype).astype(np.float64)
    o = y_as_f32(y_ora, y_dtype).astype(np.float64)
    assert g.shape == o.shape, (g.shape, o.shape)
    tol = TOL[y_dtype]
    err = np.abs(g - o)
    bad = err > tol * np.abs(o)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{where}: {bad.sum()} outputs out of tolerance, e.g. "
                             + ", ".join(f"{tuple(i)} gpu={g[tuple(i)]!r} oracle={o[tuple(i)]!r}" for i in idx))


def gamma_agrees(g_gpu, w):
    """gamma from the device equals the oracle's, or both are the two fp32
    neighbours of a value that sits (within fp64 summation error) on their
    rounding midpoint -- then either rounding is a correct result."""
    g_ora = O.absmean_gamma(w)
    if np.float32(g_gpu) == g_ora:
        return True
    exact = np.abs(w.astype(np.float64)).sum() / w.size
    lo, hi = sorted([float(g_gpu), float(g_ora)])
    mid = (lo + hi) / 2
    return np.nextafter(np.float32(lo), np.float32(np.inf)) == np.float32(hi) and \
        abs(exact - mid) <= 1e-12 * abs(exact)
