"""Full-size parity of the 100B-class layer and of the launch configurations
the benchmark times, against the CPU oracle: every output row, the whole
packed buffer, every x~ and s, no sampling.

The oracle's integer product is a float64 matmul of integer-valued arrays
(exact, see oracle.contract); it runs in chunks of output rows to bound host
memory.  Codes are computed with the gamma the device reports, after checking
that gamma against the oracle's (gpu_util.gamma_agrees)."""
import numpy as np
import pytest

import datagen
import oracle as O
from gpu_util import assert_y_close, dev, dev_bf16, gamma_agrees, host, log

pytestmark = pytest.mark.gpu

ROW_CHUNK = 4096           # output rows per oracle chunk (a multiple of 64)


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_gemm_int8_amd as B
    return B


class Packed:
    """One matrix: packed on the device, its oracle codes on the host."""

    def __init__(self, B, wl, name):
        n, k, relu2, group = wl.matrices[name]
        w = datagen.workload_weights(wl, name)
        self.packed, self.gamma = B.pack_weights(dev(w))
        self.g = host(self.gamma)[0]
        assert gamma_agrees(self.g, w), name
        self.codes = O.ternary_codes(w, self.g)
        self.n, self.k, self.relu2, self.group, self.name = n, k, relu2, group, name


def _check_packed(p):
    """The whole packed buffer, 64-row blocks in chunks: rows [r0, r1) are
    bytes [r0 * K_pad / 4, r1 * K_pad / 4) of the layout."""
    got = host(p.packed)
    kp4 = O.padded_k(p.k) // 4
    assert got.size == O.packed_bytes(p.n, p.k)
    for r0 in range(0, p.n, ROW_CHUNK):
        r1 = min(r0 + ROW_CHUNK, p.n)
        ref = O.pack_ternary(p.codes[r0:r1])
        np.testing.assert_array_equal(got[r0 * kp4: r0 * kp4 + ref.size], ref,
                                      err_msg=f"{p.name} packed rows {r0}..{r1}")


def _oracle_acc(oq, codes):
    n = codes.shape[0]
    acc = np.empty((oq.shape[0], n), np.int32)
    for r0 in range(0, n, ROW_CHUNK):
        acc[:, r0:r0 + ROW_CHUNK] = O.contract(oq, codes[r0:r0 + ROW_CHUNK])
    return acc


def _x(wl, group, m):
    bits, _ = datagen.activations(wl, group, m)
    return dev_bf16(bits), datagen.bf16_bits_to_f32(bits)


def _check_outputs(p, xo, xq, s, acc, y, where):
    """x~ / s (when given), acc and y of one product against the oracle."""
    oq, os_ = O.quant_act(xo)
    if xq is not None:
        np.testing.assert_array_equal(xq[:, :p.k], oq, err_msg=f"{where} x~")
        assert not xq[:, p.k:].any(), f"{where} x~ padding"
    if s is not None:
        np.testing.assert_array_equal(s, os_, err_msg=f"{where} s")
    racc = _oracle_acc(oq, p.codes)
    np.testing.assert_array_equal(acc, racc, err_msg=f"{where} acc")
    assert_y_close(y, O.round_output(O.dequant(racc, p.g, os_, p.relu2), "bf16"), "bf16", where)


# ------------------------------------------------------------- 100B class --
C5 = datagen.WORKLOADS["c5"]


@pytest.fixture(scope="module")
def c5(B):
    return {}


def _c5_matrix(B, c5, name):
    if name not in c5:
        log(f"c5 {name}: packing and oracle codes")
        c5[name] = Packed(B, C5, name)
    return c5[name]


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "up", "down"])
def test_c5_matrix_full(B, c5, name):
    """Each matrix of the layer: the whole packed buffer, then quant_act +
    forward at 1, 16 and 512 tokens (the dot4 GEMV, the windowed MFMA GEMV,
    and the GEMM or token-blocked MFMA GEMV), every row."""
    import torch
    p = _c5_matrix(B, c5, name)
    _check_packed(p)
    for m in C5.batches:
        log(f"c5 {name} m={m}")
        xd, xo = _x(C5, p.group, m)
        xq, s = B.quant_act(xd)
        y, acc = B.forward(xq, s, p.packed, p.gamma, p.n, p.k, relu2=p.relu2,
                           out_dtype=torch.bfloat16, acc_out=True)
        _check_outputs(p, xo, host(xq), host(s), host(acc), host(y), f"c5 {name} m={m}")


def _fused(B, mats, xs, m):
    """One bitlinear_forward_fused launch over `mats` (activations xs[group])
    with every optional output; returns the per-entry host results."""
    import torch
    ops = []
    for p in mats:
        ops.append(dict(x=xs[p.group][0], packed=p.packed, gamma=p.gamma, n=p.n, k=p.k,
                        relu2=p.relu2,
                        y=torch.empty((m, p.n), dtype=torch.bfloat16, device="cuda"),
                        acc_out=torch.empty((m, p.n), dtype=torch.int32, device="cuda"),
                        xq_out=torch.full((m, O.padded_k(p.k)), 99, dtype=torch.int8,
                                          device="cuda"),
                        scale_out=torch.empty(m, dtype=torch.float32, device="cuda")))
    B.forward_fused(ops)
    return [(host(o["xq_out"]), host(o["scale_out"]), host(o["acc_out"]), host(o["y"]))
            for o in ops]


@pytest.mark.parametrize("m", [1, 16])
def test_c5_layer_fused_steps(B, c5, m):
    """The decode step of the layer as the benchmark launches it: one fused
    launch (activation quant in the kernel) per group of products sharing an
    input -- q/k/v, then o, up, down."""
    mats = {nm: _c5_matrix(B, c5, nm) for nm in ("q", "k", "v", "o", "up", "down")}
    xs = {g: _x(C5, g, m) for g in C5.groups()}
    for grp in (("q", "k", "v"), ("o",), ("up",), ("down",)):
        log(f"c5 fused {'/'.join(grp)} m={m}")
        res = _fused(B, [mats[nm] for nm in grp], xs, m)
        for nm, (xq, s, acc, y) in zip(grp, res):
            _check_outputs(mats[nm], xs[mats[nm].group][1], xq, s, acc, y, f"c5 fused {nm} m={m}")


@pytest.mark.parametrize("m", [16, 512])
def test_c5_qkv_multi(B, c5, m):
    """q, k and v over one shared x~ in one bitlinear_forward_multi call (one
    GEMM grid at 512 tokens), as the benchmark's layer leg runs them."""
    import torch
    mats = [_c5_matrix(B, c5, nm) for nm in ("q", "k", "v")]
    xd, xo = _x(C5, "attn_in", m)
    xq, s = B.quant_act(xd)
    ops = [dict(packed=p.packed, gamma=p.gamma, n=p.n, relu2=p.relu2,
                y=torch.empty((m, p.n), dtype=torch.bfloat16, device="cuda"),
                acc_out=torch.empty((m, p.n), dtype=torch.int32, device="cuda")) for p in mats]
    log(f"c5 multi q/k/v m={m}")
    B.forward_multi(xq, s, 8192, ops)
    for p, o in zip(mats, ops):
        _check_outputs(p, xo, None, None, host(o["acc_out"]), host(o["y"]), f"c5 multi {p.name} m={m}")


# -------------------------------------------------------------- 2B stack --
C3 = datagen.WORKLOADS["c3"]


@pytest.fixture(scope="module")
def c3(B):
    return {nm: Packed(B, C3, nm) for nm in C3.matrices}


@pytest.mark.parametrize("m", [1, 8, 32, 64])
def test_c3_stack_launches(B, c3, m):
    """One layer of the 2B-class stack at 1/8/32/64 tokens with Student-t
    activations, in the launch configuration of the stack benchmark: fused
    steps per input group at 1-2 tokens, a fused q/k/v step at 3-64 tokens,
    and quant_act + forward for o, up, down at 3-64 tokens."""
    import torch
    xs = {g: _x(C3, g, m) for g in C3.groups()}
    for grp in (("q", "k", "v"), ("o",), ("up",), ("down",)):
        mats = [c3[nm] for nm in grp]
        if m <= 2 or len(grp) > 1:
            log(f"c3 fused {'/'.join(grp)} m={m}")
            res = _fused(B, mats, xs, m)
            for p, (xq, s, acc, y) in zip(mats, res):
                _check_outputs(p, xs[p.group][1], xq, s, acc, y, f"c3 fused {p.name} m={m}")
        else:
            p = mats[0]
            log(f"c3 {p.name} m={m}")
            xq, s = B.quant_act(xs[p.group][0])
            y, acc = B.forward(xq, s, p.packed, p.gamma, p.n, p.k, relu2=p.relu2,
                               out_dtype=torch.bfloat16, acc_out=True)
            _check_outputs(p, xs[p.group][1], host(xq), host(s), host(acc), host(y),
                           f"c3 {p.name} m={m}")


# ------------------------------------------------- fused plan, large sets --
# (tokens, entries (n, k, relu2), whether the plan splits K over workgroups)
LARGE_SETS = [
    # the streaming matrix-core kernel (x~ of every token within the LDS)
    (1, [(4096, 32768, False), (8192, 4096, True)], False),
    (1, [(16384, 8192, True)], False),
    (2, [(16384, 8192, True)], False),
    # rows too long for it: the dot4 kernel's large-set rules (at one token
    # up to 8 splits and 4 waves, at two at most 2 splits and 8 waves)
    (1, [(2048, 65536, False), (8192, 4096, True)], True),
    (2, [(4096, 32768, False), (8192, 4096, True)], True),
]


@pytest.mark.parametrize("m,shapes,splits", LARGE_SETS)
def test_fused_large_sets_vs_oracle(B, m, shapes, splits):
    """Sets of >= 2^27 weights in one fused launch: every x~, s, acc and y
    against the oracle, and a split plan leaves its workspace zero-filled."""
    import torch
    mats, xs = [], {}
    for i, (n, k, relu2) in enumerate(shapes):
        w = datagen.gaussian_weights(900 + m, "q" if i == 0 else "up", n, k)
        p = Packed.__new__(Packed)
        p.packed, p.gamma = B.pack_weights(dev(w))
        p.g = host(p.gamma)[0]
        assert gamma_agrees(p.g, w)
        p.codes = O.ternary_codes(w, p.g)
        del w
        p.n, p.k, p.relu2, p.group, p.name = n, k, relu2, f"in{i}", f"entry{i}"
        _, x = datagen.random_case(950 + 7 * i + m, m, 1, k)
        from datagen import to_bf16_bits
        bits = to_bf16_bits(x)
        xs[p.group] = (dev_bf16(bits), datagen.bf16_bits_to_f32(bits))
        mats.append(p)
    ops = [dict(x=xs[p.group][0], packed=p.packed, gamma=p.gamma, n=p.n, k=p.k, relu2=p.relu2,
                y=torch.empty((m, p.n), dtype=torch.bfloat16, device="cuda"),
                acc_out=torch.empty((m, p.n), dtype=torch.int32, device="cuda"),
                xq_out=torch.full((m, O.padded_k(p.k)), 99, dtype=torch.int8, device="cuda"),
                scale_out=torch.empty(m, dtype=torch.float32, device="cuda")) for p in mats]
    step = B.FusedStep(ops, workspace=B.Workspace())
    assert (step.nbytes > 0) == splits
    log(f"fused large set m={m} {shapes}")
    step()
    for p, o in zip(mats, ops):
        _check_outputs(p, xs[p.group][1], host(o["xq_out"]), host(o["scale_out"]),
                       host(o["acc_out"]), host(o["y"]), f"large {p.name} m={m}")
    torch.cuda.synchronize()
    assert step.ws.buf is None or not host(step.ws.buf).any()
