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


@pytest.mark.parametrize("m", [1, 2])
@pytest.mark.parametrize("shapes", [[(4096, 32768, False), (8192, 4096, True)],
                                    [(16384, 8192, True)]])
def test_fused_large_sets_agree_with_unfused(B, m, shapes):
    """Sets of >= 2^27 weights take the plan's large-set rules (a split entry
    beside an unsplit one; one unsplit entry; 4 or 8 waves, at most 2 splits
    at two tokens): the fused step equals bitlinear_quant_act followed by
    bitlinear_forward bit for bit, and leaves its workspace zero-filled."""
    import torch
    gen = torch.Generator(device="cuda").manual_seed(11)
    ops = []
    for n, k, relu2 in shapes:
        w = torch.randn((n, k), generator=gen, device="cuda") * 0.02
        packed, gamma = B.pack_weights(w)
        del w
        x = torch.randn((m, k), generator=gen, device="cuda").to(torch.bfloat16)
        ops.append(dict(x=x, packed=packed, gamma=gamma, n=n, k=k, relu2=relu2,
                        y=torch.empty((m, n), dtype=torch.bfloat16, device="cuda"),
                        acc_out=torch.empty((m, n), dtype=torch.int32, device="cuda")))
    step = B.FusedStep(ops, workspace=B.Workspace())
    assert (step.nbytes > 0) == (len(shapes) == 2)     # only the first set splits an entry
    step()
    for o in ops:
        xq, s = B.quant_act(o["x"])
        y, acc = B.forward(xq, s, o["packed"], o["gamma"], o["n"], o["k"], relu2=o["relu2"],
                           out_dtype=torch.bfloat16, acc_out=True)
        assert torch.equal(acc, o["acc_out"])
        assert torch.equal(y.view(torch.int16), o["y"].view(torch.int16))
    torch.cuda.synchronize()
    assert step.ws.buf is None or not host(step.ws.buf).any()


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


def test_fused_rejects(B):
    import torch
    m = B.BL_FUSED_MAX_M + 1
    x = torch.zeros((m, 256), dtype=torch.float32, device="cuda")
    packed, gamma = B.pack_weights(torch.zeros((64, 256), dtype=torch.float32, device="cuda"))
    y = torch.empty((m, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(B.BitLinearError) as e:
        B.forward_fused([dict(x=x, packed=packed, gamma=gamma, n=64, k=256, y=y)])
    assert e.value.status == 2        # m above the limit
