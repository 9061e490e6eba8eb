"""Python binding of libbitlinear (BitLinear W1.58A8 forward on MI355X).

Argument marshalling only: every step of the pass runs in the library's HIP
kernels.  PyTorch provides device memory and the current stream.  The names
follow the C ABI in include/bitlinear.h:

    pack_weights(w, eps)            -> (packed uint8, gamma fp32[1])
    quant_act(x, eps)               -> (xq int8 [M, K_pad], scale fp32 [M])
    forward(xq, scale, packed, gamma, n, k, relu2, out_dtype)  -> y [M, N]

The library must be built (``python -m bit_gemm_int8_amd.build_lib`` or
``__graft_entry__.build()``); importing fails loudly if it is missing.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbitlinear.so")

BL_OK = 0
BL_ERR_INVALID_ARG, BL_ERR_UNSUPPORTED_SHAPE, BL_ERR_MISALIGNED = 1, 2, 3
BL_ERR_WORKSPACE, BL_ERR_HIP = 4, 5
BL_F32, BL_BF16 = 0, 1
BL_EPI_NONE, BL_EPI_RELU2 = 0, 1
BL_MAX_K = 262144
BL_MAX_MN = 16777216
EPS_DEFAULT = 1e-5

STATUS_NAMES = {0: "BL_OK", 1: "BL_ERR_INVALID_ARG", 2: "BL_ERR_UNSUPPORTED_SHAPE",
                3: "BL_ERR_MISALIGNED", 4: "BL_ERR_WORKSPACE", 5: "BL_ERR_HIP"}

# Every symbol declared in include/bitlinear.h.
EXPORTS = [
    "bitlinear_padded_n", "bitlinear_padded_k", "bitlinear_packed_bytes", "bitlinear_xq_bytes",
    "bitlinear_pack_workspace_bytes", "bitlinear_pack_weights", "bitlinear_quant_act",
    "bitlinear_forward_workspace_bytes", "bitlinear_forward", "bitlinear_workspace_init",
    "bitlinear_status_string", "bitlinear_abi_version",
    "bitlinear_forward_fused_workspace_bytes", "bitlinear_forward_fused",
    "bitlinear_forward_multi_workspace_bytes", "bitlinear_forward_multi",
    "bitlinear_forward_noalloc", "bitlinear_rmsnorm_quant_act",
    "bitlinear_forward_kernel", "bitlinear_forward_fused_kernel",
]
NORM_EPS_DEFAULT = 2.0 ** -23       # fp32 machine epsilon, nn.RMSNorm's default
BL_NOALLOC_SCRATCH_BYTES = 262144
BL_MAX_FUSED = 16
BL_FUSED_MAX_M = 64
BL_MAX_MULTI = 16
# kernels a call can run (bitlinear_forward_kernel / _fused_kernel)
KERNEL_NAMES = {0: "dot4_gemv", 1: "gemm", 2: "mfma_gemv", 3: "stream_gemv", 4: "stream_mt",
                5: "two_pass"}


class BLLinear(ctypes.Structure):
    """bl_linear of include/bitlinear.h."""
    _fields_ = [("x", ctypes.c_void_p), ("x_dtype", ctypes.c_int), ("packed", ctypes.c_void_p),
                ("gamma", ctypes.c_void_p), ("n", ctypes.c_int64), ("k", ctypes.c_int64),
                ("epilogue", ctypes.c_int), ("y_dtype", ctypes.c_int), ("y", ctypes.c_void_p),
                ("acc_out", ctypes.c_void_p), ("xq_out", ctypes.c_void_p),
                ("scale_out", ctypes.c_void_p), ("rmsnorm", ctypes.c_int),
                ("norm_eps", ctypes.c_float), ("norm_weight", ctypes.c_void_p)]


class BLProduct(ctypes.Structure):
    """bl_product of include/bitlinear.h."""
    _fields_ = [("packed", ctypes.c_void_p), ("gamma", ctypes.c_void_p), ("n", ctypes.c_int64),
                ("epilogue", ctypes.c_int), ("y_dtype", ctypes.c_int), ("y", ctypes.c_void_p),
                ("acc_out", ctypes.c_void_p)]


class BitLinearError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)} ({msg})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libbitlinear.so is not built ({LIB_PATH}); run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    i64, sz, vp, f32, i32 = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float, ctypes.c_int
    sig = {
        "bitlinear_padded_n": (i64, [i64]),
        "bitlinear_padded_k": (i64, [i64]),
        "bitlinear_packed_bytes": (sz, [i64, i64]),
        "bitlinear_xq_bytes": (sz, [i64, i64]),
        "bitlinear_pack_workspace_bytes": (sz, [i64, i64]),
        "bitlinear_pack_weights": (i32, [vp, i32, i64, i64, f32, vp, vp, vp, vp, sz, vp]),
        "bitlinear_quant_act": (i32, [vp, i32, i64, i64, f32, vp, vp, vp]),
        "bitlinear_forward_workspace_bytes": (sz, [i64, i64, i64]),
        "bitlinear_forward": (i32, [vp, vp, vp, vp, i64, i64, i64, i32, i32, vp, vp, vp, sz, vp]),
        "bitlinear_workspace_init": (i32, [vp, sz, vp]),
        "bitlinear_status_string": (ctypes.c_char_p, [i32]),
        "bitlinear_abi_version": (i32, []),
        "bitlinear_forward_fused_workspace_bytes": (sz, [vp, i32, i64]),
        "bitlinear_forward_fused": (i32, [vp, i32, i64, f32, vp, sz, vp]),
        "bitlinear_forward_multi_workspace_bytes": (sz, [vp, i32, i64, i64]),
        "bitlinear_forward_multi": (i32, [vp, vp, i64, i64, vp, i32, vp, sz, vp]),
        "bitlinear_forward_noalloc": (i32, [vp, vp, vp, vp, i64, i64, i64, i32, i32, vp, vp, vp]),
        "bitlinear_rmsnorm_quant_act": (i32, [vp, i32, i64, i64, vp, f32, f32, vp, vp, vp]),
        "bitlinear_forward_kernel": (i32, [i64, i64, i64]),
        "bitlinear_forward_fused_kernel": (i32, [vp, i32, i64]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def _check(fn: str, status: int) -> None:
    if status != BL_OK:
        raise BitLinearError(fn, status, lib.bitlinear_status_string(status).decode())


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _dtype_code(dt) -> int:
    import torch
    if dt == torch.float32:
        return BL_F32
    if dt == torch.bfloat16:
        return BL_BF16
    raise TypeError(f"unsupported dtype {dt}")


# ------------------------------------------------------------------ sizes --
def padded_k(k: int) -> int:
    return int(lib.bitlinear_padded_k(k))


def padded_n(n: int) -> int:
    return int(lib.bitlinear_padded_n(n))


def packed_bytes(n: int, k: int) -> int:
    return int(lib.bitlinear_packed_bytes(n, k))


def forward_kernel(m: int, n: int, k: int) -> str:
    """Name of the kernel bitlinear_forward runs for (m, n, k) (KERNEL_NAMES)."""
    r = int(lib.bitlinear_forward_kernel(int(m), int(n), int(k)))
    if r < 0:
        _check("bitlinear_forward_kernel", -r)
    return KERNEL_NAMES[r]


def forward_workspace_bytes(m: int, n: int, k: int) -> int:
    return int(lib.bitlinear_forward_workspace_bytes(m, n, k))


# ------------------------------------------------------------ workspaces --
class Workspace:
    """A zero-filled forward workspace that grows on demand (device memory
    from torch).  The library leaves it zero-filled after every call."""

    def __init__(self, device=None):
        self.buf = None
        self.device = device

    def get(self, nbytes: int, stream=None):
        import torch
        if nbytes == 0:
            return None
        if self.buf is None or self.buf.numel() < nbytes:
            size = max(nbytes, 1 << 20)
            self.buf = torch.empty(size, dtype=torch.uint8, device=self.device or "cuda")
            _check("bitlinear_workspace_init",
                   lib.bitlinear_workspace_init(_ptr(self.buf), size, _stream(stream)))
        return self.buf


_default_ws = {}


def _workspace_for(device, stream=None) -> Workspace:
    """The default workspace of a (device, stream) pair: calls that share a
    workspace must be ordered, and calls on one stream are."""
    key = (str(device), _stream(stream))
    if key not in _default_ws:
        _default_ws[key] = Workspace(device)
    return _default_ws[key]


# ---------------------------------------------------------------- entries --
def pack_weights(w, eps: float = EPS_DEFAULT, gamma_in=None, stream=None):
    """bitlinear_pack_weights: w [N, K] fp32/bf16 (cuda) -> (packed uint8, gamma fp32[1])."""
    import torch
    if w.dim() != 2 or not w.is_contiguous():
        raise ValueError("w must be a contiguous [N, K] tensor")
    n, k = w.shape
    packed = torch.empty(max(packed_bytes(n, k), 1), dtype=torch.uint8, device=w.device)
    gamma = torch.empty(1, dtype=torch.float32, device=w.device)
    wsb = int(lib.bitlinear_pack_workspace_bytes(n, k))
    ws = None if gamma_in is not None else torch.empty(max(wsb, 8), dtype=torch.uint8, device=w.device)
    _check("bitlinear_pack_weights", lib.bitlinear_pack_weights(
        _ptr(w), _dtype_code(w.dtype), n, k, float(eps), _ptr(gamma_in), _ptr(packed),
        _ptr(gamma), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))
    return packed, gamma


def quant_act(x, eps: float = EPS_DEFAULT, stream=None) -> Tuple:
    """bitlinear_quant_act: x [M, K] fp32/bf16 -> (xq int8 [M, K_pad], scale fp32 [M])."""
    import torch
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [M, K] tensor")
    m, k = x.shape
    kp = padded_k(k)
    xq = torch.empty((m, kp), dtype=torch.int8, device=x.device)
    scale = torch.empty(m, dtype=torch.float32, device=x.device)
    _check("bitlinear_quant_act", lib.bitlinear_quant_act(
        _ptr(x), _dtype_code(x.dtype), m, k, float(eps), _ptr(xq), _ptr(scale), _stream(stream)))
    return xq, scale


def rmsnorm_quant_act(x, weight=None, norm_eps: float = NORM_EPS_DEFAULT,
                      eps: float = EPS_DEFAULT, stream=None) -> Tuple:
    """bitlinear_rmsnorm_quant_act: RMSNorm of x [M, K] (gain `weight` fp32
    [K], or ones) then absmax int8 -> (xq int8 [M, K_pad], scale fp32 [M])."""
    import torch
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [M, K] tensor")
    m, k = x.shape
    if weight is not None and (weight.dtype != torch.float32 or weight.shape != (k,)):
        raise ValueError("weight must be fp32 [K]")
    xq = torch.empty((m, padded_k(k)), dtype=torch.int8, device=x.device)
    scale = torch.empty(m, dtype=torch.float32, device=x.device)
    _check("bitlinear_rmsnorm_quant_act", lib.bitlinear_rmsnorm_quant_act(
        _ptr(x), _dtype_code(x.dtype), m, k, _ptr(weight), float(norm_eps), float(eps), _ptr(xq),
        _ptr(scale), _stream(stream)))
    return xq, scale


def forward(xq, scale, packed, gamma, n: int, k: int, relu2: bool = False,
            out_dtype=None, acc_out: bool = False, y=None, workspace: Optional[Workspace] = None,
            stream=None):
    """bitlinear_forward: returns y [M, N] (and the int32 accumulator if asked)."""
    import torch
    out_dtype = out_dtype or torch.float32
    m = xq.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=out_dtype, device=xq.device)
    acc = torch.empty((m, n), dtype=torch.int32, device=xq.device) if acc_out else None
    nbytes = forward_workspace_bytes(m, n, k)
    ws = (workspace or _workspace_for(xq.device, stream)).get(nbytes, stream)
    _check("bitlinear_forward", lib.bitlinear_forward(
        _ptr(xq), _ptr(scale), _ptr(packed), _ptr(gamma), m, n, k,
        BL_EPI_RELU2 if relu2 else BL_EPI_NONE, _dtype_code(y.dtype), _ptr(y), _ptr(acc),
        _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))
    return (y, acc) if acc_out else y


def forward_noalloc(xq, scale, packed, gamma, n: int, k: int, relu2: bool = False,
                    out_dtype=None, y=None, acc_out=None, stream=None):
    """bitlinear_forward_noalloc: bitlinear_forward without a workspace (the
    library's per-device scratch holds the split-K slots).  y and acc_out may
    be given as preallocated tensors; returns y."""
    import torch
    m = xq.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=out_dtype or torch.float32, device=xq.device)
    _check("bitlinear_forward_noalloc", lib.bitlinear_forward_noalloc(
        _ptr(xq), _ptr(scale), _ptr(packed), _ptr(gamma), m, n, k,
        BL_EPI_RELU2 if relu2 else BL_EPI_NONE, _dtype_code(y.dtype), _ptr(y), _ptr(acc_out),
        _stream(stream)))
    return y


class FusedStep:
    """A prepared bitlinear_forward_fused call: a table of BitLinear products
    sharing the token count m, each quantizing its own activations.

    ops: list of dicts with keys x, packed, gamma, n, k, y and optional
    relu2, acc_out, xq_out, scale_out (tensors on the device), rmsnorm (bool),
    norm_weight (fp32 [k] tensor or None), norm_eps."""

    def __init__(self, ops, eps: float = EPS_DEFAULT, workspace: Optional[Workspace] = None):
        if not 1 <= len(ops) <= BL_MAX_FUSED:
            raise ValueError(f"1..{BL_MAX_FUSED} entries")
        self.ops = ops
        self.m = int(ops[0]["x"].shape[0])
        self.eps = float(eps)
        arr = (BLLinear * len(ops))()
        for i, o in enumerate(ops):
            x, y = o["x"], o["y"]
            if x.shape[0] != self.m or y.shape != (self.m, o["n"]):
                raise ValueError("every entry needs x [m, k] and y [m, n] with the same m")
            arr[i] = BLLinear(_ptr(x), _dtype_code(x.dtype), _ptr(o["packed"]), _ptr(o["gamma"]),
                              int(o["n"]), int(o["k"]),
                              BL_EPI_RELU2 if o.get("relu2") else BL_EPI_NONE,
                              _dtype_code(y.dtype), _ptr(y), _ptr(o.get("acc_out")),
                              _ptr(o.get("xq_out")), _ptr(o.get("scale_out")),
                              1 if o.get("rmsnorm") else 0,
                              float(o.get("norm_eps", NORM_EPS_DEFAULT)),
                              _ptr(o.get("norm_weight")))
        self.arr = arr
        self.nbytes = int(lib.bitlinear_forward_fused_workspace_bytes(arr, len(ops), self.m))
        self.ws = workspace or Workspace(ops[0]["x"].device)
        self.ws.get(self.nbytes)

    def kernel(self) -> str:
        """Name of the kernel this step launches (KERNEL_NAMES)."""
        r = int(lib.bitlinear_forward_fused_kernel(self.arr, len(self.ops), self.m))
        if r < 0:
            _check("bitlinear_forward_fused_kernel", -r)
        return KERNEL_NAMES[r]

    def __call__(self, stream=None):
        ws = self.ws.get(self.nbytes, stream)
        _check("bitlinear_forward_fused", lib.bitlinear_forward_fused(
            self.arr, len(self.ops), self.m, self.eps, _ptr(ws), 0 if ws is None else ws.numel(),
            _stream(stream)))


def forward_multi(xq, scale, k: int, ops, workspace: Optional[Workspace] = None,
                  stream=None) -> None:
    """bitlinear_forward_multi: several products sharing x~ and s.

    ops: list of dicts with keys packed, gamma, n, y and optional relu2,
    acc_out (tensors on the device); y's dtype picks the output type."""
    if not 1 <= len(ops) <= BL_MAX_MULTI:
        raise ValueError(f"1..{BL_MAX_MULTI} entries")
    m = int(xq.shape[0])
    arr = (BLProduct * len(ops))()
    for e, o in zip(arr, ops):
        e.packed, e.gamma, e.n = _ptr(o["packed"]), _ptr(o["gamma"]), int(o["n"])
        e.epilogue = BL_EPI_RELU2 if o.get("relu2") else BL_EPI_NONE
        e.y_dtype, e.y = _dtype_code(o["y"].dtype), _ptr(o["y"])
        e.acc_out = _ptr(o.get("acc_out"))
    nbytes = int(lib.bitlinear_forward_multi_workspace_bytes(arr, len(ops), m, int(k)))
    ws = (workspace or _workspace_for(xq.device, stream)).get(nbytes, stream)
    _check("bitlinear_forward_multi", lib.bitlinear_forward_multi(
        _ptr(xq), _ptr(scale), m, int(k), arr, len(ops), _ptr(ws),
        0 if ws is None else ws.numel(), _stream(stream)))


def forward_fused(ops, eps: float = EPS_DEFAULT, workspace: Optional[Workspace] = None,
                  stream=None) -> None:
    """bitlinear_forward_fused over a list of entries (see FusedStep)."""
    FusedStep(ops, eps, workspace)(stream)


class BitLinearW158A8:
    """Inference-only BitLinear layer (ternary weights, int8 activations) on
    the library's kernels: the page's BitLinear(in_features, out_features,
    bias=False) without its training state ("BitNet b1.58 2B4T Guide",
    section "End-to-End Implementation: Building a Native BitLinear Layer").
    The weights are packed once (bitlinear_pack_weights); a call runs the
    RMSNorm (the listing's self.rms_norm, gain initialised to ones; off with
    rmsnorm=False), the per-token absmax quantization, the ternary x int8
    product and the rescale -- one fused launch up to BL_FUSED_MAX_M tokens,
    else the quantization and bitlinear_forward.  x: [..., in_features] fp32
    or bf16 on the device; returns [..., out_features] (out_dtype, default
    the dtype of x).  Argument marshalling only."""

    def __init__(self, in_features: int, out_features: int, bias: bool = False,
                 rmsnorm: bool = True, relu2: bool = False, eps: float = EPS_DEFAULT,
                 norm_eps: float = NORM_EPS_DEFAULT, out_dtype=None, device="cuda"):
        import torch
        if bias:
            raise ValueError("BitLinear W1.58A8 has no bias terms")
        self.in_features, self.out_features = int(in_features), int(out_features)
        self.rmsnorm, self.relu2 = bool(rmsnorm), bool(relu2)
        self.eps, self.norm_eps = float(eps), float(norm_eps)
        self.out_dtype, self.device = out_dtype, device
        self.norm_weight = torch.ones(self.in_features, dtype=torch.float32, device=device)
        self.packed = self.gamma = None
        self.workspace = Workspace(device)

    def load_weight(self, weight, eps: Optional[float] = None):
        """Pack W [out_features, in_features] (fp32 or bf16, on the device)."""
        if tuple(weight.shape) != (self.out_features, self.in_features):
            raise ValueError(f"weight must be [{self.out_features}, {self.in_features}]")
        self.packed, self.gamma = pack_weights(weight.contiguous(),
                                               self.eps if eps is None else eps)
        return self

    def __call__(self, x):
        import torch
        if self.packed is None:
            raise RuntimeError("no weights: call load_weight first")
        if x.shape[-1] != self.in_features:
            raise ValueError(f"x must end in {self.in_features}")
        lead = x.shape[:-1]
        x2 = x.reshape(-1, self.in_features).contiguous()
        m = x2.shape[0]
        ydt = self.out_dtype or x.dtype
        y = torch.empty((m, self.out_features), dtype=ydt, device=x.device)
        if m == 0:
            return y.reshape(*lead, self.out_features)
        if m <= BL_FUSED_MAX_M:
            FusedStep([dict(x=x2, packed=self.packed, gamma=self.gamma, n=self.out_features,
                            k=self.in_features, y=y, relu2=self.relu2, rmsnorm=self.rmsnorm,
                            norm_weight=self.norm_weight, norm_eps=self.norm_eps)],
                      eps=self.eps, workspace=self.workspace)()
        else:
            if self.rmsnorm:
                xq, s = rmsnorm_quant_act(x2, self.norm_weight, self.norm_eps, self.eps)
            else:
                xq, s = quant_act(x2, self.eps)
            forward(xq, s, self.packed, self.gamma, self.out_features, self.in_features,
                    relu2=self.relu2, y=y, workspace=self.workspace)
        return y.reshape(*lead, self.out_features)
