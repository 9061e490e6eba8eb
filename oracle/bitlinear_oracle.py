"""CPU oracle for the BitLinear W1.58A8 forward pass.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only the tests, the smoke check
in ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
or run this module.  It shares no code with the HIP library (no kernels,
headers, tables or helpers); both sides only receive the same seeded inputs.

The oracle is plain numpy, written for a reader to check by eye against the
pages.  Sources (page title, then the section or equation):

  [P1] "BitNet b1.58 2B4T Guide: Scaling Native 1-Bit LLMs"
       - "Ternary Weight Quantization: absmean Scaling": gamma = mean |W_ij|
         over all d_out*d_in entries; W~ = Clip(Round(W/(gamma+eps)), -1, 1).
       - "8-Bit Activation Quantization: absmax Scaling": beta = max_j |x_j|
         per token; x~ = Clip(Round(x*Q_b/(beta+eps)), ...), Q_b = 127.
       - "Matrix Multiplication as Pure Integer Addition": y = (x~ W~^T) *
         beta*gamma/Q_b, and the sum over W~=+1 minus the sum over W~=-1.
       - "End-to-End Implementation: Building a Native BitLinear Layer"
         (the PyTorch listing): eps = 1e-5, torch.round (half to even),
         activations clamped to [-128, 127] after multiplying by 127/beta.
  [P2] winbuzzer.com, "Microsoft Releases BitNet b1.58 2B4T", section
       "Under the Hood: The BitNet Approach": per-token absmax int8
       activations (W1.58A8), ReLU^2 in the FFN, no bias terms; section "The
       Catch": GPU kernels must pack and unpack the weights.

Readings where the pages are silent or disagree (each is listed, with its
reason, in the design notes of the repository):

  R1  eps = 1e-5 (the only value the pages give), passed in as an argument.
  R2  weight divisor d = fp32(gamma + eps), as in the equation, not the
      listing's max(gamma, 1e-5).
  R3  activation scale s = fp32(127 / max(beta, eps)) (the listing's clamp),
      then x~ = clamp(rint(fp32(x * s)), -128, 127).
  R4  "Round" is round-half-to-even (torch.round, np.rint).
  R5  gamma is accumulated in fp64 and rounded once to fp32.
  R6  the output is y = acc * gamma / s evaluated in fp64, ReLU^2 (when
      asked) applied in fp64, then rounded once to fp32 and, for a bf16
      output, fp32 -> bf16 round-to-nearest-even.
  R7  the 2-bit packing layout is this library's own (the pages only say
      that weights are packed two bits each); it is specified in
      ``pack_ternary`` below and in the C header.
  R8  the activation eps must be positive with fp32(127/eps) finite; then
      s is finite for every token, an all-zero token quantizes to x~ = 0
      and y = 0.  eps = 0 (or a value whose 127/eps overflows) is refused.
  R9  the RMSNorm ahead of the activation quant (the listing's
      nn.RMSNorm(in_features), with torch's defaults: eps = fp32 machine
      epsilon 2^-23, a weight vector initialised to ones, out =
      x * rsqrt(mean(x^2) + eps) * weight): mean(x^2) is the exact sum of the
      squares (fp64, correctly rounded) over K, rounded to fp32; r =
      fp32(1 / sqrt(fp32(ms + eps))) evaluated in fp64; y = fp32(fp32(x * r)
      * w).  The norm eps must be positive and finite.

Floating point that decides an integer (codes and int8 activations) is done
in fp32, the precision of the pages' listing (torch's default dtype).
"""
from __future__ import annotations

import numpy as np

EPS_DEFAULT = np.float32(1e-5)
QB = np.float32(127.0)

ROW_BLOCK = 64      # rows per packed block
SUPER_K = 256       # k values per packed super-chunk


# ---------------------------------------------------------------------------
# Sizes of the packed layout (R7)
# ---------------------------------------------------------------------------
def padded_n(n: int) -> int:
    return ROW_BLOCK * ((n + ROW_BLOCK - 1) // ROW_BLOCK)


def padded_k(k: int) -> int:
    return SUPER_K * ((k + SUPER_K - 1) // SUPER_K)


def packed_bytes(n: int, k: int) -> int:
    return padded_n(n) * padded_k(k) // 4


# ---------------------------------------------------------------------------
# Step 1: absmean scale  [P1 "Ternary Weight Quantization", gamma equation]
# ---------------------------------------------------------------------------
def absmean_gamma(w: np.ndarray) -> np.float32:
    """gamma = (1/(d_out*d_in)) * sum_ij |W_ij|, one scalar per tensor.

    Accumulated in fp64 (numpy's sum of a float64 array) and rounded once to
    fp32 (R5).  Every |W_ij| is an fp32 value, exact in fp64."""
    w = np.asarray(w, dtype=np.float32)
    if w.size == 0:
        raise ValueError("gamma of an empty weight tensor is undefined")
    s = np.abs(w.astype(np.float64)).sum()
    return np.float32(s / np.float64(w.size))


# ---------------------------------------------------------------------------
# Step 2: ternary codes  [P1 "Ternary Weight Quantization", W~ equation]
# ---------------------------------------------------------------------------
def ternary_codes(w: np.ndarray, gamma, eps=EPS_DEFAULT,
                  divisor: str = "gamma_plus_eps") -> np.ndarray:
    """W~ = Clip(Round(W / (gamma + eps)), -1, 1) as int8.

    fp32 throughout: d = fp32(gamma + eps), q = fp32(W / d) (IEEE division),
    Round = rint (half to even, R4), then clip.  ``divisor="max"`` gives the
    listing's max(gamma, eps) form instead; it exists only so tests can show
    where the two readings part (R2).  When d == 0 (all-zero W with eps == 0)
    every weight is zero and so is every code."""
    w = np.asarray(w, dtype=np.float32)
    g = np.float32(gamma)
    e = np.float32(eps)
    if divisor == "gamma_plus_eps":
        d = np.float32(g + e)
    elif divisor == "max":
        d = np.maximum(g, e)
    else:
        raise ValueError(divisor)
    if d == 0:
        return np.zeros(w.shape, dtype=np.int8)
    with np.errstate(over="ignore"):
        q = w / d                                  # fp32 / fp32 -> fp32
    r = np.rint(q)
    return np.clip(r, -1.0, 1.0).astype(np.int8)


# ---------------------------------------------------------------------------
# Packing (R7).  The pages: weights are packed two bits each for GPU kernels
# [P2 "The Catch"]; the layout itself is this library's.
#
#   N_pad = 64*ceil(N/64), K_pad = 256*ceil(K/256), NC = K_pad/256.
#   For weight (n, k):  b = n // 64, r = n % 64, c = k // 256,
#                       kk = k % 256 = 64*j + 16*q + t   (j, q in 0..3, t in 0..15)
#   it lives in 32-bit little-endian word
#        word = (((b*NC + c)*4 + q)*64 + r)*4 + j
#   at bits [8*(t % 4) + 2*(t // 4), +2), as a 2-bit two's complement number:
#        0 -> 0b00, +1 -> 0b01, -1 -> 0b11   (0b10 is never written).
#   Rows n >= N and columns k >= K are zero codes.
# ---------------------------------------------------------------------------
def packed_word_index(n: int, k: int, n_rows: int, k_cols: int):
    """(word index, bit shift) of weight (n, k) in the packed buffer."""
    nc = padded_k(k_cols) // SUPER_K
    b, r = divmod(n, ROW_BLOCK)
    c, kk = divmod(k, SUPER_K)
    j, rem = divmod(kk, 64)
    q, t = divmod(rem, 16)
    word = (((b * nc + c) * 4 + q) * 64 + r) * 4 + j
    shift = 8 * (t % 4) + 2 * (t // 4)
    return word, shift


def _code_to_field(codes: np.ndarray) -> np.ndarray:
    c = codes.astype(np.int64)
    if np.any((c < -1) | (c > 1)):
        raise ValueError("codes must be in {-1, 0, +1}")
    return np.where(c == 1, 1, np.where(c == -1, 3, 0)).astype(np.uint32)


def pack_ternary(codes: np.ndarray) -> np.ndarray:
    """Pack int8 codes [N, K] into the layout above; returns uint8 bytes."""
    codes = np.asarray(codes)
    n, k = codes.shape
    npad, kpad = padded_n(n), padded_k(k)
    full = np.zeros((npad, kpad), dtype=np.int8)
    full[:n, :k] = codes
    field = _code_to_field(full)
    nb, nc = npad // ROW_BLOCK, kpad // SUPER_K
    # k = 256*c + 64*j + 16*q + 4*i + e, with t = 4*i + e (e = t % 4, i = t // 4)
    f = field.reshape(nb, ROW_BLOCK, nc, 4, 4, 4, 4)      # b, r, c, j, q, i, e
    shift = (8 * np.arange(4)[None, :] + 2 * np.arange(4)[:, None]).astype(np.uint32)  # [i, e]
    words = (f << shift).sum(axis=(5, 6), dtype=np.uint64).astype(np.uint32)  # b, r, c, j, q
    words = words.transpose(0, 2, 4, 1, 3)                 # b, c, q, r, j
    return np.ascontiguousarray(words).reshape(-1).view(np.uint8)


def unpack_ternary(packed: np.ndarray, n: int, k: int, rows=None) -> np.ndarray:
    """Inverse of ``pack_ternary`` by direct lookup of every (n, k); with
    ``rows`` only those rows of the N x K matrix are read."""
    words = np.ascontiguousarray(packed).view(np.uint32)
    row_ids = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    nn, kk = np.meshgrid(row_ids, np.arange(k), indexing="ij")
    nc = padded_k(k) // SUPER_K
    b, r = nn // ROW_BLOCK, nn % ROW_BLOCK
    c, rem256 = kk // SUPER_K, kk % SUPER_K
    j, rem = rem256 // 64, rem256 % 64
    q, t = rem // 16, rem % 16
    idx = (((b * nc + c) * 4 + q) * 64 + r) * 4 + j
    sh = 8 * (t % 4) + 2 * (t // 4)
    field = (words[idx] >> sh.astype(np.uint32)) & np.uint32(3)
    if np.any(field == 2):
        raise ValueError("reserved 2-bit pattern 0b10 found")
    return np.where(field == 1, 1, np.where(field == 3, -1, 0)).astype(np.int8)


# ---------------------------------------------------------------------------
# Step 3: activation quantization  [P1 "8-Bit Activation Quantization"]
# ---------------------------------------------------------------------------
def quant_act(x: np.ndarray, eps=EPS_DEFAULT):
    """Per-token absmax int8 quantization (R3, R4).

    beta_m = max_j |x_mj| (fp32); s_m = fp32(127 / max(beta_m, eps));
    x~ = clamp(rint(fp32(x * s_m)), -128, 127).  Returns (x~ int8 [M, K],
    s fp32 [M]).

    eps must be positive with fp32(127 / eps) finite (R8): the page's
    listing only ever clamps beta at a positive eps, and with eps = 0 an
    all-zero token would give s = 127/0 = inf and x * s = 0 * inf = NaN, a
    result no rounding rule defines.  Other values raise ValueError."""
    e32 = np.float32(eps)
    with np.errstate(divide="ignore", over="ignore"):
        smax = QB / e32 if e32 > 0 else np.float32(np.inf)
    if not (np.isfinite(e32) and e32 > 0 and np.isfinite(smax)):
        raise ValueError(f"activation eps must be > 0 with 127/eps finite in fp32, got {eps!r}")
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("x must be [M, K]")
    m, k = x.shape
    if k == 0:
        beta = np.zeros(m, dtype=np.float32)
    else:
        beta = np.abs(x).max(axis=1)
    s = QB / np.maximum(beta, np.float32(eps))       # fp32 / fp32 -> fp32
    prod = x * s[:, None]                            # fp32 * fp32 -> fp32
    xq = np.clip(np.rint(prod), -128.0, 127.0).astype(np.int8)
    return xq, s.astype(np.float32)


# ---------------------------------------------------------------------------
# RMSNorm ahead of the activation quant [P1 listing, BitLinear.forward step 1:
# self.rms_norm = nn.RMSNorm(in_features) applied to x; P2 "Under the Hood":
# subln normalization; P3 "Mathematical Foundations": the five-step flow
# begins by normalizing the input activations] (R9).
# ---------------------------------------------------------------------------
NORM_EPS_DEFAULT = np.float32(2.0 ** -23)      # fp32 machine epsilon


def mean_square(x_row) -> np.float32:
    """fp32(fp64(sum of x_j^2) / K): the squares of fp32 values are exact in
    fp64 and math.fsum returns their exact sum correctly rounded to fp64."""
    import math
    r = np.asarray(x_row, dtype=np.float32).astype(np.float64)
    s = math.fsum((r * r).tolist())
    return np.float32(s / np.float64(r.size))


def rmsnorm(x: np.ndarray, weight=None, eps=NORM_EPS_DEFAULT, ms=None) -> np.ndarray:
    """y = x * r * w per token with r = 1/sqrt(mean(x^2) + eps) (R9).

    Returns fp32 [M, K].  ``weight`` is the fp32 [K] gain (None: ones, the
    listing's initial value).  ``ms`` may give the per-token fp32 mean
    squares (for a caller that checks a neighbouring rounding); by default
    they come from mean_square."""
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("x must be [M, K]")
    e = np.float32(eps)
    if not (np.isfinite(e) and e > 0):
        raise ValueError(f"norm eps must be positive and finite, got {eps!r}")
    m, k = x.shape
    w = np.ones(k, np.float32) if weight is None else np.asarray(weight, dtype=np.float32)
    if w.shape != (k,):
        raise ValueError("weight must be [K]")
    ms = np.array([mean_square(x[i]) for i in range(m)], np.float32) if ms is None \
        else np.asarray(ms, np.float32)
    v = (ms + e).astype(np.float32)                               # fp32 add
    r = (1.0 / np.sqrt(v.astype(np.float64))).astype(np.float32)  # fp64, rounded once
    xr = (x * r[:, None]).astype(np.float32)                      # fp32 multiply
    return (xr * w[None, :]).astype(np.float32)                   # fp32 multiply


# ---------------------------------------------------------------------------
# Step 4: integer contraction  [P1 "Matrix Multiplication as Pure Integer
# Addition"]:  acc[i, k] = sum_j x~[i, j] * W~[k, j]
# ---------------------------------------------------------------------------
def contract(xq: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """acc = x~ W~^T, exact, returned as int32 [M, N].

    The product is taken as a float64 matmul.  That is exact here: every
    factor is an integer with |x~| <= 128 and |W~| <= 1, so every partial sum
    in any order is an integer of magnitude <= 128*K < 2**53 and no float64
    addition rounds.  The int32 range is then checked, as the pages name an
    integer accumulator."""
    xq = np.asarray(xq)
    codes = np.asarray(codes)
    k = xq.shape[1]
    if codes.shape[1] != k:
        raise ValueError("inner dimensions differ")
    if 128 * k >= 2 ** 53:
        raise ValueError("K too large for an exact float64 contraction")
    acc = xq.astype(np.float64) @ codes.astype(np.float64).T
    if acc.size and np.abs(acc).max() >= 2 ** 31:
        raise OverflowError("accumulator leaves int32")
    return acc.astype(np.int64).astype(np.int32)


def contract_addsub(xq: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """The same product written as the page's second form: the sum of x~ over
    W~ = +1 minus the sum over W~ = -1 (int64 sums)."""
    xq = np.asarray(xq).astype(np.int64)
    codes = np.asarray(codes)
    plus = (codes == 1).astype(np.int64)
    minus = (codes == -1).astype(np.int64)
    m, n = xq.shape[0], codes.shape[0]
    out = np.zeros((m, n), dtype=np.int64)
    for i in range(m):
        out[i] = (plus * xq[i][None, :]).sum(axis=1) - (minus * xq[i][None, :]).sum(axis=1)
    return out.astype(np.int32)


# ---------------------------------------------------------------------------
# Step 5: dequantization [P1 "Matrix Multiplication as Pure Integer Addition",
# the rescale by beta*gamma/Q_b; with s = Q_b/beta that is gamma/s] and the
# FFN's ReLU^2 [P2 "Under the Hood"].
# ---------------------------------------------------------------------------
def dequant(acc: np.ndarray, gamma, s: np.ndarray, relu2: bool = False) -> np.ndarray:
    """y = acc * gamma / s_m in float64 (R6); ReLU^2 = max(y, 0)^2."""
    y = np.asarray(acc, dtype=np.float64) * np.float64(np.float32(gamma))
    y = y / np.asarray(s, dtype=np.float32).astype(np.float64)[:, None]
    if relu2:
        y = np.where(y > 0, y * y, 0.0)
    return y


def f32_to_bf16_bits(y32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 with round-to-nearest-even, as uint16 bit patterns.

    Keep the top 16 bits; add half of the dropped range, plus one when the
    kept part is odd, so that exact halves go to the even neighbour."""
    u = np.ascontiguousarray(y32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(np.asarray(y32, dtype=np.float32))
    out[nan] = np.uint16(0x7FC0)
    return out


def round_output(y64: np.ndarray, y_dtype: str) -> np.ndarray:
    """Round the float64 output once to fp32; bf16 output then rounds that
    fp32 value to bf16 (returned as uint16 bits)."""
    y32 = np.asarray(y64, dtype=np.float64).astype(np.float32)
    if y_dtype == "f32":
        return y32
    if y_dtype == "bf16":
        return f32_to_bf16_bits(y32)
    raise ValueError(y_dtype)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# The whole pass (P1's figure "The BitLinear Computation Pipeline", without the
# listing's RMSNorm and bias, which the pass excludes).
# ---------------------------------------------------------------------------
def forward(x: np.ndarray, w: np.ndarray, eps=EPS_DEFAULT, relu2: bool = False,
            y_dtype: str = "f32", gamma=None, act_eps=None, norm=False, norm_weight=None,
            norm_eps=NORM_EPS_DEFAULT, norm_ms=None):
    """Returns a dict with every intermediate of the pass.  ``eps`` serves
    both quantizers unless ``act_eps`` gives the activations their own; with
    ``norm`` the activations go through rmsnorm first (the listing's order)."""
    g = absmean_gamma(w) if gamma is None else np.float32(gamma)
    codes = ternary_codes(w, g, eps)
    xn = rmsnorm(x, norm_weight, norm_eps, norm_ms) if norm else x
    xq, s = quant_act(xn, eps if act_eps is None else act_eps)
    acc = contract(xq, codes)
    y64 = dequant(acc, g, s, relu2)
    return {"gamma": g, "codes": codes, "xq": xq, "s": s, "acc": acc,
            "y64": y64, "y": round_output(y64, y_dtype)}
