"""Plain CPU oracle for weight-only quantised decode linears.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the GPU
library and imports nothing from it.  It is deliberately slow and literal:
NumPy, float64 wherever the pages leave the precision open, no blocking and no
fusion, so that each step can be compared with the pages by eye.

Sources (the pages are cited by title and section):

* [ELG] "Open Origin - ELG Stream Layer" README, section "Technical
  Architecture": "INT8 Quantization & Direct Mapping" (the scale and int8
  equations) and "FP16 On-The-Fly GPU Reconstruction" (the reconstruction
  line).
* [OTF] "On-The-Fly Weight Synthesizer (OTF-LLM Engine)" PyPI page, section
  "Architecture & Key Innovations": the architecture diagram (global static
  permutation, 1% FP16 outlier channels, 99% INT4 background in [-7, +7], 2:1
  uint8 packing, zero-point 0, outlier GEMM plus background GEMM added into one
  FP16 output), innovation item 3 (top-1% channels by |W| x |X_profile|) and
  item 4 (INT8 vocabulary tables; an outlier-aware INT4 lm_head that may share
  the embedding matrix).

Readings where the pages are silent (each one is listed in the design notes):

* INT8 "per-parameter scaling" is one fp32 scale per weight tensor.
* "round" is round-half-to-even (the reconstruction line is PyTorch code, and
  PyTorch rounds half to even); W/scale is an IEEE fp32 division; codes are
  clamped to +-127 / +-7.
* the INT4 scale of a group is fp16(fp32(max|W_g| / 7)) over 128 consecutive
  background channels of one output row; codes are computed against that
  stored fp16 scale, so dequantisation is exactly code * scale.
* "1%" is ceil(K / 100) channels; the score of channel j is
  mean_t |X_profile[t, j]| * sum over every linear reading that input space of
  sum_n |W[n, j]|, in float64; ties go to the lower channel index.
* the permutation lists the background channels in ascending order, then the
  outlier channels in ascending order.
* a nibble holds a two's-complement code (zero-point 0), the low nibble of a
  byte is the even channel, packing runs along the input dimension.
* the background is zero-padded to a whole number of 128-channel groups.
* the INT8 vocabulary table uses the same per-tensor INT8 scheme; looking up a
  token applies the [ELG] reconstruction to its row: the code times the fp32
  scale evaluated in fp32, then rounded to fp16 (PyTorch evaluates half
  arithmetic in fp32).  A token id outside the table gives a zero row.

Parity status: every function here is pinned by the CPU tests (closed forms,
constructed ties, exhaustive nibble tables, exact integer products, planted-set
recovery and byte totals printed on the pages).  No page prints a worked
numeric example of a full product, so no end-to-end output value is pinned to
a number printed on a page.
"""
from __future__ import annotations

import numpy as np

GROUP = 128
INT8_QMAX = 127
INT4_QMAX = 7


# --------------------------------------------------------------------------
# [ELG] INT8 symmetric per-tensor quantisation
# --------------------------------------------------------------------------

def quantize_int8(W: np.ndarray, rows: np.ndarray | None = None):
    """[ELG] "INT8 Quantization & Direct Mapping": scale = max|W| / 127 and
    int8 = round(W / scale).

    W is float32 [N, K].  Returns (q int8 [N, K] (or [len(rows), K] when
    ``rows`` selects output rows; the scale still comes from the whole tensor),
    scale float32).  An all-zero tensor, or one whose scale underflows fp32, has
    scale 0 and all-zero codes; a non-finite weight raises ValueError.
    """
    W = np.asarray(W, dtype=np.float32)
    if not np.all(np.isfinite(W)):
        raise ValueError("non-finite weight")
    m = np.float32(np.max(np.abs(W))) if W.size else np.float32(0.0)
    sel = W if rows is None else W[np.asarray(rows)]
    s = np.float32(m / np.float32(INT8_QMAX))           # fp32 division
    if s == 0:                                          # all zero, or the scale underflows
        return np.zeros(sel.shape, np.int8), np.float32(0.0)
    t = sel / s                                           # fp32 IEEE division, elementwise
    q = np.clip(np.rint(t), -INT8_QMAX, INT8_QMAX)        # half to even
    return q.astype(np.int8), s


def dequantize_int8(q: np.ndarray, s) -> np.ndarray:
    """[ELG] "FP16 On-The-Fly GPU Reconstruction": weight = int8 * scale.

    Returned exactly, in float64 (the page rounds the product to fp16; the
    oracle keeps the exact product so that any kernel that factors the scale
    out of the sum is compared against the same value)."""
    return np.asarray(q, np.float64) * np.float64(s)


def linear_int8(q: np.ndarray, s, x: np.ndarray) -> np.ndarray:
    """y[b, n] = sum_k (q[n, k] * s) * x[b, k]  (x fp16 [b, K], output float64 [b, N])."""
    return np.asarray(x, np.float64) @ dequantize_int8(q, s).T


def linear_int8_abs(q: np.ndarray, s, x: np.ndarray) -> np.ndarray:
    """sum_k |q[n, k] * s| * |x[b, k]| in float64 [b, N]: the scale of the
    rounding error a floating-point evaluation of linear_int8 can make in
    element (b, n) (the denominator of the componentwise error)."""
    return np.abs(np.asarray(x, np.float64)) @ np.abs(dequantize_int8(q, s)).T


def embed_int8(q: np.ndarray, s, ids) -> np.ndarray:
    """[OTF] item 4 (INT8 vocabulary tables) with the [ELG] "FP16 On-The-Fly
    GPU Reconstruction" applied to the looked-up rows.

    q int8 [V, H] and s are the table's INT8 codes and scale (quantize_int8 of
    the embedding matrix); ids int [b].  Returns fp16 [b, H]:
    fp16(fp32(q[id, :] * s)), both roundings to nearest even.  The product of
    a code (at most 7 bits) and an fp32 scale is exact in float64, so the two
    casts below are exactly the two roundings.  Rows of ids outside [0, V)
    are zero.
    """
    q = np.asarray(q)
    ids = np.asarray(ids, np.int64).reshape(-1)
    V, H = q.shape
    out = np.zeros((ids.size, H), np.float16)
    s64 = np.float64(np.float32(s))
    for r, t in enumerate(ids):
        if 0 <= t < V:
            exact = q[t].astype(np.float64) * s64
            with np.errstate(over="ignore"):                 # overflow gives +-inf, as intended
                out[r] = exact.astype(np.float32).astype(np.float16)
    return out


# --------------------------------------------------------------------------
# [OTF] outlier-aware INT4
# --------------------------------------------------------------------------

def n_outliers(K: int) -> int:
    """[OTF] item 3 / diagram: the top 1% of input channels, rounded up."""
    return (K + 99) // 100


def int4o_geometry(K: int, n_out: int | None = None, group: int = GROUP) -> dict:
    """Sizes of the split: K_bg background channels in G groups of ``group``,
    zero-padded to K_pad = G * group."""
    n_out = n_outliers(K) if n_out is None else n_out
    K_bg = K - n_out
    G = -(-K_bg // group)
    return {"K": K, "n_out": n_out, "K_bg": K_bg, "G": G, "K_pad": G * group, "group": group}


def column_abs_sum(W: np.ndarray) -> np.ndarray:
    """sum_n |W[n, j]| in float64 for every input channel j of one linear."""
    return np.abs(np.asarray(W, np.float64)).sum(axis=0)


def space_column_abs_sum(Ws) -> np.ndarray:
    """[OTF] item 3 over a whole model: the float64 sum, over every linear in
    ``Ws`` (all reading one input space, all layers), of column_abs_sum."""
    Ws = list(Ws)
    total = np.zeros(np.asarray(Ws[0]).shape[1], np.float64)
    for W in Ws:
        total = total + column_abs_sum(W)
    return total


def outlier_scores(colabs: np.ndarray, xprof: np.ndarray) -> np.ndarray:
    """[OTF] item 3: channel importance |W| x |X_profile|.

    ``colabs`` is the float64 sum of column_abs_sum over every linear that
    reads this input space (all layers: one table for the whole model);
    ``xprof`` is the fp16 activation profile [T, K]."""
    mean_absx = np.abs(np.asarray(xprof, np.float64)).mean(axis=0)
    return mean_absx * np.asarray(colabs, np.float64)


def select_outliers(scores: np.ndarray, n_out: int) -> np.ndarray:
    """The n_out channels with the largest score (ties: lower index first),
    returned in ascending channel order."""
    K = scores.shape[0]
    order = np.lexsort((np.arange(K), -np.asarray(scores, np.float64)))
    return np.sort(order[:n_out]).astype(np.int64)


def global_perm(K: int, outliers: np.ndarray) -> np.ndarray:
    """[OTF] diagram "Global Static Permutation": background channels in
    ascending order followed by the outlier channels in ascending order."""
    is_out = np.zeros(K, bool)
    is_out[np.asarray(outliers, np.int64)] = True
    bg = np.flatnonzero(~is_out)
    return np.concatenate([bg, np.sort(np.flatnonzero(is_out))]).astype(np.int32)


def quantize_int4o(W: np.ndarray, perm: np.ndarray, n_out: int, group: int = GROUP):
    """[OTF] diagram: outlier columns kept as pure FP16, background columns as
    INT4 in [-7, +7] with zero-point 0 and one fp16 scale per output row per
    ``group`` background channels.

    W is float32 [N, K] in original channel order.  Returns
    (codes int8 [N, K_pad] in [-7, 7] with zero padding,
     scales float16 [N, G], w_out float16 [N, n_out]).
    Raises ValueError for a non-finite weight or a group scale that overflows fp16.
    """
    W = np.asarray(W, np.float32)
    if not np.all(np.isfinite(W)):
        raise ValueError("non-finite weight")
    N, K = W.shape
    geo = int4o_geometry(K, n_out, group)
    K_bg, G, K_pad = geo["K_bg"], geo["G"], geo["K_pad"]
    Wp = W[:, np.asarray(perm, np.int64)]
    w_out = Wp[:, K_bg:].astype(np.float16)
    codes = np.zeros((N, K_pad), np.int8)
    scales = np.zeros((N, G), np.float16)
    for g in range(G):
        lo, hi = g * group, min(g * group + group, K_bg)
        blk = Wp[:, lo:hi]
        m = np.max(np.abs(blk), axis=1)                           # fp32, per output row
        with np.errstate(over="ignore"):                          # overflow is reported just below
            s16 = (m / np.float32(INT4_QMAX)).astype(np.float16)  # fp32 division, then fp16
        if not np.all(np.isfinite(s16)):
            raise ValueError("group scale overflows fp16")
        s32 = s16.astype(np.float32)
        with np.errstate(divide="ignore", invalid="ignore"):
            t = blk / s32[:, None]                                 # fp32 IEEE division
        q = np.where(s32[:, None] == 0, 0.0, np.clip(np.rint(t), -INT4_QMAX, INT4_QMAX))
        codes[:, lo:hi] = q.astype(np.int8)
        scales[:, g] = s16
    return codes, scales, w_out


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """[OTF] diagram "2:1 Packing (uint8)": byte j of a row holds code 2j in
    its low nibble and code 2j+1 in its high nibble, two's complement."""
    c = np.asarray(codes, np.int16)
    assert c.shape[-1] % 2 == 0
    lo = c[..., 0::2] & 0xF
    hi = c[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_int4: nibble v in 0..15 means v - 16 when v >= 8."""
    p = np.asarray(packed, np.int16)
    lo = p & 0xF
    hi = (p >> 4) & 0xF
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.int16)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    out = np.where(out >= 8, out - 16, out)
    return out.astype(np.int8)


def permute_split(x: np.ndarray, perm: np.ndarray, n_out: int, group: int = GROUP):
    """[OTF] diagram: permute the input vector with the global table, then
    split it into the background part (zero-padded to K_pad) and the outlier
    part.  x is fp16 [b, K]; returns (x_bg fp16 [b, K_pad], x_out fp16 [b, n_out])."""
    x = np.asarray(x, np.float16)
    b, K = x.shape
    geo = int4o_geometry(K, n_out, group)
    xp = x[:, np.asarray(perm, np.int64)]
    x_bg = np.zeros((b, geo["K_pad"]), np.float16)
    x_bg[:, : geo["K_bg"]] = xp[:, : geo["K_bg"]]
    return x_bg, np.ascontiguousarray(xp[:, geo["K_bg"]:])


def dequantize_int4o(codes: np.ndarray, scales: np.ndarray, group: int = GROUP) -> np.ndarray:
    """Background weights code * scale, exactly, in float64 [N, K_pad]."""
    N, K_pad = codes.shape
    G = scales.shape[1]
    assert K_pad == G * group
    c = np.asarray(codes, np.float64).reshape(N, G, group)
    return (c * np.asarray(scales, np.float64)[:, :, None]).reshape(N, K_pad)


def linear_int4o(codes, scales, w_out, x_bg, x_out, group: int = GROUP) -> np.ndarray:
    """[OTF] diagram "Continuous GEMM Addition": y = X_out W_out^T + X_bg deq(W_bg)^T.

    All inputs as returned by quantize_int4o / permute_split; output float64 [b, N]."""
    y_bg = np.asarray(x_bg, np.float64) @ dequantize_int4o(codes, scales, group).T
    y_out = np.asarray(x_out, np.float64) @ np.asarray(w_out, np.float64).T
    return y_out + y_bg


def linear_int4o_abs(codes, scales, w_out, x_bg, x_out, group: int = GROUP) -> np.ndarray:
    """linear_int4o with every term taken in absolute value, float64 [b, N]:
    sum_i |w_out[n, i] x_out[i]| + sum_k |deq[n, k] x_bg[k]|."""
    y_bg = np.abs(np.asarray(x_bg, np.float64)) @ np.abs(dequantize_int4o(codes, scales, group)).T
    y_out = np.abs(np.asarray(x_out, np.float64)) @ np.abs(np.asarray(w_out, np.float64)).T
    return y_out + y_bg


def reconstruct_int4o(codes, scales, w_out, perm, group: int = GROUP) -> np.ndarray:
    """The dequantised weight matrix in original channel order, float64 [N, K]."""
    N = codes.shape[0]
    n_out = w_out.shape[1]
    K = perm.shape[0]
    K_bg = K - n_out
    Wp = np.concatenate([dequantize_int4o(codes, scales, group)[:, :K_bg],
                         np.asarray(w_out, np.float64)], axis=1)
    W = np.empty((N, K), np.float64)
    W[:, np.asarray(perm, np.int64)] = Wp
    return W


# --------------------------------------------------------------------------
# bookkeeping
# --------------------------------------------------------------------------

def algorithmic_bytes_int8(N: int, K: int, b: int) -> int:
    """Bytes an INT8 linear must move per call: codes, one fp32 scale, fp16 x and y."""
    return N * K + 4 + 2 * b * (K + N)


def algorithmic_bytes_int4o(N: int, K: int, b: int, n_out: int | None = None, group: int = GROUP) -> int:
    """Bytes an outlier-INT4 linear must move per call: packed background codes
    (unpadded), fp16 group scales, fp16 outlier columns, fp16 x and y."""
    geo = int4o_geometry(K, n_out, group)
    return (N * geo["K_bg"]) // 2 + 2 * N * geo["G"] + 2 * N * geo["n_out"] + 2 * b * (K + N)


def normwise_rel_err(y, yref) -> float:
    """max|y - yref| / max|yref| (0 when both are all zero)."""
    y = np.asarray(y, np.float64)
    yref = np.asarray(yref, np.float64)
    den = np.max(np.abs(yref)) if yref.size else 0.0
    num = np.max(np.abs(y - yref)) if yref.size else 0.0
    if den == 0:
        return 0.0 if num == 0 else float("inf")
    return float(num / den)


def componentwise_rel_err(y, yref, absref) -> float:
    """max over the elements with absref > 0 of |y - yref| / absref, where
    absref is the sum of the absolute terms of each output (linear_*_abs):
    the componentwise relative error of a summation.  Elements whose terms are
    all zero are left out (0 when none remain)."""
    y = np.asarray(y, np.float64)
    yref = np.asarray(yref, np.float64)
    absref = np.asarray(absref, np.float64)
    m = absref > 0
    if not np.any(m):
        return 0.0
    return float(np.max(np.abs(y - yref)[m] / absref[m]))
