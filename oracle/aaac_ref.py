"""Plain fp64 CPU oracle for activation-aware adaptive dual-codebook (AAAC) 4-bit weight quantization.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the bench's CPU-baseline leg may import
this module. It shares no code with the HIP package and imports nothing from it; the two meet only
through the seeded inputs in ``synth``.

Source: the gist.science summary page "기술 요약: AAAC (활성화 인식 적응형 코드북)"
(arXiv 2605.08692), cited below as "AAAC summary" with its section:
  §1 problem statement (fixed 4-bit grids; dequantized values decide what inference uses),
  §2 method, mechanisms 1 (two adaptive tables with the format's entry count, 15 for NVFP4 and 16
     for INT4), 2 (per-group table choice by activation-weighted error, importance
     I_k = sum_t X[t,k]^2), 3 (BF16 tables, selector in the sign bit of the positive group scale,
     selection group S vs scale group g), 4 (quantile init with T1 shifted half a step; alternate
     assign and activation-weighted k-means refine),
  §4 results (NVFP4 g=16 and INT4 g=128 layouts; S=16 costs 0.0625 bit per weight).

Notation: W is [R, C] (out, in), row-major; a scale group is g consecutive weights of a row, a
selection group S consecutive weights (S | g | C); I is [C]; T[c] (c = 0, 1) has n entries;
u = w / s is the normalized weight.

Readings taken where the page is silent (each is restated where it is used):
  R1  s = max |w| over the scale group (bf16-exact); u = 0 when s = 0; zero is unsigned (+0).
  R2  one table pair per weight matrix; groups run along the input dimension.
  R3  init ranks: T0[j] = V[floor((2j+1) N / 2n)], T1[j] = V[min(N-1, floor((j+1) N / n))] over the
      ascending sorted u of the whole matrix (no interpolation, unweighted).
  R4  nearest entry: argmin_j (u - T[j])^2, ties to the lowest j.
  R5  selection error E_c(H) = sum_{k in H} I_k (w_k - s T_c[q_c(k)])^2; sigma = 1 iff E_1 < E_0.
  R6  refine: T_c[j] <- sum I s w / sum I s^2 over the cell (sigma = c, q = j), i.e. the
      I s^2-weighted centroid of u; an empty cell keeps its entry.
  R7  loop: iters x (assign, refine), then tables rounded to bf16 (ties to even), then a final
      assign against the rounded tables.
  R8  storage: code byte = q[2i] | q[2i+1] << 4; S == g: scale word = bf16(s) | sigma << 15;
      S < g: scale sign 0 and an LSB-first bitmap over the row-major selection groups.
  R9  dequant: w_hat = bf16(|s| * T~_sigma[q]).
  R14 decode GEMV: y = sum_c |s| T~_sigma[q] x_c with the exact product of scale and entry; the
      bf16 rounding of R9 belongs to materializing W_hat, which the GEMV never does.
  R15 AWQ composition: quantize bf16(W * a) with importance I / a^2 for a caller-given a > 0.

Pins (tests/test_oracle_pins.py): every function below is pinned against something other than
itself -- torch's bf16 conversion, integer-exact sums, np.partition, exhaustive code search on tiny
groups, the single-table round-to-nearest special case, scikit-learn's weighted Lloyd step, the
monotone-error invariant, and the page's storage figures (tests/golden/). No function here is
parity-unpinned; the converged end-to-end values themselves are not printed on the page and are
only constrained through those pins.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_round", "bf16_bits", "bits_to_float",
    "importance", "group_scales", "normalized",
    "init_tables", "nearest", "assign", "refine_sums", "refine_update", "refine",
    "total_error", "quantize", "pack", "dequant", "storage_bytes",
    "decoded_weights", "gemv", "awq_prescale",
]


# ----------------------------------------------------------------------------------------------
# bf16 (1 sign, 8 exponent, 7 fraction bits) written from the IEEE-754 rounding definition.
# ----------------------------------------------------------------------------------------------

def bf16_round(x):
    """Round to the nearest bfloat16 value, ties to even, overflow to infinity; keeps the sign of
    zero. Exact fp64 arithmetic: the quantum of each binade is a power of two.
    (AAAC summary §2 mechanism 3: table entries are stored as BF16.)"""
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    nz = (x != 0) & np.isfinite(x)
    ax = np.abs(x[nz])
    _, e = np.frexp(ax)                 # ax = m 2^e, m in [0.5, 1)  ->  2^(e-1) <= ax < 2^e
    e = np.maximum(e - 1, -126)         # subnormals share the quantum of the lowest binade
    quantum = np.ldexp(1.0, e - 7)      # 8 significant bits
    r = np.rint(ax / quantum) * quantum  # np.rint: round half to even
    r = np.where(r >= 2.0 ** 128, np.inf, r)
    out[nz] = np.copysign(r, x[nz])
    return out


def bf16_bits(x):
    """uint16 bit patterns of values that are already bf16-exact."""
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)
    if not np.array_equal(f.astype(np.float64), x, equal_nan=True):
        raise ValueError("value is not representable in fp32")
    b = f.view(np.uint32)
    if np.any(b & 0xFFFF):
        raise ValueError("value is not bf16-exact")
    return (b >> 16).astype(np.uint16)


def bits_to_float(bits):
    """fp64 values of uint16 bf16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------------------------
# Importance (AAAC summary §2 mechanism 2): I_k = sum_t X[t, k]^2 over the calibration tokens.
# ----------------------------------------------------------------------------------------------

def importance(X):
    """fp64 [K] column sums of squares of the calibration activations X [T, K]."""
    X = np.asarray(X, dtype=np.float64)
    return np.sum(X * X, axis=0)


# ----------------------------------------------------------------------------------------------
# Group scale and normalized weights (reading R1; "positive scale" in §2 mechanism 3,
# "normalized weight distribution" in §2 mechanism 4).
# ----------------------------------------------------------------------------------------------

def _check_shape(W, g, S=None):
    R, C = W.shape
    if C % g:
        raise ValueError("C must be a multiple of g")
    if S is not None and g % S:
        raise ValueError("g must be a multiple of S")
    return R, C


def group_scales(W, g):
    """s [R, C/g] = max |w| over each scale group."""
    W = np.asarray(W, dtype=np.float64)
    R, C = _check_shape(W, g)
    return np.abs(W.reshape(R, C // g, g)).max(axis=2)


def _per_weight(vals, width):
    """Repeat a per-group array [R, C/width] to per-weight [R, C]."""
    return np.repeat(vals, width, axis=1)


def normalized(W, g):
    """u [R, C] = w / s with s the group scale; u = +0 where s = 0 (and zero is unsigned)."""
    W = np.asarray(W, dtype=np.float64)
    s = _per_weight(group_scales(W, g), g)
    u = np.divide(W, s, out=np.zeros_like(W), where=s > 0)
    u[u == 0] = 0.0
    return u


# ----------------------------------------------------------------------------------------------
# Init (§2 mechanism 4): equally spaced quantiles of the normalized weights; T1 half a step up.
# ----------------------------------------------------------------------------------------------

def init_ranks(N, n):
    """Order-statistic indices of reading R3."""
    j = np.arange(n, dtype=np.int64)
    r0 = ((2 * j + 1) * N) // (2 * n)
    r1 = np.minimum(N - 1, ((j + 1) * N) // n)
    return r0, r1


def init_tables(W, g, n):
    """(T0, T1) fp64 [n] each: quantiles of all u of the matrix at p = (j + 1/2)/n and (j + 1)/n."""
    V = np.sort(normalized(W, g).ravel())
    r0, r1 = init_ranks(V.size, n)
    return V[r0].copy(), V[r1].copy()


# ----------------------------------------------------------------------------------------------
# Assign (§2 mechanisms 2 and 4): nearest entry per table, then the table with the lower
# activation-weighted reconstruction error per selection group.
# ----------------------------------------------------------------------------------------------

def nearest(u, T):
    """argmin_j (u - T[j])^2 per element, ties to the lowest j (reading R4; np.argmin returns the
    first minimum)."""
    u = np.asarray(u, dtype=np.float64)
    T = np.asarray(T, dtype=np.float64)
    d = (u[..., None] - T) ** 2
    return np.argmin(d, axis=-1)


def assign(W, I, T0, T1, g, S):
    """One assign step.

    Returns a dict with
      q0, q1  [R, C] nearest entry in T0 and in T1,
      E0, E1  [R, C/S] fp64 selection errors sum_H I_k (w_k - s T_c[q_c])^2 (reading R5),
      sel     [R, C/S] uint8, 1 iff E1 < E0 (ties keep T0),
      codes   [R, C] the chosen table's entry index.
    """
    W = np.asarray(W, dtype=np.float64)
    I = np.asarray(I, dtype=np.float64)
    R, C = _check_shape(W, g, S)
    s = _per_weight(group_scales(W, g), g)
    u = normalized(W, g)
    out = {}
    for c, T in enumerate((T0, T1)):
        T = np.asarray(T, dtype=np.float64)
        q = nearest(u, T)
        resid = W - s * T[q]
        err = (I[None, :] * resid * resid).reshape(R, C // S, S).sum(axis=2)
        out["q%d" % c] = q
        out["E%d" % c] = err
    sel = (out["E1"] < out["E0"]).astype(np.uint8)
    out["sel"] = sel
    out["codes"] = np.where(_per_weight(sel, S).astype(bool), out["q1"], out["q0"])
    return out


# ----------------------------------------------------------------------------------------------
# Refine (§2 mechanism 4): activation-weighted k-means update of every table entry.
# ----------------------------------------------------------------------------------------------

def refine_sums(W, I, codes, sel, g, S, n):
    """(num, den) fp64 [2, n]: num = sum I_k s w_k, den = sum I_k s^2 over each cell
    (sigma = c, q = j). The update T = num / den minimizes sum I (w - s T)^2 over the cell."""
    W = np.asarray(W, dtype=np.float64)
    I = np.asarray(I, dtype=np.float64)
    R, C = _check_shape(W, g, S)
    s = _per_weight(group_scales(W, g), g)
    cell = _per_weight(np.asarray(sel, dtype=np.int64), S) * n + np.asarray(codes, dtype=np.int64)
    a = I[None, :] * s
    num = np.bincount(cell.ravel(), weights=(a * W).ravel(), minlength=2 * n)
    den = np.bincount(cell.ravel(), weights=(a * s).ravel(), minlength=2 * n)
    return num.reshape(2, n), den.reshape(2, n)


def refine_update(num, den, T0, T1):
    """New tables: num / den where the cell has weight, else the old entry (reading R6)."""
    old = np.stack([np.asarray(T0, dtype=np.float64), np.asarray(T1, dtype=np.float64)])
    new = np.divide(num, den, out=old.copy(), where=den > 0)
    return new[0], new[1]


def refine(W, I, codes, sel, T0, T1, g, S):
    n = len(T0)
    num, den = refine_sums(W, I, codes, sel, g, S, n)
    return refine_update(num, den, T0, T1)


def total_error(W, I, codes, sel, T0, T1, g, S):
    """sum_k I_k (w_k - s T_sigma[q_k])^2 over the whole matrix."""
    W = np.asarray(W, dtype=np.float64)
    I = np.asarray(I, dtype=np.float64)
    R, C = _check_shape(W, g, S)
    s = _per_weight(group_scales(W, g), g)
    Ts = np.stack([np.asarray(T0, np.float64), np.asarray(T1, np.float64)])
    sig = _per_weight(np.asarray(sel, dtype=np.int64), S)
    resid = W - s * Ts[sig, np.asarray(codes, dtype=np.int64)]
    return float(np.sum(I[None, :] * resid * resid))


# ----------------------------------------------------------------------------------------------
# The whole loop (reading R7) and the storage format (readings R8, R9).
# ----------------------------------------------------------------------------------------------

def quantize(W, I, g, S, n, iters, tables=None):
    """Init (unless tables are given), iters x (assign, refine), bf16 tables, final assign.

    Returns a dict with the final assign result, the bf16 tables (values), and the history of the
    total error after every half-step (assign, then refine), for the monotonicity check."""
    W = np.asarray(W, dtype=np.float64)
    if tables is None:
        T0, T1 = init_tables(W, g, n)
    else:
        T0, T1 = (np.asarray(t, dtype=np.float64).copy() for t in tables)
    history = []
    for _ in range(iters):
        a = assign(W, I, T0, T1, g, S)
        history.append(total_error(W, I, a["codes"], a["sel"], T0, T1, g, S))
        T0, T1 = refine(W, I, a["codes"], a["sel"], T0, T1, g, S)
        history.append(total_error(W, I, a["codes"], a["sel"], T0, T1, g, S))
    T0b, T1b = bf16_round(T0), bf16_round(T1)
    final = assign(W, I, T0b, T1b, g, S)
    return {"tables": (T0, T1), "tables_bf16": (T0b, T1b), "final": final,
            "history": np.asarray(history)}


def pack(W, codes, sel, tables_bf16, g, S):
    """Packed artifacts of reading R8.

    codes [R, C] ints in [0, 16); sel [R, C/S]; tables_bf16 two bf16-exact arrays.
    Returns dict(codes uint8 [R, C/2], scales uint16 [R, C/g], bitmap uint8 or None,
    tables uint16 [2, n])."""
    W = np.asarray(W, dtype=np.float64)
    R, C = _check_shape(W, g, S)
    q = np.asarray(codes, dtype=np.int64).reshape(R, C // 2, 2)
    code_bytes = (q[:, :, 0] | (q[:, :, 1] << 4)).astype(np.uint8)
    scale_bits = bf16_bits(group_scales(W, g)).astype(np.uint16)
    sel = np.asarray(sel, dtype=np.uint8)
    if S == g:
        scale_bits = scale_bits | (sel.astype(np.uint16) << 15)
        bitmap = None
    else:
        flat = sel.ravel()
        nbytes = (flat.size + 7) // 8
        bitmap = np.zeros(nbytes, dtype=np.uint8)
        for bit in range(8):
            idx = np.arange(bit, flat.size, 8)
            bitmap[idx // 8] |= (flat[idx] << bit).astype(np.uint8)
    tables = np.stack([bf16_bits(tables_bf16[0]), bf16_bits(tables_bf16[1])])
    return {"codes": code_bytes, "scales": scale_bits.astype(np.uint16), "bitmap": bitmap,
            "tables": tables}


def unpack_codes(code_bytes, R, C):
    b = np.asarray(code_bytes, dtype=np.uint8).reshape(R, C // 2).astype(np.int64)
    q = np.empty((R, C), dtype=np.int64)
    q[:, 0::2] = b & 15
    q[:, 1::2] = b >> 4
    return q


def unpack_selectors(scales, bitmap, R, C, g, S):
    scales = np.asarray(scales, dtype=np.uint16).reshape(R, C // g)
    if S == g:
        return (scales >> 15).astype(np.uint8)
    count = R * (C // S)
    bm = np.asarray(bitmap, dtype=np.uint8)
    i = np.arange(count)
    return ((bm[i // 8] >> (i % 8)) & 1).astype(np.uint8).reshape(R, C // S)


def dequant(code_bytes, scales, bitmap, tables_u16, R, C, g, S):
    """w_hat [R, C] fp64 (bf16 values) = bf16(|s| * T~_sigma[q]) (§1: the dequantized values are
    what inference uses; §2 mechanism 3: the selector lives in the sign bit or the bitmap)."""
    q = unpack_codes(code_bytes, R, C)
    sel = unpack_selectors(scales, bitmap, R, C, g, S)
    s = bits_to_float(np.asarray(scales, dtype=np.uint16).reshape(R, C // g) & 0x7FFF)
    tabs = np.stack([bits_to_float(tables_u16[0]), bits_to_float(tables_u16[1])])
    vals = _per_weight(s, g) * tabs[_per_weight(sel.astype(np.int64), S), q]
    return bf16_round(vals)


# ----------------------------------------------------------------------------------------------
# Inference side of the packed format (AAAC summary §1: W4A16 deployment, the dequantized values
# are the weights inference uses) and the AWQ composition (§4).
# ----------------------------------------------------------------------------------------------

def decoded_weights(code_bytes, scales, bitmap, tables_u16, R, C, g, S):
    """[R, C] fp64 |s| * T~_sigma[q] straight from the packed format, without the bf16 rounding
    that dequant applies to store W_hat (reading R14). Both factors are bf16 values, so the product
    is exact."""
    q = unpack_codes(code_bytes, R, C)
    sel = unpack_selectors(scales, bitmap, R, C, g, S)
    s = bits_to_float(np.asarray(scales, dtype=np.uint16).reshape(R, C // g) & 0x7FFF)
    tabs = np.stack([bits_to_float(tables_u16[0]), bits_to_float(tables_u16[1])])
    return _per_weight(s, g) * tabs[_per_weight(sel.astype(np.int64), S), q]


def gemv(code_bytes, scales, bitmap, tables_u16, R, C, g, S, x):
    """Decode GEMV on the packed format: y[b, r] = sum_c |s| T~_sigma[q] x[b, c] in fp64 (every
    product is exact: three bf16 factors), for x [B, C] of bf16 values. Returns (y [B, R],
    a [B, R]) where a = sum_c |term| scales the rounding bound of an fp32 evaluation."""
    Wd = decoded_weights(code_bytes, scales, bitmap, tables_u16, R, C, g, S)
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    return x @ Wd.T, np.abs(x) @ np.abs(Wd).T


def awq_prescale(W, a, I=None):
    """Inputs for quantizing W diag(a) (AAAC after AWQ's weight scaling, §4; reading R15):
    W_scaled = bf16(W * a) per column, from the exact fp64 product, and, if I is given,
    I_scaled = fp32(I / a^2) from one fp64 division of exact operands. The scaled matrix sees the
    inputs x / a at inference, whose energy is I / a^2, so the weighted error of W_scaled under
    I_scaled is the error of the original matrix."""
    W = np.asarray(W, dtype=np.float64)
    a = np.asarray(a, dtype=np.float32).astype(np.float64)
    Ws = bf16_round(W * a[None, :])
    if I is None:
        return Ws, None
    I = np.asarray(I, dtype=np.float32).astype(np.float64)
    return Ws, (I / (a * a)).astype(np.float32)


def storage_bytes(n, num_matrices=1):
    """Bytes of the two bf16 tables, per matrix times the matrix count (§2 mechanism 3)."""
    return 2 * n * 2 * num_matrices


def selector_bits_per_weight(g, S):
    """Extra bits per weight for the table choice: none when the sign bit of the scale holds it
    (S == g), one bit per selection group otherwise (§2 mechanism 3, §4)."""
    return 0.0 if S == g else 1.0 / S
