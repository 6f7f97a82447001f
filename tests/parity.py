"""Comparison helpers for the GPU parity tests: HIP results against the fp64 oracle.

Tolerances (each derived from the arithmetic of the kernel it checks):
  * codes: bit-exact, except a weight whose GPU entry is strictly farther than the oracle's nearest
    one by less than CODE_BAND (relative squared distance); equal distances must pick the lower
    index, so value ties are never exempt;
  * selectors: bit-exact, except groups with |E1 - E0| < SEL_BAND * max(E0, E1) (oracle fp64);
    a code in such a group is compared against the table the GPU chose;
  * tables after refine: 1e-5 relative, plus an absolute allowance for the fp64 summation order
    of each cell: both sides add the same exact fp64 terms in different orders, each sum of N
    terms within N 2^-53 of sum |term|, so an entry num / den may differ by
    2 N 2^-53 (sum |I s w| / den + |T|) (the cell nearest zero, whose terms cancel, needs it);
  * importance: 1e-12 relative in fp64 (summation order only);
  * init tables, packed bytes and dequantized weights: bit-exact.
"""

from __future__ import annotations

import numpy as np
import torch

from oracle import aaac_ref as ref

CODE_BAND = 1e-6
SEL_BAND = 1e-6
TABLE_RTOL = 1e-5
SUM_EPS = 2.0 ** -53


def to_np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64) if t.dtype in (
        torch.bfloat16, torch.float16, torch.float32) else t.detach().cpu().numpy().astype(np.float64)


def unpack_gpu_codes(codes: torch.Tensor, R: int, C: int) -> np.ndarray:
    return ref.unpack_codes(codes.cpu().numpy().reshape(R, C // 2), R, C)


def oracle_assign_rows(W64, I64, T0, T1, g, S, chunk_rows=256):
    """Oracle assign over row chunks (rows are independent; identical to one call)."""
    parts = {"q0": [], "q1": [], "E0": [], "E1": [], "sel": [], "codes": []}
    for r0 in range(0, W64.shape[0], chunk_rows):
        a = ref.assign(W64[r0:r0 + chunk_rows], I64, T0, T1, g, S)
        for k in parts:
            parts[k].append(a[k])
    return {k: np.concatenate(v, axis=0) for k, v in parts.items()}


def check_assign(W64, I64, tables, g, S, gpu_codes, gpu_sel, gpu_err=None, chunk_rows=256):
    """Compare one GPU assign with the oracle on the same inputs. Returns a dict of counts and
    raises AssertionError on a mismatch outside the bands."""
    T0 = np.asarray(tables[0], dtype=np.float64)
    T1 = np.asarray(tables[1], dtype=np.float64)
    R, C = W64.shape
    a = oracle_assign_rows(W64, I64, T0, T1, g, S, chunk_rows)
    sel_g = np.asarray(gpu_sel).reshape(R, C // S).astype(np.uint8)
    q_g = np.asarray(gpu_codes).reshape(R, C)
    E0, E1 = a["E0"], a["E1"]
    sel_diff = sel_g != a["sel"]
    sel_exempt = np.abs(E1 - E0) <= SEL_BAND * np.maximum(E0, E1)
    bad_sel = sel_diff & ~sel_exempt
    assert not bad_sel.any(), "selector mismatch outside the band at %s (E0=%r E1=%r)" % (
        np.argwhere(bad_sel)[:5].tolist(), E0[bad_sel][:5], E1[bad_sel][:5])
    # codes against the table the GPU chose
    chosen = np.repeat(sel_g, S, axis=1).astype(bool)
    q_o = np.where(chosen, a["q1"], a["q0"])
    s = np.repeat(ref.group_scales(W64, g), g, axis=1)
    code_diff = q_g != q_o
    bad_code = np.zeros_like(code_diff)
    if code_diff.any():
        idx = np.argwhere(code_diff)
        r, c = idx[:, 0], idx[:, 1]
        T = np.where(chosen[r, c], 1, 0)
        Ts = np.stack([T0, T1])
        d_g = (W64[r, c] - s[r, c] * Ts[T, q_g[r, c]]) ** 2
        d_o = (W64[r, c] - s[r, c] * Ts[T, q_o[r, c]]) ** 2
        ok = (d_g > d_o) & (d_g - d_o <= CODE_BAND * d_g)
        bad_code[r[~ok], c[~ok]] = True
        detail = ["(r=%d c=%d w=%r s=%r table=%d gpu q=%d T=%r d=%r | oracle q=%d T=%r d=%r)" % (
            r[i], c[i], W64[r[i], c[i]], s[r[i], c[i]], T[i], q_g[r[i], c[i]],
            Ts[T[i], q_g[r[i], c[i]]], d_g[i], q_o[r[i], c[i]], Ts[T[i], q_o[r[i], c[i]]], d_o[i])
            for i in np.flatnonzero(~ok)[:6]]
    assert not bad_code.any(), "%d code mismatches outside the band: %s" % (
        int(bad_code.sum()), "\n".join(detail))
    if gpu_err is not None:
        e = np.asarray(gpu_err, dtype=np.float64).reshape(R, C // S, 2)
        for k, Eo in ((0, E0), (1, E1)):
            tol = 2e-6 * np.maximum(Eo, 1e-300) + 1e-300
            bad = np.abs(e[..., k] - Eo) > tol
            assert not bad.any(), "E%d mismatch at %s: gpu %r oracle %r" % (
                k, np.argwhere(bad)[:5].tolist(), e[..., k][bad][:5], Eo[bad][:5])
    return {"sel_exempt": int((sel_diff & sel_exempt).sum()), "code_exempt": int(code_diff.sum()),
            "oracle": a}


def _tolerance(oracle, bound, rtol):
    tol = rtol * np.abs(oracle)
    if bound is not None:
        tol = tol + np.asarray(bound, dtype=np.float64).reshape(oracle.shape)
    return tol


def check_tables(gpu, oracle, bound=None, rtol=TABLE_RTOL):
    """|gpu - oracle| <= rtol |oracle| + bound per entry (bound: the summation allowance that
    oracle_refine returns, or None)."""
    gpu = np.asarray(gpu, dtype=np.float64).reshape(2, -1)
    oracle = np.asarray(oracle, dtype=np.float64).reshape(2, -1)
    tol = _tolerance(oracle, bound, rtol)
    err = np.abs(gpu - oracle)
    ok = (err <= tol) | (gpu == oracle)
    assert ok.all(), "table mismatch at %s:\n gpu=%r\n ora=%r" % (
        np.argwhere(~ok).tolist(), gpu, oracle)
    nz = np.abs(oracle) > 0
    return float((err[nz] / np.abs(oracle[nz])).max()) if nz.any() else 0.0


def check_tables_bf16(gpu, oracle, bound=None, rtol=TABLE_RTOL):
    """Tables rounded to bf16 on the last refine: each GPU entry must be the bf16 rounding of a
    value within the table tolerance of the oracle's (a value that close to a rounding midpoint may
    round either way)."""
    gpu = np.asarray(gpu, dtype=np.float64).reshape(2, -1)
    oracle = np.asarray(oracle, dtype=np.float64).reshape(2, -1)
    assert np.array_equal(ref.bf16_round(gpu), gpu), "tables are not bf16 values"
    tol = _tolerance(oracle, bound, rtol)
    lo = ref.bf16_round(oracle - tol)
    hi = ref.bf16_round(oracle + tol)
    ok = (gpu >= np.minimum(lo, hi)) & (gpu <= np.maximum(lo, hi))
    assert ok.all(), "bf16 table mismatch at %s:\n gpu=%r\n ora=%r" % (
        np.argwhere(~ok).tolist(), gpu, oracle)


def oracle_refine(W64, I64, codes, sel, T_in, g, S, chunk_rows=1024):
    """The oracle's refine on the GPU's codes and selectors: (new tables, num, den, bound), with
    bound the per-entry allowance for the fp64 summation order (see the module docstring)."""
    n = T_in.shape[1]
    num = np.zeros((2, n))
    den = np.zeros((2, n))
    absnum = np.zeros((2, n))
    count = np.zeros((2, n))
    for r0 in range(0, W64.shape[0], chunk_rows):
        Wc = W64[r0:r0 + chunk_rows]
        qc = codes[r0:r0 + chunk_rows]
        sc = sel[r0:r0 + chunk_rows]
        a, b = ref.refine_sums(Wc, I64, qc, sc, g, S, n)
        num += a
        den += b
        # sum |I s w| per cell: the same sums on |W| (the scales only see |w|)
        absnum += ref.refine_sums(np.abs(Wc), I64, qc, sc, g, S, n)[0]
        cell = np.repeat(np.asarray(sc, dtype=np.int64), S, axis=1) * n + qc
        count += np.bincount(cell.ravel(), minlength=2 * n).reshape(2, n)
    new = np.stack(ref.refine_update(num, den, T_in[0], T_in[1]))
    with np.errstate(divide="ignore", invalid="ignore"):
        bound = np.where(den > 0, 2.0 * count * SUM_EPS * (absnum / den + np.abs(new)), 0.0)
    return new, num, den, bound


def total_error_rows(W64, I64, codes, sel, T, g, S, chunk_rows=1024):
    """The oracle's total weighted error of a given assignment, over row chunks (rows are
    independent; the same sum as one call up to the order of the chunk totals)."""
    T = np.asarray(T, dtype=np.float64).reshape(2, -1)
    tot = 0.0
    for r0 in range(0, W64.shape[0], chunk_rows):
        tot += ref.total_error(W64[r0:r0 + chunk_rows], I64, codes[r0:r0 + chunk_rows],
                               sel[r0:r0 + chunk_rows], T[0], T[1], g, S)
    return tot
