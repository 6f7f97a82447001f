"""ctypes binding of libaaac.so (the C ABI in include/aaac.h).

Argument marshalling only: every function here checks dtypes and devices of torch tensors, passes
their device pointers and the current HIP stream to the C entry point of the same name, and turns
a non-zero status into an exception. All arithmetic runs in the library's kernels. There is no
fallback: if the library is missing or no GPU is visible, the calls raise.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libaaac.so")

AAAC_OK = 0
AAAC_ERR_INVALID_ARG = 1
AAAC_ERR_UNSUPPORTED_SHAPE = 2
AAAC_ERR_WORKSPACE_TOO_SMALL = 3
AAAC_ERR_HIP = 4

OP_IMPORTANCE, OP_INIT, OP_ASSIGN, OP_REFINE = 0, 1, 2, 3
REFINE_ROUND_BF16 = 1
REFINE_W2_KNOWN = 2
MAX_BATCH = 8

EXPORTED = (
    "aaac_status_string", "aaac_last_error", "aaac_workspace_bytes", "aaac_importance",
    "aaac_init_quantiles", "aaac_assign", "aaac_refine", "aaac_pack", "aaac_dequant",
    "aaac_batch_workspace_bytes", "aaac_assign_batch", "aaac_refine_batch", "aaac_awq_prescale",
    "aaac_gemv", "aaac_gemv_batch", "aaac_assign_refine_batch", "aaac_init_quantiles_batch",
    "aaac_pack_batch", "aaac_dequant_batch", "aaac_refine_batch_noalloc",
)


class AAACError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


_lib = None

c_i64 = ctypes.c_int64
c_int = ctypes.c_int
c_vp = ctypes.c_void_p
c_size = ctypes.c_size_t
P = ctypes.POINTER


def load(path: str = LIB_PATH):
    """Load the library (once) and declare every entry point's signature."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            "libaaac.so not found at %s: build it with `python -m "
            "post_weight_quantization_06_amd.build` (hipcc, gfx950)" % path)
    lib = ctypes.CDLL(path)
    sig = {
        "aaac_status_string": (ctypes.c_char_p, [c_int]),
        "aaac_last_error": (ctypes.c_char_p, []),
        "aaac_workspace_bytes": (c_size, [c_int, c_i64, c_i64, c_int, c_int, c_int]),
        "aaac_batch_workspace_bytes": (c_size, [c_int, c_int, P(c_i64), P(c_i64), c_int, c_int,
                                                c_int]),
        "aaac_importance": (c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_size, c_vp]),
        "aaac_init_quantiles": (c_int, [c_vp, c_i64, c_i64, c_int, c_int, c_vp, c_vp, c_size,
                                        c_vp]),
        "aaac_assign": (c_int, [c_vp, c_i64, c_i64, c_int, c_int, c_int, c_vp, c_vp, c_vp, c_vp,
                                c_vp, c_vp, c_vp, c_size, c_vp]),
        "aaac_refine": (c_int, [c_vp, c_i64, c_i64, c_int, c_int, c_int, c_vp, c_vp, c_vp, c_vp,
                                c_vp, c_int, c_vp, c_vp, c_vp, c_size, c_vp]),
        "aaac_pack": (c_int, [c_vp, c_i64, c_i64, c_int, c_int, c_int, c_vp, c_vp, c_vp, c_vp,
                              c_vp, c_vp, c_vp, c_vp]),
        "aaac_dequant": (c_int, [c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_int, c_int, c_int, c_vp,
                                 c_vp]),
        "aaac_init_quantiles_batch": (c_int, [c_int, P(c_vp), P(c_i64), P(c_i64), c_int, c_int,
                                              P(c_vp), c_vp, c_size, c_vp]),
        "aaac_pack_batch": (c_int, [c_int, P(c_vp), P(c_i64), P(c_i64), c_int, c_int, c_int,
                                    P(c_vp), P(c_vp), P(c_vp), P(c_vp), P(c_vp), c_vp]),
        "aaac_dequant_batch": (c_int, [c_int, P(c_vp), P(c_vp), P(c_vp), P(c_vp), P(c_i64),
                                       P(c_i64), c_int, c_int, c_int, P(c_vp), c_vp]),
        "aaac_assign_batch": (c_int, [c_int, P(c_vp), P(c_i64), P(c_i64), c_int, c_int, c_int,
                                      P(c_vp), P(c_vp), P(c_vp), P(c_vp), c_vp, c_vp, c_size,
                                      c_vp]),
        "aaac_refine_batch": (c_int, [c_int, P(c_vp), P(c_i64), P(c_i64), c_int, c_int, c_int,
                                      P(c_vp), P(c_vp), P(c_vp), P(c_vp), c_int, c_vp, c_vp,
                                      c_vp, c_size, c_vp]),
        "aaac_awq_prescale": (c_int, [c_vp, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp]),
        "aaac_refine_batch_noalloc": (c_int, [c_int, P(c_vp), P(c_i64), P(c_i64), c_int, c_int,
                                              c_int, P(c_vp), P(c_vp), P(c_vp), P(c_vp), c_int,
                                              c_vp, c_vp, c_vp]),
        "aaac_assign_refine_batch": (c_int, [c_int, P(c_vp), P(c_i64), P(c_i64), c_int, c_int,
                                             c_int, P(c_vp), P(c_vp), P(c_vp), P(c_vp), c_int,
                                             c_vp, c_vp, c_vp, c_size, c_vp]),
        "aaac_gemv": (c_int, [c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_int, c_int, c_int, c_vp,
                              c_int, c_vp, c_vp]),
        "aaac_gemv_batch": (c_int, [c_int, P(c_vp), P(c_vp), P(c_vp), P(c_vp), P(c_i64),
                                    P(c_i64), c_int, c_int, c_int, P(c_vp), c_int, P(c_vp),
                                    c_vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int, what: str):
    if status != AAAC_OK:
        lib = load()
        detail = lib.aaac_last_error().decode()
        raise AAACError(status, "%s failed: %s (%s)" % (
            what, lib.aaac_status_string(status).decode(), detail))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, numel: Optional[int] = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on the GPU (got %s)" % (name, t.device))
    if t.dtype != dtype:
        raise TypeError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if numel is not None and t.numel() != numel:
        raise ValueError("%s must hold %d elements (got %d)" % (name, numel, t.numel()))


def workspace_bytes(op: int, R: int, C: int, g: int = 128, S: int = 128, n: int = 16) -> int:
    return int(load().aaac_workspace_bytes(op, R, C, g, S, n))


def batch_workspace_bytes(op: int, Rs: Sequence[int], Cs: Sequence[int], g: int, S: int,
                          n: int) -> int:
    k = len(Rs)
    R = (c_i64 * k)(*Rs)
    C = (c_i64 * k)(*Cs)
    return int(load().aaac_batch_workspace_bytes(op, k, R, C, g, S, n))


def workspace(nbytes: int, device) -> torch.Tensor:
    """Zero-filled device workspace of at least nbytes (torch allocations are 256-byte aligned)."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------------------------------------
# Entry points (same names as the C ABI).
# ------------------------------------------------------------------------------------------------

def aaac_importance(X: torch.Tensor, I_acc: torch.Tensor, I_out: Optional[torch.Tensor] = None,
                    ws: Optional[torch.Tensor] = None, stream=None):
    """I_acc += sum_t X[t, :]^2 (fp64); I_out = fp32(I_acc) if given. X: fp32 [T, K], row stride
    X.stride(0)."""
    lib = load()
    if X.dim() != 2 or X.stride(1) != 1:
        raise ValueError("X must be 2-D with unit column stride")
    if X.device.type != "cuda" or X.dtype != torch.float32:
        raise TypeError("X must be fp32 on the GPU")
    T, K = X.shape
    _need(I_acc, "I_acc", torch.float64, K)
    if I_out is not None:
        _need(I_out, "I_out", torch.float32, K)
    nb = lib.aaac_workspace_bytes(OP_IMPORTANCE, T, K, 0, 0, 0)
    if ws is None:
        ws = workspace(nb, X.device)
    st = lib.aaac_importance(_ptr(X), T, K, X.stride(0), _ptr(I_acc), _ptr(I_out), _ptr(ws),
                             ws.numel(), _stream(stream))
    _check(st, "aaac_importance")
    return I_acc


def aaac_init_quantiles(W: torch.Tensor, g: int, n: int, tables: torch.Tensor,
                        ws: Optional[torch.Tensor] = None, stream=None):
    lib = load()
    R, C = W.shape
    _need(W, "W", torch.bfloat16)
    _need(tables, "tables", torch.float32, 2 * n)
    if ws is None:
        ws = workspace(lib.aaac_workspace_bytes(OP_INIT, R, C, g, 0, n), W.device)
    st = lib.aaac_init_quantiles(_ptr(W), R, C, g, n, _ptr(tables), _ptr(ws), ws.numel(),
                                 _stream(stream))
    _check(st, "aaac_init_quantiles")
    return tables


def aaac_assign(W: torch.Tensor, g: int, S: int, n: int, I: torch.Tensor, tables: torch.Tensor,
                codes: torch.Tensor, sel: torch.Tensor, err: Optional[torch.Tensor] = None,
                err_total: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                stream=None):
    """err: fp64 [R*C/S*2] (E0, E1) per selection group or None; err_total: fp64 [1] receiving
    the sum of the chosen errors, or None (then ws is not needed)."""
    lib = load()
    R, C = W.shape
    _need(W, "W", torch.bfloat16)
    _need(I, "I", torch.float32, C)
    _need(tables, "tables", torch.float32, 2 * n)
    _need(codes, "codes", torch.uint8, R * C // 2)
    _need(sel, "sel", torch.uint8, R * C // S)
    if err is not None:
        _need(err, "err", torch.float64, 2 * (R * C // S))
    if err_total is not None:
        _need(err_total, "err_total", torch.float64, 1)
        if ws is None:
            ws = workspace(lib.aaac_workspace_bytes(OP_ASSIGN, R, C, g, S, n), W.device)
    st = lib.aaac_assign(_ptr(W), R, C, g, S, n, _ptr(I), _ptr(tables), _ptr(codes), _ptr(sel),
                         _ptr(err), _ptr(err_total), _ptr(ws), 0 if ws is None else ws.numel(),
                         _stream(stream))
    _check(st, "aaac_assign")


def aaac_refine(W: torch.Tensor, g: int, S: int, n: int, I: torch.Tensor, codes: torch.Tensor,
                sel: torch.Tensor, tables_in: torch.Tensor, tables_out: torch.Tensor,
                flags: int = 0, ws: Optional[torch.Tensor] = None, err: Optional[torch.Tensor] = None,
                w2: Optional[torch.Tensor] = None, stream=None):
    """err: fp64 [2] receiving the assignment's error before and after the update, with w2 fp64
    [1] (sum I w^2: written, or read with REFINE_W2_KNOWN), or both None."""
    lib = load()
    R, C = W.shape
    _need(W, "W", torch.bfloat16)
    _need(I, "I", torch.float32, C)
    _need(codes, "codes", torch.uint8, R * C // 2)
    _need(sel, "sel", torch.uint8, R * C // S)
    _need(tables_in, "tables_in", torch.float32, 2 * n)
    _need(tables_out, "tables_out", torch.float32, 2 * n)
    if err is not None:
        _need(err, "err", torch.float64, 2)
    if w2 is not None:
        _need(w2, "w2", torch.float64, 1)
    if ws is None:
        ws = workspace(lib.aaac_workspace_bytes(OP_REFINE, R, C, g, S, n), W.device)
    st = lib.aaac_refine(_ptr(W), R, C, g, S, n, _ptr(I), _ptr(codes), _ptr(sel),
                         _ptr(tables_in), _ptr(tables_out), flags, _ptr(err), _ptr(w2),
                         _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "aaac_refine")


def aaac_pack(W: torch.Tensor, g: int, S: int, n: int, sel: torch.Tensor, tables: torch.Tensor,
              scales: torch.Tensor, bitmap: Optional[torch.Tensor], tables_bf16: torch.Tensor,
              codes_u8: Optional[torch.Tensor] = None, codes_out: Optional[torch.Tensor] = None,
              stream=None):
    """codes_u8 (u8 [R*C], one code per byte) and codes_out (u8 [R*C/2]): pack codes given one per
    byte into the two-per-byte layout, or both None."""
    lib = load()
    R, C = W.shape
    _need(W, "W", torch.bfloat16)
    _need(sel, "sel", torch.uint8, R * C // S)
    _need(tables, "tables", torch.float32, 2 * n)
    _need(scales, "scales", torch.int16, R * C // g)
    _need(tables_bf16, "tables_bf16", torch.int16, 2 * n)
    if bitmap is not None:
        _need(bitmap, "bitmap", torch.uint8, (R * C // S + 7) // 8)
    if codes_u8 is not None:
        _need(codes_u8, "codes_u8", torch.uint8, R * C)
    if codes_out is not None:
        _need(codes_out, "codes_out", torch.uint8, R * C // 2)
    st = lib.aaac_pack(_ptr(W), R, C, g, S, n, _ptr(sel), _ptr(tables), _ptr(codes_u8),
                       _ptr(codes_out), _ptr(scales), _ptr(bitmap), _ptr(tables_bf16),
                       _stream(stream))
    _check(st, "aaac_pack")


def aaac_dequant(codes: torch.Tensor, scales: torch.Tensor, bitmap: Optional[torch.Tensor],
                 tables_bf16: torch.Tensor, R: int, C: int, g: int, S: int, n: int,
                 W_hat: torch.Tensor, stream=None):
    lib = load()
    _need(codes, "codes", torch.uint8, R * C // 2)
    _need(scales, "scales", torch.int16, R * C // g)
    _need(tables_bf16, "tables_bf16", torch.int16, 2 * n)
    _need(W_hat, "W_hat", torch.bfloat16, R * C)
    if bitmap is not None:
        _need(bitmap, "bitmap", torch.uint8, (R * C // S + 7) // 8)
    st = lib.aaac_dequant(_ptr(codes), _ptr(scales), _ptr(bitmap), _ptr(tables_bf16), R, C, g, S,
                          n, _ptr(W_hat), _stream(stream))
    _check(st, "aaac_dequant")


def aaac_pack_batch(Ws: Sequence[torch.Tensor], g: int, S: int, n: int,
                    sels: Sequence[torch.Tensor], tables: Sequence[torch.Tensor],
                    scales: Sequence[torch.Tensor], bitmaps: Optional[Sequence[torch.Tensor]],
                    tables_bf16: Sequence[torch.Tensor], stream=None):
    """aaac_pack for up to MAX_BATCH matrices in one set of launches (see aaac.h); bitmaps is None
    when S == g."""
    lib = load()
    k = len(Ws)
    Rs = [W.shape[0] for W in Ws]
    Cs = [W.shape[1] for W in Ws]
    for i in range(k):
        R, C = Rs[i], Cs[i]
        _need(Ws[i], "W[%d]" % i, torch.bfloat16)
        _need(sels[i], "sel[%d]" % i, torch.uint8, R * C // S)
        _need(tables[i], "tables[%d]" % i, torch.float32, 2 * n)
        _need(scales[i], "scales[%d]" % i, torch.int16, R * C // g)
        _need(tables_bf16[i], "tables_bf16[%d]" % i, torch.int16, 2 * n)
        if bitmaps is not None:
            _need(bitmaps[i], "bitmap[%d]" % i, torch.uint8, (R * C // S + 7) // 8)
    st = lib.aaac_pack_batch(
        k, _arr(c_vp, [t.data_ptr() for t in Ws]), _arr(c_i64, Rs), _arr(c_i64, Cs), g, S, n,
        _arr(c_vp, [t.data_ptr() for t in sels]), _arr(c_vp, [t.data_ptr() for t in tables]),
        _arr(c_vp, [t.data_ptr() for t in scales]),
        None if bitmaps is None else _arr(c_vp, [t.data_ptr() for t in bitmaps]),
        _arr(c_vp, [t.data_ptr() for t in tables_bf16]), _stream(stream))
    _check(st, "aaac_pack_batch")


def aaac_dequant_batch(codes: Sequence[torch.Tensor], scales: Sequence[torch.Tensor],
                       bitmaps: Optional[Sequence[torch.Tensor]],
                       tables_bf16: Sequence[torch.Tensor], Rs: Sequence[int], Cs: Sequence[int],
                       g: int, S: int, n: int, W_hats: Sequence[torch.Tensor], stream=None):
    """aaac_dequant for up to MAX_BATCH matrices in one launch (see aaac.h); bitmaps is None when
    S == g."""
    lib = load()
    k = len(codes)
    for i in range(k):
        R, C = Rs[i], Cs[i]
        _need(codes[i], "codes[%d]" % i, torch.uint8, R * C // 2)
        _need(scales[i], "scales[%d]" % i, torch.int16, R * C // g)
        _need(tables_bf16[i], "tables_bf16[%d]" % i, torch.int16, 2 * n)
        _need(W_hats[i], "W_hat[%d]" % i, torch.bfloat16, R * C)
        if bitmaps is not None:
            _need(bitmaps[i], "bitmap[%d]" % i, torch.uint8, (R * C // S + 7) // 8)
    st = lib.aaac_dequant_batch(
        k, _arr(c_vp, [t.data_ptr() for t in codes]), _arr(c_vp, [t.data_ptr() for t in scales]),
        None if bitmaps is None else _arr(c_vp, [t.data_ptr() for t in bitmaps]),
        _arr(c_vp, [t.data_ptr() for t in tables_bf16]), _arr(c_i64, list(Rs)),
        _arr(c_i64, list(Cs)), g, S, n, _arr(c_vp, [t.data_ptr() for t in W_hats]),
        _stream(stream))
    _check(st, "aaac_dequant_batch")


def _arr(ctype, values):
    return (ctype * len(values))(*values)


def aaac_init_quantiles_batch(Ws: Sequence[torch.Tensor], g: int, n: int,
                              tables: Sequence[torch.Tensor], ws: Optional[torch.Tensor] = None,
                              stream=None):
    """Init tables of up to MAX_BATCH matrices in one set of launches (see aaac.h)."""
    lib = load()
    k = len(Ws)
    Rs = [W.shape[0] for W in Ws]
    Cs = [W.shape[1] for W in Ws]
    for i in range(k):
        _need(Ws[i], "W[%d]" % i, torch.bfloat16)
        _need(tables[i], "tables[%d]" % i, torch.float32, 2 * n)
    if ws is None:
        ws = workspace(batch_workspace_bytes(OP_INIT, Rs, Cs, g, 8, n), Ws[0].device)
    st = lib.aaac_init_quantiles_batch(
        k, _arr(c_vp, [t.data_ptr() for t in Ws]), _arr(c_i64, Rs), _arr(c_i64, Cs), g, n,
        _arr(c_vp, [t.data_ptr() for t in tables]), _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "aaac_init_quantiles_batch")


def aaac_assign_batch(Ws: Sequence[torch.Tensor], g: int, S: int, n: int,
                      Is: Sequence[torch.Tensor], tables: Sequence[torch.Tensor],
                      codes: Sequence[torch.Tensor], sels: Sequence[torch.Tensor],
                      err_total: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                      stream=None):
    """err_total: fp64 [len(Ws)] receiving each matrix's sum of chosen errors, or None."""
    lib = load()
    k = len(Ws)
    Rs = [W.shape[0] for W in Ws]
    Cs = [W.shape[1] for W in Ws]
    for i in range(k):
        _need(Ws[i], "W[%d]" % i, torch.bfloat16)
        _need(Is[i], "I[%d]" % i, torch.float32, Cs[i])
        _need(tables[i], "tables[%d]" % i, torch.float32, 2 * n)
        _need(codes[i], "codes[%d]" % i, torch.uint8, Rs[i] * Cs[i] // 2)
        _need(sels[i], "sel[%d]" % i, torch.uint8, Rs[i] * Cs[i] // S)
    if err_total is not None:
        _need(err_total, "err_total", torch.float64, k)
        if ws is None:
            ws = workspace(batch_workspace_bytes(OP_ASSIGN, Rs, Cs, g, S, n), Ws[0].device)
    st = lib.aaac_assign_batch(
        k, _arr(c_vp, [t.data_ptr() for t in Ws]), _arr(c_i64, Rs), _arr(c_i64, Cs), g, S, n,
        _arr(c_vp, [t.data_ptr() for t in Is]), _arr(c_vp, [t.data_ptr() for t in tables]),
        _arr(c_vp, [t.data_ptr() for t in codes]), _arr(c_vp, [t.data_ptr() for t in sels]),
        _ptr(err_total), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream))
    _check(st, "aaac_assign_batch")


def aaac_refine_batch(Ws: Sequence[torch.Tensor], g: int, S: int, n: int,
                      Is: Sequence[torch.Tensor], codes: Sequence[torch.Tensor],
                      sels: Sequence[torch.Tensor], tables: Sequence[torch.Tensor],
                      flags: int = 0, ws: Optional[torch.Tensor] = None,
                      err: Optional[torch.Tensor] = None, w2: Optional[torch.Tensor] = None,
                      stream=None):
    """err: fp64 [2, len(Ws)] (row 0: each matrix's assignment error before the update, row 1:
    after it) and w2: fp64 [len(Ws)] (sum I w^2 per matrix: written, or read with
    REFINE_W2_KNOWN), or both None."""
    lib = load()
    k = len(Ws)
    Rs = [W.shape[0] for W in Ws]
    Cs = [W.shape[1] for W in Ws]
    for i in range(k):
        _need(Ws[i], "W[%d]" % i, torch.bfloat16)
        _need(Is[i], "I[%d]" % i, torch.float32, Cs[i])
        _need(tables[i], "tables[%d]" % i, torch.float32, 2 * n)
        _need(codes[i], "codes[%d]" % i, torch.uint8, Rs[i] * Cs[i] // 2)
        _need(sels[i], "sel[%d]" % i, torch.uint8, Rs[i] * Cs[i] // S)
    if err is not None:
        _need(err, "err", torch.float64, 2 * k)
    if w2 is not None:
        _need(w2, "w2", torch.float64, k)
    if ws is None:
        ws = workspace(batch_workspace_bytes(OP_REFINE, Rs, Cs, g, S, n), Ws[0].device)
    st = lib.aaac_refine_batch(
        k, _arr(c_vp, [t.data_ptr() for t in Ws]), _arr(c_i64, Rs), _arr(c_i64, Cs), g, S, n,
        _arr(c_vp, [t.data_ptr() for t in Is]), _arr(c_vp, [t.data_ptr() for t in codes]),
        _arr(c_vp, [t.data_ptr() for t in sels]), _arr(c_vp, [t.data_ptr() for t in tables]),
        flags, _ptr(err), _ptr(w2), _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "aaac_refine_batch")


def aaac_assign_refine_batch(Ws: Sequence[torch.Tensor], g: int, S: int, n: int,
                             Is: Sequence[torch.Tensor], tables: Sequence[torch.Tensor],
                             codes: Sequence[torch.Tensor], sels: Sequence[torch.Tensor],
                             flags: int = 0, ws: Optional[torch.Tensor] = None,
                             err: Optional[torch.Tensor] = None, w2: Optional[torch.Tensor] = None,
                             stream=None):
    """One assign + refine iteration in one launch (tables updated in place); flags, err (fp64
    [2, len(Ws)]) and w2 as for aaac_refine_batch."""
    lib = load()
    k = len(Ws)
    Rs = [W.shape[0] for W in Ws]
    Cs = [W.shape[1] for W in Ws]
    for i in range(k):
        _need(Ws[i], "W[%d]" % i, torch.bfloat16)
        _need(Is[i], "I[%d]" % i, torch.float32, Cs[i])
        _need(tables[i], "tables[%d]" % i, torch.float32, 2 * n)
        _need(codes[i], "codes[%d]" % i, torch.uint8, Rs[i] * Cs[i] // 2)
        _need(sels[i], "sel[%d]" % i, torch.uint8, Rs[i] * Cs[i] // S)
    if err is not None:
        _need(err, "err", torch.float64, 2 * k)
    if w2 is not None:
        _need(w2, "w2", torch.float64, k)
    if ws is None:
        ws = workspace(batch_workspace_bytes(OP_REFINE, Rs, Cs, g, S, n), Ws[0].device)
    st = lib.aaac_assign_refine_batch(
        k, _arr(c_vp, [t.data_ptr() for t in Ws]), _arr(c_i64, Rs), _arr(c_i64, Cs), g, S, n,
        _arr(c_vp, [t.data_ptr() for t in Is]), _arr(c_vp, [t.data_ptr() for t in tables]),
        _arr(c_vp, [t.data_ptr() for t in codes]), _arr(c_vp, [t.data_ptr() for t in sels]),
        flags, _ptr(err), _ptr(w2), _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "aaac_assign_refine_batch")


def aaac_awq_prescale(W: torch.Tensor, a: torch.Tensor, W_scaled: torch.Tensor,
                      I: Optional[torch.Tensor] = None, I_scaled: Optional[torch.Tensor] = None,
                      stream=None):
    """W_scaled = bf16(W * a) per column, I_scaled = fp32(I / a^2) (in place allowed)."""
    lib = load()
    R, C = W.shape
    _need(W, "W", torch.bfloat16)
    _need(a, "a", torch.float32, C)
    _need(W_scaled, "W_scaled", torch.bfloat16, R * C)
    if I is not None:
        _need(I, "I", torch.float32, C)
    if I_scaled is not None:
        _need(I_scaled, "I_scaled", torch.float32, C)
    st = lib.aaac_awq_prescale(_ptr(W), R, C, _ptr(a), _ptr(I), _ptr(W_scaled), _ptr(I_scaled),
                               _stream(stream))
    _check(st, "aaac_awq_prescale")


def aaac_gemv(codes: torch.Tensor, scales: torch.Tensor, bitmap: Optional[torch.Tensor],
              tables_bf16: torch.Tensor, R: int, C: int, g: int, S: int, n: int,
              x: torch.Tensor, y: torch.Tensor, stream=None):
    """y [B, R] fp32 = decoded packed weights times x [B, C] bf16 (see aaac.h)."""
    lib = load()
    B = x.shape[0] if x.dim() == 2 else 1
    _need(codes, "codes", torch.uint8, R * C // 2)
    _need(scales, "scales", torch.int16, R * C // g)
    _need(tables_bf16, "tables_bf16", torch.int16, 2 * n)
    _need(x, "x", torch.bfloat16, B * C)
    _need(y, "y", torch.float32, B * R)
    if bitmap is not None:
        _need(bitmap, "bitmap", torch.uint8, (R * C // S + 7) // 8)
    st = lib.aaac_gemv(_ptr(codes), _ptr(scales), _ptr(bitmap), _ptr(tables_bf16), R, C, g, S, n,
                       _ptr(x), B, _ptr(y), _stream(stream))
    _check(st, "aaac_gemv")


def aaac_gemv_batch(codes: Sequence[torch.Tensor], scales: Sequence[torch.Tensor],
                    bitmaps: Optional[Sequence[torch.Tensor]], tables_bf16: Sequence[torch.Tensor],
                    Rs: Sequence[int], Cs: Sequence[int], g: int, S: int, n: int,
                    xs: Sequence[torch.Tensor], ys: Sequence[torch.Tensor], stream=None):
    lib = load()
    k = len(codes)
    B = xs[0].shape[0] if xs[0].dim() == 2 else 1
    for i in range(k):
        R, C = Rs[i], Cs[i]
        _need(codes[i], "codes[%d]" % i, torch.uint8, R * C // 2)
        _need(scales[i], "scales[%d]" % i, torch.int16, R * C // g)
        _need(tables_bf16[i], "tables_bf16[%d]" % i, torch.int16, 2 * n)
        _need(xs[i], "x[%d]" % i, torch.bfloat16, B * C)
        _need(ys[i], "y[%d]" % i, torch.float32, B * R)
        if bitmaps is not None:
            _need(bitmaps[i], "bitmap[%d]" % i, torch.uint8, (R * C // S + 7) // 8)
    bm = None if bitmaps is None else _arr(c_vp, [t.data_ptr() for t in bitmaps])
    st = lib.aaac_gemv_batch(
        k, _arr(c_vp, [t.data_ptr() for t in codes]), _arr(c_vp, [t.data_ptr() for t in scales]),
        bm, _arr(c_vp, [t.data_ptr() for t in tables_bf16]), _arr(c_i64, list(Rs)),
        _arr(c_i64, list(Cs)), g, S, n, _arr(c_vp, [t.data_ptr() for t in xs]), B,
        _arr(c_vp, [t.data_ptr() for t in ys]), _stream(stream))
    _check(st, "aaac_gemv_batch")


def aaac_refine_batch_noalloc(Ws: Sequence[torch.Tensor], g: int, S: int, n: int,
                              Is: Sequence[torch.Tensor], codes: Sequence[torch.Tensor],
                              sels: Sequence[torch.Tensor], tables: Sequence[torch.Tensor],
                              flags: int = 0, err: Optional[torch.Tensor] = None,
                              w2: Optional[torch.Tensor] = None, stream=None):
    """aaac_refine_batch with the library's fixed device scratch instead of a workspace (see
    aaac.h): the call itself allocates nothing."""
    lib = load()
    k = len(Ws)
    Rs = [W.shape[0] for W in Ws]
    Cs = [W.shape[1] for W in Ws]
    for i in range(k):
        _need(Ws[i], "W[%d]" % i, torch.bfloat16)
        _need(Is[i], "I[%d]" % i, torch.float32, Cs[i])
        _need(tables[i], "tables[%d]" % i, torch.float32, 2 * n)
        _need(codes[i], "codes[%d]" % i, torch.uint8, Rs[i] * Cs[i] // 2)
        _need(sels[i], "sel[%d]" % i, torch.uint8, Rs[i] * Cs[i] // S)
    if err is not None:
        _need(err, "err", torch.float64, 2 * k)
    if w2 is not None:
        _need(w2, "w2", torch.float64, k)
    st = lib.aaac_refine_batch_noalloc(
        k, _arr(c_vp, [t.data_ptr() for t in Ws]), _arr(c_i64, Rs), _arr(c_i64, Cs), g, S, n,
        _arr(c_vp, [t.data_ptr() for t in Is]), _arr(c_vp, [t.data_ptr() for t in codes]),
        _arr(c_vp, [t.data_ptr() for t in sels]), _arr(c_vp, [t.data_ptr() for t in tables]),
        flags, _ptr(err), _ptr(w2), _stream(stream))
    _check(st, "aaac_refine_batch_noalloc")
