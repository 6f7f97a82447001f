"""Loop driver over the C ABI (AAAC summary §2 mechanism 4): init, iters x (assign, refine), bf16
tables, final assign, pack.

Control flow only: every step is one library call enqueued on the current stream; the host does not
synchronize inside the loop. Device buffers come from torch.
"""

from __future__ import annotations

import dataclasses
from typing import Iterable, List, Optional, Sequence

import torch

from . import _lib as L


@dataclasses.dataclass
class QuantizedMatrix:
    R: int
    C: int
    g: int
    S: int
    n: int
    codes: torch.Tensor          # uint8 [R, C/2], low nibble = even column
    sel: torch.Tensor            # uint8 [R, C/S]
    tables: torch.Tensor         # fp32 [2, n] (bf16-exact after the loop)
    scales: torch.Tensor         # int16 [R, C/g] bf16 bits, sign bit = selector when S == g
    bitmap: Optional[torch.Tensor]  # uint8 [ceil(R C / S / 8)] when S < g
    tables_bf16: torch.Tensor    # int16 [2, n] bf16 bits

    def dequant(self, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        if out is None:
            out = torch.empty(self.R, self.C, dtype=torch.bfloat16, device=self.codes.device)
        L.aaac_dequant(self.codes, self.scales, self.bitmap, self.tables_bf16, self.R, self.C,
                       self.g, self.S, self.n, out)
        return out

    def gemv(self, x: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """fp32 [B, R] = the packed weights times x (bf16 [B, C] or [C], B <= 4), decoded on the
        fly (AAAC summary §1: the dequantized values are what inference uses)."""
        x2 = x.reshape(-1, self.C).contiguous()
        if out is None:
            out = torch.empty(x2.shape[0], self.R, dtype=torch.float32, device=x.device)
        L.aaac_gemv(self.codes, self.scales, self.bitmap, self.tables_bf16, self.R, self.C,
                    self.g, self.S, self.n, x2, out)
        return out


def importance(chunks: Iterable[torch.Tensor], K: int, device) -> torch.Tensor:
    """fp32 [K] I_k = sum over all chunks of X[:, k]^2, accumulated in fp64 on the device."""
    acc = torch.zeros(K, dtype=torch.float64, device=device)
    out = torch.empty(K, dtype=torch.float32, device=device)
    ws = None
    any_chunk = False
    for X in chunks:
        need = L.workspace_bytes(L.OP_IMPORTANCE, X.shape[0], K)
        if ws is None or ws.numel() < need:
            ws = L.workspace(need, device)
        L.aaac_importance(X, acc, out, ws)
        any_chunk = True
    if not any_chunk:
        L.aaac_importance(torch.empty(0, K, dtype=torch.float32, device=device), acc, out)
    return out


class Workspaces:
    """Zero-filled workspaces reused across the calls of one quantization run."""

    def __init__(self, device):
        self.device = device
        self._ws = {}

    def get(self, key, nbytes) -> torch.Tensor:
        t = self._ws.get(key)
        if t is None or t.numel() < nbytes:
            t = L.workspace(nbytes, self.device)
            self._ws[key] = t
        return t


def _batches(seq, k=L.MAX_BATCH):
    for i in range(0, len(seq), k):
        yield i, seq[i:i + k]


def quantize_matrices(Ws: Sequence[torch.Tensor], Is: Sequence[torch.Tensor], g: int, S: int,
                      n: int, iters: int, tables: Optional[Sequence[torch.Tensor]] = None,
                      workspaces: Optional[Workspaces] = None) -> List[QuantizedMatrix]:
    """Quantize matrices that share (g, S, n); matrix i uses importance Is[i] (fp32 [C_i])."""
    if iters < 1:
        raise ValueError("iters must be >= 1 (the last refine rounds the tables to bf16)")
    dev = Ws[0].device
    wsp = workspaces or Workspaces(dev)
    k = len(Ws)
    Rs = [W.shape[0] for W in Ws]
    Cs = [W.shape[1] for W in Ws]
    codes = [torch.empty(R * C // 2, dtype=torch.uint8, device=dev) for R, C in zip(Rs, Cs)]
    sels = [torch.empty(R * C // S, dtype=torch.uint8, device=dev) for R, C in zip(Rs, Cs)]
    if tables is None:
        tabs = [torch.empty(2 * n, dtype=torch.float32, device=dev) for _ in range(k)]
        for b0, group in _batches(list(range(k))):
            sl = slice(b0, b0 + len(group))
            need = L.batch_workspace_bytes(L.OP_INIT, Rs[sl], Cs[sl], g, 8, n)
            L.aaac_init_quantiles_batch(Ws[sl], g, n, tabs[sl], wsp.get("init", need))
    else:
        tabs = [t.reshape(-1).to(torch.float32).clone() for t in tables]
    for it in range(iters):
        flags = L.REFINE_ROUND_BF16 if it == iters - 1 else 0
        for b0, group in _batches(list(range(k))):
            sl = slice(b0, b0 + len(group))
            Wb, Ib = Ws[sl], Is[sl]
            L.aaac_assign_batch(Wb, g, S, n, Ib, tabs[sl], codes[sl], sels[sl])
            ws_r = wsp.get(("refine", b0), L.batch_workspace_bytes(
                L.OP_REFINE, Rs[sl], Cs[sl], g, S, n))
            L.aaac_refine_batch(Wb, g, S, n, Ib, codes[sl], sels[sl], tabs[sl], flags, ws_r)
    for b0, group in _batches(list(range(k))):
        sl = slice(b0, b0 + len(group))
        L.aaac_assign_batch(Ws[sl], g, S, n, Is[sl], tabs[sl], codes[sl], sels[sl])
    scales = [torch.empty(R * C // g, dtype=torch.int16, device=dev) for R, C in zip(Rs, Cs)]
    bitmaps = ([torch.empty((R * C // S + 7) // 8, dtype=torch.uint8, device=dev)
                for R, C in zip(Rs, Cs)] if S < g else None)
    tbs = [torch.empty(2 * n, dtype=torch.int16, device=dev) for _ in range(k)]
    for b0, group in _batches(list(range(k))):
        sl = slice(b0, b0 + len(group))
        L.aaac_pack_batch(Ws[sl], g, S, n, sels[sl], tabs[sl], scales[sl],
                          bitmaps[sl] if bitmaps is not None else None, tbs[sl])
    out = []
    for i in range(k):
        R, C = Rs[i], Cs[i]
        out.append(QuantizedMatrix(R, C, g, S, n, codes[i].view(R, C // 2),
                                   sels[i].view(R, C // S), tabs[i].view(2, n),
                                   scales[i].view(R, C // g),
                                   bitmaps[i] if bitmaps is not None else None,
                                   tbs[i].view(2, n)))
    return out


def quantize_matrix(W: torch.Tensor, I: torch.Tensor, g: int = 128, S: int = 128, n: int = 16,
                    iters: int = 10, tables=None) -> QuantizedMatrix:
    return quantize_matrices([W], [I], g, S, n, iters,
                             None if tables is None else [tables])[0]


def awq_prescale(W: torch.Tensor, a: torch.Tensor, I: Optional[torch.Tensor] = None):
    """Inputs for quantizing W diag(a) after AWQ-style weight scaling (AAAC summary §4):
    (bf16(W * a), fp32(I / a^2) or None). The inference side then feeds x / a."""
    Ws = torch.empty_like(W)
    Is = None if I is None else torch.empty_like(I)
    L.aaac_awq_prescale(W, a, Ws, I, Is)
    return Ws, Is
