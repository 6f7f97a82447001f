"""Loop driver over the C ABI (AAAC summary §2 mechanism 4): importance, init, iters x (assign,
refine), bf16 tables, final assign, pack -- for a set of matrices, a decoder layer, or a whole model
streamed layer by layer (§4: models up to 32B; every layer is quantized on its own, from its own
activations).

Control flow only: every step is one library call enqueued on the current stream; the host does not
synchronize inside the loop. Device buffers come from torch.

The total weighted error after every half-step is kept on the device in a history
[2 iters + 1, matrices]: rows 2t and 2t + 1 are the error of iteration t's assignment under the
tables it was chosen with and under the tables refine t wrote, both reported by that refine from
its cell sums (W2 = sum I w^2 is one register sum per thread on the first refine), and the last row
is the final assign's own err_total against the bf16 tables. The alternation is a descent (each
half-step minimizes the error over its own variables), so the history never increases except
across the last refine, whose entries are rounded to bf16; `check_history` verifies that after the
loop (one host read).
"""

from __future__ import annotations

import dataclasses
from typing import Callable, Dict, Iterable, List, Optional, Sequence, Tuple

import torch

from . import _lib as L

# relative slack of the monotonicity check: the error totals are fp64 sums of fp32-rounded terms
# (relative error below 2.4e-7), and decisions inside the 1e-6 tie band may go either way
MONOTONE_RTOL = 1e-6


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
    # fp64 [2 iters + 1]: the total error after every half-step (assign 0, refine 0, assign 1, ...,
    # refine iters-1 on bf16 tables, the final assign)
    err_history: Optional[torch.Tensor] = None

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


class Workspaces:
    """Zero-filled workspaces reused across the calls of one quantization run (each call leaves its
    counters zero again, so a workspace serves any later call it is large enough for)."""

    def __init__(self, device):
        self.device = device
        self._ws = {}

    def get(self, key, nbytes) -> torch.Tensor:
        t = self._ws.get(key)
        if t is None or t.numel() < nbytes:
            t = L.workspace(nbytes, self.device)
            self._ws[key] = t
        return t


def importance(chunks: Iterable[torch.Tensor], K: int, device,
               workspaces: Optional[Workspaces] = None, acc: Optional[torch.Tensor] = None,
               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp32 [K] I_k = sum over all chunks of X[:, k]^2, accumulated in fp64 on the device (AAAC
    summary §2 mechanism 2). chunks: fp32 [T_i, K] tensors (one resident tensor is one chunk)."""
    wsp = workspaces or Workspaces(device)
    acc = torch.zeros(K, dtype=torch.float64, device=device) if acc is None else acc.zero_()
    out = torch.empty(K, dtype=torch.float32, device=device) if out is None else out
    any_chunk = False
    for X in chunks:
        L.aaac_importance(X, acc, out, wsp.get(("importance", K),
                                               L.workspace_bytes(L.OP_IMPORTANCE, X.shape[0], K)))
        any_chunk = True
    if not any_chunk:
        L.aaac_importance(torch.empty(0, K, dtype=torch.float32, device=device), acc, out)
    return out


def _batches(k, size=L.MAX_BATCH):
    for b0 in range(0, k, size):
        yield slice(b0, min(k, b0 + size))


class LayerBuffers:
    """Device outputs of one set of matrices that share (g, S, n): codes, selectors, fp32 and bf16
    tables, scales, bitmaps and the error history. Allocated once; a run overwrites them."""

    def __init__(self, shapes: Sequence[Tuple[int, int]], g: int, S: int, n: int, iters: int,
                 device):
        self.shapes = [tuple(s) for s in shapes]
        self.g, self.S, self.n, self.iters = g, S, n, iters
        self.device = device
        dev = device
        self.codes = [torch.empty(R * C // 2, dtype=torch.uint8, device=dev) for R, C in shapes]
        self.sels = [torch.empty(R * C // S, dtype=torch.uint8, device=dev) for R, C in shapes]
        self.tables = [torch.empty(2 * n, dtype=torch.float32, device=dev) for _ in shapes]
        self.scales = [torch.empty(R * C // g, dtype=torch.int16, device=dev) for R, C in shapes]
        self.bitmaps = ([torch.empty((R * C // S + 7) // 8, dtype=torch.uint8, device=dev)
                         for R, C in shapes] if S < g else None)
        self.tables_bf16 = [torch.empty(2 * n, dtype=torch.int16, device=dev) for _ in shapes]
        # error history, one tensor per batch of matrices (the calls write a batch's rows whole):
        # row 2t = total error of iteration t's assignment under the tables it was chosen with,
        # row 2t + 1 = the same assignment under the tables refine t wrote (both from refine t),
        # row 2 iters = the final assign's; w2[i] = sum I w^2 of matrix i (summed by the first
        # refine, read by the others)
        self.batches = list(_batches(len(shapes)))
        self.err_b = [torch.zeros(2 * iters + 1, b.stop - b.start, dtype=torch.float64,
                                  device=dev) for b in self.batches]
        self.w2 = torch.zeros(len(shapes), dtype=torch.float64, device=dev)

    @property
    def err(self) -> torch.Tensor:
        """fp64 [2 iters + 1, matrices]: the half-step error history of every matrix."""
        return self.err_b[0] if len(self.err_b) == 1 else torch.cat(self.err_b, dim=1)

    def results(self) -> List[QuantizedMatrix]:
        out = []
        err = self.err
        for i, (R, C) in enumerate(self.shapes):
            out.append(QuantizedMatrix(
                R, C, self.g, self.S, self.n, self.codes[i].view(R, C // 2),
                self.sels[i].view(R, C // self.S), self.tables[i].view(2, self.n),
                self.scales[i].view(R, C // self.g),
                self.bitmaps[i] if self.bitmaps is not None else None,
                self.tables_bf16[i].view(2, self.n), err[:, i]))
        return out


class Probe:
    """Hooks the loop calls on the host as it enqueues work (for timing with stream events).
    The default does nothing."""

    def loop_begin(self):
        pass

    def before_assign(self, it):
        pass

    def before_refine(self, it):
        pass

    def after_refine(self, it):
        pass

    def loop_end(self):
        pass


def run_loop(Ws: Sequence[torch.Tensor], Is: Sequence[torch.Tensor], buf: LayerBuffers,
             wsp: Workspaces, init: bool = True, pack: bool = True,
             probe: Optional[Probe] = None, totals: bool = True,
             fused: bool = False) -> LayerBuffers:
    """Enqueue the quantization of matrices Ws (bf16 [R_i, C_i]) with importances Is (fp32 [C_i])
    into buf: batched init (unless init is False: then buf.tables hold the starting tables),
    buf.iters x (batched assign, batched refine; the last refine rounds the tables to bf16), the
    final assign, and pack. With totals, every refine reports the error of the assignment it
    consumes before and after its update and the final assign its own (buf.err: every half-step),
    and the first refine sums buf.w2. With fused,
    each iteration is one aaac_assign_refine_batch call instead of the two (bitwise the same
    results; the probe's assign interval then covers the whole call)."""
    g, S, n, iters = buf.g, buf.S, buf.n, buf.iters
    if iters < 1:
        raise ValueError("iters must be >= 1 (the last refine rounds the tables to bf16)")
    k = len(Ws)
    Rs = [W.shape[0] for W in Ws]
    Cs = [W.shape[1] for W in Ws]
    if [tuple(W.shape) for W in Ws] != buf.shapes:
        raise ValueError("matrix shapes do not match the buffers")
    pr = probe or Probe()
    sl = buf.batches
    if init:
        for b in sl:
            need = L.batch_workspace_bytes(L.OP_INIT, Rs[b], Cs[b], g, 8, n)
            L.aaac_init_quantiles_batch(Ws[b], g, n, buf.tables[b], wsp.get("init", need))

    pr.loop_begin()
    for it in range(iters):
        flags = L.REFINE_ROUND_BF16 if it == iters - 1 else 0
        if totals and it > 0:
            flags |= L.REFINE_W2_KNOWN
        pr.before_assign(it)
        if fused:
            for bi, b in enumerate(sl):
                ws_r = wsp.get(("refine", b.start), L.batch_workspace_bytes(
                    L.OP_REFINE, Rs[b], Cs[b], g, S, n))
                L.aaac_assign_refine_batch(Ws[b], g, S, n, Is[b], buf.tables[b], buf.codes[b],
                                           buf.sels[b], flags, ws_r,
                                           buf.err_b[bi][2 * it:2 * it + 2] if totals else None,
                                           buf.w2[b] if totals else None)
            pr.before_refine(it)
        else:
            for b in sl:
                L.aaac_assign_batch(Ws[b], g, S, n, Is[b], buf.tables[b], buf.codes[b],
                                    buf.sels[b])
            pr.before_refine(it)
            for bi, b in enumerate(sl):
                ws_r = wsp.get(("refine", b.start), L.batch_workspace_bytes(
                    L.OP_REFINE, Rs[b], Cs[b], g, S, n))
                L.aaac_refine_batch(Ws[b], g, S, n, Is[b], buf.codes[b], buf.sels[b],
                                    buf.tables[b], flags, ws_r,
                                    buf.err_b[bi][2 * it:2 * it + 2] if totals else None,
                                    buf.w2[b] if totals else None)
        pr.after_refine(it)
    pr.loop_end()
    for bi, b in enumerate(sl):
        ws_a = (wsp.get(("assign", b.start), L.batch_workspace_bytes(L.OP_ASSIGN, Rs[b], Cs[b],
                                                                        g, S, n))
                if totals else None)
        L.aaac_assign_batch(Ws[b], g, S, n, Is[b], buf.tables[b], buf.codes[b], buf.sels[b],
                            buf.err_b[bi][2 * iters] if totals else None, ws_a)
    if pack:
        for b in sl:
            L.aaac_pack_batch(Ws[b], g, S, n, buf.sels[b], buf.tables[b], buf.scales[b],
                              buf.bitmaps[b] if buf.bitmaps is not None else None,
                              buf.tables_bf16[b])
    return buf


def check_history(err: torch.Tensor, rtol: float = MONOTONE_RTOL,
                  w2: Optional[torch.Tensor] = None, half_steps: bool = True):
    """Raise if the total error of some matrix increased along its history. With half_steps, err is
    the [2 iters + 1, matrices] history of run_loop (after every assign and every refine): every
    step may only lower the error, except the last refine, whose entries are rounded to bf16 (the
    final assign against them may then only lower it again). Without, err holds one row per
    iteration's assignment and a last row against the bf16 tables, which is not compared. The
    slack is rtol of the earlier value (the tie band of the decisions) plus, with w2 (sum I w^2 per
    matrix), the 1e-15 W2 accuracy of the errors refine reports. Reads the history from the device
    (synchronizes)."""
    h = err.detach().double().cpu()
    if h.dim() == 1:
        h = h[:, None]
    rows = h.shape[0]
    if half_steps:
        steps = [r for r in range(rows - 1) if r != rows - 3]
    else:
        steps = list(range(rows - 2))
    extra = 0.0 if w2 is None else 1e-13 * w2.detach().double().cpu().reshape(1, -1)
    for r in steps:
        slack = h[r:r + 1] * rtol + extra
        bad = h[r + 1:r + 2] > h[r:r + 1] + slack
        if bool(bad.any()):
            m = int(bad.nonzero()[0][1])
            raise RuntimeError("total error increased for matrix %d from history row %d to %d: "
                               "%.17g -> %.17g" % (m, r, r + 1, float(h[r, m]),
                                                   float(h[r + 1, m])))
    return h


def quantize_matrices(Ws: Sequence[torch.Tensor], Is: Sequence[torch.Tensor], g: int, S: int,
                      n: int, iters: int, tables: Optional[Sequence[torch.Tensor]] = None,
                      workspaces: Optional[Workspaces] = None,
                      check: bool = True) -> List[QuantizedMatrix]:
    """Quantize matrices that share (g, S, n); matrix i uses importance Is[i] (fp32 [C_i]).
    With check, the error history is verified to be non-increasing (one synchronization)."""
    dev = Ws[0].device
    wsp = workspaces or Workspaces(dev)
    buf = LayerBuffers([tuple(W.shape) for W in Ws], g, S, n, iters, dev)
    if tables is not None:
        for t, src in zip(buf.tables, tables):
            t.copy_(src.reshape(-1).to(torch.float32))
    run_loop(Ws, Is, buf, wsp, init=tables is None)
    if check:
        check_history(buf.err, w2=buf.w2)
    return buf.results()


def quantize_matrix(W: torch.Tensor, I: torch.Tensor, g: int = 128, S: int = 128, n: int = 16,
                    iters: int = 10, tables=None) -> QuantizedMatrix:
    return quantize_matrices([W], [I], g, S, n, iters,
                             None if tables is None else [tables])[0]


@dataclasses.dataclass
class Layer:
    """One decoder layer to quantize: its matrices, and for each matrix the id of the activation
    stream that feeds it (matrices that read the same input share a stream); streams maps each id
    to an iterable of fp32 [T_i, K] chunks of that input over the calibration tokens (or to one
    resident tensor)."""
    Ws: Sequence[torch.Tensor]
    stream_of: Sequence[int]
    streams: Dict[int, object]


def quantize_layer(layer: Layer, g: int, S: int, n: int, iters: int,
                   workspaces: Optional[Workspaces] = None,
                   buffers: Optional[LayerBuffers] = None,
                   probe: Optional[Probe] = None) -> LayerBuffers:
    """Importance of every activation stream of the layer, then run_loop over its matrices."""
    dev = layer.Ws[0].device
    wsp = workspaces or Workspaces(dev)
    Is_by = {}
    for sid, src in layer.streams.items():
        chunks = [src] if isinstance(src, torch.Tensor) else src
        K = next(W.shape[1] for W, s in zip(layer.Ws, layer.stream_of) if s == sid)
        Is_by[sid] = importance(chunks, K, dev, wsp)
    Is = [Is_by[s] for s in layer.stream_of]
    buf = buffers or LayerBuffers([tuple(W.shape) for W in layer.Ws], g, S, n, iters, dev)
    return run_loop(layer.Ws, Is, buf, wsp, probe=probe)


def quantize_model(layers: Iterable[Layer], g: int, S: int, n: int, iters: int,
                   on_layer: Optional[Callable[[int, List[QuantizedMatrix]], None]] = None,
                   check: bool = True) -> List[List[QuantizedMatrix]]:
    """Quantize a model layer after layer (AAAC summary §4: models up to 32B; §2 mechanism 4: each
    layer needs only its own activations, so layers are independent). The weights of every layer
    stay where the caller keeps them; the layers' outputs are kept and returned in order. One
    workspace set serves all layers. on_layer(i, results) runs after layer i is enqueued."""
    wsp = None
    out = []
    for i, layer in enumerate(layers):
        if wsp is None:
            wsp = Workspaces(layer.Ws[0].device)
        buf = quantize_layer(layer, g, S, n, iters, wsp)
        if check:
            check_history(buf.err, w2=buf.w2)
        res = buf.results()
        out.append(res)
        if on_layer is not None:
            on_layer(i, res)
    return out


def awq_prescale(W: torch.Tensor, a: torch.Tensor, I: Optional[torch.Tensor] = None):
    """Inputs for quantizing W diag(a) after AWQ-style weight scaling (AAAC summary §4):
    (bf16(W * a), fp32(I / a^2) or None). The inference side then feeds x / a."""
    Ws = torch.empty_like(W)
    Is = None if I is None else torch.empty_like(I)
    L.aaac_awq_prescale(W, a, Ws, I, Is)
    return Ws, Is
