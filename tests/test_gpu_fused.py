"""GPU tests of the one-launch iteration (aaac_assign_refine_batch): bitwise equal to the assign
launch followed by the refine launch, and step-wise parity with the fp64 oracle."""

import numpy as np
import pytest
import torch

from oracle import aaac_ref as ref
from synth import layers as syn
from tests import parity as par

pytestmark = pytest.mark.gpu

P = pytest.importorskip("post_weight_quantization_06_amd")
L = P._lib

DEV = "cuda"


def _say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    L.load()
    yield


def _np(t):
    return t.detach().cpu().numpy()


def _setup(shapes, g, S, n, seed):
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    Ws = [syn.make_weight(R, C, seed * 31 + i, DEV) for i, (R, C) in enumerate(shapes)]
    Is = [torch.rand(C, device=DEV, generator=gen) * 4.0 + 0.05 for _, C in shapes]
    tabs = []
    for W in Ws:
        t = torch.empty(2 * n, dtype=torch.float32, device=DEV)
        L.aaac_init_quantiles(W, g, n, t)
        tabs.append(t)
    return Ws, Is, tabs


def _buffers(shapes, S):
    codes = [torch.empty(R * C // 2, dtype=torch.uint8, device=DEV) for R, C in shapes]
    sels = [torch.empty(R * C // S, dtype=torch.uint8, device=DEV) for R, C in shapes]
    return codes, sels


def _run_both(shapes, g, S, n, iters, seed):
    Ws, Is, tabs = _setup(shapes, g, S, n, seed)
    tf = [t.clone() for t in tabs]
    t2 = [t.clone() for t in tabs]
    cf, sf = _buffers(shapes, S)
    c2, s2 = _buffers(shapes, S)
    Rs = [R for R, _ in shapes]
    Cs = [C for _, C in shapes]
    wsf = L.workspace(L.batch_workspace_bytes(L.OP_REFINE, Rs, Cs, g, S, n), DEV)
    ws2 = L.workspace(L.batch_workspace_bytes(L.OP_REFINE, Rs, Cs, g, S, n), DEV)
    k = len(shapes)
    ef, e2 = (torch.zeros(2, k, dtype=torch.float64, device=DEV) for _ in range(2))
    wf, w2 = (torch.zeros(k, dtype=torch.float64, device=DEV) for _ in range(2))
    for it in range(iters):
        # the error outputs every iteration: I w^2 summed on the first, read back after that
        flags = (L.REFINE_ROUND_BF16 if it == iters - 1 else 0) | (L.REFINE_W2_KNOWN if it else 0)
        L.aaac_assign_refine_batch(Ws, g, S, n, Is, tf, cf, sf, flags, wsf, err=ef, w2=wf)
        L.aaac_assign_batch(Ws, g, S, n, Is, t2, c2, s2)
        L.aaac_refine_batch(Ws, g, S, n, Is, c2, s2, t2, flags, ws2, err=e2, w2=w2)
        torch.cuda.synchronize()
        for i in range(k):
            assert torch.equal(cf[i], c2[i]), ("codes", it, shapes[i])
            assert torch.equal(sf[i], s2[i]), ("sel", it, shapes[i])
            assert torch.equal(tf[i], t2[i]), ("tables", it, shapes[i], _np(tf[i]), _np(t2[i]))
        assert torch.equal(ef, e2), ("err", it, _np(ef), _np(e2))
        assert torch.equal(wf, w2), ("w2", it, _np(wf), _np(w2))
    # and without error outputs
    L.aaac_assign_refine_batch(Ws, g, S, n, Is, tf, cf, sf, 0, wsf)
    L.aaac_assign_batch(Ws, g, S, n, Is, t2, c2, s2)
    L.aaac_refine_batch(Ws, g, S, n, Is, c2, s2, t2, 0, ws2)
    torch.cuda.synchronize()
    for i in range(k):
        assert torch.equal(cf[i], c2[i]) and torch.equal(sf[i], s2[i])
        assert torch.equal(tf[i], t2[i])
    # the workspaces are left zeroed for the next call
    assert int(wsf[:256].count_nonzero()) == 0
    return Ws, Is, tf, cf, sf


@pytest.mark.parametrize("g,S,n", [(128, 128, 16), (128, 16, 16), (16, 16, 15), (64, 32, 16),
                                   (128, 8, 16)])
def test_fused_bitwise_equal_to_two_launches(g, S, n):
    # ragged shapes: rows not a multiple of a task, a partial last slab, a one-row matrix, and a
    # row length whose codes do not end on a cache line
    shapes = [(37, 1152), (16, 4096), (300, 2048), (1, 256)]
    shapes = [(R, C) for R, C in shapes if C % g == 0]
    _say("fused vs two launches", g, S, n, shapes)
    _run_both(shapes, g, S, n, iters=3, seed=g + S + n)


def test_fused_step_parity_with_oracle():
    g, S, n = 128, 128, 16
    shapes = [(64, 1024), (24, 3072)]
    _say("fused step parity", shapes)
    Ws, Is, tabs = _setup(shapes, g, S, n, 5)
    codes, sels = _buffers(shapes, S)
    Rs = [R for R, _ in shapes]
    Cs = [C for _, C in shapes]
    ws = L.workspace(L.batch_workspace_bytes(L.OP_REFINE, Rs, Cs, g, S, n), DEV)
    for it in range(2):
        T_in = [_np(t).astype(np.float64).reshape(2, n) for t in tabs]
        L.aaac_assign_refine_batch(Ws, g, S, n, Is, tabs, codes, sels, 0, ws)
        torch.cuda.synchronize()
        for i, (R, C) in enumerate(shapes):
            W64 = par.to_np64(Ws[i])
            I64 = par.to_np64(Is[i])
            q = par.unpack_gpu_codes(codes[i], R, C)
            s = _np(sels[i]).reshape(R, C // S)
            par.check_assign(W64, I64, T_in[i], g, S, q, s)
            want, _, _, bound = par.oracle_refine(W64, I64, q, s, T_in[i], g, S)
            par.check_tables(_np(tabs[i]).astype(np.float64).reshape(2, n), want, bound)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("cfg_id", [2, 3, 4, 5])
def test_fused_full_size_layers(cfg_id):
    """Whole layers of the 8B-shaped (INT4 and NVFP4-style), 13B-shaped (S = 16 bitmap) and
    32B-shaped workloads over all their iterations, bitwise against the two launches."""
    cfg = syn.config(cfg_id)
    shapes = [(m.rows, m.cols) for m in cfg.matrices]
    _say("fused full size", cfg.name)
    _run_both(shapes, cfg.g, cfg.S, cfg.n, iters=cfg.iters, seed=cfg_id)


@pytest.mark.parametrize("kind", ["edge", "up", "down"])
def test_fused_extreme_group_scales(kind):
    """Groups whose scales leave the fast range (zero, subnormal, 3e30 and 2^+-100 scales: the
    exact scan) through the fused iteration, bitwise against the two launches."""
    from tests import test_gpu_parity as gp

    g, S, n = 128, 128, 16
    W = gp._edge_matrix(kind, 64, 512)
    _say("fused extreme scales", kind)
    gen = torch.Generator(device=DEV).manual_seed(73)
    I = torch.rand(512, device=DEV, generator=gen) * 4.0 + 0.05
    if kind == "edge":
        I[:32] = 0
        I[100:104] = 1e20
    tabs = torch.empty(2 * n, dtype=torch.float32, device=DEV)
    L.aaac_init_quantiles(W, g, n, tabs)
    Ws, Is = [W], [I]
    tf, t2 = [tabs.clone()], [tabs.clone()]
    cf, sf = _buffers([(64, 512)], S)
    c2, s2 = _buffers([(64, 512)], S)
    wsb = L.batch_workspace_bytes(L.OP_REFINE, [64], [512], g, S, n)
    wsf, ws2 = L.workspace(wsb, DEV), L.workspace(wsb, DEV)
    ef, e2 = (torch.zeros(2, 1, dtype=torch.float64, device=DEV) for _ in range(2))
    wf, w2 = (torch.zeros(1, dtype=torch.float64, device=DEV) for _ in range(2))
    for it in range(3):
        flags = (L.REFINE_ROUND_BF16 if it == 2 else 0) | (L.REFINE_W2_KNOWN if it else 0)
        L.aaac_assign_refine_batch(Ws, g, S, n, Is, tf, cf, sf, flags, wsf, err=ef, w2=wf)
        L.aaac_assign_batch(Ws, g, S, n, Is, t2, c2, s2)
        L.aaac_refine_batch(Ws, g, S, n, Is, c2, s2, t2, flags, ws2, err=e2, w2=w2)
        torch.cuda.synchronize()
        assert torch.equal(cf[0], c2[0]) and torch.equal(sf[0], s2[0]), (kind, it)
        assert torch.equal(tf[0], t2[0]), (kind, it, _np(tf[0]), _np(t2[0]))
        assert bool(torch.isfinite(tf[0]).all())
        assert torch.equal(ef, e2) and torch.equal(wf, w2)



@pytest.mark.parametrize("g,S,n", [(128, 128, 16), (128, 16, 16)])
def test_run_loop_fused_equals_two_launch_loop(g, S, n):
    """quantize.run_loop with one fused launch per iteration: every output and the error history
    bitwise those of the two-launch loop."""
    shapes = [(37, 1152), (16, 4096), (300, 2048)]
    shapes = [(R, C) for R, C in shapes if C % g == 0]
    _say("run_loop fused", g, S, n, shapes)
    Ws, Is, _ = _setup(shapes, g, S, n, 9)
    out = []
    for fused in (False, True):
        buf = P.LayerBuffers(shapes, g, S, n, 6, DEV)
        P.run_loop(Ws, Is, buf, P.Workspaces(DEV), fused=fused)
        torch.cuda.synchronize()
        out.append(buf)
    a, b = out
    for i in range(len(shapes)):
        assert torch.equal(a.codes[i], b.codes[i]) and torch.equal(a.sels[i], b.sels[i])
        assert torch.equal(a.tables[i], b.tables[i]) and torch.equal(a.scales[i], b.scales[i])
        assert torch.equal(a.tables_bf16[i], b.tables_bf16[i])
    assert torch.equal(a.err, b.err) and torch.equal(a.w2, b.w2)
    P.check_history(b.err, w2=b.w2)
