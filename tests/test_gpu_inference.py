"""GPU parity of the inference-side entry points against the fp64 oracle: the AWQ pre-scale hook
(bit-exact) and the decode GEMV on the packed format (within the fp32 rounding bound)."""

import numpy as np
import pytest
import torch

from oracle import aaac_ref as ref
from synth import layers as syn

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


def _bits(t):
    return _np(t.view(torch.int16)).view(np.uint16)


# ------------------------------------------------------------------ AWQ pre-scale

@pytest.mark.parametrize("R,C", [(1, 8), (3, 24), (64, 4096), (257, 1032)])
def test_awq_prescale_bit_exact(R, C):
    _say("awq_prescale", R, C)
    rng = np.random.default_rng(R * 131 + C)
    W = syn.make_weight(R, C, syn.seed_for(1, 0, 0) + R + C, DEV)
    a = np.exp(rng.normal(0.0, 0.7, size=C)).astype(np.float32)
    I = (np.exp(rng.normal(0.0, 2.0, size=C)) * 1e3).astype(np.float32)
    a_t = torch.from_numpy(a).to(DEV)
    I_t = torch.from_numpy(I).to(DEV)
    Ws = torch.empty_like(W)
    Is = torch.empty_like(I_t)
    L.aaac_awq_prescale(W, a_t, Ws, I_t, Is)
    torch.cuda.synchronize()
    want_w, want_i = ref.awq_prescale(_np(W.float()).astype(np.float64), a, I)
    assert np.array_equal(_bits(Ws).reshape(R, C), ref.bf16_bits(want_w))
    assert np.array_equal(_np(Is), want_i)


def test_awq_prescale_edge_values_and_in_place():
    _say("awq_prescale edges")
    C = 16
    # zeros of both signs, bf16 subnormals, products that become subnormal, tie cases, overflow
    w = np.array([0.0, -0.0, 2.0 ** -130, -(2.0 ** -133), 1.0, -1.0, 3.0, 1.0 + 2 ** -7,
                  2.0 ** 120, -(2.0 ** 120), 0.5, 1.5, 2.0 ** -100, 7.0, -7.0, 0.0078125])
    a = np.array([3.0, 3.0, 0.75, 1.0, 1.0 + 2 ** -8, 1.0 + 2 ** -8, 1.0 / 3.0, 1.0 + 2 ** -9,
                  2.0 ** 9, 2.0 ** 7, 2.0 ** -30, 1.00390625, 2.0 ** -30, 1.1, 0.9, 1.0],
                 dtype=np.float32)
    W = torch.from_numpy(w.astype(np.float32)).to(torch.bfloat16).reshape(1, C).to(DEV)
    W0 = W.clone()
    a_t = torch.from_numpy(a).to(DEV)
    I_t = torch.from_numpy(np.linspace(0.5, 8.0, C).astype(np.float32)).to(DEV)
    I0 = I_t.clone()
    L.aaac_awq_prescale(W, a_t, W, I_t, I_t)        # in place
    torch.cuda.synchronize()
    want_w, want_i = ref.awq_prescale(_np(W0.float()).astype(np.float64), a, _np(I0))
    got = _bits(W).reshape(1, C)
    assert np.array_equal(got[np.isfinite(want_w)], ref.bf16_bits(want_w[np.isfinite(want_w)]))
    inf = ~np.isfinite(want_w)
    assert inf.any()
    assert np.array_equal(got[inf], np.where(want_w[inf] > 0, 0x7F80, 0xFF80).astype(np.uint16))
    assert np.array_equal(_np(I_t), want_i)


def test_awq_prescale_without_importance():
    W = syn.make_weight(8, 64, 77, DEV)
    a = torch.full((64,), 2.0, dtype=torch.float32, device=DEV)
    Ws = torch.empty_like(W)
    L.aaac_awq_prescale(W, a, Ws)
    torch.cuda.synchronize()
    assert torch.equal(Ws.float(), W.float() * 2.0)


# ------------------------------------------------------------------ decode GEMV

def _packed_inputs(rng, R, C, g, S, n):
    """A seeded packed matrix: bell-shaped codes, sorted bf16 tables, positive bf16 scales with the
    selector in the sign bit (S == g) or an LSB-first bitmap (S < g)."""
    q = np.clip(np.rint(rng.normal((n - 1) / 2.0, n / 5.0, size=(R, C))), 0, n - 1).astype(np.uint8)
    code_bytes = (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)
    sel = (rng.random((R, C // S)) < 0.4).astype(np.uint8)
    s = np.abs(rng.normal(0.05, 0.02, size=(R, C // g))) + 1e-3
    s_bits = ref.bf16_bits(ref.bf16_round(s)).astype(np.uint16)
    T = np.sort(rng.uniform(-1.0, 1.0, size=(2, n)), axis=1)
    tables = ref.bf16_bits(ref.bf16_round(T)).astype(np.uint16)
    if S == g:
        scales = s_bits | (sel.astype(np.uint16) << 15)
        bitmap = None
    else:
        scales = s_bits
        bits = sel.reshape(-1)
        pad = (-bits.size) % 8
        bits = np.concatenate([bits, np.zeros(pad, np.uint8)]).reshape(-1, 8)
        bitmap = (bits << np.arange(8, dtype=np.uint8)).sum(axis=1).astype(np.uint8)
    return code_bytes, scales, bitmap, tables


def _bf16_x(rng, B, C):
    return ref.bf16_round(rng.standard_normal((B, C)))


def _to_dev(code_bytes, scales, bitmap, tables, x):
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(DEV).view(dt).reshape(-1)  # noqa
    xb = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(DEV)
    return (t(code_bytes, torch.uint8), t(scales.astype(np.uint16).view(np.int16), torch.int16),
            None if bitmap is None else t(bitmap, torch.uint8),
            t(tables.astype(np.uint16).view(np.int16), torch.int16), xb.reshape(-1))


def _gemv_bound(C, g):
    """Rounding bound of the fp32 evaluation, relative to sum |term|: per lane 16 code bytes per
    2048-column slab, each v_dot2 at most two roundings, one scaling per scale group, then a
    six-level butterfly over the lanes."""
    nslab = -(-C // 2048)
    gpl = 1 if g >= 32 else 32 // g
    return (32 * nslab + gpl * nslab + 6 + 2) * 2.0 ** -24


def _check_gemv(y_gpu, y_ref, a_ref, C, g):
    bound = _gemv_bound(C, g) * a_ref + 1e-30
    err = np.abs(y_gpu - y_ref)
    assert np.all(err <= bound), "max err/bound %.3g" % np.max(err / bound)


@pytest.mark.parametrize("R,C,g,S,n,B", [
    (16, 2048, 128, 128, 16, 1),     # one slab, one task
    (37, 5120, 128, 128, 16, 1),     # ragged rows, partial last slab
    (33, 4096, 128, 16, 16, 2),      # selection bitmap
    (20, 6144, 16, 16, 15, 1),       # NVFP4-style groups: two scales per lane row
    (9, 2080, 8, 8, 16, 3),          # g = 8: four scales per lane row, 32-column tail slab
    (12, 1024, 32, 8, 16, 4),        # S = 8 < g: four selection groups per lane row
    (18, 3072, 16, 8, 12, 1),        # g = 16, S = 8
])
def test_gemv_parity(R, C, g, S, n, B):
    _say("gemv", R, C, g, S, n, B)
    rng = np.random.default_rng(R * 1000 + C + g + S + n + B)
    cb, sc, bm, tb = _packed_inputs(rng, R, C, g, S, n)
    x = _bf16_x(rng, B, C)
    dcb, dsc, dbm, dtb, dx = _to_dev(cb, sc, bm, tb, x)
    y = torch.full((B * R,), float("nan"), dtype=torch.float32, device=DEV)
    L.aaac_gemv(dcb, dsc, dbm, dtb, R, C, g, S, n, dx.reshape(B, C), y)
    torch.cuda.synchronize()
    y_ref, a_ref = ref.gemv(cb, sc, bm, tb.reshape(2, n), R, C, g, S, x)
    _check_gemv(_np(y).reshape(B, R).astype(np.float64), y_ref, a_ref, C, g)
    # the same inputs through the dequantized bf16 weights differ only by that storage rounding
    W_hat = ref.dequant(cb, sc, bm, tb.reshape(2, n), R, C, g, S)
    assert np.all(np.abs(_np(y).reshape(B, R) - x @ W_hat.T) <= 2.0 ** -8 * a_ref + 1e-30)


def test_gemv_batch_matches_single_calls_bitwise():
    _say("gemv batch")
    rng = np.random.default_rng(7)
    shapes = [(48, 4096), (16, 14336), (64, 2048), (5, 5120)]
    g, S, n, B = 128, 128, 16, 2
    ins, xs, ys, singles = [], [], [], []
    for R, C in shapes:
        cb, sc, bm, tb = _packed_inputs(rng, R, C, g, S, n)
        x = _bf16_x(rng, B, C)
        d = _to_dev(cb, sc, bm, tb, x)
        ins.append(d)
        xs.append(d[4].reshape(B, C))
        ys.append(torch.empty(B * R, dtype=torch.float32, device=DEV))
        y1 = torch.empty(B * R, dtype=torch.float32, device=DEV)
        L.aaac_gemv(d[0], d[1], None, d[3], R, C, g, S, n, xs[-1], y1)
        singles.append(y1)
    L.aaac_gemv_batch([d[0] for d in ins], [d[1] for d in ins], None, [d[3] for d in ins],
                      [s[0] for s in shapes], [s[1] for s in shapes], g, S, n, xs, ys)
    torch.cuda.synchronize()
    for a, b in zip(ys, singles):
        assert torch.equal(a, b)


def test_gemv_full_size_layer_sampled_rows():
    # every linear of the 8B-shaped decoder layer in one batched launch, as the bench times it
    _say("gemv full size 8B layer")
    cfg = syn.config(2)
    rng = np.random.default_rng(11)
    g, S, n = cfg.g, cfg.S, cfg.n
    devs, xs, ys, hosts = [], [], [], []
    for m in cfg.matrices:
        cb, sc, bm, tb = _packed_inputs(rng, m.rows, m.cols, g, S, n)
        x = _bf16_x(rng, 1, m.cols)
        d = _to_dev(cb, sc, bm, tb, x)
        devs.append(d)
        xs.append(d[4].reshape(1, m.cols))
        ys.append(torch.empty(m.rows, dtype=torch.float32, device=DEV))
        hosts.append((cb, sc, tb, x))
    L.aaac_gemv_batch([d[0] for d in devs], [d[1] for d in devs], None, [d[3] for d in devs],
                      [m.rows for m in cfg.matrices], [m.cols for m in cfg.matrices], g, S, n,
                      xs, ys)
    torch.cuda.synchronize()
    for m, (cb, sc, tb, x), y in zip(cfg.matrices, hosts, ys):
        rows = np.sort(rng.choice(m.rows, size=48, replace=False))
        y_ref, a_ref = ref.gemv(cb[rows], sc[rows], None, tb.reshape(2, n), rows.size, m.cols,
                                g, S, x)
        _check_gemv(_np(y)[rows][None, :].astype(np.float64), y_ref, a_ref, m.cols, g)
