"""Pins for the fp64 oracle against things other than itself (CPU only).

Each pin is chosen so that a plausible slip in the oracle -- a dropped weight, a wrong rank, a
flipped tie, a transposed operand -- fails at least one of them. The last section plants such
slips in copies of oracle functions and checks that the pins catch them.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import aaac_ref as ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16_matrix(rng, R, C, scale=0.02, outliers=0.01):
    z = rng.standard_normal((R, C)) * scale
    z *= np.where(rng.random((R, C)) < outliers, 20.0, 1.0)
    return torch.from_numpy(z.astype(np.float32)).to(torch.bfloat16).float().numpy().astype(np.float64)


# ------------------------------------------------------------------ bf16 rounding

def test_bf16_round_matches_torch_conversion():
    rng = np.random.default_rng(1)
    vals = [rng.standard_normal(20000) * 10.0 ** rng.integers(-40, 38, 20000)]
    # exact halfway cases with even and odd kept parts, and their neighbours
    hi = rng.integers(0, 0x7F7F, 4000, dtype=np.uint32)
    for low in (0x8000, 0x7FFF, 0x8001, 0x0000):
        bits = (hi << 16) | low
        vals.append(bits.view(np.float32).astype(np.float64))
        vals.append(-bits.view(np.float32).astype(np.float64))
    # subnormal fp32 inputs, and values near the overflow threshold
    vals.append((np.arange(1, 5000, dtype=np.uint32) * 97).view(np.float32).astype(np.float64))
    vals.append(np.array([3.3895e38, 3.39e38, 3.4e38, -3.4e38, 1e-45, -0.0, 0.0]))
    x = np.concatenate(vals).astype(np.float32).astype(np.float64)
    x = x[np.isfinite(x)]
    got = ref.bf16_round(x)
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).float().numpy()
    assert np.array_equal(np.signbit(got), np.signbit(want.astype(np.float64)))
    assert np.array_equal(got, want.astype(np.float64))


def test_bf16_bits_roundtrip():
    bits = np.arange(0, 0x7F80, 7, dtype=np.uint16)
    vals = ref.bits_to_float(bits)
    assert np.array_equal(ref.bf16_bits(vals), bits)
    assert np.array_equal(ref.bf16_bits(-vals[1:]), bits[1:] | 0x8000)
    with pytest.raises(ValueError):
        ref.bf16_bits(np.array([1.0 + 2.0 ** -10]))


# ------------------------------------------------------------------ importance

def test_importance_integer_exact():
    rng = np.random.default_rng(2)
    X = rng.integers(-1000, 1000, size=(777, 37)).astype(np.float32)
    want = [sum(int(v) * int(v) for v in X[:, k]) for k in range(X.shape[1])]
    got = ref.importance(X)
    assert got.dtype == np.float64
    assert [int(v) for v in got] == want


def test_importance_is_squared_column_norm():
    # column norm from the library's own BLAS-free routine, computed in fp64
    rng = np.random.default_rng(3)
    X = rng.standard_t(4, size=(300, 50)).astype(np.float32)
    assert np.allclose(ref.importance(X), np.linalg.norm(X.astype(np.float64), axis=0) ** 2,
                       rtol=1e-13, atol=0)


# ------------------------------------------------------------------ scales / normalization

def test_group_scales_and_normalized_bruteforce():
    rng = np.random.default_rng(4)
    W = _bf16_matrix(rng, 5, 24)
    W[1, 8:16] = 0.0                      # an all-zero group
    W[2, 0:8] = -0.0
    s = ref.group_scales(W, 8)
    u = ref.normalized(W, 8)
    for r in range(5):
        for G in range(3):
            grp = W[r, 8 * G:8 * G + 8]
            m = max(abs(v) for v in grp)
            assert s[r, G] == m
            for i, v in enumerate(grp):
                expect = 0.0 if m == 0 else v / m
                assert u[r, 8 * G + i] == expect
                if expect == 0:
                    assert not math.copysign(1.0, u[r, 8 * G + i]) < 0
    assert np.all(np.abs(u) <= 1.0)


# ------------------------------------------------------------------ init

@pytest.mark.parametrize("n", [2, 3, 15, 16])
def test_init_tables_match_partition(n):
    rng = np.random.default_rng(5 + n)
    W = _bf16_matrix(rng, 37, 64)
    T0, T1 = ref.init_tables(W, 16, n)
    u = ref.normalized(W, 16).ravel()
    N = u.size
    for j in range(n):
        k0 = ((2 * j + 1) * N) // (2 * n)
        k1 = min(N - 1, ((j + 1) * N) // n)
        assert T0[j] == np.partition(u, k0)[k0]
        assert T1[j] == np.partition(u, k1)[k1]
    assert T1[-1] == u.max()
    # half-step interleave: T0[j] <= T1[j] <= T0[j+1]
    assert np.all(T0 <= T1) and np.all(T1[:-1] <= T0[1:])


def test_init_tables_tiny_sorted_list():
    W = np.array([[4.0, -2.0, 1.0, 0.5, -1.0, 3.0, 0.25, -4.0]])
    T0, T1 = ref.init_tables(W, 4, 2)
    # u of the two groups: [1, -0.5, 0.25, 0.125] and [-0.25, 0.75, 0.0625, -1]
    V = sorted([1, -0.5, 0.25, 0.125, -0.25, 0.75, 0.0625, -1])
    assert list(T0) == [V[2], V[6]]            # floor(1*8/4) = 2, floor(3*8/4) = 6
    assert list(T1) == [V[4], V[7]]            # floor(8/2) = 4, min(7, 8) = 7


# ------------------------------------------------------------------ assign

def _bruteforce_group(w, I, s, T):
    """Minimum and minimizers of sum I (w - s T[q])^2 over all code vectors."""
    best, arg = None, []
    for qv in itertools.product(range(len(T)), repeat=len(w)):
        e = sum(I[k] * (w[k] - s * T[qv[k]]) ** 2 for k in range(len(w)))
        if best is None or e < best - 1e-300:
            best, arg = e, [qv]
        elif e == best:
            arg.append(qv)
    return best, arg


@pytest.mark.parametrize("g,S,n", [(2, 2, 16), (4, 4, 3), (4, 2, 4), (4, 4, 2)])
def test_assign_matches_exhaustive_search(g, S, n):
    rng = np.random.default_rng(10 * g + n)
    W = _bf16_matrix(rng, 3, 2 * g, outliers=0.2)
    I = rng.random(2 * g) * 5
    I[1] = 0.0
    T0 = np.sort(rng.uniform(-1, 1, n))
    T1 = np.sort(rng.uniform(-1, 1, n))
    a = ref.assign(W, I, T0, T1, g, S)
    s = ref.group_scales(W, g)
    for r in range(W.shape[0]):
        for H in range(W.shape[1] // S):
            cols = range(H * S, H * S + S)
            sg = s[r, (H * S) // g]
            w = [W[r, k] for k in cols]
            Ik = [I[k] for k in cols]
            mins = []
            for c, T in enumerate((T0, T1)):
                best, arg = _bruteforce_group(w, Ik, sg, T)
                assert a["E%d" % c][r, H] == pytest.approx(best, rel=1e-12, abs=1e-300)
                mins.append(best)
                qv = tuple(a["q%d" % c][r, k] for k in cols)
                # the per-weight nearest entries always achieve the minimum
                e_q = sum(Ik[i] * (w[i] - sg * T[qv[i]]) ** 2 for i in range(S))
                assert e_q == pytest.approx(best, rel=1e-12, abs=1e-300)
            assert a["sel"][r, H] == (1 if mins[1] < mins[0] * (1 - 1e-12) else a["sel"][r, H])
            assert a["sel"][r, H] == (1 if a["E1"][r, H] < a["E0"][r, H] else 0)


def test_assign_nearest_is_bruteforce_argmin_with_lowest_index_ties():
    T = np.array([-0.5, 0.0, 0.0, 0.5, 0.25])
    u = np.array([0.0, 0.125, 0.25, 0.375, -0.25, -1.0, 1.0, 0.3])
    got = ref.nearest(u, T)
    for x, q in zip(u, got):
        d = [abs(x - t) for t in T]
        assert q == d.index(min(d))
    assert list(got[:5]) == [1, 1, 4, 3, 0]


def test_assign_single_table_is_round_to_nearest():
    """T0 = T1 = {j/8}: nearest index = clamp(ceil(8u - 1/2), -8, 7) + 8 exactly (half-way
    points go down, the lower index), and every group keeps T0 (equal errors)."""
    rng = np.random.default_rng(7)
    W = _bf16_matrix(rng, 16, 256, outliers=0.05)
    # make exact half-way points appear: weights at (k + 1/2)/8 of the group scale
    W[0, 0] = 1.0
    W[0, 1:16] = (np.arange(-8, 7) + 0.5) / 8.0
    T = np.arange(-8, 8) / 8.0
    a = ref.assign(W, np.ones(256), T, T, 128, 128)
    u = ref.normalized(W, 128)
    want = np.clip(np.ceil(8 * u - 0.5), -8, 7).astype(np.int64) + 8
    assert np.array_equal(a["q0"], want)
    assert np.array_equal(a["codes"], want)
    assert not a["sel"].any()


# ------------------------------------------------------------------ refine

def test_refine_is_weighted_centroid_grid_search():
    rng = np.random.default_rng(8)
    W = _bf16_matrix(rng, 4, 32, outliers=0.1)
    I = rng.random(32) + 0.1
    T0 = np.linspace(-0.9, 0.9, 4)
    T1 = T0 + 0.1
    a = ref.assign(W, I, T0, T1, 8, 8)
    N0, N1 = ref.refine(W, I, a["codes"], a["sel"], T0, T1, 8, 8)
    s = np.repeat(ref.group_scales(W, 8), 8, axis=1)
    sel_w = np.repeat(a["sel"], 8, axis=1)
    for c, (Told, Tnew) in enumerate(((T0, N0), (T1, N1))):
        for j in range(4):
            m = (sel_w == c) & (a["codes"] == j)
            if not m.any():
                assert Tnew[j] == Told[j]
                continue
            f = lambda t: np.sum(I[None, :].repeat(4, 0)[m] * (W[m] - s[m] * t) ** 2)  # noqa: E731
            grid = np.linspace(Tnew[j] - 1e-3, Tnew[j] + 1e-3, 2001)
            vals = np.array([f(t) for t in grid])
            assert abs(grid[np.argmin(vals)] - Tnew[j]) <= 1.5e-6
            # stationarity: sum I s (w - s t) = 0 at the update
            resid = np.sum(I[None, :].repeat(4, 0)[m] * s[m] * (W[m] - s[m] * Tnew[j]))
            scale = np.sum(I[None, :].repeat(4, 0)[m] * np.abs(s[m] * W[m]))
            assert abs(resid) <= 1e-12 * scale


def _lloyd_setup(seed, n, R=64, C=128, g=32):
    """Matrix whose every scale group has the same absmax, so I s^2 = I * const."""
    rng = np.random.default_rng(seed)
    W = _bf16_matrix(rng, R, C, scale=0.02, outliers=0.0)
    top = 0.125
    W = np.clip(W, -top * 0.99, top * 0.99)
    W = ref.bf16_round(W)
    W[:, ::g] = top                          # force absmax = top in every group
    return rng, W


@pytest.mark.parametrize("weighted", [False, True])
def test_refine_loop_equals_sklearn_lloyd(weighted):
    from sklearn.cluster import KMeans

    n, g, iters = 8, 32, 5
    rng, W = _lloyd_setup(11, n)
    C = W.shape[1]
    I = rng.random(C) * 3 + 0.5 if weighted else np.ones(C)
    T0, T1 = ref.init_tables(W, g, n)
    T0 = np.unique(T0)
    assert T0.size == n
    u = ref.normalized(W, g)
    Ts = T0.copy()
    for _ in range(iters):
        a = ref.assign(W, I, Ts, Ts, g, g)
        assert not a["sel"].any()            # identical tables: every group keeps T0
        num, den = ref.refine_sums(W, I, a["codes"], a["sel"], g, g, n)
        assert np.all(den[0] > 0)            # sklearn relocates empty clusters; keep none empty
        Ts, _ = ref.refine_update(num, den, Ts, Ts)
    km = KMeans(n_clusters=n, init=T0.reshape(-1, 1), n_init=1, max_iter=iters, tol=0.0,
                algorithm="lloyd")
    km.fit(u.reshape(-1, 1), sample_weight=np.tile(I, W.shape[0]))
    want = np.sort(km.cluster_centers_.ravel())
    assert np.allclose(Ts, want, rtol=0, atol=1e-12)


# ------------------------------------------------------------------ the loop

@pytest.mark.parametrize("g,S,n", [(16, 16, 15), (32, 8, 16), (64, 64, 4)])
def test_total_error_never_increases(g, S, n):
    rng = np.random.default_rng(g + S + n)
    W = _bf16_matrix(rng, 48, 128)
    I = rng.standard_t(4, size=(64, 128)).astype(np.float32)
    I = ref.importance(I * np.exp(rng.standard_normal(128)))
    out = ref.quantize(W, I, g, S, n, iters=6)
    h = out["history"]
    assert np.all(np.diff(h) <= 1e-12 * h[:-1])
    fin = out["final"]
    # the stored codes are nearest entries of the stored (bf16) tables
    u = ref.normalized(W, g)
    for c in range(2):
        assert np.array_equal(fin["q%d" % c], ref.nearest(u, out["tables_bf16"][c]))


# ------------------------------------------------------------------ storage format

def test_pack_roundtrip_and_page_storage_figures():
    with open(os.path.join(GOLDEN, "storage_overhead.json")) as fh:
        gold = json.load(fh)
    rng = np.random.default_rng(12)
    for g, S, n in ((128, 128, 16), (128, 16, 16), (16, 16, 15)):
        W = _bf16_matrix(rng, 6, 256)
        I = rng.random(256)
        out = ref.quantize(W, I, g, S, n, iters=2)
        fin = out["final"]
        p = ref.pack(W, fin["codes"], fin["sel"], out["tables_bf16"], g, S)
        R, C = W.shape
        assert np.array_equal(ref.unpack_codes(p["codes"], R, C), fin["codes"])
        assert np.array_equal(ref.unpack_selectors(p["scales"], p["bitmap"], R, C, g, S),
                              fin["sel"])
        tb = p["tables"].size * 2
        assert tb == ref.storage_bytes(n)
        assert abs(tb - gold["table_bytes_per_layer"]["value"]) <= \
            gold["table_bytes_per_layer"]["tolerance_bytes"]
        sel_bits = 0 if p["bitmap"] is None else p["bitmap"].size * 8
        want_bpw = gold["selector_bpw"]["S_eq_g"] if S == g else gold["selector_bpw"]["S_16"]
        assert sel_bits / W.size == pytest.approx(want_bpw)
        assert ref.selector_bits_per_weight(g, S) == pytest.approx(want_bpw)
        if S == g:
            # the scale stays positive apart from the selector in its sign bit
            assert np.array_equal(p["scales"] & 0x7FFF, ref.bf16_bits(ref.group_scales(W, g)))
    model = gold["table_bytes_7b_model"]
    assert ref.storage_bytes(16, model["linears"]) / 1024 == pytest.approx(model["value_kib"],
                                                                           abs=0.5)
    assert gold["entries"]["NVFP4"] == 15 and gold["entries"]["INT4"] == 16


def test_pack_bitmap_layout_lsb_first():
    W = np.ones((1, 64))
    sel = np.zeros((1, 4), dtype=np.uint8)
    sel[0, 1] = 1
    sel[0, 3] = 1
    p = ref.pack(W, np.zeros((1, 64), dtype=np.int64), sel,
                 (np.zeros(16), np.zeros(16)), 64, 16)
    assert p["bitmap"].tolist() == [0b1010]
    assert p["scales"].tolist() == [[0x3F80]]
    p = ref.pack(W, np.arange(64).reshape(1, 64) % 16, np.ones((1, 1), np.uint8),
                 (np.zeros(16), np.zeros(16)), 64, 64)
    assert p["scales"].tolist() == [[0xBF80]]
    assert p["codes"][0, :2].tolist() == [0x10, 0x32]


def test_dequant_matches_torch_product_rounding():
    rng = np.random.default_rng(13)
    R, C, g, S, n = 8, 256, 16, 16, 15
    W = _bf16_matrix(rng, R, C)
    I = rng.random(C)
    out = ref.quantize(W, I, g, S, n, iters=2)
    fin = out["final"]
    p = ref.pack(W, fin["codes"], fin["sel"], out["tables_bf16"], g, S)
    got = ref.dequant(p["codes"], p["scales"], p["bitmap"], p["tables"], R, C, g, S)
    s = torch.from_numpy(np.repeat(ref.group_scales(W, g), g, axis=1).astype(np.float32))
    Ts = torch.from_numpy(np.stack(out["tables_bf16"]).astype(np.float32))
    sig = torch.from_numpy(np.repeat(fin["sel"], S, axis=1).astype(np.int64))
    q = torch.from_numpy(fin["codes"])
    want = (s * Ts[sig, q]).to(torch.bfloat16).float().numpy().astype(np.float64)
    assert np.array_equal(got, want)


# ------------------------------------------------------------------ planted mistakes

def test_pins_catch_planted_mistakes(monkeypatch):
    """Copies of oracle steps with one slip each; the pins above must reject every one."""
    rng = np.random.default_rng(14)
    W = _bf16_matrix(rng, 16, 256, outliers=0.05)
    W[0, 0] = 1.0
    W[0, 1:16] = (np.arange(-8, 7) + 0.5) / 8.0
    T = np.arange(-8, 8) / 8.0
    u = ref.normalized(W, 128)
    want = np.clip(np.ceil(8 * u - 0.5), -8, 7).astype(np.int64) + 8

    # 1. ties to the highest index
    def nearest_last(u, T):
        d = (np.asarray(u)[..., None] - np.asarray(T)) ** 2
        return T.size - 1 - np.argmin(d[..., ::-1], axis=-1)
    assert not np.array_equal(nearest_last(u, T), want)

    # 2. refine weighting by I alone (dropping s^2): the centroid moves off the grid-search optimum
    T0 = np.linspace(-0.9, 0.9, 4)
    I = rng.random(256) + 0.1
    a = ref.assign(W, I, T0, T0 + 0.1, 128, 128)
    sel_w = np.repeat(a["sel"], 128, axis=1)
    counts = {(c, j): int(np.sum((sel_w == c) & (a["codes"] == j)))
              for c in range(2) for j in range(4)}
    c, j = max(counts, key=counts.get)
    m = (sel_w == c) & (a["codes"] == j)
    s = np.repeat(ref.group_scales(W, 128), 128, axis=1)
    Iw = np.broadcast_to(I, W.shape)
    wrong = np.sum(Iw[m] * u[m]) / np.sum(Iw[m])
    right = ref.refine(W, I, a["codes"], a["sel"], T0, T0 + 0.1, 128, 128)[c][j]
    f = lambda t: np.sum(Iw[m] * (W[m] - s[m] * t) ** 2)  # noqa: E731
    assert f(right) < f(wrong)

    # 3. T1 not shifted (both tables at the same quantiles) fails the interleave pin
    T0i, T1i = ref.init_tables(W, 128, 16)
    assert not np.array_equal(T0i, T1i)
    assert np.any(T0i < T1i)

    # 4. selection on the wrong comparison (E1 <= E0) flips all exact ties to T1
    a = ref.assign(W, np.ones(256), T, T, 128, 128)
    assert np.all(a["E0"] == a["E1"]) and not a["sel"].any()
