"""Pins for the parts of the oracle that a single-layer check cannot see: the
layer chaining of the decode stack, the temporal tier across tokens, a
per-element RMSNorm weight, and the rounding points of the prefill. Each is
compared with the independent pure-Python brute force (``oracle/brute.py``) at
1e-12, on weights whose per-layer MoE contribution is far from zero, and each
test also shows that dropping the pinned step moves the result by much more
than that tolerance (so a mistake there would fail the comparison). CPU only.

Definitions: "Flash-MoE - Chạy mô hình 397 tỷ tham số trên laptop"
(vi.news.hada.io), sections "Kiến trúc mô hình" (60 layers, K of 512 experts)
and "Deferred GPU Expert Compute" (combine + norm + residual feed the next
layer); "Autoresearch impulsa a Qwen3.5-397B ..." (openclawradar.com), section
"Optimizaciones Efectivas" (27% of a token's experts repeat the previous
token's, read as a selection tier); the prefill rounding points follow the
expert-grouped bf16 contraction of the batched-prefill workload.
"""
import numpy as np

import workload as wl
from oracle import brute
from oracle import ref

TOL = 1e-12


def zero_mean_canon(rng, H, I, bits=4, s_sigma=0.1, b_sigma=0.02):
    """Canonical expert whose dequantised weights have zero mean: bias is minus
    the code midpoint times the scale, plus a little noise. Gate pre-activations
    then stay O(1) and every layer adds a visible contribution."""
    cs, ss, bs = [], [], []
    mid = ((1 << bits) - 1) / 2.0
    for m in range(3):
        r, c = (I, H) if m < 2 else (H, I)
        cs.append(rng.integers(0, 1 << bits, size=(r, c), dtype=np.uint8))
        s = wl.bf16_bits_from_f32(np.abs(rng.normal(0, s_sigma, (r, c // 64))).astype(np.float32))
        sf = wl.bf16_bits_to_f32(s).astype(np.float64)
        b = wl.bf16_bits_from_f32((-mid * sf + rng.normal(0, b_sigma, sf.shape)).astype(np.float32))
        ss.append(s)
        bs.append(b)
    return cs, ss, bs


def tolist(c):
    return ([m.tolist() for m in c[0]], [m.tolist() for m in c[1]], [m.tolist() for m in c[2]])


def _stack_setup(seed, H=64, I=64, E=8, K=2, L=3, T=4):
    rng = np.random.default_rng(seed)
    experts = {(l, e): zero_mean_canon(rng, H, I) for l in range(L) for e in range(E)}
    shared = {l: [zero_mean_canon(rng, H, I)] for l in range(L)}
    routers = [rng.normal(0, 0.3, (E, H)).astype(np.float32) for _ in range(L)]
    gammas = [(1.0 + 0.3 * rng.normal(size=H)).astype(np.float32) for _ in range(L)]
    xs = rng.normal(size=(T, H))
    boost = (rng.random((T, L, K)) < 0.5).astype(np.uint8)
    boost[0] = 0
    return H, I, E, K, L, T, experts, shared, routers, gammas, xs, boost


def _brute_layers(L, E, experts, shared, routers, gammas):
    return [{"router": [list(map(float, r)) for r in routers[l]],
             "experts": [tolist(experts[(l, e)]) for e in range(E)],
             "shared": [tolist(s) for s in shared[l]],
             "gamma": [float(g) for g in gammas[l]]} for l in range(L)]


def test_stack_chaining_tier_and_gamma_match_brute_force():
    H, I, E, K, L, T, experts, shared, routers, gammas, xs, boost = _stack_setup(40)
    ys, sets, _ = ref.stack_decode(xs, L, lambda l: routers[l], lambda l, e: experts[(l, e)],
                                   lambda l: shared[l], K, boost=boost, gamma_of=lambda l: gammas[l])
    by, bsets = brute.stack([list(x) for x in xs], _brute_layers(L, E, experts, shared, routers, gammas), K,
                            boost=boost.tolist())
    for t in range(T):
        assert [list(map(int, s)) for s in sets[t]] == bsets[t], f"token {t}: selected sets differ"
        scale = max(abs(v) for v in by[t])
        np.testing.assert_allclose(ys[t], by[t], rtol=0, atol=TOL * scale)
    # the tier was exercised: some boosted expert would not have been selected on score alone
    assert boost[1:].sum() > 0


def test_stack_pin_sees_every_layer():
    """Every layer's MoE contribution is far above the comparison tolerance, so a
    stack that dropped the chaining (each layer fed the token's input) or a layer
    would fail the brute-force comparison above."""
    H, I, E, K, L, T, experts, shared, routers, gammas, xs, boost = _stack_setup(40)
    for t in range(T):
        x = xs[t]
        for l in range(L):
            r = ref.layer_decode(x, routers[l], lambda e, l=l: experts[(l, e)], shared[l], K, gamma=gammas[l])
            delta = np.abs(r.y - x).max()
            assert delta > 1e6 * TOL * np.abs(r.y).max(), f"token {t} layer {l}: MoE delta too small"
            x = r.y
    # without chaining, the last layer sees the token input: a different output
    unchained = ref.layer_decode(xs[1], routers[L - 1], lambda e: experts[(L - 1, e)], shared[L - 1], K,
                                 gamma=gammas[L - 1]).y
    ys, _, _ = ref.stack_decode(xs, L, lambda l: routers[l], lambda l, e: experts[(l, e)],
                                lambda l: shared[l], K, boost=boost, gamma_of=lambda l: gammas[l])
    assert np.abs(unchained - ys[1]).max() > 1e6 * TOL * np.abs(ys[1]).max()


def test_stack_tier_changes_the_selection():
    """The boost mask changes some token's set (so a dropped tier fails the pin)."""
    H, I, E, K, L, T, experts, shared, routers, gammas, xs, boost = _stack_setup(40)
    args = (xs, L, lambda l: routers[l], lambda l, e: experts[(l, e)], lambda l: shared[l], K)
    _, with_tier, _ = ref.stack_decode(*args, boost=boost, gamma_of=lambda l: gammas[l])
    _, without, _ = ref.stack_decode(*args, boost=None, gamma_of=lambda l: gammas[l])
    assert not np.array_equal(with_tier, without)


def test_layer_with_random_gamma_matches_brute_force():
    rng = np.random.default_rng(41)
    H, I, E, K = 128, 64, 8, 2
    experts = [zero_mean_canon(rng, H, I) for _ in range(E)]
    shared = [zero_mean_canon(rng, H, I)]
    W = rng.normal(0, 0.3, (E, H)).astype(np.float32)
    gamma = (1.0 + 0.5 * rng.normal(size=H)).astype(np.float32)
    x = rng.normal(size=H)
    r = ref.layer_decode(x, W, lambda e: experts[e], shared, K, gamma=gamma)
    yb, ib, wb = brute.layer(list(x), [list(map(float, row)) for row in W], [tolist(e) for e in experts],
                             [tolist(s) for s in shared], K, gamma=[float(g) for g in gamma])
    assert list(r.idx) == ib
    np.testing.assert_allclose(r.w, wb, rtol=1e-13)
    scale = max(abs(v) for v in yb)
    np.testing.assert_allclose(r.y, yb, rtol=0, atol=TOL * scale)
    # gamma matters: with unit gamma the output moves far beyond the tolerance
    y1, _, _ = brute.layer(list(x), [list(map(float, row)) for row in W], [tolist(e) for e in experts],
                           [tolist(s) for s in shared], K)
    assert max(abs(a - b) for a, b in zip(y1, yb)) > 1e6 * TOL * scale


def _prefill_setup(seed, H=128, I=64, E=8, K=2):
    rng = np.random.default_rng(seed)
    experts = [zero_mean_canon(rng, H, I) for _ in range(E)]
    shared = [zero_mean_canon(rng, H, I)]
    W = rng.normal(0, 0.3, (E, H)).astype(np.float32)
    gamma = (1.0 + 0.3 * rng.normal(size=H)).astype(np.float32)
    x = rng.normal(size=H).astype(np.float32)    # float32, generally off the bf16 grid
    sel = rng.normal(size=E)
    return experts, shared, W, gamma, x, sel, K


def _brute_prefill(experts, shared, W, gamma, x, sel, K, points=True, by_sel=True):
    return brute.layer([float(v) for v in x], [list(map(float, row)) for row in W], [tolist(e) for e in experts],
                       [tolist(s) for s in shared], K, gamma=[float(g) for g in gamma], sel=list(sel),
                       by_sel=by_sel, bf16_points=points)


def test_prefill_rounding_points_match_brute_force():
    experts, shared, W, gamma, x, sel, K = _prefill_setup(42)
    off_grid = wl.bf16_bits_to_f32(wl.bf16_bits_from_f32(x)) != x
    assert off_grid.mean() > 0.9                 # the input rounding x_b is not a no-op here
    for by_sel in (True, False):
        p = ref.prefill_token(x, W, lambda e: experts[e], shared, K, sel, gamma=gamma, by_sel=by_sel)
        yb, ib, wb = _brute_prefill(experts, shared, W, gamma, x, sel, K, by_sel=by_sel)
        assert list(p.idx) == ib
        np.testing.assert_allclose(p.w, wb, rtol=1e-13)
        scale = max(abs(v) for v in yb)
        np.testing.assert_allclose(p.y, yb, rtol=0, atol=TOL * scale)


def test_prefill_each_rounding_point_is_visible():
    """Dropping any one of the four rounding points (x_b, the expert input, the
    weights, h_b) moves the output by far more than the comparison tolerance."""
    experts, shared, W, gamma, x, sel, K = _prefill_setup(42)
    full, _, _ = _brute_prefill(experts, shared, W, gamma, x, sel, K)
    scale = max(abs(v) for v in full)
    for drop in ("x", "a", "w", "h"):
        pts = {"x", "a", "w", "h"} - {drop}
        other, _, _ = _brute_prefill(experts, shared, W, gamma, x, sel, K, points=pts)
        assert max(abs(a - b) for a, b in zip(other, full)) > 1e6 * TOL * scale, f"rounding point {drop}"


def test_brute_bf16_rounding_matches_the_bit_definition():
    """The brute force's own bf16 rounding (on the float64 bit pattern) agrees with
    the float32 -> bf16 round-to-nearest-even of the workload generator on float32
    values, ties included."""
    rng = np.random.default_rng(43)
    f = np.concatenate([rng.normal(0, 1, 3000), rng.normal(0, 1e-3, 500),
                        [1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -8 * 255.5]]).astype(np.float32)
    want = wl.bf16_bits_to_f32(wl.bf16_bits_from_f32(f)).astype(np.float64)
    got = np.array([brute.bf16_round(float(v)) for v in f])
    assert np.array_equal(got, want)
