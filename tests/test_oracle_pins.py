"""Pins for the CPU oracle: closed forms, invariants, library routines and an
independent brute force, chosen so that a dropped term, a wrong sign or index,
or a transposed operand in the oracle fails at least one test. CPU only."""
import json
import math
import os

import numpy as np
import pytest

import workload as wl
from oracle import brute
from oracle import ref

GOLD = os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")
BF16_ONE = 0x3F80


def rand_canon(rng, H, I, bits=4, s_sigma=0.02, b_sigma=0.01):
    cs, ss, bs = [], [], []
    for m in range(3):
        r, c = (I, H) if m < 2 else (H, I)
        cs.append(rng.integers(0, 1 << bits, size=(r, c), dtype=np.uint8))
        ss.append(wl.bf16_bits_from_f32(np.abs(rng.normal(0, s_sigma, (r, c // 64))).astype(np.float32)))
        bs.append(wl.bf16_bits_from_f32(rng.normal(0, b_sigma, (r, c // 64)).astype(np.float32)))
    return cs, ss, bs


def deq_np(q, s, b):
    """float32 dequantisation with numpy's IEEE single ops (no fusion)."""
    sf = np.repeat(wl.bf16_bits_to_f32(s), 64, axis=1)
    bf = np.repeat(wl.bf16_bits_to_f32(b), 64, axis=1)
    return (q.astype(np.float32) * sf + bf).astype(np.float32)


# ---------------------------------------------------------------- page constants

def test_expert_bytes_closed_form_matches_page():
    g = json.load(open(GOLD))
    H = g["hidden"]["value"]
    I = 1024
    per_expert = 3 * H * I * 4 // 8 + 3 * H * I // 64 * 4  # codes + bf16 (scale, bias) per group
    assert per_expert == 7_077_888
    assert per_expert / 2 ** 20 == g["expert_mib_4bit"]["value"]
    assert 3 * H * I * 2 // 8 + 3 * H * I // 64 * 4 == 3_932_160  # 2-bit
    q3 = 3 * H * I * 3 // 8 + 3 * H * I // 64 * 4  # 3-bit
    assert q3 == 5_505_024
    # a 3-bit group-affine expert is about as much smaller than a 4-bit one as the
    # page's 3-bit experts are (within one percentage point)
    assert abs((1 - q3 / per_expert) - g["q3_size_reduction"]["value"]) < 0.01


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_generator_codes_are_bit_slices_of_the_word_stream(bits):
    # element k is bits [b*(k % per), +b) of word k // per, per = 64 // b
    key = wl.stream_key(3, wl.KIND_CODES, 1, 2, 0)
    n = 3 * (64 // bits) + 5
    got = wl.codes(key, n, bits)
    words = [int(v) for v in wl.words(key, 0, n)]
    per = 64 // bits
    want = [(words[k // per] >> (bits * (k % per))) % (1 << bits) for k in range(n)]
    assert got.tolist() == want
    assert got.max() < (1 << bits)


def test_fma_rewrite_identity_exact():
    # The page's rewrite (q*s+b)*x == fma(q, s*x, b*x) holds exactly in real
    # arithmetic; with dyadic values it holds exactly in float64 too.
    rng = np.random.default_rng(1)
    for _ in range(1000):
        q = int(rng.integers(0, 16))
        s, b, x = (float(rng.integers(-512, 512)) / 256 for _ in range(3))
        assert (q * s + b) * x == q * (s * x) + b * x


# ---------------------------------------------------------------- mat-vec pins

def test_matvec_integer_core_exact():
    rng = np.random.default_rng(2)
    R, C = 96, 4096
    q = rng.integers(0, 16, size=(R, C), dtype=np.uint8)
    s = np.full((R, C // 64), BF16_ONE, np.uint16)
    b = np.zeros((R, C // 64), np.uint16)
    x = rng.integers(-8, 9, size=C).astype(np.float64)
    y = ref.matvec(q, s, b, x)
    exact = q.astype(np.int64) @ x.astype(np.int64)
    assert np.array_equal(y, exact.astype(np.float64))


def test_matvec_bias_only_closed_form():
    rng = np.random.default_rng(3)
    R, C = 40, 1024
    q = rng.integers(0, 16, size=(R, C), dtype=np.uint8)
    s = np.zeros((R, C // 64), np.uint16)
    b = wl.bf16_bits_from_f32(rng.normal(0, 1, (R, C // 64)).astype(np.float32))
    x = rng.integers(-4, 5, size=C).astype(np.float64)
    y = ref.matvec(q, s, b, x)
    X = x.reshape(C // 64, 64).sum(axis=1)            # per-group sums of x
    expect = wl.bf16_bits_to_f32(b).astype(np.float64) @ X
    np.testing.assert_allclose(y, expect, rtol=0, atol=1e-12)


def test_matvec_one_hot_reads_one_column():
    rng = np.random.default_rng(4)
    R, C = 16, 256
    q = rng.integers(0, 16, size=(R, C), dtype=np.uint8)
    s = np.full((R, C // 64), BF16_ONE, np.uint16)
    b = np.zeros((R, C // 64), np.uint16)
    for k in (0, 1, 63, 64, 130, 255):
        x = np.zeros(C)
        x[k] = 1.0
        assert np.array_equal(ref.matvec(q, s, b, x), q[:, k].astype(np.float64))
    # bias-only one-hot: column k reads the bias of group k // 64
    s0 = np.zeros_like(s)
    bb = wl.bf16_bits_from_f32(rng.normal(0, 1, (R, C // 64)).astype(np.float32))
    for k in (0, 65, 200):
        x = np.zeros(C)
        x[k] = 1.0
        assert np.array_equal(ref.matvec(q, s0, bb, x), wl.bf16_bits_to_f32(bb[:, k // 64]).astype(np.float64))


def test_matvec_matches_numpy_dense():
    rng = np.random.default_rng(5)
    q, s, b = (a[0] for a in rand_canon(rng, 512, 64))
    x = rng.normal(size=512)
    np.testing.assert_allclose(ref.matvec(q, s, b, x), deq_np(q, s, b).astype(np.float64) @ x,
                               rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- norm / bf16

def test_rmsnorm_closed_form():
    for c in (3.0, -0.5, 1e-3):
        xn = ref.rmsnorm(np.full(4096, c))
        np.testing.assert_allclose(xn, c / math.sqrt(c * c + 1e-6), rtol=1e-12)  # 4096-term fp64 sum


def test_round_bf16_matches_bit_rounding():
    rng = np.random.default_rng(6)
    f = np.concatenate([rng.normal(0, 1, 5000), rng.normal(0, 1e-3, 1000)]).astype(np.float32)
    # ties: 1 + 2^-8 -> 1 (even), 1 + 3*2^-8 -> 1 + 2^-6
    f = np.concatenate([f, np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)], np.float32)])
    want = wl.bf16_bits_to_f32(wl.bf16_bits_from_f32(f)).astype(np.float64)
    got = ref.round_bf16(f.astype(np.float64))
    assert np.array_equal(got, want)
    assert got[-3] == 1.0 and got[-2] == 1 + 2 ** -6


# ---------------------------------------------------------------- routing

def test_select_equals_full_sort_and_weights_sum_to_one():
    rng = np.random.default_rng(7)
    for trial in range(50):
        E, K = 512, 4
        logits = rng.normal(0, 1.28, E)
        idx, w, gap = ref.select(logits, K)
        order = np.argsort(-logits, kind="stable")
        assert list(idx) == list(order[:K])
        assert abs(w.sum() - 1.0) < 1e-12
        assert np.all(np.diff(w) <= 0)                  # weights follow logit order
        assert gap == pytest.approx(logits[order[K - 1]] - logits[order[K]])
        p = np.exp(logits - logits.max())
        np.testing.assert_allclose(w, p[idx] / p[idx].sum(), rtol=1e-13)


def test_select_ties_prefer_lower_index_and_tier_first():
    logits = np.zeros(8)
    idx, w, gap = ref.select(logits, 3)
    assert list(idx) == [0, 1, 2] and gap == 0.0
    np.testing.assert_allclose(w, [1 / 3] * 3)
    logits = np.arange(8, dtype=np.float64)
    idx, _, _ = ref.select(logits, 3, boosted=(0, 2))
    assert list(idx) == [2, 0, 7]                      # tier 1 (by score), then best of the rest


def test_select_k1_bias_gives_unit_weight_and_by_sel_ignores_logits():
    logits = np.random.default_rng(8).normal(size=64)
    sel = np.zeros(64)
    sel[17] = 100.0
    idx, w, _ = ref.select(logits, 1, sel=sel)
    assert list(idx) == [17] and w[0] == 1.0
    idx, w, _ = ref.select(logits, 2, sel=-np.arange(64.0), by_sel=True)
    assert list(idx) == [0, 1]


# ---------------------------------------------------------------- expert / layer

def test_one_hot_routing_equals_dense_expert():
    rng = np.random.default_rng(9)
    H, I, E = 256, 128, 8
    experts = [rand_canon(rng, H, I) for _ in range(E)]
    W = rng.normal(0, 0.02, (E, H)).astype(np.float32)
    x = rng.normal(size=H)
    W[5] = np.sign(x).astype(np.float32)               # logit_5 = sum|x_n|: expert 5 is the top-1
    r = ref.layer_decode(x, W, lambda e: experts[e], [], K=1)
    assert list(r.idx) == [5] and r.w[0] == 1.0
    G, U, D = (deq_np(experts[5][0][m], experts[5][1][m], experts[5][2][m]).astype(np.float64) for m in range(3))
    xn = x / np.sqrt(np.mean(x * x) + 1e-6)
    g, u = G @ xn, U @ xn
    expect = x + D @ (g / (1 + np.exp(-g)) * u)
    np.testing.assert_allclose(r.y, expect, rtol=1e-11, atol=1e-9)


@pytest.mark.parametrize("rms,res", [(True, True), (False, False)])
def test_layer_matches_pure_python_brute_force(rms, res):
    rng = np.random.default_rng(10)
    H, I, E, K = 64, 64, 8, 2
    experts = [rand_canon(rng, H, I, s_sigma=0.1, b_sigma=0.05) for _ in range(E)]
    shared = [rand_canon(rng, H, I, s_sigma=0.1, b_sigma=0.05)]
    W = rng.normal(0, 0.3, (E, H)).astype(np.float32)
    x = rng.normal(size=H)

    def tolist(c):
        return ([m.tolist() for m in c[0]], [m.tolist() for m in c[1]], [m.tolist() for m in c[2]])

    yb, ib, wb = brute.layer(list(x), [list(map(float, r)) for r in W], [tolist(e) for e in experts],
                             [tolist(s) for s in shared], K, rmsnorm=rms, residual=res)
    r = ref.layer_decode(x, W, lambda e: experts[e], shared, K, rmsnorm_on=rms, residual=res)
    assert list(r.idx) == ib
    np.testing.assert_allclose(r.w, wb, rtol=1e-13)
    scale = max(abs(v) for v in yb)
    np.testing.assert_allclose(r.y, yb, rtol=0, atol=1e-12 * scale)


def test_layer_with_shared_gate_matches_pure_python_brute_force():
    rng = np.random.default_rng(15)
    H, I, E, K = 64, 64, 8, 2
    experts = [rand_canon(rng, H, I, s_sigma=0.1, b_sigma=0.05) for _ in range(E)]
    shared = [rand_canon(rng, H, I, s_sigma=0.1, b_sigma=0.05)]
    W = rng.normal(0, 0.3, (E, H)).astype(np.float32)
    G = rng.normal(0, 0.3, (1, H)).astype(np.float32)
    x = rng.normal(size=H)

    def tolist(c):
        return ([m.tolist() for m in c[0]], [m.tolist() for m in c[1]], [m.tolist() for m in c[2]])

    yb, ib, wb = brute.layer(list(x), [list(map(float, r)) for r in W], [tolist(e) for e in experts],
                             [tolist(s) for s in shared], K, shared_gate=[list(map(float, r)) for r in G])
    r = ref.layer_decode(x, W, lambda e: experts[e], shared, K, shared_gate=G)
    assert list(r.idx) == ib
    scale = max(abs(v) for v in yb)
    np.testing.assert_allclose(r.y, yb, rtol=0, atol=1e-12 * scale)


def _gate_layers(seed):
    rng = np.random.default_rng(seed)
    H, I, E, K = 128, 64, 8, 2
    experts = [rand_canon(rng, H, I) for _ in range(E)]
    shared = [rand_canon(rng, H, I, s_sigma=0.05)]
    W = rng.normal(0, 0.02, (E, H)).astype(np.float32)
    x = rng.normal(size=H)
    full = ref.layer_decode(x, W, lambda e: experts[e], shared, K)
    # the same routed part without the shared expert: combine of the same selection
    o_r = np.stack([ref.expert(experts[int(e)], full.xn) for e in full.idx])
    none = ref.combine(x, full.w, o_r, np.zeros((0, H)))
    return x, W, experts, shared, K, full, none


def test_shared_gate_zero_vector_halves_the_shared_expert():
    x, W, experts, shared, K, full, none = _gate_layers(16)
    g = ref.layer_decode(x, W, lambda e: experts[e], shared, K, shared_gate=np.zeros((1, x.size), np.float32))
    # sigmoid(0) = 1/2 exactly: the gated output is the midpoint of "shared weight 1"
    # and "no shared expert" (the combine is linear in the shared weight)
    np.testing.assert_allclose(g.y, 0.5 * (full.y + none), rtol=0, atol=1e-13 * np.abs(full.y).max())
    assert list(g.idx) == list(full.idx)


@pytest.mark.parametrize("k,m", [(3, 2.0), (77, -1.5), (0, 40.0)])
def test_shared_gate_one_hot_row_closed_form(k, m):
    x, W, experts, shared, K, full, none = _gate_layers(17)
    G = np.zeros((1, x.size), np.float32)
    G[0, k] = m
    g = ref.layer_decode(x, W, lambda e: experts[e], shared, K, shared_gate=G)
    c = 1.0 / (1.0 + math.exp(-m * full.xn[k]))   # the textbook logistic of one product
    expect = none + c * (full.y - none)
    np.testing.assert_allclose(g.y, expect, rtol=0, atol=1e-12 * np.abs(full.y).max())


def test_shared_gate_saturates_to_no_shared_expert():
    x, W, experts, shared, K, full, none = _gate_layers(18)
    G = (-1000.0 * np.sign(full.xn)).astype(np.float32)[None, :]   # G . x_n = -1000 sum|x_n|
    g = ref.layer_decode(x, W, lambda e: experts[e], shared, K, shared_gate=G)
    np.testing.assert_array_equal(g.y, none)


def test_zero_experts_stack_is_identity():
    rng = np.random.default_rng(11)
    H, I, E, K, L = 128, 64, 16, 4, 5
    zero = ([np.full((I, H), 7, np.uint8), np.full((I, H), 3, np.uint8), np.full((H, I), 9, np.uint8)],
            [np.zeros((I, H // 64), np.uint16), np.zeros((I, H // 64), np.uint16), np.zeros((H, I // 64), np.uint16)],
            [np.zeros((I, H // 64), np.uint16), np.zeros((I, H // 64), np.uint16), np.zeros((H, I // 64), np.uint16)])
    Ws = [rng.normal(0, 0.02, (E, H)).astype(np.float32) for _ in range(L)]
    xs = rng.normal(size=(3, H))
    ys, sets, _ = ref.stack_decode(xs, L, lambda l: Ws[l], lambda l, e: zero, lambda l: [zero], K)
    assert np.array_equal(ys, xs)


def test_prefill_without_rounding_points_reduces_to_decode():
    rng = np.random.default_rng(12)
    H, I, E, K = 128, 64, 16, 2
    experts = [rand_canon(rng, H, I) for _ in range(E)]
    shared = [rand_canon(rng, H, I)]
    W = rng.normal(0, 0.02, (E, H)).astype(np.float32)
    # x already on the bf16 grid makes x_b = x; the prefill token must then equal
    # the decode layer's selection and weights, and the decode combine applied to
    # experts evaluated with the bf16 rounding points.
    x = wl.bf16_bits_to_f32(wl.bf16_bits_from_f32(rng.normal(size=H).astype(np.float32))).astype(np.float64)
    sel = rng.normal(size=E)
    d = ref.layer_decode(x, W, lambda e: experts[e], shared, K, sel=sel, by_sel=True)
    xn = ref.rmsnorm(x)
    a = ref.round_bf16(xn)
    o_r = np.stack([ref.expert(experts[e], a, bf16_points=True) for e in d.idx])
    o_s = np.stack([ref.expert(shared[0], a, bf16_points=True)])
    p = ref.prefill_token(x.astype(np.float32), W, lambda e: experts[e], shared, K, sel=sel)
    assert list(p.idx) == list(d.idx)
    np.testing.assert_allclose(p.w, d.w, rtol=1e-14)
    np.testing.assert_allclose(p.y, ref.combine(x, d.w, o_r, o_s), rtol=1e-14)
    # and the rounding points matter at the 1e-3 level (they are not no-ops)
    rel = np.linalg.norm(p.y - d.y) / np.linalg.norm(d.y)
    assert 1e-5 < rel < 3e-2


def test_prefill_bf16_weights_one_hot_readout():
    rng = np.random.default_rng(13)
    q, s, b = (a[0] for a in rand_canon(rng, 256, 32))
    W = deq_np(q, s, b)
    Wb = wl.bf16_bits_to_f32(wl.bf16_bits_from_f32(W)).astype(np.float64)
    for k in (0, 77, 255):
        x = np.zeros(256)
        x[k] = 1.0
        assert np.array_equal(ref.matvec(q, s, b, x, round_w_bf16=True), Wb[:, k])


# ---------------------------------------------------------------- workload statistics

def test_temporal_mask_rate():
    m = wl.boost_mask(0, 256, 60, 4)
    frac = m[1:].mean()
    assert abs(frac - 0.27) < 0.005            # 61,200 Bernoulli(0.27) slots: sigma ~ 0.0018
    assert m[0].sum() == 0


def test_oracle_stack_realises_boosted_repeats():
    rng = np.random.default_rng(14)
    H, I, E, K, L, T = 64, 64, 32, 4, 3, 40
    experts = {(l, e): rand_canon(rng, H, I) for l in range(L) for e in range(E)}
    Ws = [rng.normal(0, 0.02, (E, H)).astype(np.float32) for _ in range(L)]
    xs = rng.normal(size=(T, H))
    boost = wl.boost_mask(3, T, L, K)
    ys, sets, _ = ref.stack_decode(xs, L, lambda l: Ws[l], lambda l, e: experts[(l, e)], lambda l: [], K,
                                   boost=boost)
    for t in range(1, T):
        for l in range(L):
            for j in range(K):
                if boost[t, l, j]:
                    assert sets[t - 1, l, j] in set(sets[t, l])


def test_zipf_gumbel_first_pick_follows_power_law():
    T, E = 20000, 512
    s, rank = wl.zipf_gumbel_scores(5, T, E, 1.1)
    first = rank[np.argmax(s, axis=1)]
    p = np.arange(1, E + 1, dtype=np.float64) ** -1.1
    p /= p.sum()
    top = 20
    obs = np.array([(first == r).sum() for r in range(1, top + 1)], dtype=np.float64)
    exp = p[:top] * T
    chi2 = ((obs - exp) ** 2 / exp).sum()
    assert chi2 < 45.3                           # chi-square, 20 dof, p = 0.001


# ---------------------------------------------------------------- expert cache (host-memory tier)

def test_expert_cache_hand_worked_trace():
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "expert_cache_trace.json")))
    hits = ref.expert_cache_hits(g["sets"], g["cache_slots"])
    assert [sorted(h) for h in hits] == g["hits"]


def test_expert_cache_of_k_slots_hits_exactly_the_repeats_from_the_token_before():
    rng = np.random.default_rng(21)
    for K, E in [(4, 16), (2, 5), (6, 12)]:
        sets = [rng.choice(E, K, replace=False) for _ in range(40)]
        hits = ref.expert_cache_hits(sets, K)
        assert hits[0] == set()
        for t in range(1, len(sets)):
            assert hits[t] == set(sets[t].tolist()) & set(sets[t - 1].tolist())


def test_expert_cache_never_full_hits_every_expert_seen_before():
    rng = np.random.default_rng(22)
    K, E = 4, 20
    sets = [rng.choice(E, K, replace=False) for _ in range(30)]
    hits = ref.expert_cache_hits(sets, E)
    seen = set()
    for t, st in enumerate(sets):
        assert hits[t] == set(st.tolist()) & seen
        seen |= set(st.tolist())


def test_expert_cache_holds_the_current_set_and_at_most_c_experts():
    # after each token the current set is cached (a later token repeating it hits
    # in full when nothing else came between), for any C >= K
    rng = np.random.default_rng(23)
    K, E = 4, 24
    for C in (4, 5, 8, 13):
        sets = [rng.choice(E, K, replace=False) for _ in range(25)]
        for t in range(len(sets)):
            again = sets[:t + 1] + [sets[t]]
            assert ref.expert_cache_hits(again, C)[-1] == set(sets[t].tolist())


# ---------------------------------------------------------------- fused Q/K/V projection

def _qkv_closed_form_mats(rng, H, rq, rk, rv):
    G = H // 64
    ones = np.full((rq, G), BF16_ONE, np.uint16)
    wq = (np.ones((rq, H), np.uint8), ones, np.zeros((rq, G), np.uint16))  # every row sums x_n
    bk = wl.bf16_bits_from_f32(rng.normal(0, 1, (rk, G)).astype(np.float32))
    wk = (rng.integers(0, 16, (rk, H), dtype=np.uint8), np.zeros((rk, G), np.uint16), bk)  # bias only
    cols = rng.integers(0, H, rv)
    cv = np.zeros((rv, H), np.uint8)
    cv[np.arange(rv), cols] = 1
    wv = (cv, np.full((rv, G), BF16_ONE, np.uint16), np.zeros((rv, G), np.uint16))  # reads one column
    return [wq, wk, wv], bk, cols


def test_qkv_each_output_has_its_own_closed_form():
    rng = np.random.default_rng(31)
    H, rq, rk, rv = 512, 7, 5, 6
    mats, bk, cols = _qkv_closed_form_mats(rng, H, rq, rk, rv)
    x = rng.integers(-8, 9, H).astype(np.float64)
    q, k, v = ref.qkv(mats, x)
    assert np.array_equal(q, np.full(rq, x.sum()))
    Xg = x.reshape(H // 64, 64).sum(axis=1)
    np.testing.assert_allclose(k, wl.bf16_bits_to_f32(bk).astype(np.float64) @ Xg, rtol=0, atol=1e-9)
    assert np.array_equal(v, x[cols])


def test_qkv_normalises_the_input_once():
    # x = c * ones: RMSNorm gives c / sqrt(c^2 + eps) * gamma for every element
    rng = np.random.default_rng(32)
    H, rq, rk, rv = 256, 3, 2, 4
    mats, bk, cols = _qkv_closed_form_mats(rng, H, rq, rk, rv)
    c, eps = 2.5, 1e-6
    gamma = np.full(H, 0.75, np.float32)
    xn = c / math.sqrt(c * c + eps) * 0.75
    q, k, v = ref.qkv(mats, np.full(H, c), gamma=gamma, norm=True, eps=eps)
    np.testing.assert_allclose(q, np.full(rq, H * xn), rtol=1e-12)
    np.testing.assert_allclose(v, np.full(rv, xn), rtol=1e-12)
    np.testing.assert_allclose(k, wl.bf16_bits_to_f32(bk).astype(np.float64) @ np.full(H // 64, 64 * xn),
                               rtol=1e-12, atol=1e-12)
    # without the norm only gamma scales the input
    q2, _, v2 = ref.qkv(mats, np.full(H, c), gamma=gamma)
    np.testing.assert_allclose(q2, np.full(rq, H * c * 0.75), rtol=1e-12)
    np.testing.assert_allclose(v2, np.full(rv, c * 0.75), rtol=1e-12)

