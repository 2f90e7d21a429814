"""GPU parity of the batched prefill (moe_layer_forward with MOE_F_PREFILL_BF16:
token grouping by expert + expert-grouped bf16 MFMA GEMM) against the oracle's
prefill token (bf16 rounding points), through the C ABI."""
import numpy as np
import pytest

import quantized_expert_mat_amd as q
import workload as wl
from oracle import ref
from tests.helpers import (NEAR_TIE, DeviceCanonicalLayer, DeviceLayer, HostLayer, config_for, parity,
                           same_set)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

PREFILL = wl.PREFILL1155  # 1155 tokens, H 4096, I 1024, E 512, Zipf(1.1) routing


def small(**kw):
    base = dict(name="small-prefill", hidden=512, inter=256, n_experts=16, top_k=4, n_shared=1)
    base.update(kw)
    return wl.WorkloadConfig(**base)


def run_prefill(w, dl, x, sel=None, boosted=None, flags_extra=q.MOE_F_SELECT_BY_BIAS, gamma=None):
    T = x.shape[0]
    cfg = config_for(w, q.MOE_F_PREFILL_BF16 | flags_extra)
    ws = torch.empty(q.moe_workspace_bytes(cfg, T, 1), dtype=torch.uint8, device="cuda")
    xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    y = torch.empty_like(xd)
    idx = torch.empty((T, w.top_k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, w.top_k), dtype=torch.float32, device="cuda")
    sd = torch.from_numpy(np.ascontiguousarray(sel)).cuda() if sel is not None else None
    bd = torch.from_numpy(np.ascontiguousarray(boosted)).cuda() if boosted is not None else None
    lw = dl.weights() if gamma is None else q.layer_weights(dl.experts, dl.shared if w.n_shared else None,
                                                          dl.router, gamma)
    q.moe_layer_forward(cfg, lw, T, xd, y, ws, sel_bias=sd, boosted=bd, idx_out=idx, w_out=wts)
    q.moe_device_status(ws)
    return y.cpu().numpy(), idx.cpu().numpy(), wts.cpu().numpy()


def check_tokens(w, hl, x, yh, ih, wh, sel, tokens, by_sel=True, boosted=None, gamma=None, what=""):
    for t in tokens:
        b = tuple(int(v) for v in boosted[t] if v >= 0) if boosted is not None else ()
        kw = dict(by_sel=by_sel, boosted=b, rmsnorm_on=w.rmsnorm, residual=w.residual, gamma=gamma)
        s = sel[t] if sel is not None else None
        r = ref.prefill_token(x[t], hl.router, hl.expert, hl.shared(), w.top_k, s, **kw)
        if by_sel:
            # the scores are the same float32 values on both sides: the order is exact
            assert np.array_equal(np.asarray(r.idx), ih[t]), f"{what} token {t}: {r.idx} vs {ih[t]}"
        elif not same_set(r.idx, ih[t]):
            assert r.gap < NEAR_TIE, f"{what} token {t}: sets differ, gap {r.gap}"
            r = ref.prefill_token(x[t], hl.router, hl.expert, hl.shared(), w.top_k, s, force_idx=ih[t], **kw)
        order = [list(r.idx).index(e) for e in ih[t]] if by_sel else range(w.top_k)
        if by_sel:
            np.testing.assert_allclose(wh[t], np.asarray(r.w)[order], rtol=2e-5, atol=1e-7)
        parity(yh[t], r.y, f"{what} token {t}")


@pytest.mark.parametrize("bits,T", [(4, 37), (2, 37), (4, 1), (4, 130)])
def test_prefill_parity_small(bits, T):
    w = small(bits=bits, sigma_scale=0.02 if bits == 4 else 0.06)
    dl, hl = DeviceLayer(w, 0), HostLayer(w, 0)
    x = wl.tokens_x(w.seed + 1000, T, w.hidden)
    sel, _ = wl.zipf_gumbel_scores(w.seed + 3, T, w.n_experts, 1.1)
    yh, ih, wh = run_prefill(w, dl, x, sel)
    check_tokens(w, hl, x, yh, ih, wh, sel, range(T), what=f"{bits}-bit T={T}")


def test_prefill_hot_expert_spans_m_tiles():
    """One expert takes every token (rows beyond one 128-row m-tile, ragged tail), the
    others split the rest; H 256 / I 64 also exercise the smallest tile shapes."""
    w = small(hidden=256, inter=64, n_experts=8, top_k=2)
    T = 300
    dl, hl = DeviceLayer(w, 0), HostLayer(w, 0)
    x = wl.tokens_x(w.seed + 1001, T, w.hidden)
    sel, _ = wl.zipf_gumbel_scores(w.seed + 4, T, w.n_experts, 1.1)
    sel = sel.copy()
    sel[:, 3] += 100.0  # expert 3 is in every token's set
    yh, ih, wh = run_prefill(w, dl, x, sel)
    assert (ih == 3).any(axis=1).all()
    check_tokens(w, hl, x, yh, ih, wh, sel, range(T), what="hot expert")


def test_prefill_router_selection_and_boosted_tier():
    """Selection by logit + sel_bias (router GEMM path) with a boosted tier, and by
    the logits alone; near-ties follow the GPU's set."""
    w = small(n_experts=40, top_k=3, n_shared=2)
    T = 29
    dl, hl = DeviceLayer(w, 0), HostLayer(w, 0)
    x = wl.tokens_x(w.seed + 1002, T, w.hidden)
    sel, _ = wl.zipf_gumbel_scores(w.seed + 5, T, w.n_experts, 1.1)
    sel = (0.01 * sel).astype(np.float32)
    boosted = np.full((T, w.top_k), -1, dtype=np.int32)
    boosted[::3, 0] = 7
    boosted[1::4, 1] = 21
    yh, ih, wh = run_prefill(w, dl, x, sel, boosted=boosted, flags_extra=0)
    check_tokens(w, hl, x, yh, ih, wh, sel, range(T), by_sel=False, boosted=boosted, what="logit+bias")
    for t in range(T):
        for e in boosted[t]:
            if e >= 0:
                assert e in ih[t]
    yh, ih, wh = run_prefill(w, dl, x, None, flags_extra=0)
    check_tokens(w, hl, x, yh, ih, wh, None, range(T), by_sel=False, what="logits")


def test_prefill_flags_gamma_and_no_residual():
    w = small(rmsnorm=True, residual=False, n_shared=0, top_k=1, n_experts=8)
    T = 17
    dl, hl = DeviceLayer(w, 0), HostLayer(w, 0)
    x = wl.tokens_x(w.seed + 1003, T, w.hidden)
    sel, _ = wl.zipf_gumbel_scores(w.seed + 6, T, w.n_experts, 1.1)
    gamma = (1.0 + 0.25 * wl.tokens_x(99, 1, w.hidden)[0]).astype(np.float32)
    yh, ih, wh = run_prefill(w, dl, x, sel, gamma=torch.from_numpy(gamma).cuda())
    check_tokens(w, hl, x, yh, ih, wh, sel, range(T), gamma=gamma.astype(np.float64), what="gamma")
    w2 = small(rmsnorm=False, residual=True, hidden=128, inter=128)
    dl2, hl2 = DeviceLayer(w2, 0), HostLayer(w2, 0)
    x2 = wl.tokens_x(w2.seed + 1004, T, w2.hidden)
    sel2, _ = wl.zipf_gumbel_scores(w2.seed + 7, T, w2.n_experts, 1.1)
    yh, ih, wh = run_prefill(w2, dl2, x2, sel2)
    check_tokens(w2, hl2, x2, yh, ih, wh, sel2, range(T), what="no norm")


def test_prefill_more_tokens_than_one_pass():
    """2100 tokens: the entry point runs them as two passes (2048 + 52)."""
    w = small(hidden=64, inter=64, n_experts=8, top_k=2)
    T = 2100
    dl, hl = DeviceLayer(w, 0), HostLayer(w, 0)
    x = wl.tokens_x(w.seed + 1005, T, w.hidden)
    sel, _ = wl.zipf_gumbel_scores(w.seed + 8, T, w.n_experts, 1.1)
    yh, ih, wh = run_prefill(w, dl, x, sel)
    check_tokens(w, hl, x, yh, ih, wh, sel, list(range(0, T, 7)) + [2047, 2048, 2099], what="2 passes")


def test_prefill_deterministic_and_zero_tokens():
    w = small()
    dl = DeviceLayer(w, 0)
    x = wl.tokens_x(w.seed + 1006, 50, w.hidden)
    sel, _ = wl.zipf_gumbel_scores(w.seed + 9, 50, w.n_experts, 1.1)
    y1, i1, _ = run_prefill(w, dl, x, sel)
    y2, i2, _ = run_prefill(w, dl, x, sel)
    assert np.array_equal(y1, y2) and np.array_equal(i1, i2)
    cfg = config_for(w, q.MOE_F_PREFILL_BF16 | q.MOE_F_SELECT_BY_BIAS)
    ws = torch.empty(q.moe_workspace_bytes(cfg, 1, 1), dtype=torch.uint8, device="cuda")
    xd = torch.zeros((1, w.hidden), dtype=torch.float32, device="cuda")
    y = torch.full_like(xd, 7.0)
    q.moe_layer_forward(cfg, dl.weights(), 0, xd, y, ws, sel_bias=xd)
    q.moe_device_status(ws)
    assert (y == 7.0).all()


def test_prefill_full_size_sampled():
    """The 1155-token prefill at the flash-moe layer shape with Zipf(1.1) routing:
    every token's experts and weights against the oracle's selection, sampled tokens'
    outputs against the oracle's prefill token."""
    w = PREFILL
    T = w.n_tokens
    dl = DeviceLayer(w, 0)
    x = wl.tokens_x(w.seed + 1000, T, w.hidden)
    sel, _ = wl.zipf_gumbel_scores(w.seed + 11, T, w.n_experts, w.zipf)
    yh, ih, wh = run_prefill(w, dl, x, sel)
    cl = DeviceCanonicalLayer(w, 0)
    for t in range(T):
        r_idx, _, _ = ref.select(np.zeros(w.n_experts), w.top_k, sel=sel[t], by_sel=True)
        assert np.array_equal(np.asarray(r_idx), ih[t]), f"token {t}"
    counts = np.bincount(ih.reshape(-1), minlength=w.n_experts)
    hot = int(np.argmax(counts))
    assert counts.max() > 128  # the hottest expert spans several m-tiles
    tokens = [0, 1, 577, T - 1] + [int(t) for t in np.nonzero((ih == hot).any(axis=1))[0][[0, -1]]]
    check_tokens(w, cl, x, yh, ih, wh, sel, tokens, what="prefill1155")


@pytest.mark.parametrize("T", [37, 1700])
def test_prefill_top10(T):
    """Top-10 routing; at 1700 tokens the pass holds at most 16384 routed pairs, so two passes."""
    w = small(top_k=10, n_experts=32, hidden=256, inter=128)
    dl, hl = DeviceLayer(w, 0), HostLayer(w, 0)
    x = wl.tokens_x(w.seed + 1000, T, w.hidden)
    sel, _ = wl.zipf_gumbel_scores(w.seed + 3, T, w.n_experts, 1.1)
    yh, ih, wh = run_prefill(w, dl, x, sel)
    toks = range(T) if T <= 64 else list(range(0, T, 97)) + [1637, 1638, 1639, T - 1]
    check_tokens(w, hl, x, yh, ih, wh, sel, toks, what=f"top-10 T={T}")


def test_prefill_repeat_calls_bit_identical():
    """Rows of an expert are placed by LDS atomics, so their order may change between
    calls; every row is computed on its own, so the outputs may not."""
    w = small(n_experts=8)
    T = 300
    dl = DeviceLayer(w, 0)
    x = wl.tokens_x(w.seed + 1000, T, w.hidden)
    sel, _ = wl.zipf_gumbel_scores(w.seed + 3, T, w.n_experts, 1.1)
    outs = [run_prefill(w, dl, x, sel) for _ in range(3)]
    for y, idx, wts in outs[1:]:
        assert np.array_equal(y, outs[0][0])
        assert np.array_equal(idx, outs[0][1])
        assert np.array_equal(wts, outs[0][2])
