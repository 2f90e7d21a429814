"""GPU parity at the limits the C ABI accepts: 1024 routed experts, top-16, two
shared experts, intermediate width 4096 (with hidden 4096 and with hidden 64),
through decode (layer and stack) and prefill, against the oracle."""
import numpy as np
import pytest

import quantized_expert_mat_amd as q
import workload as wl
from oracle import ref
from tests.helpers import NEAR_TIE, DeviceLayer, HostLayer, config_for, parity, same_set

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def ws_for(cfg, T=1, L=1):
    return torch.empty(q.moe_workspace_bytes(cfg, T, L), dtype=torch.uint8, device="cuda")


def xs(w, T):
    return wl.tokens_x(w.seed + 1000, T, w.hidden)


MAX_COUNTS = wl.WorkloadConfig("max-counts", 256, 64, 1024, top_k=16, n_shared=2)


@pytest.mark.parametrize("wcfg,T", [
    (MAX_COUNTS, 2),
    (wl.WorkloadConfig("max-inter", 1024, 4096, 8, top_k=2, n_shared=1), 2),
    (wl.WorkloadConfig("min-hidden-max-inter", 64, 4096, 6, top_k=3, n_shared=1), 2),
])
def test_layer_forward_at_limits(wcfg, T):
    cfg = config_for(wcfg)
    dl, hl = DeviceLayer(wcfg, 0, chunk=8), HostLayer(wcfg, 0)
    x = xs(wcfg, T)
    xd = torch.from_numpy(x).cuda()
    y = torch.empty_like(xd)
    idx = torch.empty((T, wcfg.top_k), dtype=torch.int32, device="cuda")
    ws = ws_for(cfg, T)
    q.moe_layer_forward(cfg, dl.weights(), T, xd, y, ws, idx_out=idx)
    q.moe_device_status(ws)
    yh, ih = y.cpu().numpy(), idx.cpu().numpy()
    for t in range(T):
        r = ref.layer_decode(x[t], hl.router, hl.expert, hl.shared(), wcfg.top_k)
        if not same_set(r.idx, ih[t]):
            assert r.gap < NEAR_TIE, f"token {t}: sets differ, gap {r.gap}"
            r = ref.layer_decode(x[t], hl.router, hl.expert, hl.shared(), wcfg.top_k, force_idx=ih[t])
        parity(yh[t], r.y, f"{wcfg.name} token {t}")


def test_expert_forward_max_dims():
    w = wl.WorkloadConfig("max-dims", 4096, 4096, 1, top_k=1, n_shared=0)
    cfg = config_for(w)
    dl, hl = DeviceLayer(w, 0), HostLayer(w, 0)
    T = 2
    x = xs(w, T)
    xd = torch.from_numpy(x).cuda()
    y = torch.empty_like(xd)
    ws = ws_for(cfg, T)
    q.moe_expert_forward(cfg, dl.experts, T, xd, y, ws)
    q.moe_device_status(ws)
    for t in range(T):
        parity(y.cpu().numpy()[t], ref.expert(hl.expert(0), x[t]), f"hidden 4096 inter 4096 token {t}")


def test_stack_at_max_counts_with_tier():
    w = MAX_COUNTS.replace(n_layers=2, n_tokens=3, temporal_p=0.27)
    L, T, K = w.n_layers, w.n_tokens, w.top_k
    cfg = config_for(w)
    dls = [DeviceLayer(w, l, chunk=8) for l in range(L)]
    hls = [HostLayer(w, l) for l in range(L)]
    x = xs(w, T)
    mask = wl.boost_mask(w.seed + 5, T, L, K, 0.5)
    y = torch.empty((T, w.hidden), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, L, K), dtype=torch.int32, device="cuda")
    ws = ws_for(cfg, T, L)
    q.moe_stack_decode(cfg, [d.weights() for d in dls], T, torch.from_numpy(x).cuda(), y, ws,
                       boost_mask=torch.from_numpy(mask).cuda(), idx_trace=idx)
    q.moe_device_status(ws)
    ih = idx.cpu().numpy()

    def follow(t, l, oi, gap):
        if same_set(oi, ih[t, l]):
            return None
        assert gap < NEAR_TIE, f"t={t} l={l}: sets differ, gap {gap}"
        return ih[t, l]

    ys, sets, _ = ref.stack_decode(x, L, lambda l: hls[l].router, lambda l, e: hls[l].expert(e),
                                   lambda l: hls[l].shared(), K, boost=mask, follow=follow)
    for t in range(T):
        parity(y.cpu().numpy()[t], ys[t], f"max-counts stack token {t}")


def test_prefill_at_max_counts():
    w = MAX_COUNTS
    T = 40
    dl, hl = DeviceLayer(w, 0, chunk=8), HostLayer(w, 0)
    x = xs(w, T)
    sel, _ = wl.zipf_gumbel_scores(w.seed + 3, T, w.n_experts, 1.1)
    cfg = config_for(w, q.MOE_F_PREFILL_BF16 | q.MOE_F_SELECT_BY_BIAS)
    ws = ws_for(cfg, T)
    xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    y = torch.empty_like(xd)
    idx = torch.empty((T, w.top_k), dtype=torch.int32, device="cuda")
    q.moe_layer_forward(cfg, dl.weights(), T, xd, y, ws, sel_bias=torch.from_numpy(sel).cuda(), idx_out=idx)
    q.moe_device_status(ws)
    yh, ih = y.cpu().numpy(), idx.cpu().numpy()
    for t in range(T):
        r = ref.prefill_token(x[t], hl.router, hl.expert, hl.shared(), w.top_k, sel[t])
        assert np.array_equal(np.asarray(r.idx), ih[t])
        parity(yh[t], r.y, f"max-counts prefill token {t}")
