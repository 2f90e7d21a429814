"""GPU parity of the shared-expert gate: shared expert s enters the combine scaled by
sigmoid(g_s . x_n) (moe_layer_weights.shared_gate), for the decode layer, the
decode stack and the batched prefill, against the oracle through the C ABI."""
import numpy as np
import pytest

import quantized_expert_mat_amd as q
import workload as wl
from oracle import ref
from tests.helpers import NEAR_TIE, DeviceLayer, HostLayer, config_for, parity, same_set

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

LAYER = wl.LAYER_H4096  # H 4096, I 1024, E 512, norm + residual


def small(**kw):
    base = dict(name="small-gate", hidden=512, inter=128, n_experts=24, top_k=4, n_shared=1)
    base.update(kw)
    return wl.WorkloadConfig(**base)


def xs(w, T):
    return wl.tokens_x(w.seed + 1000, T, w.hidden)


def ws_for(cfg, T=1, L=1):
    return torch.empty(q.moe_workspace_bytes(cfg, T, L), dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("wcfg,T,phased", [
    (small(), 3, False),
    (small(n_shared=2, top_k=3, n_experts=12), 2, False),
    (small(), 2, True),
    (LAYER, 1, False),
])
def test_layer_forward_shared_gate(wcfg, T, phased):
    cfg = config_for(wcfg, q.MOE_F_PHASED if phased else 0)
    dl = DeviceLayer(wcfg, 0, gated=True)
    hl = HostLayer(wcfg, 0)
    G = hl.shared_gate()
    x = xs(wcfg, T)
    xd = torch.from_numpy(x).cuda()
    y = torch.empty_like(xd)
    idx = torch.empty((T, wcfg.top_k), dtype=torch.int32, device="cuda")
    ws = ws_for(cfg, T)
    q.moe_layer_forward(cfg, dl.weights(), T, xd, y, ws, idx_out=idx)
    q.moe_device_status(ws)
    yh, ih = y.cpu().numpy(), idx.cpu().numpy()
    for t in range(T):
        r = ref.layer_decode(x[t], hl.router, hl.expert, hl.shared(), wcfg.top_k, shared_gate=G)
        if not same_set(r.idx, ih[t]):
            assert r.gap < NEAR_TIE, f"token {t}: sets differ, gap {r.gap}"
            r = ref.layer_decode(x[t], hl.router, hl.expert, hl.shared(), wcfg.top_k, shared_gate=G,
                                 force_idx=ih[t])
        parity(yh[t], r.y, f"{wcfg.name} gated token {t}")
        # the gate changed the output: it is not a no-op on this input
        u = ref.layer_decode(x[t], hl.router, hl.expert, hl.shared(), wcfg.top_k, force_idx=ih[t])
        assert np.abs(u.y - r.y).max() > 1e-4 * np.abs(r.y).max()


def test_stack_decode_shared_gate_mixed_layers():
    """Gated and ungated layers in one stack (layer 1 has no gate)."""
    w = small(n_layers=3, n_tokens=4, n_experts=16)
    L, T, K = w.n_layers, w.n_tokens, w.top_k
    cfg = config_for(w)
    dls = [DeviceLayer(w, l, gated=(l != 1)) for l in range(L)]
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
                                   lambda l: hls[l].shared(), K, boost=mask, follow=follow,
                                   shared_gate_of=lambda l: None if l == 1 else hls[l].shared_gate())
    for t in range(T):
        parity(y.cpu().numpy()[t], ys[t], f"gated stack token {t}")


@pytest.mark.parametrize("n_shared", [1, 2])
def test_prefill_shared_gate(n_shared):
    w = wl.WorkloadConfig(name="small-prefill-gate", hidden=512, inter=256, n_experts=16, top_k=4,
                          n_shared=n_shared)
    T = 37
    dl, hl = DeviceLayer(w, 0, gated=True), HostLayer(w, 0)
    G = hl.shared_gate()
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
        r = ref.prefill_token(x[t], hl.router, hl.expert, hl.shared(), w.top_k, sel[t], shared_gate=G)
        assert np.array_equal(np.asarray(r.idx), ih[t])
        parity(yh[t], r.y, f"gated prefill S={n_shared} token {t}")
