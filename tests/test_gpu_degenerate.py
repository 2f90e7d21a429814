"""Degenerate cases of the method on the GPU, through the C ABI: equal router logits
(ties go to the lower expert index, the boosted tier first), every expert selected
(E == K), and an all-zero input (zero output, exactly)."""
import numpy as np
import pytest

import quantized_expert_mat_amd as q
import workload as wl
from oracle import ref
from tests.helpers import DeviceLayer, HostLayer, config_for, parity

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def small(**kw):
    base = dict(name="degenerate", hidden=512, inter=128, n_experts=16, top_k=4, n_shared=1)
    base.update(kw)
    return wl.WorkloadConfig(**base)


def ws_for(cfg, T=1, L=1):
    return torch.empty(q.moe_workspace_bytes(cfg, T, L), dtype=torch.uint8, device="cuda")


def layer_call(w, dl, x, flags=0, sel=None):
    T = x.shape[0]
    cfg = config_for(w, flags)
    xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    y = torch.empty_like(xd)
    idx = torch.empty((T, w.top_k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, w.top_k), dtype=torch.float32, device="cuda")
    ws = ws_for(cfg, T)
    sd = torch.from_numpy(sel).cuda() if sel is not None else None
    q.moe_layer_forward(cfg, dl.weights(), T, xd, y, ws, sel_bias=sd, idx_out=idx, w_out=wts)
    q.moe_device_status(ws)
    return y.cpu().numpy(), idx.cpu().numpy(), wts.cpu().numpy()


@pytest.mark.parametrize("prefill", [False, True])
def test_equal_logits_pick_the_lowest_indices(prefill):
    w = small()
    dl, hl = DeviceLayer(w, 0), HostLayer(w, 0)
    dl.router.zero_()
    hl.router = np.zeros_like(hl.router)
    x = wl.tokens_x(w.seed + 1000, 3, w.hidden)
    y, idx, wts = layer_call(w, dl, x, q.MOE_F_PREFILL_BF16 if prefill else 0)
    for t in range(3):
        assert idx[t].tolist() == [0, 1, 2, 3]
        np.testing.assert_allclose(wts[t], 0.25, rtol=0, atol=1e-7)
        if prefill:
            r = ref.prefill_token(x[t], hl.router, hl.expert, hl.shared(), w.top_k, None, by_sel=False)
        else:
            r = ref.layer_decode(x[t], hl.router, hl.expert, hl.shared(), w.top_k)
        assert list(r.idx) == [0, 1, 2, 3]
        parity(y[t], r.y, f"equal logits token {t}")


def test_equal_logits_boosted_tier_first():
    w = small()
    hl = HostLayer(w, 0)
    T = 2
    cfg = config_for(w)
    x = wl.tokens_x(w.seed + 1000, T, w.hidden)
    router = torch.zeros((w.n_experts, w.hidden), dtype=torch.float32, device="cuda")
    boosted = np.array([[9, 5, -1, -1], [-1, 13, -1, -1]], np.int32)
    idx = torch.empty((T, w.top_k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, w.top_k), dtype=torch.float32, device="cuda")
    ws = ws_for(cfg, T)
    q.moe_route(cfg, T, torch.from_numpy(x).cuda(), router, idx, wts, ws, boosted=torch.from_numpy(boosted).cuda())
    q.moe_device_status(ws)
    ih = idx.cpu().numpy()
    # the tier first (ties inside it by lower index), then the lowest other indices
    assert ih[0].tolist() == [5, 9, 0, 1]
    assert ih[1].tolist() == [13, 0, 1, 2]
    for t in range(T):
        b = [int(v) for v in boosted[t] if v >= 0]
        oi, ow, _ = ref.select(np.zeros(w.n_experts), w.top_k, boosted=b)
        assert sorted(oi) == sorted(ih[t].tolist())
    del hl


@pytest.mark.parametrize("prefill", [False, True])
def test_every_expert_selected(prefill):
    w = small(n_experts=4, top_k=4)
    dl, hl = DeviceLayer(w, 0), HostLayer(w, 0)
    T = 5
    x = wl.tokens_x(w.seed + 1000, T, w.hidden)
    y, idx, wts = layer_call(w, dl, x, q.MOE_F_PREFILL_BF16 if prefill else 0)
    for t in range(T):
        assert sorted(idx[t].tolist()) == [0, 1, 2, 3]
        assert abs(float(wts[t].sum()) - 1.0) < 1e-5
        if prefill:
            r = ref.prefill_token(x[t], hl.router, hl.expert, hl.shared(), w.top_k, None, by_sel=False)
        else:
            r = ref.layer_decode(x[t], hl.router, hl.expert, hl.shared(), w.top_k)
        parity(y[t], r.y, f"E == K token {t}")


@pytest.mark.parametrize("prefill", [False, True])
def test_zero_input_gives_exactly_zero(prefill):
    """x = 0: the normalised input, every expert input and every expert output are
    zero, so y = x + 0 = 0 exactly; the equal logits select experts 0..K-1."""
    w = small()
    dl = DeviceLayer(w, 0)
    x = np.zeros((3, w.hidden), np.float32)
    y, idx, _ = layer_call(w, dl, x, q.MOE_F_PREFILL_BF16 if prefill else 0)
    assert np.array_equal(y, np.zeros_like(y))
    assert all(idx[t].tolist() == [0, 1, 2, 3] for t in range(3))
