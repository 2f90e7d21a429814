"""GPU parity of 3-bit group-affine experts (codes 0..7, one bf16 (scale, bias) per
64-group; a synthetic stand-in for the 3-bit experts of the autoresearch page,
section "Optimizaciones Efectivas") through pack, expert forward, one layer, the
decode stack and the batched prefill, against the oracle through the C ABI."""
import numpy as np
import pytest

import quantized_expert_mat_amd as q
import workload as wl
from oracle import ref
from tests.helpers import NEAR_TIE, DeviceLayer, HostLayer, config_for, parity, same_set
from workload import device as wdev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SIGMA3 = 0.04
LAYER3 = wl.LAYER_H4096.replace(name="layer-h4096-e512-3bit", bits=3, sigma_scale=SIGMA3)


def small(**kw):
    base = dict(name="small-3bit", hidden=512, inter=128, n_experts=24, top_k=4, n_shared=1, bits=3,
                sigma_scale=SIGMA3)
    base.update(kw)
    return wl.WorkloadConfig(**base)


def xs(w, T):
    return wl.tokens_x(w.seed + 1000, T, w.hidden)


def ws_for(cfg, T=1, L=1):
    return torch.empty(q.moe_workspace_bytes(cfg, T, L), dtype=torch.uint8, device="cuda")


def test_device_generator_3bit_codes_match_host():
    spec = wl.ExpertSpec(256, 128, bits=3)
    codes = torch.empty((1, 3, 256 * 128), dtype=torch.uint8, device="cuda")
    sc = torch.empty((1, 3, 512), dtype=torch.int16, device="cuda")
    bi = torch.empty((1, 3, 512), dtype=torch.int16, device="cuda")
    keep = wdev.experts_canonical(spec, 7, 3, [5], codes, sc, bi)
    torch.cuda.synchronize()
    cs, _, _ = wl.expert_canonical(spec, 7, 3, 5)
    for m in range(3):
        assert np.array_equal(codes[0, m].cpu().numpy(), cs[m].reshape(-1))
    assert int(codes.max()) == 7
    del keep


@pytest.mark.parametrize("H,I", [(512, 128), (4096, 1024), (64, 64)])
def test_expert_forward_integer_exact_3bit(H, I):
    """scale 1, bias 0, integer x: every bit of every code reaches the result, so a
    misplaced bit in the packed layout or its unpacking shows as an integer error."""
    cfg = q.Config.make(H, I, 1, 1, 0, 3)
    rng = np.random.default_rng(11)
    codes = rng.integers(0, 8, size=(1, 3, H * I), dtype=np.uint8)
    ones = np.full((1, 3, H * I // 64), 0x3F80, np.uint16)
    zeros = np.zeros_like(ones)
    ones[0, 2] = wl.bf16_bits_from_f32(np.full(H * I // 64, 2.0 ** -20, np.float32))
    packed = torch.empty(q.moe_packed_expert_bytes(cfg), dtype=torch.uint8, device="cuda")
    ws = ws_for(cfg, 2)
    q.moe_pack_weights(cfg, 1, torch.from_numpy(codes).cuda(), torch.from_numpy(ones.view(np.int16)).cuda(),
                       torch.from_numpy(zeros.view(np.int16)).cuda(), packed, ws)
    x = rng.integers(-8, 9, size=(2, H)).astype(np.float32) / 64.0
    xd = torch.from_numpy(x).cuda()
    y = torch.empty_like(xd)
    q.moe_expert_forward(cfg, packed, 2, xd, y, ws)
    q.moe_device_status(ws)
    canon = ([codes[0, 0].reshape(I, H), codes[0, 1].reshape(I, H), codes[0, 2].reshape(H, I)],
             [ones[0, 0].reshape(I, H // 64), ones[0, 1].reshape(I, H // 64), ones[0, 2].reshape(H, I // 64)],
             [zeros[0, 0].reshape(I, H // 64), zeros[0, 1].reshape(I, H // 64), zeros[0, 2].reshape(H, I // 64)])
    for t in range(2):
        o = ref.expert(canon, x[t])
        np.testing.assert_allclose(y.cpu().numpy()[t], o, rtol=2e-6, atol=1e-6 * np.abs(o).max())


def test_pack_rejects_code_above_7():
    cfg = q.Config.make(64, 64, 1, 1, 0, 3)
    codes = np.zeros((1, 3, 64 * 64), np.uint8)
    codes[0, 1, 77] = 8
    s = np.full((1, 3, 64), 0x3F80, np.uint16).view(np.int16)
    packed = torch.empty(q.moe_packed_expert_bytes(cfg), dtype=torch.uint8, device="cuda")
    ws = ws_for(cfg)
    q.moe_pack_weights(cfg, 1, torch.from_numpy(codes).cuda(), torch.from_numpy(s).cuda(),
                       torch.from_numpy(s).cuda(), packed, ws)
    with pytest.raises(q.MoeError):
        q.moe_device_status(ws)


@pytest.mark.parametrize("H,I", [(1024, 256), (256, 64), (4096, 1024)])
def test_expert_forward_parity_3bit(H, I):
    w = small(hidden=H, inter=I, n_experts=2, top_k=1, n_shared=0)
    dl, hl = DeviceLayer(w, 0), HostLayer(w, 0)
    T = 3
    cfg = config_for(w)
    x = xs(w, T)
    xd = torch.from_numpy(x).cuda()
    y = torch.empty_like(xd)
    ws = ws_for(cfg, T)
    for e in range(2):
        q.moe_expert_forward(cfg, dl.experts[e * dl.expert_bytes:(e + 1) * dl.expert_bytes], T, xd, y, ws)
        q.moe_device_status(ws)
        yh = y.cpu().numpy()
        for t in range(T):
            parity(yh[t], ref.expert(hl.expert(e), x[t]), f"3-bit expert {e} token {t}")


@pytest.mark.parametrize("wcfg,T,phased,gated", [
    (small(), 3, False, False),
    (small(), 2, True, False),
    (LAYER3, 2, False, False),
    (LAYER3, 1, False, True),
])
def test_layer_forward_parity_3bit(wcfg, T, phased, gated):
    cfg = config_for(wcfg, q.MOE_F_PHASED if phased else 0)
    dl, hl = DeviceLayer(wcfg, 0, gated=gated), HostLayer(wcfg, 0)
    G = hl.shared_gate() if gated else None
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
        parity(yh[t], r.y, f"{wcfg.name} token {t}")


def test_stack_decode_parity_3bit():
    w = small(hidden=512, inter=128, n_experts=16, n_layers=4, n_tokens=6, temporal_p=0.27)
    L, T, K = w.n_layers, w.n_tokens, w.top_k
    cfg = config_for(w)
    dls = [DeviceLayer(w, l) for l in range(L)]
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
        for l in range(L):
            assert same_set(sets[t, l], ih[t, l])
        parity(y.cpu().numpy()[t], ys[t], f"3-bit stack token {t}")


@pytest.mark.parametrize("T", [37, 130])
def test_prefill_parity_3bit(T):
    w = small(inter=256, n_experts=16)
    dl, hl = DeviceLayer(w, 0), HostLayer(w, 0)
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
        parity(yh[t], r.y, f"3-bit prefill T={T} token {t}")
