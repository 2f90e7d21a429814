"""GPU parity of the streamed decode stack (moe_stack_decode_streamed): routed
experts in pinned host memory, read over PCIe, recently used ones kept in an HBM
cache. Outputs and expert sets against the oracle; the per-expert hit pattern
against the oracle's cache policy; outputs against the resident stack."""
import numpy as np
import pytest

import quantized_expert_mat_amd as q
import workload as wl
from oracle import ref
from tests.helpers import NEAR_TIE, DeviceCanonicalLayer, DeviceLayer, HostLayer, config_for, parity, same_set

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def small(**kw):
    base = dict(name="small-streamed", hidden=512, inter=128, n_experts=16, top_k=4, n_shared=1, n_layers=3,
                n_tokens=8, temporal_p=0.27)
    base.update(kw)
    return wl.WorkloadConfig(**base)


def host_layers(dls):
    """Pinned host copies of every layer's routed experts, and the layer weights
    that point at them."""
    pins, lws = [], []
    for d in dls:
        h = torch.empty(d.experts.numel(), dtype=torch.uint8, pin_memory=True)
        h.copy_(d.experts)
        pins.append(h)
        lws.append(q.layer_weights(h, d.shared if d.w.n_shared else None, d.router, None, d.sgate))
    torch.cuda.synchronize()
    return pins, lws


def run_streamed(w, dls, x, mask, C, cfg=None):
    L, T, K = w.n_layers, x.shape[0], w.top_k
    cfg = cfg or config_for(w)
    pins, lws = host_layers(dls)
    cache = torch.empty(L * C * q.moe_packed_expert_bytes(cfg), dtype=torch.uint8, device="cuda")
    ws = torch.empty(q.moe_workspace_bytes(cfg, T, L), dtype=torch.uint8, device="cuda")
    y = torch.empty((T, w.hidden), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, L, K), dtype=torch.int32, device="cuda")
    hit = torch.empty((T, L, K), dtype=torch.uint8, device="cuda")
    q.moe_stack_decode_streamed(cfg, lws, T, torch.from_numpy(x).cuda(), y, ws, cache, C,
                                boost_mask=None if mask is None else torch.from_numpy(mask).cuda(),
                                idx_trace=idx, hit_trace=hit)
    q.moe_device_status(ws)
    del pins
    return y.cpu().numpy(), idx.cpu().numpy(), hit.cpu().numpy()


def check_against_oracle(w, hls, x, mask, yh, ih, hh, C, tokens=None):
    L, K = w.n_layers, w.top_k

    def follow(t, l, oi, gap):
        if same_set(oi, ih[t, l]):
            return None
        assert gap < NEAR_TIE, f"t={t} l={l}: sets differ, gap {gap}"
        return ih[t, l]

    ys, sets, _ = ref.stack_decode(x, L, lambda l: hls[l].router, lambda l, e: hls[l].expert(e),
                                   lambda l: hls[l].shared(), K, boost=mask, follow=follow)
    for t in range(x.shape[0]):
        parity(yh[t], ys[t], f"streamed token {t}")
    n_hits = 0
    for l in range(L):
        want = ref.expert_cache_hits([sets[t, l] for t in range(x.shape[0])], C)
        for t in range(x.shape[0]):
            got = {int(e) for e, h in zip(ih[t, l], hh[t, l]) if h}
            assert got == want[t], f"t={t} l={l}: hits {sorted(got)} vs oracle {sorted(want[t])}"
            n_hits += len(got)
    return n_hits


@pytest.mark.parametrize("C", [4, 6, 16])
def test_streamed_stack_parity_and_cache_hits(C):
    w = small()
    dls = [DeviceLayer(w, l) for l in range(w.n_layers)]
    hls = [HostLayer(w, l) for l in range(w.n_layers)]
    x = wl.tokens_x(w.seed + 1000, w.n_tokens, w.hidden)
    mask = wl.boost_mask(w.seed + 5, w.n_tokens, w.n_layers, w.top_k, 0.5)
    yh, ih, hh = run_streamed(w, dls, x, mask, C)
    n_hits = check_against_oracle(w, hls, x, mask, yh, ih, hh, C)
    assert n_hits > 0  # the boosted repeats are served from the cache


def test_streamed_equals_resident_stack():
    """Same kernels' arithmetic on the same bytes: the streamed stack's outputs are
    bit-identical to the resident stack's."""
    w = small(n_layers=2, n_tokens=6, bits=3, sigma_scale=0.04)
    dls = [DeviceLayer(w, l) for l in range(w.n_layers)]
    x = wl.tokens_x(w.seed + 1000, w.n_tokens, w.hidden)
    mask = wl.boost_mask(w.seed + 5, w.n_tokens, w.n_layers, w.top_k, 0.5)
    ys, is_, _ = run_streamed(w, dls, x, mask, 6)
    cfg = config_for(w)
    T, L, K = w.n_tokens, w.n_layers, w.top_k
    ws = torch.empty(q.moe_workspace_bytes(cfg, T, L), dtype=torch.uint8, device="cuda")
    y = torch.empty((T, w.hidden), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, L, K), dtype=torch.int32, device="cuda")
    q.moe_stack_decode(cfg, [d.weights() for d in dls], T, torch.from_numpy(x).cuda(), y, ws,
                       boost_mask=torch.from_numpy(mask).cuda(), idx_trace=idx)
    q.moe_device_status(ws)
    assert np.array_equal(idx.cpu().numpy(), is_)
    assert np.array_equal(y.cpu().numpy(), ys)


def test_streamed_full_layer_shape():
    """Hidden 4096, I 1024, 512 experts, top-4 + shared: two layers, 7.2 GB of
    pinned host experts."""
    w = wl.LAYER_H4096.replace(name="streamed-h4096", n_layers=2, n_tokens=3, temporal_p=0.27)
    dls = [DeviceLayer(w, l) for l in range(w.n_layers)]
    hls = [DeviceCanonicalLayer(w, l) for l in range(w.n_layers)]
    x = wl.tokens_x(w.seed + 1000, w.n_tokens, w.hidden)
    mask = wl.boost_mask(w.seed + 5, w.n_tokens, w.n_layers, w.top_k, 0.5)
    yh, ih, hh = run_streamed(w, dls, x, mask, 8)
    check_against_oracle(w, hls, x, mask, yh, ih, hh, 8)


def test_streamed_full_shape_zero_mean():
    """The host-memory tier on zero-mean weights, where routing stays token-dependent
    (the regime of the 27% repeats): three full-shape layers x 4 tokens with the
    tier, outputs, sets and the per-expert hit pattern against the oracle."""
    w = wl.STACK60_4BIT_ZM.replace(name="streamed-zm", n_layers=3, n_tokens=4)
    dls = [DeviceLayer(w, l, chunk=8) for l in range(w.n_layers)]
    hls = [DeviceCanonicalLayer(w, l) for l in range(w.n_layers)]
    x = wl.tokens_x(w.seed + 1000, w.n_tokens, w.hidden)
    mask = wl.boost_mask(w.seed + 7, w.n_tokens, w.n_layers, w.top_k, w.temporal_p)
    yh, ih, hh = run_streamed(w, dls, x, mask, w.top_k)
    n_hits = check_against_oracle(w, hls, x, mask, yh, ih, hh, w.top_k)
    # with C = K a hit is exactly a repeat from the token before; every promoted
    # expert repeats, so there are at least as many hits as promoted slots
    assert n_hits >= int(mask[1:].astype(bool).sum())


def test_streamed_rejects_pageable_experts():
    w = small(n_layers=1, n_tokens=1)
    d = DeviceLayer(w, 0)
    cfg = config_for(w)
    pageable = d.experts.cpu()  # ordinary host memory: the device cannot read it
    lw = q.layer_weights(pageable, d.shared, d.router)
    cache = torch.empty(4 * q.moe_packed_expert_bytes(cfg), dtype=torch.uint8, device="cuda")
    ws = torch.empty(q.moe_workspace_bytes(cfg, 1, 1), dtype=torch.uint8, device="cuda")
    x = torch.zeros((1, w.hidden), device="cuda")
    y = torch.empty_like(x)
    with pytest.raises(q.MoeError) as ei:
        q.moe_stack_decode_streamed(cfg, [lw], 1, x, y, ws, cache, 4)
    assert ei.value.status == q.MOE_ERR_ARG
