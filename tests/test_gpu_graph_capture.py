"""Entry points captured into a HIP graph (torch.cuda.CUDAGraph) and replayed: the
resident stack (with a workspace and allocation-free), the streamed stack (routed
experts in pinned host memory), the single-layer decode call, the 1155-token
prefill and the fused Q/K/V projection. Every replay, with
eager work and a synchronisation between replays, gives the eager call's outputs
bit for bit, including after the input buffer is rewritten between replays. The
weight memory stays alive while a graph may replay (a capture made with torch
begins by returning freed cached memory to the device)."""
import numpy as np
import pytest

import quantized_expert_mat_amd as q
import workload as wl
from workload.device_layer import DeviceLayer, config_for

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def eager(cfg, lws, T, x, mask, L, K, H):
    ws = torch.empty(q.moe_workspace_bytes(cfg, T, L), dtype=torch.uint8, device="cuda")
    y = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((T, L, K), -1, dtype=torch.int32, device="cuda")
    q.moe_stack_decode(cfg, lws, T, x, y, ws, boost_mask=mask, idx_trace=idx)
    q.moe_device_status(ws)
    return y.cpu().numpy(), idx.cpu().numpy()


def capture_case(w, L, T, noalloc):
    cfg = config_for(w)
    K, H = w.top_k, w.hidden
    # the layers own the device tensors that the weight pointers point into: they
    # must stay alive (capture begins by returning freed cached memory to the device)
    dls = [DeviceLayer(w, l, chunk=8) for l in range(L)]
    lws = [d.weights() for d in dls]
    x = torch.from_numpy(wl.tokens_x(w.seed + 1000, T, H)).cuda()
    x2 = torch.from_numpy(wl.tokens_x(w.seed + 2000, T, H)).cuda()
    mask = torch.from_numpy(wl.boost_mask(w.seed + 7, T, L, K, w.temporal_p or 0.27)).cuda()
    y_ref, i_ref = eager(cfg, lws, T, x, mask, L, K, H)
    y2_ref, i2_ref = eager(cfg, lws, T, x2, mask, L, K, H)
    assert not np.array_equal(y_ref, y2_ref)

    y = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((T, L, K), -1, dtype=torch.int32, device="cuda")
    err = torch.zeros((1,), dtype=torch.int32, device="cuda")
    ws = torch.empty(q.moe_workspace_bytes(cfg, T, L), dtype=torch.uint8, device="cuda")
    xin = x.clone()
    s = torch.cuda.Stream()

    def call():
        if noalloc:
            q.moe_stack_decode_noalloc(cfg, lws, T, xin, y, boost_mask=mask, idx_trace=idx, dev_err=err,
                                       stream=s)
        else:
            q.moe_stack_decode(cfg, lws, T, xin, y, ws, boost_mask=mask, idx_trace=idx, stream=s)

    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()  # eager warm-up on the capture stream: one-time set-up happens here
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    torch.cuda.synchronize()
    for r in range(4):
        print(f"graph ({'noalloc' if noalloc else 'workspace'}) L={L} T={T} H={H}: replay {r}", flush=True)
        y.fill_(float("nan"))
        idx.fill_(-1)
        err.fill_(0x7FFFFFFF)
        second = r >= 2
        xin.copy_(x2 if second else x)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        yr, ir = (y2_ref, i2_ref) if second else (y_ref, i_ref)
        assert np.array_equal(idx.cpu().numpy(), ir)
        assert np.array_equal(y.cpu().numpy().view(np.uint32), yr.view(np.uint32))
        if noalloc:
            assert int(err.item()) == 0
    if not noalloc:
        q.moe_device_status(ws)
    del g
    torch.cuda.synchronize()
    del dls


@pytest.mark.parametrize("noalloc", [False, True])
def test_stack_graph_replays_full_shape(noalloc):
    capture_case(wl.STACK60_4BIT.replace(n_layers=3, n_tokens=4), 3, 4, noalloc)


@pytest.mark.parametrize("noalloc", [False, True])
def test_stack_graph_replays_general_shape(noalloc):
    small = wl.WorkloadConfig(name="small", hidden=512, inter=128, n_experts=24, top_k=4, n_shared=1,
                              n_layers=2, n_tokens=3)
    capture_case(small, 2, 3, noalloc)


def _fill(outs):
    for o in outs:
        o.fill_(float("nan") if o.dtype.is_floating_point else -1)


def graph_vs_eager(what, run, xin, inputs, outs):
    """Eager results of run(stream) for each input, then the same call captured into a
    graph: four replays (inputs[0] twice, then inputs[1] twice), each compared bit for
    bit with the eager result of its input."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    refs = []
    for xv in inputs:
        xin.copy_(xv)
        _fill(outs)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            run(s)
        torch.cuda.synchronize()
        refs.append([o.cpu().numpy().copy() for o in outs])
    assert not np.array_equal(refs[0][0], refs[1][0])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run(s)
    torch.cuda.synchronize()
    for r in range(4):
        print(f"graph {what}: replay {r}", flush=True)
        i = 0 if r < 2 else 1
        _fill(outs)
        xin.copy_(inputs[i])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, ref in zip(outs, refs[i]):
            got = o.cpu().numpy()
            assert np.array_equal(got.view(np.uint8), ref.view(np.uint8)), what
    del g
    torch.cuda.synchronize()


def test_layer_decode_graph_replays():
    w = wl.LAYER_H4096.replace(n_tokens=2)
    T = 2
    cfg = config_for(w)
    dl = DeviceLayer(w, 0)
    lw = dl.weights()
    ws = torch.empty(q.moe_workspace_bytes(cfg, T, 1), dtype=torch.uint8, device="cuda")
    xs = [torch.from_numpy(wl.tokens_x(w.seed + 100 + i, T, w.hidden)).cuda() for i in range(2)]
    xin = xs[0].clone()
    y = torch.empty_like(xin)
    idx = torch.empty((T, w.top_k), dtype=torch.int32, device="cuda")
    wt = torch.empty((T, w.top_k), dtype=torch.float32, device="cuda")

    def run(s):
        q.moe_layer_forward(cfg, lw, T, xin, y, ws, idx_out=idx, w_out=wt, stream=s)

    graph_vs_eager("layer decode", run, xin, xs, [y, idx, wt])
    q.moe_device_status(ws)


def test_prefill_graph_replays():
    w = wl.PREFILL1155
    T = w.n_tokens
    cfg = config_for(w, q.MOE_F_PREFILL_BF16 | q.MOE_F_SELECT_BY_BIAS)
    dl = DeviceLayer(w, 0)
    lw = dl.weights()
    ws = torch.empty(q.moe_workspace_bytes(cfg, T, 1), dtype=torch.uint8, device="cuda")
    sel, _ = wl.zipf_gumbel_scores(w.seed, T, w.n_experts, 1.1)
    sd = torch.from_numpy(np.ascontiguousarray(sel)).cuda()
    xs = [torch.from_numpy(wl.tokens_x(w.seed + 200 + i, T, w.hidden)).cuda() for i in range(2)]
    xin = xs[0].clone()
    y = torch.empty_like(xin)
    idx = torch.empty((T, w.top_k), dtype=torch.int32, device="cuda")
    wt = torch.empty((T, w.top_k), dtype=torch.float32, device="cuda")

    def run(s):
        q.moe_layer_forward(cfg, lw, T, xin, y, ws, sel_bias=sd, idx_out=idx, w_out=wt, stream=s)

    graph_vs_eager("prefill", run, xin, xs, [y, idx, wt])
    q.moe_device_status(ws)


def test_qkv_graph_replays():
    H, rows, T = 4096, (4096, 512, 512), 3
    rng = np.random.default_rng(5)
    cfg = q.QkvConfig.make(H, *rows, bits=4, flags=q.MOE_F_RMSNORM)
    R = sum(rows)
    codes = rng.integers(0, 16, size=(R, H), dtype=np.uint8)
    sc = wl.bf16_bits_from_f32(np.abs(rng.normal(0, 0.02, (R, H // 64))).astype(np.float32))
    bi = wl.bf16_bits_from_f32(rng.normal(0, 0.01, (R, H // 64)).astype(np.float32))
    packed = torch.empty(q.moe_qkv_packed_bytes(cfg), dtype=torch.uint8, device="cuda")
    pws = torch.empty(1024, dtype=torch.uint8, device="cuda")
    q.moe_qkv_pack(cfg, torch.from_numpy(codes).cuda(), torch.from_numpy(sc.view(np.int16)).cuda(),
                   torch.from_numpy(bi.view(np.int16)).cuda(), packed, pws)
    q.moe_device_status(pws)
    gamma = torch.from_numpy((1.0 + 0.1 * rng.normal(size=H)).astype(np.float32)).cuda()
    xs = [torch.from_numpy(wl.tokens_x(300 + i, T, H)).cuda() for i in range(2)]
    xin = xs[0].clone()
    outs = [torch.empty((T, r), dtype=torch.float32, device="cuda") for r in rows]

    def run(s):
        q.moe_qkv_forward(cfg, packed, T, xin, *outs, gamma=gamma, stream=s)

    graph_vs_eager("qkv", run, xin, xs, outs)


def test_streamed_stack_graph_replays():
    w = wl.WorkloadConfig(name="small-streamed", hidden=512, inter=128, n_experts=16, top_k=4, n_shared=1,
                          n_layers=3, n_tokens=8, temporal_p=0.27)
    L, T, K, C = w.n_layers, w.n_tokens, w.top_k, 6
    cfg = config_for(w)
    dls = [DeviceLayer(w, l) for l in range(L)]
    pins, lws = [], []
    for d in dls:
        h = torch.empty(d.experts.numel(), dtype=torch.uint8, pin_memory=True)
        h.copy_(d.experts)
        pins.append(h)
        lws.append(q.layer_weights(h, d.shared, d.router))
    torch.cuda.synchronize()
    cache = torch.empty(L * C * q.moe_packed_expert_bytes(cfg), dtype=torch.uint8, device="cuda")
    ws = torch.empty(q.moe_workspace_bytes(cfg, T, L), dtype=torch.uint8, device="cuda")
    mask = torch.from_numpy(wl.boost_mask(w.seed + 7, T, L, K, 0.27)).cuda()
    xs = [torch.from_numpy(wl.tokens_x(w.seed + 400 + i, T, w.hidden)).cuda() for i in range(2)]
    xin = xs[0].clone()
    y = torch.empty_like(xin)
    idx = torch.empty((T, L, K), dtype=torch.int32, device="cuda")
    hit = torch.empty((T, L, K), dtype=torch.uint8, device="cuda")

    def run(s):
        q.moe_stack_decode_streamed(cfg, lws, T, xin, y, ws, cache, C, boost_mask=mask, idx_trace=idx,
                                    hit_trace=hit, stream=s)

    graph_vs_eager("streamed stack", run, xin, xs, [y, idx, hit])
    q.moe_device_status(ws)
    del pins
