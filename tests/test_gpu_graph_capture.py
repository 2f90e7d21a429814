"""The resident stack entry points captured into a HIP graph (torch.cuda.CUDAGraph)
and replayed: every replay, with eager work and a synchronisation between
replays, gives the eager call's outputs bit for bit, including after the input
buffer is rewritten between replays."""
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
