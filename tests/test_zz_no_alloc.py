"""moe_stack_decode_noalloc (the library's fixed scratch array instead of a caller
workspace) against moe_stack_decode on the same inputs, through the C ABI: two
calls in a row, the second smaller, each bit-identical to the workspace call
(both run the same kernels), with the device error word copied out as 0."""
import numpy as np
import pytest

import quantized_expert_mat_amd as q
import workload as wl
from workload.device_layer import DeviceLayer, config_for

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def run_both(w, L, T, seed_shift):
    cfg = config_for(w)
    K = w.top_k
    dls = [DeviceLayer(w, l, chunk=8) for l in range(L)]
    lws = [d.weights() for d in dls]
    x = torch.from_numpy(wl.tokens_x(w.seed + 1000 + seed_shift, T, w.hidden)).cuda()
    mask = torch.from_numpy(wl.boost_mask(w.seed + 7 + seed_shift, T, L, K, w.temporal_p or 0.27)).cuda()
    ws = torch.empty(q.moe_workspace_bytes(cfg, T, L), dtype=torch.uint8, device="cuda")
    outs = []
    for noalloc in (False, True):
        y = torch.full((T, w.hidden), float("nan"), dtype=torch.float32, device="cuda")
        idx = torch.full((T, L, K), -1, dtype=torch.int32, device="cuda")
        wt = torch.full((T, L, K), float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            err = torch.full((1,), 0x7FFFFFFF, dtype=torch.int32, device="cuda")
            q.moe_stack_decode_noalloc(cfg, lws, T, x, y, boost_mask=mask, idx_trace=idx, w_trace=wt,
                                       dev_err=err)
            torch.cuda.synchronize()
            assert int(err.item()) == 0
        else:
            q.moe_stack_decode(cfg, lws, T, x, y, ws, boost_mask=mask, idx_trace=idx, w_trace=wt)
            q.moe_device_status(ws)
        outs.append((y.cpu().numpy(), idx.cpu().numpy(), wt.cpu().numpy()))
    (y0, i0, w0), (y1, i1, w1) = outs
    assert np.isfinite(y1).all()
    assert np.array_equal(i0, i1)
    assert np.array_equal(w0.view(np.uint32), w1.view(np.uint32))
    assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32))


def test_noalloc_matches_workspace_call_twice_second_smaller():
    # the launch the benchmark times (hidden 4096, I 1024, 512 experts, top-4 +
    # shared), then a smaller general shape on the same scratch array
    print("noalloc: full shape L=3 T=4", flush=True)
    run_both(wl.STACK60_4BIT.replace(n_layers=3, n_tokens=4), 3, 4, 0)
    print("noalloc: small shape L=2 T=3", flush=True)
    small = wl.WorkloadConfig(name="small", hidden=512, inter=128, n_experts=24, top_k=4, n_shared=1,
                              n_layers=2, n_tokens=3)
    run_both(small, 2, 3, 1)


def test_noalloc_layer_table_past_the_launch_arguments():
    """70 layers: the first 64 layer-table entries travel in the launch arguments,
    the rest are written into the scratch array by a second kernel; the result is
    the workspace call's, bit for bit."""
    print("noalloc: 70 small layers, T=2", flush=True)
    w = wl.WorkloadConfig(name="small70", hidden=256, inter=128, n_experts=16, top_k=2, n_shared=1,
                          n_layers=70, n_tokens=2)
    run_both(w, 70, 2, 2)
