"""Shared helpers for the GPU tests: seeded workloads on the device (packed with
moe_pack_weights), the same experts in canonical form on the host for the
oracle, and the parity bar."""
import numpy as np

import quantized_expert_mat_amd as q
import workload as wl
from workload import device as wdev

NEAR_TIE = 1e-5  # oracle selection margin under which a different set is tie-ambiguous


def config_for(w: wl.WorkloadConfig, extra_flags=0):
    flags = (q.MOE_F_RMSNORM if w.rmsnorm else 0) | (q.MOE_F_RESIDUAL if w.residual else 0) | extra_flags
    return q.Config.make(w.hidden, w.inter, w.n_experts, w.top_k, w.n_shared, w.bits, flags=flags)


class DeviceLayer:
    """One layer of packed experts, shared experts and router weights on the GPU."""

    def __init__(self, w: wl.WorkloadConfig, layer: int, device="cuda", chunk=32, ws=None, gated=False):
        import torch
        self.w, self.layer = w, layer
        self.sgate = None
        if gated and w.n_shared:
            self.sgate = torch.from_numpy(wl.shared_gate_weights(w.seed, layer, w.n_shared, w.hidden)).to(device)
        self.cfg = config_for(w)
        spec = w.expert_spec()
        nb = q.moe_packed_expert_bytes(self.cfg)
        assert nb > 0, q.moe_last_error()
        self.expert_bytes = nb
        E, S, H, I = w.n_experts, w.n_shared, w.hidden, w.inter
        self.experts = torch.empty(E * nb, dtype=torch.uint8, device=device)
        self.shared = torch.empty(max(S, 1) * nb, dtype=torch.uint8, device=device)
        self.router = torch.empty((E, H), dtype=torch.float32, device=device)
        own_ws = ws is None
        if own_ws:
            ws = torch.empty(q.moe_workspace_bytes(self.cfg, 1, 1), dtype=torch.uint8, device=device)
        n = min(chunk, E + S)
        codes = torch.empty((n, 3, H * I), dtype=torch.uint8, device=device)
        scales = torch.empty((n, 3, H * I // 64), dtype=torch.int16, device=device)
        biases = torch.empty((n, 3, H * I // 64), dtype=torch.int16, device=device)
        ids = list(range(E + S))  # shared expert s uses generator id E + s
        for i0 in range(0, E + S, n):
            part = ids[i0:i0 + n]
            keep = wdev.experts_canonical(spec, w.seed, layer, part, codes, scales, biases)
            # split the chunk into routed and shared destinations
            r = [e for e in part if e < E]
            if r:
                dst = self.experts[r[0] * nb:(r[-1] + 1) * nb]
                q.moe_pack_weights(self.cfg, len(r), codes, scales, biases, dst, ws)
            sh = [e for e in part if e >= E]
            if sh:
                o = len(r)
                dst = self.shared[(sh[0] - E) * nb:(sh[-1] - E + 1) * nb]
                q.moe_pack_weights(self.cfg, len(sh), codes[o:], scales[o:], biases[o:], dst, ws)
            torch.cuda.current_stream().synchronize()
            del keep
        wdev.router(w.seed, layer, E, H, self.router, sigma=w.sigma_router)
        torch.cuda.current_stream().synchronize()
        q.moe_device_status(ws)

    def weights(self):
        return q.layer_weights(self.experts, self.shared if self.w.n_shared else None, self.router,
                               shared_gate=self.sgate)


class HostLayer:
    """The same layer in canonical form on the host (experts generated on demand)."""

    def __init__(self, w: wl.WorkloadConfig, layer: int):
        self.w, self.layer = w, layer
        self.spec = w.expert_spec()
        self._cache = {}
        self.router = wl.router_weights(w.seed, layer, w.n_experts, w.hidden, w.sigma_router)

    def expert(self, e):
        if e not in self._cache:
            if len(self._cache) > 64:
                self._cache.clear()
            self._cache[e] = wl.expert_canonical(self.spec, self.w.seed, self.layer, e)
        return self._cache[e]

    def shared(self):
        return [self.expert(self.w.n_experts + s) for s in range(self.w.n_shared)]

    def shared_gate(self):
        return wl.shared_gate_weights(self.w.seed, self.layer, self.w.n_shared, self.w.hidden)


class DeviceCanonicalLayer:
    """Canonical experts of one layer for the oracle, produced with the device
    generator (same bits as the host generator) and copied to the host: fast
    enough to regenerate the experts a 60-layer replay touches. Time spent
    generating is accumulated in ``gen_seconds``."""

    def __init__(self, w: wl.WorkloadConfig, layer: int, router=None):
        import time
        import torch
        self.w, self.layer = w, layer
        self.spec = w.expert_spec()
        self._cache = {}
        self.gen_seconds = 0.0
        t0 = time.perf_counter()
        if router is not None:
            self.router = router
        else:
            r = torch.empty((w.n_experts, w.hidden), dtype=torch.float32, device="cuda")
            wdev.router(w.seed, layer, w.n_experts, w.hidden, r, sigma=w.sigma_router)
            self.router = r.cpu().numpy()
        self.gen_seconds += time.perf_counter() - t0

    def expert(self, e):
        import time
        import torch
        if e in self._cache:
            return self._cache[e]
        t0 = time.perf_counter()
        H, I = self.w.hidden, self.w.inter
        codes = torch.empty((1, 3, H * I), dtype=torch.uint8, device="cuda")
        sc = torch.empty((1, 3, H * I // 64), dtype=torch.int16, device="cuda")
        bi = torch.empty((1, 3, H * I // 64), dtype=torch.int16, device="cuda")
        keep = wdev.experts_canonical(self.spec, self.w.seed, self.layer, [e], codes, sc, bi)
        torch.cuda.synchronize()
        c, s_, b = codes.cpu().numpy()[0], sc.cpu().numpy()[0].view(np.uint16), bi.cpu().numpy()[0].view(np.uint16)
        del keep
        shapes = [(I, H), (I, H), (H, I)]
        canon = ([c[m].reshape(shapes[m]) for m in range(3)],
                 [s_[m].reshape(shapes[m][0], -1) for m in range(3)],
                 [b[m].reshape(shapes[m][0], -1) for m in range(3)])
        if len(self._cache) > self.w.n_shared + self.w.top_k:
            # keep the shared experts; routed ones are reused only within one token
            self._cache = {k: v for k, v in self._cache.items() if k >= self.w.n_experts}
        self._cache[e] = canon
        self.gen_seconds += time.perf_counter() - t0
        return canon

    def shared(self):
        return [self.expert(self.w.n_experts + s) for s in range(self.w.n_shared)]


def parity(y, y_ref, what=""):
    """The bar for float32 outputs: max|err| <= 2e-3 max|y_ref| and rel-L2 <= 1e-4."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    err = np.abs(y - y_ref).max()
    scale = np.abs(y_ref).max()
    rel = np.linalg.norm(y - y_ref) / max(np.linalg.norm(y_ref), 1e-300)
    assert err <= 2e-3 * scale, f"{what}: max|err| {err:.3e} > 2e-3 * {scale:.3e}"
    assert rel <= 1e-4, f"{what}: rel-L2 {rel:.3e} > 1e-4"
    return err / max(scale, 1e-300), rel


def same_set(a, b):
    return sorted(int(v) for v in a) == sorted(int(v) for v in b)
