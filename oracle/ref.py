"""Oracle for the MoE FFN step with group-affine quantized experts (fp64, CPU).

TEST INFRASTRUCTURE: imported only by tests, the smoke check and the
benchmark's CPU-baseline leg. Shares no code with the HIP path.

Steps, in the order the flash-moe page runs them for one token and one layer
("Flash-MoE - Chạy mô hình 397 tỷ tham số trên laptop", vi.news.hada.io,
sections "Kiến trúc mô hình", "Kernel dequant tối ưu FMA", "Metal Compute
Shaders", "Deferred GPU Expert Compute"):

1. RMSNorm of the residual stream (optional: the tiny workload has none).
2. Router logits, a plain mat-vec with float32 router weights.
3. Top-K selection (the temporal tier first, then score, then lower index);
   softmax over all logits and renormalisation over the selected K.
4. Each selected expert and the shared expert: dequant mat-vec for gate and up,
   SwiGLU (silu on gate), dequant mat-vec for down.
5. Weighted combine plus the shared expert plus the residual. Optionally each
   shared expert is scaled by a gate, sigmoid(g_s . x_n) (the "gate" of the page's
   combine kernel, read as the shared-expert gate of this model family).

Prefill (one layer, T tokens) adds the bf16 rounding points of a bf16 GEMM:
x_b = bf16(x); x_n = RMSNorm(x_b); router from the unrounded x_n; expert input
bf16(x_n); weights bf16(deq); h bf16(silu(g)*u); y = x_b + sum w o + o_shared.

Pins (see tests/test_oracle_*.py): integer-exact mat-vec (scale 1, bias 0),
the bias-only closed form, one-hot column read-out, closed-form RMSNorm,
softmax weights summing to 1, brute-force sort for selection, one-hot routing
against a numpy float64 dense expert, zero experts giving the identity through
a stack, the bf16-free prefill reducing to the decode oracle, and the
independent pure-Python brute force (``oracle/brute.py``) on tiny shapes for the
single layer, a per-element RMSNorm weight, the multi-layer stack with the
temporal tier (layer chaining included) and the prefill with every rounding
point (input off the bf16 grid). No function is parity unpinned.
"""
import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qmoe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libqmoe_oracle.so")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_F = ctypes.POINTER(ctypes.c_float)
_U8 = ctypes.POINTER(ctypes.c_uint8)
_U16 = ctypes.POINTER(ctypes.c_uint16)
_I = ctypes.POINTER(ctypes.c_int)


def build(force=False):
    """Compile the oracle with gcc (no fusion, no reordering)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
                               "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB_PATH)
        L.orc_round_bf16.restype = ctypes.c_double
        L.orc_round_bf16.argtypes = [ctypes.c_double]
        L.orc_rmsnorm.argtypes = [ctypes.c_int, _D, _F, ctypes.c_double, _D]
        L.orc_router.argtypes = [ctypes.c_int, ctypes.c_int, _F, _D, _D]
        L.orc_select.restype = ctypes.c_int
        L.orc_select.argtypes = [ctypes.c_int, ctypes.c_int, _D, _D, ctypes.c_int, _I, ctypes.c_int,
                                 _I, _D, _D]
        L.orc_matvec.argtypes = [ctypes.c_int, ctypes.c_int, _U8, _U16, _U16, _D, ctypes.c_int, _D]
        L.orc_expert.argtypes = [ctypes.c_int, ctypes.c_int] + [_U8, _U16, _U16] * 3 + \
            [_D, ctypes.c_int, _D, _D]
        L.orc_combine.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _D, ctypes.c_int, _D, _D, _D, _D]
        _lib = L
    return _lib


def _p(a, t):
    return a.ctypes.data_as(t)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def round_bf16(v):
    f = lib().orc_round_bf16
    return np.vectorize(lambda z: f(float(z)), otypes=[np.float64])(np.asarray(v, dtype=np.float64))


def rmsnorm(x, gamma=None, eps=1e-6):
    x = _c(x, np.float64)
    out = np.empty_like(x)
    g = _c(gamma, np.float32) if gamma is not None else None
    lib().orc_rmsnorm(x.size, _p(x, _D), _p(g, _F) if g is not None else None, eps, _p(out, _D))
    return out


def router(W, xn):
    W = _c(W, np.float32)
    xn = _c(xn, np.float64)
    out = np.empty(W.shape[0], dtype=np.float64)
    lib().orc_router(W.shape[0], W.shape[1], _p(W, _F), _p(xn, _D), _p(out, _D))
    return out


def select(logits, K, sel=None, by_sel=False, boosted=()):
    """Returns (idx[K] in key order, w[K], gap)."""
    logits = _c(logits, np.float64)
    E = logits.size
    s = _c(sel, np.float64) if sel is not None else None
    b = _c(list(boosted) if len(boosted) else [0], np.int32)
    idx = np.empty(K, dtype=np.int32)
    w = np.empty(K, dtype=np.float64)
    gap = np.empty(1, dtype=np.float64)
    rc = lib().orc_select(E, K, _p(logits, _D), _p(s, _D) if s is not None else None, int(by_sel),
                          _p(b, _I), len(boosted), _p(idx, _I), _p(w, _D), _p(gap, _D))
    if rc != 0:
        raise ValueError("orc_select: bad arguments")
    return idx, w, float(gap[0])


def weights_for(logits, idx):
    """Renormalised softmax weights of a given selected set (used when the
    oracle follows a set chosen elsewhere at a near-tie)."""
    logits = np.asarray(logits, dtype=np.float64)
    m = logits.max()
    p = np.exp(logits - m) / np.exp(logits - m).sum()
    ps = p[list(idx)].sum()
    return np.array([p[i] / ps for i in idx])


def matvec(q, s, b, x, round_w_bf16=False):
    q, s, b = _c(q, np.uint8), _c(s, np.uint16), _c(b, np.uint16)
    x = _c(x, np.float64)
    R, C = q.shape
    y = np.empty(R, dtype=np.float64)
    lib().orc_matvec(R, C, _p(q, _U8), _p(s, _U16), _p(b, _U16), _p(x, _D), int(round_w_bf16), _p(y, _D))
    return y


def expert(canon, x, bf16_points=False, return_h=False):
    """canon = (codes[3], scales[3], biases[3]) in canonical form."""
    cs, ss, bs = canon
    I, H = cs[0].shape
    arrs = []
    for m in range(3):
        arrs += [_c(cs[m], np.uint8), _c(ss[m], np.uint16), _c(bs[m], np.uint16)]
    ptrs = []
    for i, a in enumerate(arrs):
        ptrs.append(_p(a, _U8 if i % 3 == 0 else _U16))
    x = _c(x, np.float64)
    o = np.empty(H, dtype=np.float64)
    h = np.empty(I, dtype=np.float64)
    lib().orc_expert(H, I, *ptrs, _p(x, _D), int(bf16_points), _p(o, _D), _p(h, _D))
    return (o, h) if return_h else o


def sigmoid(z):
    """Logistic function in fp64 (the form that cannot overflow)."""
    if z >= 0:
        return 1.0 / (1.0 + math.exp(-z))
    e = math.exp(z)
    return e / (1.0 + e)


def shared_gates(G, xn):
    """Shared-expert gate factors sigmoid(G[s] . x_n), one per shared expert. The page
    ("Flash-MoE", section "Metal Compute Shaders") lists a gate in its combine
    kernel without defining it; the reading here is the shared-expert gate of this
    model family: a float32 vector per shared expert, the dot product accumulated
    like the router's (fp64, index order)."""
    return np.array([sigmoid(float(z)) for z in router(np.asarray(G, dtype=np.float32), xn)])


def combine(x, w, o_routed, o_shared, residual=True, gates=None):
    x = _c(x, np.float64)
    H = x.size
    o = _c(np.concatenate([np.reshape(o_routed, (-1, H)), np.reshape(o_shared, (-1, H))]), np.float64)
    w = _c(w, np.float64)
    y = np.empty(H, dtype=np.float64)
    n_r = np.reshape(o_routed, (-1, H)).shape[0]
    n_s = np.reshape(o_shared, (-1, H)).shape[0]
    c = None if gates is None else _c(gates, np.float64)
    lib().orc_combine(H, n_r, n_s, _p(x, _D), int(residual), _p(w, _D), _p(o, _D),
                      None if c is None else _p(c, _D), _p(y, _D))
    return y


class LayerResult:
    def __init__(self, y, idx, w, gap, logits, xn):
        self.y, self.idx, self.w, self.gap, self.logits, self.xn = y, idx, w, gap, logits, xn


def layer_decode(x, router_W, get_expert, shared, K, rmsnorm_on=True, residual=True, gamma=None,
                 eps=1e-6, boosted=(), sel=None, by_sel=False, force_idx=None, shared_gate=None):
    """One decode layer for one token.

    get_expert(e) -> canonical expert e; shared: list of canonical shared experts.
    force_idx: a selected set to use instead of the oracle's own (near-tie follow).
    shared_gate: [S][H] float32 or None (shared experts added with weight 1).
    """
    x = np.asarray(x, dtype=np.float64)
    xn = rmsnorm(x, gamma, eps) if rmsnorm_on else x.copy()
    logits = router(router_W, xn)
    idx, w, gap = select(logits, K, sel=sel, by_sel=by_sel, boosted=boosted)
    if force_idx is not None:
        idx = np.asarray(force_idx, dtype=np.int32)
        w = weights_for(logits, idx)
    o_r = np.stack([expert(get_expert(int(e)), xn) for e in idx])
    o_s = np.stack([expert(c, xn) for c in shared]) if shared else np.zeros((0, x.size))
    gates = shared_gates(shared_gate, xn) if (shared_gate is not None and shared) else None
    y = combine(x, w, o_r, o_s, residual, gates=gates)
    return LayerResult(y, idx, w, gap, logits, xn)


def prefill_token(x, router_W, get_expert, shared, K, sel, gamma=None, eps=1e-6, by_sel=True,
                  boosted=(), rmsnorm_on=True, residual=True, force_idx=None, shared_gate=None):
    """One token of the batched prefill with the bf16 rounding points (the input,
    the expert input, every dequantised weight and the SwiGLU output are rounded
    to bf16; the router sees the unrounded normalised input). Selection uses
    ``sel`` alone by default (Gumbel-top-k scores); by_sel=False ranks by
    logit + sel instead. force_idx: a set chosen elsewhere at a near-tie."""
    xb = np.array([float(v) for v in np.asarray(x, dtype=np.float32)], dtype=np.float64)
    xb = round_bf16(xb)
    xn = rmsnorm(xb, gamma, eps) if rmsnorm_on else xb.copy()
    logits = router(router_W, xn)
    idx, w, gap = select(logits, K, sel=sel, by_sel=by_sel, boosted=boosted)
    if force_idx is not None:
        idx = np.asarray(force_idx, dtype=np.int32)
        w = weights_for(logits, idx)
    a = round_bf16(xn)
    o_r = np.stack([expert(get_expert(int(e)), a, bf16_points=True) for e in idx])
    o_s = np.stack([expert(c, a, bf16_points=True) for c in shared]) if shared else np.zeros((0, xb.size))
    # the gate sees the unrounded x_n, as the router does
    gates = shared_gates(shared_gate, xn) if (shared_gate is not None and shared) else None
    y = combine(xb, w, o_r, o_s, residual=residual, gates=gates)
    return LayerResult(y, idx, w, gap, logits, xn)


NEAR_TIE = 1e-5


def stack_decode(x_tokens, n_layers, router_of, expert_of, shared_of, K, boost=None,
                 rmsnorm_on=True, residual=True, eps=1e-6, follow=None, tokens=None, shared_gate_of=None,
                 gamma_of=None, on_layer=None):
    """Decode stack: for each token t in order, for each layer l, x <- layer(x).
    Attention is the identity between MoE blocks.

    boost[t][l][j] = 1 boosts slot j of token t-1's selected set at layer l, with
    the set sorted by expert index (the temporal-correlation tier).
    follow(t, l, idx_oracle, gap) -> set to use (or None to keep the oracle's);
    it lets a caller follow another implementation's set at a near-tie.
    tokens: subset of token indices to evaluate (teacher-forced: token t's
    boosted set then needs ``prev_sets``, supplied through ``follow`` history).
    gamma_of(l): layer l's RMSNorm weight [H] float32, or None (all ones).
    on_layer(t, l, x_in, result): called after every layer (inspection only).
    Returns (y [T][H] float64, idx [T][L][K] sorted by expert, gaps [T][L])."""
    T = len(x_tokens)
    H = np.asarray(x_tokens[0]).size
    ys = np.zeros((T, H))
    sets = np.zeros((T, n_layers, K), dtype=np.int32)
    gaps = np.zeros((T, n_layers))
    prev = None
    for t in (range(T) if tokens is None else tokens):
        x = np.asarray(x_tokens[t], dtype=np.float64)
        for l in range(n_layers):
            boosted = ()
            if boost is not None and t > 0 and prev is not None:
                ps = np.sort(prev[l])
                boosted = tuple(int(ps[j]) for j in range(K) if boost[t][l][j])
            sg = None if shared_gate_of is None else shared_gate_of(l)
            gm = None if gamma_of is None else gamma_of(l)
            r = layer_decode(x, router_of(l), lambda e, l=l: expert_of(l, e), shared_of(l), K,
                             rmsnorm_on=rmsnorm_on, residual=residual, eps=eps, boosted=boosted,
                             shared_gate=sg, gamma=gm)
            if follow is not None:
                f = follow(t, l, r.idx, r.gap)
                if f is not None and set(int(v) for v in f) != set(int(v) for v in r.idx):
                    r = layer_decode(x, router_of(l), lambda e, l=l: expert_of(l, e), shared_of(l), K,
                                     rmsnorm_on=rmsnorm_on, residual=residual, eps=eps,
                                     boosted=boosted, force_idx=f, shared_gate=sg, gamma=gm)
            sets[t, l] = np.sort(r.idx)
            gaps[t, l] = r.gap
            if on_layer is not None:
                on_layer(t, l, x, r)
            x = r.y
        ys[t] = x
        prev = sets[t]
    return ys, sets, gaps


def silu(z):
    return z / (1.0 + math.exp(-z)) if z > -700 else 0.0 * z


def qkv(mats, x, gamma=None, norm=False, eps=1e-6):
    """Fused Q/K/V projection: three group-affine dequant mat-vecs of one input
    ("Autoresearch impulsa a Qwen3.5-397B ...", section "Optimizaciones Efectivas":
    the fused Q/K/V kernel reads the input once instead of three times; the mat-vec
    itself is that of "Flash-MoE", section "Metal Compute Shaders").
    mats: [(codes, scales, biases)] for Wq, Wk, Wv, each [R][H]. The input is
    x_n = RMSNorm(x) * gamma with norm, else x * gamma (gamma None: 1).
    Returns (q, k, v) in float64."""
    x = np.asarray(x, dtype=np.float64)
    if norm:
        xn = rmsnorm(x, gamma, eps)
    elif gamma is not None:
        xn = x * np.asarray(gamma, dtype=np.float32).astype(np.float64)
    else:
        xn = x
    return tuple(matvec(c, sc, bi, xn) for c, sc, bi in mats)


def expert_cache_hits(sets, C):
    """Host-memory tier with an HBM cache of C experts for one layer (the pages stream
    experts from SSD and find about 27% of a token's experts repeating from the token
    before: "Flash-MoE", section "SSD Expert Streaming"; "Autoresearch impulsa a
    Qwen3.5-397B ...", section "Optimizaciones Efectivas"). The cache policy is the
    library's own, stated with its streamed decode entry point:

    the cache has C numbered slots, each empty or holding one expert with the token
    at which it was last used. For token t with selected set S_t, every expert of S_t
    already held by a slot is a hit, and that slot's last use becomes t. The other
    experts of S_t, in increasing index, each go into the slot chosen as follows:
    among slots whose last use is not t, an empty one if any (lowest number first),
    else the one used least recently (lowest number on equal last use); its last use
    becomes t.

    sets: sequence over tokens of the selected experts (any order).
    Returns a list over tokens of the set of experts that were hits."""
    slots = [None] * C  # None or [expert, last_use]
    out = []
    for t, sel in enumerate(sets):
        sel = sorted(set(int(e) for e in sel))
        assert len(sel) <= C
        hits = set()
        for e in sel:
            for sl in slots:
                if sl is not None and sl[0] == e:
                    sl[1] = t
                    hits.add(e)
        for e in sel:
            if e in hits:
                continue
            free = [i for i in range(C) if slots[i] is None]
            if free:
                victim = free[0]
            else:
                cands = [i for i in range(C) if slots[i][1] != t]
                victim = min(cands, key=lambda i: (slots[i][1], i))
            slots[victim] = [e, t]
        out.append(hits)
    return out
