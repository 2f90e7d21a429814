"""Counter-based generator for synthetic MoE weights and inputs (host side).

Definition (implemented identically, bit for bit, in ``gen_device.hip``):

* ``mix64`` is the SplitMix64 output function (Steele, Lea and Flood, "Fast
  splittable pseudorandom number generators", OOPSLA 2014; constants as in
  Vigna's public-domain splitmix64.c).
* A stream key folds integer fields into a 64-bit key:
  ``k = KEY0; for f in fields: k = mix64(k ^ (f + GOLDEN))``.
* Word ``i`` of a stream is ``mix64(key + (i + 1) * GOLDEN)`` (mod 2**64), i.e.
  the i-th output of a SplitMix64 generator whose state starts at ``key``.
* ``b``-bit codes (b in {2, 3, 4}): element ``k`` of a matrix (row-major index) is
  bits ``[b*(k % (64//b)), +b)`` of word ``k // (64//b)``.
* Approximate standard normals (Irwin-Hall with 12 terms, a textbook
  approximation whose variance is exactly 1 up to discretisation): element
  ``i`` sums the twelve 16-bit halves of words ``3i, 3i+1, 3i+2`` and returns
  ``(sum - 393210) / 65536``. This is integer-exact, so device and host agree.
* A real value ``sigma * n`` is formed in float64 (one correctly rounded
  product), rounded to float32 (round-to-nearest-even) and, for bf16 tensors,
  rounded again float32 -> bf16 (round-to-nearest-even on the bit pattern).
* Bernoulli(p): word < floor(p * 2**64).
* Zero-mean experts (a conditioned variant of the workload): the bias of a
  (row, group) is ``-m * s + sigma_bias * n`` with ``m = (2**bits - 1) / 2`` the
  code midpoint, ``s`` the group's bf16 scale (as a float64) and ``n`` the
  group's bias normal; the two products and the sum are float64 operations, each
  rounded once (``m * s`` is exact), then rounded to float32 and to bf16. The
  dequantised weights q*s + b then have mean zero, so the residual stream of a
  deep stack does not drift into one common direction.

The distributions stand in for the workload description of the MoE layer at
the shapes the flash-moe page gives (512 experts, top-4, hidden 4096, group
size 64; "Kiến trúc mô hình" section of "Flash-MoE - Chạy mô hình 397 tỷ tham
số trên laptop", vi.news.hada.io).
"""
import numpy as np

__all__ = [
    "GOLDEN", "KEY0", "KIND_CODES", "KIND_SCALE", "KIND_BIAS", "KIND_ROUTER",
    "KIND_X", "KIND_BOOST", "KIND_GUMBEL", "KIND_RANK", "KIND_SGATE",
    "mix64", "stream_key", "words", "codes", "normals", "f32_from_normals",
    "bf16_bits_from_f32", "bf16_bits_to_f32", "bf16_from_normals",
    "ExpertSpec", "expert_canonical", "router_weights", "shared_gate_weights", "tokens_x",
    "boost_mask", "zipf_gumbel_scores", "WorkloadConfig", "WORKLOADS", "TINY_LAYER", "LAYER_H4096",
    "STACK60_4BIT", "STACK60_2BIT", "PREFILL1155", "STACK60_3BIT", "STACK60_4BIT_ZM",
    "zero_mean_bias_bits", "HostLayer",
]

M64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15
KEY0 = 0x243F6A8885A308D3
_C1 = np.uint64(0xBF58476D1CE4E5B9)
_C2 = np.uint64(0x94D049BB133111EB)

KIND_CODES, KIND_SCALE, KIND_BIAS, KIND_ROUTER = 1, 2, 3, 4
KIND_X, KIND_BOOST, KIND_GUMBEL, KIND_RANK = 5, 6, 7, 8
KIND_SGATE = 9


def mix64(z):
    """SplitMix64 output function on a uint64 array (wrapping arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _C1
        z = (z ^ (z >> np.uint64(27))) * _C2
        z = z ^ (z >> np.uint64(31))
    return z


def _mix64_int(z: int) -> int:
    z &= M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def stream_key(*fields) -> int:
    """Fold integer fields (seed, kind, layer, expert, sub) into a 64-bit key."""
    k = KEY0
    for f in fields:
        k = _mix64_int(k ^ ((int(f) + GOLDEN) & M64))
    return k


def words(key: int, start: int, count: int) -> np.ndarray:
    """Words ``start .. start+count-1`` of the stream with the given key."""
    idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        state = np.uint64(key) + idx * np.uint64(GOLDEN)
    return mix64(state)


def codes(key: int, n: int, bits: int) -> np.ndarray:
    """First ``n`` unsigned ``bits``-bit codes of a stream, one per uint8."""
    per = 64 // bits
    nw = (n + per - 1) // per
    w = words(key, 0, nw)
    shifts = (np.arange(per, dtype=np.uint64) * np.uint64(bits))
    c = (w[:, None] >> shifts[None, :]) & np.uint64((1 << bits) - 1)
    return c.reshape(-1)[:n].astype(np.uint8)


def normals(key: int, n: int) -> np.ndarray:
    """First ``n`` Irwin-Hall(12) approximate standard normals (float64, exact)."""
    w = words(key, 0, 3 * n).reshape(n, 3)
    s = np.zeros(n, dtype=np.int64)
    for j in range(3):
        for h in range(4):
            s += ((w[:, j] >> np.uint64(16 * h)) & np.uint64(0xFFFF)).astype(np.int64)
    return (s - 393210).astype(np.float64) / 65536.0


def f32_from_normals(n: np.ndarray, sigma: float, absolute: bool = False) -> np.ndarray:
    v = np.abs(n) if absolute else n
    return (np.float64(sigma) * v).astype(np.float32)


def bf16_bits_from_f32(f: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint32) << np.uint32(16)).view(np.float32)


def bf16_from_normals(n: np.ndarray, sigma: float, absolute: bool = False) -> np.ndarray:
    return bf16_bits_from_f32(f32_from_normals(n, sigma, absolute))


class ExpertSpec:
    """Shapes and value distributions of one expert (gate, up: [I][H]; down: [H][I])."""

    def __init__(self, hidden, inter, bits=4, group=64, sigma_scale=0.02, sigma_bias=0.01, zero_mean=False):
        self.hidden, self.inter, self.bits, self.group = hidden, inter, bits, group
        self.sigma_scale, self.sigma_bias = sigma_scale, sigma_bias
        self.zero_mean = zero_mean

    def shape(self, mat):
        return (self.inter, self.hidden) if mat < 2 else (self.hidden, self.inter)


def expert_canonical(spec: ExpertSpec, seed: int, layer: int, expert: int):
    """Canonical form of one expert: codes [3] uint8 arrays (rows, cols) one code per
    byte, scale/bias [3] uint16 (bf16 bits) arrays (rows, cols/group)."""
    cs, ss, bs = [], [], []
    for mat in range(3):
        r, c = spec.shape(mat)
        ng = r * (c // spec.group)
        cs.append(codes(stream_key(seed, KIND_CODES, layer, expert, mat), r * c, spec.bits).reshape(r, c))
        sc = bf16_from_normals(normals(stream_key(seed, KIND_SCALE, layer, expert, mat), ng),
                               spec.sigma_scale, absolute=True)
        nb = normals(stream_key(seed, KIND_BIAS, layer, expert, mat), ng)
        if spec.zero_mean:
            bi = zero_mean_bias_bits(sc, nb, spec.sigma_bias, spec.bits)
        else:
            bi = bf16_from_normals(nb, spec.sigma_bias)
        ss.append(sc.reshape(r, c // spec.group))
        bs.append(bi.reshape(r, c // spec.group))
    return cs, ss, bs


def zero_mean_bias_bits(scale_bits, n, sigma_bias, bits):
    """bf16 bias bits -m*s + sigma_bias*n (float64 ops, then float32, then bf16)."""
    m = np.float64(((1 << bits) - 1) / 2.0)
    s = bf16_bits_to_f32(scale_bits).astype(np.float64)
    v = (-m) * s + np.float64(sigma_bias) * np.asarray(n, dtype=np.float64)
    return bf16_bits_from_f32(v.astype(np.float32))


def router_weights(seed, layer, n_experts, hidden, sigma=0.02):
    n = normals(stream_key(seed, KIND_ROUTER, layer, 0, 0), n_experts * hidden)
    return f32_from_normals(n, sigma).reshape(n_experts, hidden)


def shared_gate_weights(seed, layer, n_shared, hidden, sigma=0.02):
    """Shared-expert gate vectors [n_shared][hidden] float32 ~ N(0, sigma)."""
    n = normals(stream_key(seed, KIND_SGATE, layer, 0, 0), n_shared * hidden)
    return f32_from_normals(n, sigma).reshape(n_shared, hidden)


def tokens_x(seed, n_tokens, hidden, first_token=0):
    """Activations x_t ~ N(0,1) (Irwin-Hall approximation, exact in float32)."""
    out = np.empty((n_tokens, hidden), dtype=np.float32)
    for t in range(n_tokens):
        out[t] = normals(stream_key(seed, KIND_X, 0, first_token + t, 0), hidden).astype(np.float32)
    return out


def boost_mask(seed, n_tokens, n_layers, top_k, p=0.27):
    """Temporal-correlation mask [T][L][K] (uint8): slot j of token t-1's selected set
    (sorted by expert index) is boosted at token t with probability p. Token 0 has
    no previous token, so its row is zero."""
    thr = np.uint64(int(p * 2.0 ** 64))
    out = np.zeros((n_tokens, n_layers, top_k), dtype=np.uint8)
    for t in range(1, n_tokens):
        w = words(stream_key(seed, KIND_BOOST, 0, t, 0), 0, n_layers * top_k)
        out[t] = (w < thr).reshape(n_layers, top_k)
    return out


def zipf_gumbel_scores(seed, n_tokens, n_experts, exponent=1.1):
    """Selection scores for Zipf-skewed routing by Gumbel-top-k: score[t,e] =
    -exponent*ln(rank_e) + G[t,e], with rank a seeded permutation of 1..E and G a
    standard Gumbel draw per (t, e). Taking the top-k scores samples k distinct
    experts with probability proportional to rank**-exponent (without
    replacement). Returns float32 [T][E] and the ranks."""
    rk = words(stream_key(seed, KIND_RANK, 0, 0, 0), 0, n_experts)
    rank = np.empty(n_experts, dtype=np.int64)
    rank[np.argsort(rk, kind="stable")] = np.arange(1, n_experts + 1)
    w = words(stream_key(seed, KIND_GUMBEL, 0, 0, 0), 0, n_tokens * n_experts)
    u = ((w >> np.uint64(11)).astype(np.float64) + 0.5) / float(1 << 53)
    g = -np.log(-np.log(u))
    s = -exponent * np.log(rank.astype(np.float64))[None, :] + g.reshape(n_tokens, n_experts)
    return s.astype(np.float32), rank


class WorkloadConfig:
    """One workload: shapes, distributions and the layer flags it runs with."""

    def __init__(self, name, hidden, inter, n_experts, top_k=4, n_shared=1, bits=4,
                 sigma_scale=0.02, sigma_bias=0.01, sigma_router=0.02, rmsnorm=True,
                 residual=True, n_layers=1, n_tokens=1, temporal_p=None, zipf=None, seed=0, zero_mean=False):
        self.__dict__.update(locals())
        del self.__dict__["self"]

    def expert_spec(self):
        return ExpertSpec(self.hidden, self.inter, self.bits, 64, self.sigma_scale, self.sigma_bias,
                          self.zero_mean)

    def replace(self, **kw):
        d = dict(self.__dict__)
        d.update(kw)
        return WorkloadConfig(**d)


# The five workloads: a tiny layer, one layer at the flash-moe shape, the 60-layer
# 4-bit decode stack with 27% temporal routing correlation, the same stack with
# 2-bit experts, and a 1155-token prefill through one layer with Zipf(1.1) routing.
TINY_LAYER = WorkloadConfig("tiny-layer", 1024, 256, 64, rmsnorm=False, residual=False)
LAYER_H4096 = WorkloadConfig("layer-h4096-e512", 4096, 1024, 512)
STACK60_4BIT = WorkloadConfig("stack60-4bit", 4096, 1024, 512, n_layers=60, n_tokens=256, temporal_p=0.27)
STACK60_2BIT = WorkloadConfig("stack60-2bit", 4096, 1024, 512, bits=2, sigma_scale=0.06, n_layers=60,
                              n_tokens=256, temporal_p=0.27)
PREFILL1155 = WorkloadConfig("prefill1155", 4096, 1024, 512, n_tokens=1155, zipf=1.1)
WORKLOADS = [TINY_LAYER, LAYER_H4096, STACK60_4BIT, STACK60_2BIT, PREFILL1155]

# The 60-layer decode stack with 3-bit experts: a synthetic group-affine stand-in
# for the 3-bit experts of the autoresearch page ("Optimizaciones Efectivas"),
# which it finds about 23% smaller than 4-bit ones.
STACK60_3BIT = WorkloadConfig("stack60-3bit", 4096, 1024, 512, bits=3, sigma_scale=0.04, n_layers=60,
                              n_tokens=256, temporal_p=0.27)

# The same stack with zero-mean experts (bias = -7.5 * scale + N(0, 0.01)): same
# shapes, codes, scales and bytes as stack60-4bit, but the residual stream keeps
# each token's identity through all 60 layers and every layer adds a visible
# contribution. With the stack60-4bit distributions (unsigned codes, positive
# scales, zero-mean bias) every weight has mean 7.5 * E[scale] > 0: the first layer
# pushes the residual stream into one common direction, the routing then no
# longer depends on the token, and later layers either add the same large
# vector or (gate pre-activations far below zero) nothing at all. The headline
# throughput is measured on stack60-4bit (the bytes moved are the same); parity at
# depth, the temporal tier statistics and the expert-cache hit rates use this one.
STACK60_4BIT_ZM = STACK60_4BIT.replace(name="stack60-4bit-zero-mean", zero_mean=True)


class HostLayer:
    """One layer in canonical form on the host (experts generated on demand)."""

    def __init__(self, w, layer):
        self.w, self.layer = w, layer
        self.spec = w.expert_spec()
        self._cache = {}
        self.router = router_weights(w.seed, layer, w.n_experts, w.hidden, w.sigma_router)

    def expert(self, e):
        if e not in self._cache:
            if len(self._cache) > 64:
                self._cache.clear()
            self._cache[e] = expert_canonical(self.spec, self.w.seed, self.layer, e)
        return self._cache[e]

    def shared(self):
        return [self.expert(self.w.n_experts + s) for s in range(self.w.n_shared)]

    def shared_gate(self):
        return shared_gate_weights(self.w.seed, self.layer, self.w.n_shared, self.w.hidden)
