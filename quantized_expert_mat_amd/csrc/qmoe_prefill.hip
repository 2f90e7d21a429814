// qmoe_prefill.hip -- batched prefill through one MoE layer: T tokens routed
// independently, grouped by expert, and contracted as an expert-grouped bf16 GEMM
// on the CDNA4 matrix cores (v_mfma_f32_16x16x32_bf16, float32 accumulation).
//
// What is computed is the same MoE FFN step as decode (router -> top-K experts plus
// the shared expert -> SwiGLU -> weighted combine + residual; flash-moe page,
// "Kiến trúc mô hình" and "Deferred GPU Expert Compute"), for many tokens at once:
// the batched-prefill regime that the flash-moe page mentions as an opportunity and
// that LOOM measures at 1155 prompt tokens (alessandroviola.dev, "Cosa hanno
// stabilito gli esperimenti"). The prefill defines its own rounding points: the
// input is rounded to bf16 (x_b), the expert input is bf16(RMSNorm(x_b)), every
// weight is bf16(q*s + b) rounded once from its exact float32 value (q*s is exact),
// and the SwiGLU output is rounded to bf16 before the down projection.
//
// Pipeline per pass of at most kChunkT tokens (all on one stream):
//   prep     one workgroup per token: x_b, RMSNorm, A = bf16(x_n), x_n (float32)
//   router   (only when the selection needs all logits) logits = x_n W^T, float32
//   select   one wave per token: top-K by (tier, score, lower index), softmax of the
//            selected router logits (computed here when selection is by sel_bias)
//   group    one workgroup: stable counting of (token, slot) pairs by expert via a
//            bitonic sort of (expert, pair) keys; per-expert row runs; m-tile table
//   gateup   grouped GEMM: rows of one expert x 64 intermediate columns per
//            workgroup, gate and up fused, h = bf16(silu(g) * u)
//   down     grouped GEMM: rows x 128 output columns per workgroup -> float32 rows
//   combine  y = x_b + sum_k w_k o_k + sum_s o_s, fixed order per token
//
// Weights are dequantised in registers by the lane that feeds them to the MFMA (no
// LDS round trip for B); activations are staged through LDS per 128-wide reduction
// chunk. Inside a chunk the reduction index is permuted identically for the A and B
// operands (the MFMA sums over it, so any common permutation is exact): lane group
// kk = lane/16 covers chunk positions [32kk, 32kk+32) and MFMA step i the octet
// [32kk+8i, 32kk+8i+8), which is exactly one 16-byte code chunk of the packed layout
// for 4-bit codes (half a slot for 2-bit codes).
#include <string>

#include "qmoe_internal.h"

namespace qmoe {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunkT = 2048;      // tokens per pass (bounds the workspace)
constexpr int kBM = 128;           // rows (token-expert pairs) per m-tile
constexpr int kMT = kBM / 16;      // 16-row MFMA subtiles per m-tile
constexpr int kKC = 128;           // reduction chunk: two 64-groups
constexpr int kArow = kKC * 2 + 16;  // LDS bytes per staged activation row (+pad)
constexpr int kGuCols = 64;        // intermediate columns per gate/up workgroup
constexpr int kDnCols = 128;       // output columns per down workgroup
constexpr int kSortMax = 16384;    // pairs per pass (kChunkT * kMaxK)
constexpr int kPairBits = 14;      // pair index bits in a sort key

// ---------------------------------------------------------------------------
// Workspace layout of one prefill pass
// ---------------------------------------------------------------------------
struct PLayout {
  int Tc, rows, max_tiles;
  size_t err, a, xn, logits, idx, wts, pos, rowtok, tiles, hbuf, obuf, total;
};

PLayout p_layout(const moe_config& c, int T) {
  PLayout p;
  p.Tc = T < 1 ? 1 : (T < kChunkT ? T : kChunkT);
  const int TK = p.Tc * c.top_k;
  p.rows = TK + c.n_shared * p.Tc;
  const int nz = c.n_experts < TK ? c.n_experts : TK;
  p.max_tiles = nz + (TK + kBM - 1) / kBM + c.n_shared * ((p.Tc + kBM - 1) / kBM);
  size_t o = 0;
  p.err = o; o += 256;
  p.a = o; o = align256(o + (size_t)p.Tc * c.hidden * 2);
  p.xn = o; o = align256(o + (size_t)p.Tc * c.hidden * 4);
  p.logits = o; o = align256(o + (size_t)p.Tc * c.n_experts * 4);
  p.idx = o; o = align256(o + (size_t)TK * 4);
  p.wts = o; o = align256(o + (size_t)TK * 4);
  p.pos = o; o = align256(o + (size_t)TK * 4);
  p.rowtok = o; o = align256(o + (size_t)p.rows * 4);
  p.tiles = o; o = align256(o + 16 * (size_t)(p.max_tiles + 1));
  p.hbuf = o; o = align256(o + (size_t)p.rows * c.inter * 2);
  p.obuf = o; o = align256(o + (size_t)p.rows * c.hidden * 4);
  p.total = o;
  return p;
}

// Arguments shared by the prefill kernels (one pass).
struct PArgs {
  int H, I, E, K, S, flags, n;  // n: tokens in this pass
  float eps;
  Geo geo;
  const float* x;         // [n][H] input rows of this pass
  float* y;               // [n][H]
  const float* router;    // [E][H]
  const float* gamma;     // [H] or null
  const float* sel_bias;  // [n][E] or null
  const int* boosted;     // [n][K] or null
  int* idx_out;           // [n][K] or null
  float* w_out;           // [n][K] or null
  const uint8_t* experts;
  const uint8_t* shared;
  unsigned* err;
  uint16_t* a;            // [Tc][H] bf16 expert input
  float* xn;              // [Tc][H] normalised input (router operand)
  float* logits;          // [Tc][E]
  int* idx;               // [Tc][K] selected experts
  float* wts;             // [Tc][K] routing weights
  int* pos;               // [Tc][K] row of pair (t, k) in the grouped order
  int* rowtok;            // [rows] token of each grouped row
  int4* tiles;            // [0] = {count}; [1 + i] = {expert slot, row0, nrows, 0}
  uint16_t* hbuf;         // [rows][I] bf16 SwiGLU output
  float* obuf;            // [rows][H] float32 expert outputs
};

__device__ inline float bf16_round(float v) {
  f32x2 p = {v, 0.f};
  bf16x2 b = __builtin_convertvector(p, bf16x2);
  return __uint_as_float(__builtin_bit_cast(unsigned, b) << 16);
}

__device__ inline unsigned pack_bf16(float lo, float hi) {
  f32x2 p = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(p, bf16x2));
}

__device__ inline float wave_sum_f(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ inline unsigned long long wave_max_key(unsigned long long v) {
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long w = __shfl_xor(v, o, 64);
    v = w > v ? w : v;
  }
  return v;
}

__device__ inline unsigned ord_f32(float f) {
  const unsigned u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------------
// prep: x_b = bf16(x); x_n = RMSNorm(x_b) (or x_b); A = bf16(x_n).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prep_kernel(PArgs a) {
  const int t = blockIdx.x;
  const float* xr = a.x + (size_t)t * a.H;
  __shared__ float red[4];
  float ss = 0.f;
  for (int k = threadIdx.x * 4; k < a.H; k += 1024) {
    const float4 v = *reinterpret_cast<const float4*>(xr + k);
    const float b0 = bf16_round(v.x), b1 = bf16_round(v.y), b2 = bf16_round(v.z),
                b3 = bf16_round(v.w);
    ss += b0 * b0 + b1 * b1 + b2 * b2 + b3 * b3;
  }
  float rs = 1.f;
  if (a.flags & MOE_F_RMSNORM) {
    ss = wave_sum_f(ss);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    ss = red[0] + red[1] + red[2] + red[3];
    rs = 1.f / sqrtf(ss / (float)a.H + a.eps);
  }
  for (int k = threadIdx.x * 4; k < a.H; k += 1024) {
    const float4 v = *reinterpret_cast<const float4*>(xr + k);
    float n0 = bf16_round(v.x), n1 = bf16_round(v.y), n2 = bf16_round(v.z), n3 = bf16_round(v.w);
    if (a.flags & MOE_F_RMSNORM) {
      float4 g = make_float4(1.f, 1.f, 1.f, 1.f);
      if (a.gamma) g = *reinterpret_cast<const float4*>(a.gamma + k);
      n0 = n0 * rs * g.x; n1 = n1 * rs * g.y; n2 = n2 * rs * g.z; n3 = n3 * rs * g.w;
    }
    *reinterpret_cast<float4*>(a.xn + (size_t)t * a.H + k) = make_float4(n0, n1, n2, n3);
    *reinterpret_cast<uint2*>(a.a + (size_t)t * a.H + k) =
        make_uint2(pack_bf16(n0, n1), pack_bf16(n2, n3));
  }
}

// ---------------------------------------------------------------------------
// router: logits[t][e] = sum_h x_n[t][h] W[e][h] in float32 (64 x 64 tiles).
// Used only when the selection score includes the logit.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void router_kernel(PArgs a) {
  __shared__ float xs[32][65];
  __shared__ float wsh[32][65];
  const int t0 = blockIdx.y * 64, e0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < a.H; k0 += 32) {
    for (int i = threadIdx.x; i < 64 * 32; i += 256) {
      const int r = i >> 5, kk = i & 31;
      const int t = t0 + r, e = e0 + r;
      xs[kk][r] = t < a.n ? a.xn[(size_t)t * a.H + k0 + kk] : 0.f;
      wsh[kk][r] = e < a.E ? a.router[(size_t)e * a.H + k0 + kk] : 0.f;
    }
    __syncthreads();
    for (int kk = 0; kk < 32; ++kk) {
      float xv[4], wv[4];
      for (int i = 0; i < 4; ++i) { xv[i] = xs[kk][ty + 16 * i]; wv[i] = wsh[kk][tx + 16 * i]; }
      for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(xv[i], wv[j], acc[i][j]);
    }
    __syncthreads();
  }
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) {
      const int t = t0 + ty + 16 * i, e = e0 + tx + 16 * j;
      if (t < a.n && e < a.E) a.logits[(size_t)t * a.E + e] = acc[i][j];
    }
}

// ---------------------------------------------------------------------------
// select: one wave per token. Key = (tier, ordered score, 1023 - e): the maximum key
// is the highest tier, then the highest score, then the lowest index.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void select_kernel(PArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.n) return;
  const bool by_sel = (a.flags & MOE_F_SELECT_BY_BIAS) != 0;
  int bst[kMaxK];
  for (int j = 0; j < kMaxK; ++j) {
    int b = -1;
    if (a.boosted && j < a.K) {
      b = a.boosted[(size_t)t * a.K + j];
      if (b >= a.E || b < -1) {
        if (lane == 0) set_dev_err(a.err, DEV_BAD_INDEX);
        b = -1;
      }
    }
    bst[j] = b;
  }
  constexpr int kPer = kMaxE / 64;
  unsigned long long key[kPer];
  for (int i = 0; i < kPer; ++i) {
    const int e = lane + 64 * i;
    key[i] = 0ull;
    if (e < a.E) {
      float s = 0.f;
      if (by_sel) {
        s = a.sel_bias[(size_t)t * a.E + e];
      } else {
        s = a.logits[(size_t)t * a.E + e];
        if (a.sel_bias) s += a.sel_bias[(size_t)t * a.E + e];
      }
      unsigned long long tier = 1ull;
      for (int j = 0; j < kMaxK; ++j) tier = (bst[j] == e) ? 2ull : tier;
      key[i] = (tier << 42) | ((unsigned long long)ord_f32(s) << 10) |
               (unsigned long long)(1023 - e);
    }
  }
  int sel[kMaxK];
  for (int k = 0; k < kMaxK; ++k) {
    sel[k] = 0;
    if (k >= a.K) continue;
    unsigned long long m = 0ull;
    for (int i = 0; i < kPer; ++i) m = key[i] > m ? key[i] : m;
    m = wave_max_key(m);
    const int e = 1023 - (int)(m & 1023ull);
    sel[k] = e;
    for (int i = 0; i < kPer; ++i) key[i] = key[i] == m ? 0ull : key[i];
  }
  // router logits of the selected experts
  float lg[kMaxK];
  for (int k = 0; k < kMaxK; ++k) {
    lg[k] = 0.f;
    if (k >= a.K) continue;
    if (!by_sel) {
      lg[k] = a.logits[(size_t)t * a.E + sel[k]];
    } else {
      const float* wr = a.router + (size_t)sel[k] * a.H;
      const float* xr = a.xn + (size_t)t * a.H;
      float s = 0.f;
      for (int h = lane * 4; h < a.H; h += 256) {
        const float4 w = *reinterpret_cast<const float4*>(wr + h);
        const float4 v = *reinterpret_cast<const float4*>(xr + h);
        s = fmaf(w.x, v.x, s); s = fmaf(w.y, v.y, s); s = fmaf(w.z, v.z, s); s = fmaf(w.w, v.w, s);
      }
      lg[k] = wave_sum_f(s);
    }
  }
  float mx = lg[0];
  for (int k = 1; k < kMaxK; ++k) mx = (k < a.K && lg[k] > mx) ? lg[k] : mx;
  float p[kMaxK], den = 0.f;
  for (int k = 0; k < kMaxK; ++k) {
    p[k] = k < a.K ? __expf(lg[k] - mx) : 0.f;
    den += p[k];
  }
  if (lane < a.K) {
    float wk = 0.f;
    int ek = 0;
    for (int k = 0; k < kMaxK; ++k)
      if (k == lane) { wk = p[k] / den; ek = sel[k]; }
    const size_t o = (size_t)t * a.K + lane;
    a.idx[o] = ek;
    a.wts[o] = wk;
    if (a.idx_out) a.idx_out[o] = ek;
    if (a.w_out) a.w_out[o] = wk;
  }
}

// ---------------------------------------------------------------------------
// group: one workgroup of 1024 threads. Sorting the keys (expert << 14 | pair)
// orders pairs by expert and, within an expert, by (token, slot): a stable counting
// sort. Writes rowtok, pos and the m-tile table (routed experts in index order, then
// the shared experts, whose rows are all tokens in order).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void group_kernel(PArgs a, int n2) {
  extern __shared__ unsigned gl[];
  unsigned* keys = gl;                               // [n2]
  int* first = reinterpret_cast<int*>(gl + n2);      // [E]
  int* last = first + a.E;                           // [E]
  int* scan = last + a.E;                            // [1024]
  const int tid = threadIdx.x;
  const int np = a.n * a.K;
  for (int i = tid; i < n2; i += 1024) {
    unsigned k = 0xFFFFFFFFu;
    if (i < np) {
      int e = a.idx[i];
      if (e < 0 || e >= a.E) {
        set_dev_err(a.err, DEV_BAD_INDEX);
        e = 0;
      }
      k = ((unsigned)e << kPairBits) | (unsigned)i;
    }
    keys[i] = k;
  }
  for (int e = tid; e < a.E; e += 1024) { first[e] = -1; last[e] = -2; }
  __syncthreads();
  for (int size = 2; size <= n2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < (n2 >> 1); i += 1024) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const unsigned x = keys[lo], y = keys[hi];
        if ((x > y) == up) { keys[lo] = y; keys[hi] = x; }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < np; i += 1024) {
    const unsigned k = keys[i];
    const int e = (int)(k >> kPairBits), p = (int)(k & ((1u << kPairBits) - 1));
    a.rowtok[i] = p / a.K;
    a.pos[p] = i;
    if (i == 0 || (int)(keys[i - 1] >> kPairBits) != e) first[e] = i;
    if (i == np - 1 || (int)(keys[i + 1] >> kPairBits) != e) last[e] = i;
  }
  for (int s = 0; s < a.S; ++s)
    for (int t = tid; t < a.n; t += 1024) a.rowtok[np + s * a.n + t] = t;
  __syncthreads();
  // m-tiles per expert, exclusive scan over experts (E <= 1024 = one per thread)
  int nm = 0;
  if (tid < a.E) {
    const int c = last[tid] - first[tid] + 1;
    nm = c > 0 ? (c + kBM - 1) / kBM : 0;
  }
  scan[tid] = nm;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  const int routed_tiles = scan[1023];
  if (tid < a.E && nm > 0) {
    const int t0 = scan[tid] - nm;
    const int c = last[tid] - first[tid] + 1;
    for (int m = 0; m < nm; ++m) {
      const int r = m * kBM;
      a.tiles[1 + t0 + m] = make_int4(tid, first[tid] + r, c - r < kBM ? c - r : kBM, 0);
    }
  }
  const int per_shared = (a.n + kBM - 1) / kBM;
  for (int i = tid; i < a.S * per_shared; i += 1024) {
    const int s = i / per_shared, m = i % per_shared;
    const int r = m * kBM;
    a.tiles[1 + routed_tiles + i] =
        make_int4(a.E + s, np + s * a.n + r, a.n - r < kBM ? a.n - r : kBM, 0);
  }
  if (tid == 0) a.tiles[0] = make_int4(routed_tiles + a.S * per_shared, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Grouped GEMM building blocks
// ---------------------------------------------------------------------------

// Codes and (scale, bias) of one lane for one reduction chunk of one weight row:
// 4-bit: 16 bytes = octets 0..3 of the lane's range; 2-bit: 8 bytes.
struct WFrag {
  u32x4 c;
  unsigned sb;
};

template <int BITS>
__device__ inline WFrag load_wfrag(const uint8_t* blk, int slot, int half, bool valid) {
  WFrag f;
  f.c = u32x4{0u, 0u, 0u, 0u};
  f.sb = 0u;
  if (!valid) return f;
  if (BITS == 4) {
    f.c = *reinterpret_cast<const u32x4*>(blk + half * 1024 + slot * 16);
    f.sb = *reinterpret_cast<const unsigned*>(blk + 2048 + slot * 4);
  } else {
    const uint2 v = *reinterpret_cast<const uint2*>(blk + slot * 16 + half * 8);
    f.c = u32x4{v.x, v.y, 0u, 0u};
    f.sb = *reinterpret_cast<const unsigned*>(blk + 1024 + slot * 4);
  }
  return f;
}

// bf16(q*s + b) for the 8 codes of octet i of a fragment, in reduction order.
template <int BITS>
__device__ inline bf16x8 deq_octet(const WFrag& f, int i) {
  unsigned lo, hi;
  if (BITS == 4) {
    const unsigned d = f.c[i] ^ 0x88888888u;  // stored as q ^ 8
    lo = d & 0x0F0F0F0Fu;
    hi = (d >> 4) & 0x0F0F0F0Fu;
  } else {
    const unsigned d = f.c[i >> 1] >> (2 * (i & 1));
    lo = d & 0x03030303u;
    hi = (d >> 4) & 0x03030303u;
  }
  const float s = bf16lo_to_f32(f.sb), b = bf16hi_to_f32(f.sb);
  const float w0 = fmaf((float)(lo & 0xFFu), s, b);
  const float w1 = fmaf((float)((lo >> 8) & 0xFFu), s, b);
  const float w2 = fmaf((float)((lo >> 16) & 0xFFu), s, b);
  const float w3 = fmaf((float)(lo >> 24), s, b);
  const float w4 = fmaf((float)(hi & 0xFFu), s, b);
  const float w5 = fmaf((float)((hi >> 8) & 0xFFu), s, b);
  const float w6 = fmaf((float)((hi >> 16) & 0xFFu), s, b);
  const float w7 = fmaf((float)(hi >> 24), s, b);
  u32x4 r = {pack_bf16(w0, w1), pack_bf16(w2, w3), pack_bf16(w4, w5), pack_bf16(w6, w7)};
  return __builtin_bit_cast(bf16x8, r);
}

// Activation rows of one m-tile, one reduction chunk: thread handles row
// (tid >> 4) + 16 q for q < mt_valid, 16-byte segment tid & 15.
struct AStage {
  u32x4 v[kMT];
};

__device__ inline void load_astage(AStage& st, const uint16_t* const* rowp, int k0, int Kdim,
                                   int mt_valid) {
  const int seg = threadIdx.x & 15;
  const bool ok = k0 + seg * 8 < Kdim;
#pragma unroll
  for (int q = 0; q < kMT; ++q) {
    st.v[q] = u32x4{0u, 0u, 0u, 0u};
    if (q < mt_valid && ok)
      st.v[q] = *reinterpret_cast<const u32x4*>(rowp[q] + k0 + seg * 8);
  }
}

__device__ inline void store_astage(const AStage& st, uint8_t* lds, int mt_valid) {
  const int seg = threadIdx.x & 15, r = threadIdx.x >> 4;
#pragma unroll
  for (int q = 0; q < kMT; ++q)
    if (q < mt_valid)
      *reinterpret_cast<u32x4*>(lds + (r + 16 * q) * kArow + seg * 16) = st.v[q];
}

__device__ inline bf16x8 lds_afrag(const uint8_t* lds, int mt, int i) {
  const int lane = threadIdx.x & 63;
  const int row = 16 * mt + (lane & 15), kk = lane >> 4;
  return __builtin_bit_cast(bf16x8,
                            *reinterpret_cast<const u32x4*>(lds + row * kArow + kk * 64 + i * 16));
}

// Maps a workgroup to a work item so that each XCD (blockIdx % 8) takes a contiguous
// range of the item list: neighbouring items share activation rows and weights in
// that XCD's L2. Returns -1 for workgroups without an item.
__device__ inline int work_item(int n_items) {
  const int per = (n_items + 7) >> 3;
  const int i = blockIdx.x >> 3, x = blockIdx.x & 7;
  if (i >= per) return -1;
  const int item = x * per + i;
  return item < n_items ? item : -1;
}

__device__ inline const uint8_t* expert_base(const PArgs& a, int e) {
  return e < a.E ? a.experts + (size_t)e * a.geo.expert_bytes
                 : a.shared + (size_t)(e - a.E) * a.geo.expert_bytes;
}

// ---------------------------------------------------------------------------
// gate/up: one m-tile (<= 128 rows of one expert) x 64 intermediate columns.
// Wave w owns columns j0 + 16w .. +15 of both gate and up.
// ---------------------------------------------------------------------------
template <int BITS>
__global__ __launch_bounds__(256) void gateup_kernel(PArgs a) {
  extern __shared__ uint8_t lds[];
  const int NT = a.I / kGuCols;
  const int item = work_item(a.tiles[0].x * NT);
  if (item < 0) return;
  const int4 td = a.tiles[1 + item / NT];
  const int nt = item % NT;
  const int e = td.x, row0 = td.y, nrows = td.z;
  const int mt_valid = (nrows + 15) >> 4;
  const uint8_t* W = expert_base(a, e);
  const Geo& g = a.geo;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kk = lane >> 4;
  const int j = nt * kGuCols + wave * 16 + (lane & 15);
  const uint8_t* blk_g = W + (size_t)(j / g.Ph) * g.blk;
  const uint8_t* blk_u = W + g.off_up + (size_t)(j / g.Ph) * g.blk;
  const int slot0 = (j % g.Ph) * g.Gh;

  const uint16_t* rowp[kMT];
#pragma unroll
  for (int q = 0; q < kMT; ++q) {
    int r = (threadIdx.x >> 4) + 16 * q;
    r = r < nrows ? r : nrows - 1;
    rowp[q] = a.a + (size_t)a.rowtok[row0 + r] * a.H;
  }
  const int nch = (a.H + kKC - 1) / kKC;

  f32x4 acc_g[kMT], acc_u[kMT];
#pragma unroll
  for (int q = 0; q < kMT; ++q) {
    acc_g[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc_u[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  auto wload = [&](int ch, WFrag& fg, WFrag& fu) {
    const int grp = 2 * ch + (kk >> 1);
    const bool ok = ch < nch && grp < g.Gh;
    fg = load_wfrag<BITS>(blk_g, slot0 + grp, kk & 1, ok);
    fu = load_wfrag<BITS>(blk_u, slot0 + grp, kk & 1, ok);
  };
  WFrag g0, u0, g1, u1;
  AStage st;
  wload(0, g0, u0);
  wload(1, g1, u1);
  load_astage(st, rowp, 0, a.H, mt_valid);

  auto chunk = [&](int ch, WFrag& fg, WFrag& fu) {
    __syncthreads();
    store_astage(st, lds, mt_valid);
    __syncthreads();
    if (ch + 1 < nch) load_astage(st, rowp, (ch + 1) * kKC, a.H, mt_valid);
    const WFrag cg = fg, cu = fu;
    wload(ch + 2, fg, fu);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x8 bg = deq_octet<BITS>(cg, i);
      const bf16x8 bu = deq_octet<BITS>(cu, i);
#pragma unroll
      for (int q = 0; q < kMT; ++q) {
        if (q < mt_valid) {
          const bf16x8 af = lds_afrag(lds, q, i);
          acc_g[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bg, acc_g[q], 0, 0, 0);
          acc_u[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bu, acc_u[q], 0, 0, 0);
        }
      }
    }
  };
  for (int ch = 0; ch < nch; ch += 2) {
    chunk(ch, g0, u0);
    if (ch + 1 < nch) chunk(ch + 1, g1, u1);
  }

  // epilogue: h = bf16(silu(g) * u) -> hbuf[row][j]
#pragma unroll
  for (int q = 0; q < kMT; ++q) {
    if (q < mt_valid) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 16 * q + 4 * kk + r;
        if (m < nrows) {
          const float gv = acc_g[q][r], uv = acc_u[q][r];
          const float h = gv / (1.f + __expf(-gv)) * uv;
          a.hbuf[(size_t)(row0 + m) * a.I + j] = (uint16_t)(pack_bf16(h, 0.f) & 0xFFFFu);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// down: one m-tile x 128 output columns; wave w owns columns n0 + 32w .. +31
// (two 16-column MFMA tiles).
// ---------------------------------------------------------------------------
template <int BITS>
__global__ __launch_bounds__(256) void down_kernel(PArgs a) {
  extern __shared__ uint8_t lds[];
  const int NT = (a.H + kDnCols - 1) / kDnCols;
  const int item = work_item(a.tiles[0].x * NT);
  if (item < 0) return;
  const int4 td = a.tiles[1 + item / NT];
  const int nt = item % NT;
  const int e = td.x, row0 = td.y, nrows = td.z;
  const int mt_valid = (nrows + 15) >> 4;
  const uint8_t* W = expert_base(a, e) + a.geo.off_down;
  const Geo& g = a.geo;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kk = lane >> 4;
  const int nA = nt * kDnCols + wave * 32 + (lane & 15);
  const int nB = nA + 16;
  const bool wave_on = nt * kDnCols + wave * 32 < a.H;  // wave-uniform
  const bool bon = wave_on && nt * kDnCols + wave * 32 + 16 < a.H;
  const uint8_t* blk_a = W + (size_t)((wave_on ? nA : 0) / g.Pi) * g.blk;
  const uint8_t* blk_b = W + (size_t)((bon ? nB : 0) / g.Pi) * g.blk;
  const int slot_a = ((wave_on ? nA : 0) % g.Pi) * g.Gi;
  const int slot_b = ((bon ? nB : 0) % g.Pi) * g.Gi;

  const uint16_t* rowp[kMT];
#pragma unroll
  for (int q = 0; q < kMT; ++q) {
    int r = (threadIdx.x >> 4) + 16 * q;
    r = r < nrows ? r : nrows - 1;
    rowp[q] = a.hbuf + (size_t)(row0 + r) * a.I;
  }
  const int nch = (a.I + kKC - 1) / kKC;

  f32x4 acc_a[kMT], acc_b[kMT];
#pragma unroll
  for (int q = 0; q < kMT; ++q) {
    acc_a[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc_b[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  auto wload = [&](int ch, WFrag& fa, WFrag& fb) {
    const int grp = 2 * ch + (kk >> 1);
    const bool ok = ch < nch && grp < g.Gi;
    fa = load_wfrag<BITS>(blk_a, slot_a + grp, kk & 1, ok && wave_on);
    fb = load_wfrag<BITS>(blk_b, slot_b + grp, kk & 1, ok && bon);
  };
  WFrag a0, b0, a1, b1;
  AStage st;
  wload(0, a0, b0);
  wload(1, a1, b1);
  load_astage(st, rowp, 0, a.I, mt_valid);

  auto chunk = [&](int ch, WFrag& fa, WFrag& fb) {
    __syncthreads();
    store_astage(st, lds, mt_valid);
    __syncthreads();
    if (ch + 1 < nch) load_astage(st, rowp, (ch + 1) * kKC, a.I, mt_valid);
    const WFrag ca = fa, cb = fb;
    wload(ch + 2, fa, fb);
    if (!wave_on) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x8 ba = deq_octet<BITS>(ca, i);
      const bf16x8 bb = deq_octet<BITS>(cb, i);
#pragma unroll
      for (int q = 0; q < kMT; ++q) {
        if (q < mt_valid) {
          const bf16x8 af = lds_afrag(lds, q, i);
          acc_a[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, ba, acc_a[q], 0, 0, 0);
          acc_b[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bb, acc_b[q], 0, 0, 0);
        }
      }
    }
  };
  for (int ch = 0; ch < nch; ch += 2) {
    chunk(ch, a0, b0);
    if (ch + 1 < nch) chunk(ch + 1, a1, b1);
  }
  if (!wave_on) return;
#pragma unroll
  for (int q = 0; q < kMT; ++q) {
    if (q < mt_valid) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 16 * q + 4 * kk + r;
        if (m < nrows) {
          float* orow = a.obuf + (size_t)(row0 + m) * a.H;
          orow[nA] = acc_a[q][r];
          if (bon) orow[nB] = acc_b[q][r];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// combine: y[t] = x_b[t] (residual) + sum_k w[t][k] o[pos[t][k]] + sum_s o_s[t].
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_kernel(PArgs a) {
  const int h4 = a.H / 4;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)a.n * h4) return;
  const int t = (int)(i / h4), k = (int)(i % h4) * 4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (a.flags & MOE_F_RESIDUAL) {
    const float4 v = *reinterpret_cast<const float4*>(a.x + (size_t)t * a.H + k);
    acc = make_float4(bf16_round(v.x), bf16_round(v.y), bf16_round(v.z), bf16_round(v.w));
  }
  for (int j = 0; j < a.K; ++j) {
    const float w = a.wts[(size_t)t * a.K + j];
    const float4 o =
        *reinterpret_cast<const float4*>(a.obuf + (size_t)a.pos[(size_t)t * a.K + j] * a.H + k);
    acc.x = fmaf(w, o.x, acc.x); acc.y = fmaf(w, o.y, acc.y);
    acc.z = fmaf(w, o.z, acc.z); acc.w = fmaf(w, o.w, acc.w);
  }
  const size_t np = (size_t)a.n * a.K;
  for (int s = 0; s < a.S; ++s) {
    const float4 o =
        *reinterpret_cast<const float4*>(a.obuf + (np + (size_t)s * a.n + t) * a.H + k);
    acc.x += o.x; acc.y += o.y; acc.z += o.z; acc.w += o.w;
  }
  *reinterpret_cast<float4*>(a.y + (size_t)t * a.H + k) = acc;
}

__global__ void clear_err(unsigned* err) {
  if (threadIdx.x == 0) *err = 0u;
}

int next_pow2(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

}  // namespace

size_t prefill_ws_bytes(const moe_config& c, int T) { return p_layout(c, T).total; }

moe_status prefill_forward(const moe_config& c, const moe_layer_weights* lw, int T,
                           const float* x, float* y, const float* sel_bias, const int32_t* boosted,
                           int32_t* idx_out, float* w_out, uint8_t* ws, size_t ws_bytes,
                           hipStream_t stream, std::string* msg) {
  if ((c.flags & MOE_F_SELECT_BY_BIAS) && !sel_bias) {
    *msg = "MOE_F_SELECT_BY_BIAS needs sel_bias";
    return MOE_ERR_ARG;
  }
  const PLayout pl = p_layout(c, T);
  if (ws_bytes < pl.total) {
    *msg = "workspace too small for the prefill path";
    return MOE_ERR_WORKSPACE;
  }
  PArgs a;
  a.H = c.hidden; a.I = c.inter; a.E = c.n_experts; a.K = c.top_k; a.S = c.n_shared;
  a.flags = c.flags; a.eps = c.eps;
  a.geo = make_geo(c.hidden, c.inter, c.bits);
  a.router = lw->router_w;
  a.gamma = lw->gamma;
  a.experts = static_cast<const uint8_t*>(lw->experts);
  a.shared = static_cast<const uint8_t*>(lw->shared);
  a.err = reinterpret_cast<unsigned*>(ws + pl.err);
  a.a = reinterpret_cast<uint16_t*>(ws + pl.a);
  a.xn = reinterpret_cast<float*>(ws + pl.xn);
  a.logits = reinterpret_cast<float*>(ws + pl.logits);
  a.idx = reinterpret_cast<int*>(ws + pl.idx);
  a.wts = reinterpret_cast<float*>(ws + pl.wts);
  a.pos = reinterpret_cast<int*>(ws + pl.pos);
  a.rowtok = reinterpret_cast<int*>(ws + pl.rowtok);
  a.tiles = reinterpret_cast<int4*>(ws + pl.tiles);
  a.hbuf = reinterpret_cast<uint16_t*>(ws + pl.hbuf);
  a.obuf = reinterpret_cast<float*>(ws + pl.obuf);

  static bool attr_done = false;
  const size_t group_lds_max = sizeof(unsigned) * (kSortMax + 2 * kMaxE + 1024);
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&group_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)group_lds_max);
    if (e != hipSuccess) {
      *msg = std::string("hipFuncSetAttribute: ") + hipGetErrorString(e);
      return MOE_ERR_HIP;
    }
    attr_done = true;
  }

  hipLaunchKernelGGL(clear_err, dim3(1), dim3(64), 0, stream, a.err);
  const size_t lds_ab = (size_t)kBM * kArow;
  for (int t0 = 0; t0 < T; t0 += pl.Tc) {
    const int n = T - t0 < pl.Tc ? T - t0 : pl.Tc;
    a.n = n;
    a.x = x + (size_t)t0 * c.hidden;
    a.y = y + (size_t)t0 * c.hidden;
    a.sel_bias = sel_bias ? sel_bias + (size_t)t0 * c.n_experts : nullptr;
    a.boosted = boosted ? boosted + (size_t)t0 * c.top_k : nullptr;
    a.idx_out = idx_out ? idx_out + (size_t)t0 * c.top_k : nullptr;
    a.w_out = w_out ? w_out + (size_t)t0 * c.top_k : nullptr;

    hipLaunchKernelGGL(prep_kernel, dim3(n), dim3(256), 0, stream, a);
    if (!(c.flags & MOE_F_SELECT_BY_BIAS))
      hipLaunchKernelGGL(router_kernel, dim3((c.n_experts + 63) / 64, (n + 63) / 64), dim3(256), 0,
                         stream, a);
    hipLaunchKernelGGL(select_kernel, dim3((n + 3) / 4), dim3(256), 0, stream, a);
    const int n2 = next_pow2(n * c.top_k < 2 ? 2 : n * c.top_k);
    const size_t glds = sizeof(unsigned) * ((size_t)n2 + 2 * c.n_experts + 1024);
    hipLaunchKernelGGL(group_kernel, dim3(1), dim3(1024), glds, stream, a, n2);
    // grids: an upper bound of the m-tiles this pass can have, rounded to whole XCDs
    const int TK = n * c.top_k;
    const int nz = c.n_experts < TK ? c.n_experts : TK;
    const int tiles_max = nz + (TK + kBM - 1) / kBM + c.n_shared * ((n + kBM - 1) / kBM);
    const int gu_items = tiles_max * (c.inter / kGuCols);
    const int dn_items = tiles_max * ((c.hidden + kDnCols - 1) / kDnCols);
    const unsigned gu_grid = (unsigned)(8 * ((gu_items + 7) / 8));
    const unsigned dn_grid = (unsigned)(8 * ((dn_items + 7) / 8));
    if (c.bits == 4) {
      hipLaunchKernelGGL(gateup_kernel<4>, dim3(gu_grid), dim3(256), lds_ab, stream, a);
      hipLaunchKernelGGL(down_kernel<4>, dim3(dn_grid), dim3(256), lds_ab, stream, a);
    } else {
      hipLaunchKernelGGL(gateup_kernel<2>, dim3(gu_grid), dim3(256), lds_ab, stream, a);
      hipLaunchKernelGGL(down_kernel<2>, dim3(dn_grid), dim3(256), lds_ab, stream, a);
    }
    const size_t nthreads = (size_t)n * (c.hidden / 4);
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((nthreads + 255) / 256)), dim3(256), 0,
                       stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    *msg = std::string("prefill launch: ") + hipGetErrorString(e);
    return MOE_ERR_HIP;
  }
  return MOE_OK;
}

}  // namespace qmoe
