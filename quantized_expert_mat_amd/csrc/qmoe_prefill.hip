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
//   group    one workgroup: counting sort of the (token, slot) pairs by expert
//            (counts, exclusive scan, row claims); per-expert row runs; m-tile table
//   gateup   grouped GEMM: rows of one expert x 16 intermediate columns per wave
//            (4 waves per thin-tile workgroup, 8 per thick one), gate and up fused,
//            h = bf16(silu(g) * u)
//   down     grouped GEMM: rows x 32 output columns per wave -> float32 rows
//   combine  y = x_b + sum_k w_k o_k + sum_s o_s, fixed order per token
//
// Weights are dequantised in registers by the lane that feeds them to the MFMA (no
// LDS round trip for B); activations are staged through LDS per 256-wide reduction
// chunk (four 64-groups). Inside a chunk the reduction index is permuted identically
// for the A and B operands (the MFMA sums over it, so any common permutation is
// exact): lane group kk = lane/16 covers group kk of the chunk, positions
// [64kk, 64kk+64), and MFMA step i (i = 0..7) the octet [64kk+8i, 64kk+8i+8) of it,
// so each lane dequantises whole groups of one packed slot.
#include <mutex>
#include <string>

#include "qmoe_internal.h"

namespace qmoe {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kChunkT = 2048;      // tokens per pass (bounds the workspace)
constexpr int kBM = 64;            // rows (token-expert pairs) per thick m-tile
constexpr int kGuCols = 16;        // intermediate columns per gate/up wave
constexpr int kDnCols = 32;        // output columns per down wave
constexpr int kSortMax = 16384;    // routed (token, expert) pairs per pass
constexpr int kGroupWaves = 1024 / kWave;  // waves of the grouping workgroup
constexpr int kMaxAttrDevices = 64;        // devices whose kernel attributes are tracked

// ---------------------------------------------------------------------------
// Workspace layout of one prefill pass
// ---------------------------------------------------------------------------
struct PLayout {
  int Tc, rows, max_tiles;
  size_t err, a, xn, logits, idx, wts, pos, rowtok, thin, thick, hbuf, obuf, sgc, total;
};

PLayout p_layout(const moe_config& c, int T) {
  PLayout p;
  // tokens per pass: at most kChunkT, and at most kSortMax routed pairs
  const int tmax = std::min(kChunkT, kSortMax / std::max(1, c.top_k));
  p.Tc = T < 1 ? 1 : (T < tmax ? T : tmax);
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
  p.thin = o; o = align256(o + 16 * (size_t)(p.max_tiles + 1));
  p.thick = o; o = align256(o + 16 * (size_t)(p.max_tiles + 1));
  p.hbuf = o; o = align256(o + (size_t)p.rows * c.inter * 2);
  p.obuf = o; o = align256(o + (size_t)p.rows * c.hidden * 4);
  p.sgc = o; o = align256(o + (size_t)p.Tc * kMaxShared * 4);
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
  const float* sgate;     // [S][H] shared-expert gate or null
  unsigned* err;
  uint16_t* a;            // [Tc][H] bf16 expert input
  float* xn;              // [Tc][H] normalised input (router operand)
  float* logits;          // [Tc][E]
  int* idx;               // [Tc][K] selected experts
  float* wts;             // [Tc][K] routing weights
  int* pos;               // [Tc][K] row of pair (t, k) in the grouped order
  int* rowtok;            // [rows] token of each grouped row
  int4* thin;             // m-tiles of <= 16 rows: [0] = {count}; [1 + i] = {expert slot, row0, nrows, 0}
  int4* thick;            // m-tiles of 17..64 rows, same format
  uint16_t* hbuf;         // [rows][I] bf16 SwiGLU output
  float* obuf;            // [rows][H] float32 expert outputs
  float* sgc;             // [Tc][kMaxShared] shared-expert gate factors (with sgate)
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
// prep: x_b = bf16(x); x_n = RMSNorm(x_b) (or x_b); A = bf16(x_n); with a
// shared-expert gate also c_s = sigmoid(g_s . x_n) from the unrounded x_n.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prep_kernel(PArgs a) {
  const int t = blockIdx.x;
  const float* xr = a.x + (size_t)t * a.H;
  __shared__ float red[4];
  __shared__ float gred[kMaxShared][4];
  float gz[kMaxShared] = {};
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
    if (a.sgate) {
      for (int sh = 0; sh < a.S; ++sh) {
        const float4 g = *reinterpret_cast<const float4*>(a.sgate + (size_t)sh * a.H + k);
        gz[sh] = fmaf(g.x, n0, gz[sh]);
        gz[sh] = fmaf(g.y, n1, gz[sh]);
        gz[sh] = fmaf(g.z, n2, gz[sh]);
        gz[sh] = fmaf(g.w, n3, gz[sh]);
      }
    }
  }
  if (a.sgate) {
    for (int sh = 0; sh < a.S; ++sh) {
      const float v = wave_sum_f(gz[sh]);
      if ((threadIdx.x & 63) == 0) gred[sh][threadIdx.x >> 6] = v;
    }
    __syncthreads();
    if ((int)threadIdx.x < a.S) {
      const float z = gred[threadIdx.x][0] + gred[threadIdx.x][1] + gred[threadIdx.x][2] + gred[threadIdx.x][3];
      a.sgc[(size_t)t * kMaxShared + threadIdx.x] = 1.f / (1.f + expf(-z));
    }
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
  // selection by sel_bias: the router logits of the selected experts are formed
  // here; x_n is requested now, under the selection
  constexpr int kIt = kMaxDim / 256;  // float4 of a row per lane
  float4 xv[kIt];
  if (by_sel) {
    const float* xr = a.xn + (size_t)t * a.H;
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
      const int h = lane * 4 + it * 256;
      xv[it] = h < a.H ? *reinterpret_cast<const float4*>(xr + h) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
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
  // router logits of the selected experts. By sel_bias: each selected row is
  // requested whole, the next one while the current one is reduced (one round trip
  // per row, overlapped); the products run in the same order as a plain loop over h.
  float lg[kMaxK];
  if (!by_sel) {
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) lg[k] = k < a.K ? a.logits[(size_t)t * a.E + sel[k]] : 0.f;
  } else {
    float4 wa[kIt], wb[kIt];
    auto load_row = [&](float4 (&w)[kIt], int e) {
      const float* wr = a.router + (size_t)e * a.H;
#pragma unroll
      for (int it = 0; it < kIt; ++it) {
        const int h = lane * 4 + it * 256;
        w[it] = h < a.H ? *reinterpret_cast<const float4*>(wr + h) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    };
    load_row(wa, sel[0]);
#pragma unroll
    for (int k = 0; k < kMaxK; ++k) {
      float4(&cur)[kIt] = (k & 1) ? wb : wa;
      float4(&nxt)[kIt] = (k & 1) ? wa : wb;
      if (k + 1 < a.K) load_row(nxt, sel[k + 1]);
      lg[k] = 0.f;
      if (k < a.K) {
        float s = 0.f;
#pragma unroll
        for (int it = 0; it < kIt; ++it) {
          const float4 w = cur[it], v = xv[it];
          s = fmaf(w.x, v.x, s); s = fmaf(w.y, v.y, s); s = fmaf(w.z, v.z, s); s = fmaf(w.w, v.w, s);
        }
        lg[k] = wave_sum_f(s);
      }
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
// group: one workgroup of 1024 threads, a counting sort of the (token, slot) pairs by
// expert: per-expert counts, their exclusive scan, then every pair takes the next
// free row of its expert. Writes rowtok, pos and the m-tile table (routed experts in
// index order, then the shared experts, whose rows are all tokens in order).
// ---------------------------------------------------------------------------
// (thin << 16) | thick: the m-tiles of an expert with c > 0 rows: full thick tiles
// of kBM rows, then the remainder as a thin (<= 16 rows) or a thick tile.
__device__ inline int tile_counts(int c) {
  const int full = c / kBM, rem = c % kBM;
  const int thick = full + (rem > 16 ? 1 : 0);
  const int thin = (rem > 0 && rem <= 16) ? 1 : 0;
  return (thin << 16) | thick;
}

__device__ inline void write_tiles(const PArgs& a, int e, int row0, int c, int thin_at,
                                   int thick_at) {
  const int full = c / kBM, rem = c % kBM;
  for (int m = 0; m < full; ++m)
    a.thick[1 + thick_at + m] = make_int4(e, row0 + m * kBM, kBM, 0);
  if (rem > 16) a.thick[1 + thick_at + full] = make_int4(e, row0 + full * kBM, rem, 0);
  else if (rem > 0) a.thin[1 + thin_at] = make_int4(e, row0 + full * kBM, rem, 0);
}

// Inclusive prefix sum over the 1024 threads of a workgroup: a shuffle scan inside
// each wave, then one over the 16 wave totals. wsum: 16 ints of LDS.
__device__ inline int block_scan_1024(int v, int* wsum) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  __syncthreads();  // a previous call's readers of wsum are done
  for (int o = 1; o < kWave; o <<= 1) {
    const int u = __shfl_up(v, o, kWave);
    if (lane >= o) v += u;
  }
  if (lane == kWave - 1) wsum[w] = v;
  __syncthreads();
  if (w == 0) {
    int t = lane < kGroupWaves ? wsum[lane] : 0;
    for (int o = 1; o < kGroupWaves; o <<= 1) {
      const int u = __shfl_up(t, o, kWave);
      if (lane >= o) t += u;
    }
    if (lane < kGroupWaves) wsum[lane] = t;
  }
  __syncthreads();
  return v + (w > 0 ? wsum[w - 1] : 0);
}

__global__ __launch_bounds__(1024) void group_kernel(PArgs a) {
  extern __shared__ int gl[];
  const int E = a.E;
  int* cnt = gl;              // [E] pairs per expert, then the rows placed so far
  int* off = cnt + E;         // [E] first row of each expert
  int* scan = off + E;        // [kGroupWaves] block-scan wave totals
  const int tid = threadIdx.x;
  const int np = a.n * a.K;
  for (int e = tid; e < E; e += 1024) cnt[e] = 0;
  __syncthreads();
  for (int i = tid; i < np; i += 1024) {
    int e = a.idx[i];
    if (e < 0 || e >= E) {
      set_dev_err(a.err, DEV_BAD_INDEX);
      e = 0;
    }
    atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  // exclusive scan of the counts (one expert per thread, E <= 1024): off[e]
  const int c = tid < E ? cnt[tid] : 0;
  const int c_incl = block_scan_1024(c, scan);
  if (tid < E) {
    off[tid] = c_incl - c;
    cnt[tid] = 0;
  }
  __syncthreads();
  // each pair takes the next free row of its expert (LDS atomics: the order of an
  // expert's rows varies from call to call, its rows' results do not, since every
  // row of a tile is computed on its own)
  for (int i = tid; i < np; i += 1024) {
    int e = a.idx[i];
    if (e < 0 || e >= E) e = 0;
    const int row = off[e] + atomicAdd(&cnt[e], 1);
    a.rowtok[row] = i / a.K;
    a.pos[i] = row;
  }
  for (int s = 0; s < a.S; ++s)
    for (int t = tid; t < a.n; t += 1024) a.rowtok[np + s * a.n + t] = t;
  // m-tiles of an expert with c rows: full kBM-row tiles, then the remainder as a
  // thin tile (<= 16 rows) or a thick one. Exclusive scan over experts of the packed
  // counts (thin << 16 | thick), one expert per thread (E <= 1024).
  const int tiles = c > 0 ? tile_counts(c) : 0;
  const int t_incl = block_scan_1024(tiles, scan);
  const int tot = scan[kGroupWaves - 1];
  if (tiles > 0) {
    const int ex = t_incl - tiles;
    write_tiles(a, tid, off[tid], c, ex >> 16, ex & 0xFFFF);
  }
  // shared experts after the routed ones (one thread each; S <= 2)
  if (tid == 0) {
    int thin_n = tot >> 16, thick_n = tot & 0xFFFF;
    for (int s = 0; s < a.S; ++s) {
      const int k = tile_counts(a.n);
      write_tiles(a, a.E + s, np + s * a.n, a.n, thin_n, thick_n);
      thin_n += k >> 16;
      thick_n += k & 0xFFFF;
    }
    a.thin[0] = make_int4(thin_n, 0, 0, 0);
    a.thick[0] = make_int4(thick_n, 0, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// Grouped GEMM
//
// A work item is one m-tile of one expert (<= 16 rows: "thin", or 17..64 rows:
// "thick") and a slice of output columns. Every wave owns two 16-column MFMA tiles
// ("sets"): the gate and the up rows j..j+15 of the gate/up GEMM (so silu(g) * u is
// lane-local), or two adjacent 16-row blocks of the down matrix.
//
// Reduction chunks are 256 wide (four 64-groups). Lane (n, kk) loads the codes of
// group kk of the chunk for weight row n -- the four lanes of a row read 64
// contiguous bytes of each code plane, which keeps the HBM stream dense -- and
// feeds octet i of that group to MFMA step i (i = 0..7). The activation operand
// uses the same order: lane (m, kk) at step i holds row m, chunk positions
// 64kk + 8i .. 64kk + 8i + 7. Activations are copied into LDS
// through registers, two stages deep, in a fragment-major layout
// [subtile][kk][i][row][16 B] that the MFMA reads without bank conflicts.
// ---------------------------------------------------------------------------
constexpr int kKC2 = 256;                 // reduction chunk
constexpr int kSubBytes = 16 * kKC2 * 2;  // one 16-row subtile of a chunk in LDS (8 KB)
constexpr int kThinRows = 16;
constexpr int kThickMT = 4;               // subtiles of a thick m-tile (64 rows)

// Codes and (scale, bias) of one lane's group for one chunk.
struct WFrag {
  u32x4 c0, c1;  // 4-bit: codes 0..31 and 32..63 of the group; 3-bit: c0 and c1[0..1]
  unsigned sb;   // (the packed slot's six dwords); 2-bit: c0 holds all 64
};

typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;

// q*s + b rounded once to float32, for a code q held in one 16-bit half of m as a
// field at bit 0 or bit 4 of that half (the half's other bits zero). The half read
// as a float16 is the denormal q * 2^-24 (field at bit 0) or q * 2^-20 (bit 4),
// which converts exactly, and sc is s * 2^24 or s * 2^20 to match, so the fused
// product is q*s exactly and the fma rounds the exact q*s + b once: the same value
// as fmaf((float)q, s, b). One v_fma_mix_f32 per weight instead of a byte-to-float
// conversion and an fma. (Exact while |s| < 2^104, where s * 2^24 is finite.)
__device__ inline float deq_lo(unsigned m, float sc, float b) {
  return fmaf((float)__builtin_bit_cast(f16x2, m)[0], sc, b);
}
__device__ inline float deq_hi(unsigned m, float sc, float b) {
  return fmaf((float)__builtin_bit_cast(f16x2, m)[1], sc, b);
}

// bf16(q*s + b) for the 8 codes of octet i of a group, in reduction order. The
// octet's codes sit in one dword d as two interleaved sets of four byte lanes:
// element j < 4 in bits [8j, 8j + bits), element 4 + j in bits [8j + 4, 8j + 4 + bits).
// So each 16-bit half of d holds elements at bits 0 and 4 (both inside a float16's
// mantissa) and at bits 8 and 12; one shift by 8 and four masks leave two codes per
// dword, one per half, each at bit 0 or bit 4, for deq_lo / deq_hi.
template <int BITS>
__device__ inline bf16x8 deq_octet(const WFrag& f, int i) {
  unsigned d;
  if (BITS == 4) {
    d = i < 4 ? f.c0[i & 3] : f.c1[i & 3];  // stored q ^ 8, flipped back per field below
  } else if (BITS == 3) {
    // octets 0..3 come from dwords 0..2, octets 4..7 from dwords 3..5; the fourth
    // octet of each triple is gathered from the top bits of the three dwords
    // triple t is dwords 3t..3t+2 of the slot (c0[0..2] or c0[3], c1[0], c1[1]),
    // picked by selects rather than an indexed array, which would live in scratch
    const int t = i >> 2, r = i & 3;
    const unsigned w0 = t ? f.c0[3] : f.c0[0], w1 = t ? f.c1[0] : f.c0[1], w2 = t ? f.c1[1] : f.c0[2];
    if (r < 3) {
      d = r == 0 ? w0 : r == 1 ? w1 : w2;
    } else {
      d = ((w0 >> 3) & 0x11111111u) | ((w1 >> 2) & 0x22222222u) | ((w2 >> 1) & 0x44444444u);
    }
  } else {
    d = f.c0[i >> 1] >> (2 * (i & 1));
  }
  constexpr unsigned kM = ((1u << BITS) - 1u) * 0x00010001u;  // a field at bit 0 of each half
  constexpr unsigned kX = BITS == 4 ? 0x00080008u : 0u;        // 4-bit codes are stored as q ^ 8
  const unsigned e = d >> 8;
  const unsigned m02 = (d & kM) ^ kX;                  // elements 0 (low half) and 2 (high half), bit 0
  const unsigned m13 = (e & kM) ^ kX;                  // elements 1 and 3, bit 0
  const unsigned m46 = (d & (kM << 4)) ^ (kX << 4);    // elements 4 and 6, bit 4
  const unsigned m57 = (e & (kM << 4)) ^ (kX << 4);    // elements 5 and 7, bit 4
  const float s = bf16lo_to_f32(f.sb), b = bf16hi_to_f32(f.sb);
  const float s24 = s * 16777216.0f, s20 = s * 1048576.0f;
  u32x4 r = {pack_bf16(deq_lo(m02, s24, b), deq_lo(m13, s24, b)),
             pack_bf16(deq_hi(m02, s24, b), deq_hi(m13, s24, b)),
             pack_bf16(deq_lo(m46, s20, b), deq_lo(m57, s20, b)),
             pack_bf16(deq_hi(m46, s20, b), deq_hi(m57, s20, b))};
  return __builtin_bit_cast(bf16x8, r);
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

// One work item as seen by one lane. Chunk ch of a lane's weight row starts 64*ch
// bytes after wc (code plane 0; plane 1 of 4-bit codes is 1024 bytes further) and
// 32*ch bytes after wc1 (plane 1 of 3-bit codes); the row's (scale, bias) words,
// one per 64-group, start at wsb.
struct Job {
  int row0, nrows, K, nch, G;
  const uint8_t* wc[2];    // codes of chunk 0 of this lane's row in each set
  const uint8_t* wc1[2];   // 3-bit: second code plane of chunk 0
  const unsigned* wsb[2];  // (scale, bias) word of group 0 of this lane's row
  unsigned sbmask;         // 0 where the lane's group lies beyond K (K < 256)
  int col[2];              // output column of this lane in each set
  bool on[2];              // the set has columns (wave-uniform)
};

template <int BITS>
__device__ inline void job_row(const Geo& g, const uint8_t* mat, int row, int P, int G, int kk,
                               const uint8_t*& wc, const uint8_t*& wc1, const unsigned*& wsb) {
  const int grp = kk < G ? kk : 0;
  const uint8_t* blk = mat + (size_t)(row / P) * g.blk;
  const int slot = (row % P) * G + grp;
  wc = blk + slot * 16;
  wc1 = blk + kPlane1Offset + slot * 8;
  wsb = reinterpret_cast<const unsigned*>(blk + sb_offset(BITS)) + (row % P) * G;
}

template <int BITS, bool DOWN, int NWV>
__device__ inline bool make_job(const PArgs& a, const int4* list, Job& jb) {
  const int NT = DOWN ? (a.H + NWV * kDnCols - 1) / (NWV * kDnCols) : (a.I + NWV * kGuCols - 1) / (NWV * kGuCols);
  const int item = work_item(list[0].x * NT);
  if (item < 0) return false;
  const int4 td = list[1 + item / NT];
  const int nt = item % NT;
  jb.row0 = td.y;
  jb.nrows = td.z;
  const Geo& g = a.geo;
  const uint8_t* W = expert_base(a, td.x);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kk = lane >> 4;
  jb.K = DOWN ? a.I : a.H;
  jb.nch = (jb.K + kKC2 - 1) / kKC2;
  const int G = DOWN ? g.Gi : g.Gh;
  jb.G = G;
  jb.sbmask = kk < G ? 0xFFFFFFFFu : 0u;
  if (!DOWN) {
    // a wave past the last column (wide workgroups on a narrow layer) reads row 0
    // and stores nothing
    const int base = nt * (NWV * kGuCols) + wave * kGuCols;
    jb.on[0] = jb.on[1] = base < a.I;
    const int j = jb.on[0] ? base + (lane & 15) : 0;
    job_row<BITS>(g, W, j, g.Ph, g.Gh, kk, jb.wc[0], jb.wc1[0], jb.wsb[0]);
    job_row<BITS>(g, W + g.off_up, j, g.Ph, g.Gh, kk, jb.wc[1], jb.wc1[1], jb.wsb[1]);
    jb.col[0] = jb.col[1] = j;
  } else {
    const int base = nt * (NWV * kDnCols) + wave * kDnCols;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      jb.on[s] = base + 16 * s < a.H;
      const int n = jb.on[s] ? base + 16 * s + (lane & 15) : 0;
      jb.col[s] = n;
      job_row<BITS>(g, W + g.off_down, n, g.Pi, g.Gi, kk, jb.wc[s], jb.wc1[s], jb.wsb[s]);
    }
  }
  return true;
}

// Weight fragments of chunk ch (clamped to the last chunk: loads past the end are
// in bounds and their values are never used).
template <int BITS>
__device__ inline void load_wpair(const Job& jb, int ch, WFrag& f0, WFrag& f1) {
  ch = ch < jb.nch ? ch : jb.nch - 1;
  f0.c0 = *reinterpret_cast<const u32x4*>(jb.wc[0] + ch * 64);
  f1.c0 = *reinterpret_cast<const u32x4*>(jb.wc[1] + ch * 64);
  if (BITS == 4) {
    f0.c1 = *reinterpret_cast<const u32x4*>(jb.wc[0] + kPlane1Offset + ch * 64);
    f1.c1 = *reinterpret_cast<const u32x4*>(jb.wc[1] + kPlane1Offset + ch * 64);
  } else if (BITS == 3) {
    const u32x2 h0 = *reinterpret_cast<const u32x2*>(jb.wc1[0] + ch * 32);
    const u32x2 h1 = *reinterpret_cast<const u32x2*>(jb.wc1[1] + ch * 32);
    f0.c1 = u32x4{h0[0], h0[1], 0u, 0u};
    f1.c1 = u32x4{h1[0], h1[1], 0u, 0u};
  } else {
    f0.c1 = u32x4{0u, 0u, 0u, 0u};
    f1.c1 = u32x4{0u, 0u, 0u, 0u};
  }
}

// (scale, bias) words. A chunk needs one word per lane (its group of the chunk), but
// one dword load per chunk spends a memory request on 16 bytes of each row, a third
// of the requests of the whole weight stream. So they are loaded four chunks at a
// time: for the block of chunks 4q..4q+3, lane (kk, m) loads the 16 bytes of chunk
// 4q + kk of its row m (all four groups of that chunk), the wave writes the 4 x 4
// words of each row to its own LDS area, and at chunk 4q + j lane (kk, m) reads
// word kk of the piece that lane (j, m) loaded. Chunks past the last are clamped
// (in-bounds loads of values never used). A row of fewer than four groups (K < 256,
// a single chunk) loads its words one by one, clamped to the row.
__device__ inline u32x4 load_sbpiece(const Job& jb, int q, int set) {
  const unsigned* row = set ? jb.wsb[1] : jb.wsb[0];
  if (jb.G >= 4) {
    int c = 4 * q + ((threadIdx.x & 63) >> 4);
    c = c < jb.nch ? c : jb.nch - 1;
    return *reinterpret_cast<const u32x4*>(row + 4 * c);
  }
  u32x4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = row[e < jb.G ? e : 0];
  return v;
}

// Each wave owns 4 KB of LDS: two areas (blocks q even / odd), each with 1 KB per
// set. Block q is stored one set at a time during chunks 4q - 2 and 4q - 1, while
// the other area still serves block q - 1; the workgroup barrier at the start of
// every chunk orders a block's stores before the reads of its first chunk.
__device__ inline uint8_t* sb_area(uint8_t* lds_sb, int q, int set) {
  return lds_sb + (threadIdx.x >> 6) * 4096 + (q & 1) * 2048 + set * 1024;
}

__device__ inline void store_sbpiece(uint8_t* lds_sb, int q, int set, const u32x4& v) {
  *reinterpret_cast<u32x4*>(sb_area(lds_sb, q, set) + (threadIdx.x & 63) * 16) = v;
}

__device__ inline void read_sb(uint8_t* lds_sb, int ch, unsigned& sb0, unsigned& sb1) {
  const int lane = threadIdx.x & 63;
  const uint8_t* r = sb_area(lds_sb, ch >> 2, 0) + ((ch & 3) * 16 + (lane & 15)) * 16 + (lane >> 4) * 4;
  sb0 = *reinterpret_cast<const unsigned*>(r);
  sb1 = *reinterpret_cast<const unsigned*>(r + 1024);
}

template <bool DOWN>
__device__ inline const uint16_t* a_row(const PArgs& a, const Job& jb, int r) {
  r = r < jb.nrows ? r : jb.nrows - 1;
  return DOWN ? a.hbuf + (size_t)(jb.row0 + r) * a.I
              : a.a + (size_t)a.rowtok[jb.row0 + r] * a.H;
}

// Activations of chunk ch for one LDS stage. A stage holds MT subtiles of 32
// (kk, i) pieces x 16 rows x 16 B, 512 pieces per subtile; with 64 NWV threads,
// thread t moves pieces p = t + 64 NWV v (v < 8 MT / NWV): subtile p >> 9, row
// m = p & 15 (= t & 15), piece c = (p >> 4) & 31. Positions past K (K < 256)
// re-read the row start: those products meet zero weights.
template <int MT, int NWV>
struct AStage {
  static constexpr int kN = 8 * MT / NWV;
  u32x4 v[kN];
};

template <int MT, int NWV>
__device__ inline void load_achunk(AStage<MT, NWV>& st, const uint16_t* const* rowp, int ch, int K,
                                   int mt_valid) {
#pragma unroll
  for (int v = 0; v < AStage<MT, NWV>::kN; ++v) {
    const int sub = (64 * NWV * v) >> 9;  // a compile-time constant (threadIdx.x < 64 NWV)
    if (sub >= mt_valid) continue;
    const int c = ((int)(threadIdx.x >> 4) + 4 * NWV * v) & 31;
    int k = ch * kKC2 + 64 * (c >> 3) + 8 * (c & 7);
    k = k < K ? k : 8 * (c & 7);
    st.v[v] = *reinterpret_cast<const u32x4*>(rowp[sub] + k);
  }
}

template <int MT, int NWV>
__device__ inline void store_achunk(const AStage<MT, NWV>& st, uint8_t* stage, int mt_valid) {
  const int m = threadIdx.x & 15;
#pragma unroll
  for (int v = 0; v < AStage<MT, NWV>::kN; ++v) {
    const int sub = (64 * NWV * v) >> 9;
    if (sub >= mt_valid) continue;
    const int c = ((int)(threadIdx.x >> 4) + 4 * NWV * v) & 31;
    *reinterpret_cast<u32x4*>(stage + sub * kSubBytes + c * 256 + m * 16) = st.v[v];
  }
}

__device__ inline bf16x8 lds_afrag(const uint8_t* stage, int q, int i) {
  const int lane = threadIdx.x & 63;
  const int kk = lane >> 4, m = lane & 15;
  return __builtin_bit_cast(
      bf16x8, *reinterpret_cast<const u32x4*>(stage + q * kSubBytes + (kk * 8 + i) * 256 + m * 16));
}

// Results of rows mbase..mbase+3 (this lane's C rows of one MFMA subtile).
template <bool DOWN>
__device__ inline void store_rows(const PArgs& a, const Job& jb, const f32x4& c0, const f32x4& c1,
                                  int mbase) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = mbase + r;
    if (m >= jb.nrows) continue;
    if (!DOWN) {
      if (!jb.on[0]) continue;
      const float gv = c0[r], uv = c1[r];
      const float h = gv / (1.f + __expf(-gv)) * uv;
      a.hbuf[(size_t)(jb.row0 + m) * a.I + jb.col[0]] = (uint16_t)(pack_bf16(h, 0.f) & 0xFFFFu);
    } else {
      float* orow = a.obuf + (size_t)(jb.row0 + m) * a.H;
      if (jb.on[0]) orow[jb.col[0]] = c0[r];
      if (jb.on[1]) orow[jb.col[1]] = c1[r];
    }
  }
}

template <int BITS, bool DOWN, int MT, int NWV>
__global__ __launch_bounds__(64 * NWV) void gemm_grouped(PArgs a) {
  extern __shared__ uint8_t lds[];
  Job jb;
  if (!make_job<BITS, DOWN, NWV>(a, MT == 1 ? a.thin : a.thick, jb)) return;
  const int mt_valid = (jb.nrows + 15) >> 4;
  const int lane = threadIdx.x & 63;
  const uint16_t* rowp[MT];
#pragma unroll
  for (int q = 0; q < MT; ++q) rowp[q] = a_row<DOWN>(a, jb, 16 * q + (threadIdx.x & 15));
  const int nch = jb.nch;
  f32x4 acc0[MT], acc1[MT];
#pragma unroll
  for (int q = 0; q < MT; ++q) {
    acc0[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc1[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // activations: LDS stage ch & 1 holds chunk ch, chunk ch + 1 is in registers;
  // weights: chunks ch and ch + 1 in registers, ch + 2 requested during chunk ch
  uint8_t* lds_sb = lds + 2 * MT * kSubBytes;
  AStage<MT, NWV> st;
  WFrag p0, p1, r0, r1;
  load_achunk<MT, NWV>(st, rowp, 0, jb.K, mt_valid);
  {
    const u32x4 v0 = load_sbpiece(jb, 0, 0), v1 = load_sbpiece(jb, 0, 1);
    load_wpair<BITS>(jb, 0, p0, p1);
    load_wpair<BITS>(jb, 1, r0, r1);
    store_sbpiece(lds_sb, 0, 0, v0);
    store_sbpiece(lds_sb, 0, 1, v1);
  }
  store_achunk<MT, NWV>(st, lds, mt_valid);

  auto chunk = [&](int ch, WFrag& f0, WFrag& f1) {
    const uint8_t* cur = lds + (ch & 1) * (MT * kSubBytes);
    uint8_t* nxt = lds + ((ch + 1) & 1) * (MT * kSubBytes);
    __syncthreads();  // stage cur is written; stage nxt is no longer read
    WFrag c0 = f0, c1 = f1;
    read_sb(lds_sb, ch, c0.sb, c1.sb);
    if (ch + 1 < nch) load_achunk<MT, NWV>(st, rowp, ch + 1, jb.K, mt_valid);
    // one set of the next block's (scale, bias) words: set 0 during chunk 4q - 2,
    // set 1 during chunk 4q - 1
    const int bset = ((ch + 2) & 3) == 0 ? 0 : 1;
    const int bq = (ch + 2 - bset) >> 2;
    const bool bnext = ((ch + 2 - bset) & 3) == 0 && 4 * bq < nch;
    u32x4 sbv;
    if (bnext) sbv = load_sbpiece(jb, bq, bset);
    load_wpair<BITS>(jb, ch + 2, f0, f1);
    c0.sb &= jb.sbmask;
    c1.sb &= jb.sbmask;
    if constexpr (MT > 1) {
      // A fragments one octet ahead: the reads of octet i + 1 (every subtile, also
      // those without rows: the stage is always in bounds and their products are
      // never stored) are in flight while octet i is dequantised and multiplied.
      // (A thin tile keeps one read per octet: four more registers would cost it a
      // wave per SIMD.)
      bf16x8 af[MT];
#pragma unroll
      for (int q = 0; q < MT; ++q) af[q] = lds_afrag(cur, q, 0);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        bf16x8 an[MT];
        if (i < 7) {
#pragma unroll
          for (int q = 0; q < MT; ++q) an[q] = lds_afrag(cur, q, i + 1);
        }
        const bf16x8 b0 = deq_octet<BITS>(c0, i);
        const bf16x8 b1 = deq_octet<BITS>(c1, i);
#pragma unroll
        for (int q = 0; q < MT; ++q) {
          if (q < mt_valid) {
            acc0[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[q], b0, acc0[q], 0, 0, 0);
            acc1[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[q], b1, acc1[q], 0, 0, 0);
          }
        }
        if (i < 7) {
#pragma unroll
          for (int q = 0; q < MT; ++q) af[q] = an[q];
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bf16x8 b0 = deq_octet<BITS>(c0, i);
        const bf16x8 b1 = deq_octet<BITS>(c1, i);
#pragma unroll
        for (int q = 0; q < MT; ++q) {
          if (q < mt_valid) {
            const bf16x8 af = lds_afrag(cur, q, i);
            acc0[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, b0, acc0[q], 0, 0, 0);
            acc1[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, b1, acc1[q], 0, 0, 0);
          }
        }
      }
    }
    if (ch + 1 < nch) store_achunk<MT, NWV>(st, nxt, mt_valid);
    if (bnext) store_sbpiece(lds_sb, bq, bset, sbv);
  };
  for (int ch = 0; ch < nch; ch += 2) {
    chunk(ch, p0, p1);
    if (ch + 1 < nch) chunk(ch + 1, r0, r1);
  }
#pragma unroll
  for (int q = 0; q < MT; ++q)
    if (q < mt_valid) store_rows<DOWN>(a, jb, acc0[q], acc1[q], 16 * q + 4 * (lane >> 4));
}

// ---------------------------------------------------------------------------
// combine: y[t] = x_b[t] (residual) + sum_k w[t][k] o[pos[t][k]] + sum_s c_s o_s[t]
// (c_s = 1 without a shared-expert gate).
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
    if (a.sgate) {
      const float c = a.sgc[(size_t)t * kMaxShared + s];
      acc.x = fmaf(c, o.x, acc.x); acc.y = fmaf(c, o.y, acc.y);
      acc.z = fmaf(c, o.z, acc.z); acc.w = fmaf(c, o.w, acc.w);
    } else {
      acc.x += o.x; acc.y += o.y; acc.z += o.z; acc.w += o.w;
    }
  }
  *reinterpret_cast<float4*>(a.y + (size_t)t * a.H + k) = acc;
}

__global__ void clear_err(unsigned* err) {
  if (threadIdx.x == 0) *err = 0u;
}

dim3 xcd_grid(int items) { return dim3((unsigned)(8 * ((items + 7) / 8))); }

// Waves per workgroup: a thin tile's four waves cover 64 intermediate (128 output)
// columns. A thick tile's activation chunk (32 KB from L2 through LDS per chunk)
// serves eight waves, 128 (256) columns, where the layer is that wide: half the
// activation traffic per weight, and one such workgroup (two waves per SIMD) per CU.
constexpr int kThinW = 4, kThickW = 8;

// Dynamic LDS of a GEMM workgroup: two activation stages, then each wave's 4 KB of
// (scale, bias) areas. The thick tiles' 80 / 96 KB exceed the default 64 KB limit.
constexpr size_t lds_bytes(int mt, int nwv) { return 2 * (size_t)mt * kSubBytes + 4096 * (size_t)nwv; }

template <int BITS>
hipError_t gemm_lds_attrs() {
  hipError_t e = hipSuccess;
  const void* k[4] = {reinterpret_cast<const void*>(&gemm_grouped<BITS, false, kThickMT, kThinW>),
                      reinterpret_cast<const void*>(&gemm_grouped<BITS, true, kThickMT, kThinW>),
                      reinterpret_cast<const void*>(&gemm_grouped<BITS, false, kThickMT, kThickW>),
                      reinterpret_cast<const void*>(&gemm_grouped<BITS, true, kThickMT, kThickW>)};
  const size_t b[4] = {lds_bytes(kThickMT, kThinW), lds_bytes(kThickMT, kThinW), lds_bytes(kThickMT, kThickW),
                       lds_bytes(kThickMT, kThickW)};
  for (int i = 0; i < 4 && e == hipSuccess; ++i)
    e = hipFuncSetAttribute(k[i], hipFuncAttributeMaxDynamicSharedMemorySize, (int)b[i]);
  return e;
}

// Column tiles of a gate/up or down pass for workgroups of nwv waves.
inline int nt_of(const PArgs& a, bool down, int nwv) {
  return down ? (a.H + nwv * kDnCols - 1) / (nwv * kDnCols) : (a.I + nwv * kGuCols - 1) / (nwv * kGuCols);
}

// The gate/up and down passes, thin (one m-tile) and thick (kThickMT m-tiles) items.
template <int BITS>
void launch_gemms(const PArgs& a, int thin_max, int thick_max, hipStream_t stream) {
  const dim3 thin_blk(64 * kThinW);
  const size_t lds_thin = lds_bytes(1, kThinW);
  // eight-wave thick workgroups where every wave has columns in both passes
  const bool wide = a.I >= kThickW * kGuCols && a.H >= kThickW * kDnCols;
  hipLaunchKernelGGL((gemm_grouped<BITS, false, 1, kThinW>), xcd_grid(thin_max * nt_of(a, false, kThinW)),
                     thin_blk, lds_thin, stream, a);
  if (thick_max > 0) {
    if (wide)
      hipLaunchKernelGGL((gemm_grouped<BITS, false, kThickMT, kThickW>),
                         xcd_grid(thick_max * nt_of(a, false, kThickW)), dim3(64 * kThickW),
                         lds_bytes(kThickMT, kThickW), stream, a);
    else
      hipLaunchKernelGGL((gemm_grouped<BITS, false, kThickMT, kThinW>),
                         xcd_grid(thick_max * nt_of(a, false, kThinW)), thin_blk,
                         lds_bytes(kThickMT, kThinW), stream, a);
  }
  hipLaunchKernelGGL((gemm_grouped<BITS, true, 1, kThinW>), xcd_grid(thin_max * nt_of(a, true, kThinW)),
                     thin_blk, lds_thin, stream, a);
  if (thick_max > 0) {
    if (wide)
      hipLaunchKernelGGL((gemm_grouped<BITS, true, kThickMT, kThickW>),
                         xcd_grid(thick_max * nt_of(a, true, kThickW)), dim3(64 * kThickW),
                         lds_bytes(kThickMT, kThickW), stream, a);
    else
      hipLaunchKernelGGL((gemm_grouped<BITS, true, kThickMT, kThinW>),
                         xcd_grid(thick_max * nt_of(a, true, kThinW)), thin_blk,
                         lds_bytes(kThickMT, kThinW), stream, a);
  }
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
  a.sgate = c.n_shared > 0 ? lw->shared_gate : nullptr;
  a.err = reinterpret_cast<unsigned*>(ws + pl.err);
  a.a = reinterpret_cast<uint16_t*>(ws + pl.a);
  a.xn = reinterpret_cast<float*>(ws + pl.xn);
  a.logits = reinterpret_cast<float*>(ws + pl.logits);
  a.idx = reinterpret_cast<int*>(ws + pl.idx);
  a.wts = reinterpret_cast<float*>(ws + pl.wts);
  a.pos = reinterpret_cast<int*>(ws + pl.pos);
  a.rowtok = reinterpret_cast<int*>(ws + pl.rowtok);
  a.thin = reinterpret_cast<int4*>(ws + pl.thin);
  a.thick = reinterpret_cast<int4*>(ws + pl.thick);
  a.hbuf = reinterpret_cast<uint16_t*>(ws + pl.hbuf);
  a.obuf = reinterpret_cast<float*>(ws + pl.obuf);
  a.sgc = reinterpret_cast<float*>(ws + pl.sgc);

  // the kernels' dynamic-LDS limits, raised once per device (the grouping kernel and
  // the thick GEMM tiles use more than the default 64 KB)
  {
    static std::mutex mu;
    static bool attr_done[kMaxAttrDevices] = {};
    int dev = 0;
    hipError_t e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) {
      *msg = std::string("hipStreamGetDevice: ") + hipGetErrorString(e);
      return MOE_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxAttrDevices) {
      *msg = "device ordinal beyond the library's limit";
      return MOE_ERR_UNSUPPORTED;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!attr_done[dev]) {
      const size_t group_lds_max = sizeof(int) * (2 * (size_t)kMaxE + kGroupWaves);
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&group_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)group_lds_max);
      if (e == hipSuccess) e = gemm_lds_attrs<2>();
      if (e == hipSuccess) e = gemm_lds_attrs<3>();
      if (e == hipSuccess) e = gemm_lds_attrs<4>();
      if (e != hipSuccess) {
        *msg = std::string("hipFuncSetAttribute: ") + hipGetErrorString(e);
        return MOE_ERR_HIP;
      }
      attr_done[dev] = true;
    }
  }

  hipLaunchKernelGGL(clear_err, dim3(1), dim3(64), 0, stream, a.err);
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
    const size_t glds = sizeof(int) * (2 * (size_t)c.n_experts + kGroupWaves);
    hipLaunchKernelGGL(group_kernel, dim3(1), dim3(1024), glds, stream, a);
    // grids: upper bounds of the m-tiles this pass can have, rounded to whole XCDs.
    // Every expert has at most one thin tile; a thick tile has at least 17 rows.
    const int TK = n * c.top_k;
    const int nz = c.n_experts < TK ? c.n_experts : TK;
    const int thin_max = nz + c.n_shared;
    const int thick_max = TK / 17 + c.n_shared * (n / 17);
    if (c.bits == 4) launch_gemms<4>(a, thin_max, thick_max, stream);
    else if (c.bits == 3) launch_gemms<3>(a, thin_max, thick_max, stream);
    else launch_gemms<2>(a, thin_max, thick_max, stream);
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
