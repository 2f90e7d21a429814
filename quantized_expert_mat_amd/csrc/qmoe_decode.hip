// qmoe_decode.hip -- single-token MoE decode on gfx950.
//
// One token through one layer is three phases; each depends on all of the
// previous one:
//   A  RMSNorm of x (every workgroup recomputes it from the 16 KB input), router
//      logits (float32 mat-vec), shared expert gate/up + SwiGLU -> h_shared.
//   B  top-K over the logits (every workgroup recomputes it from the logits),
//      routed experts gate/up + SwiGLU -> h_k.
//   C  down projections of the routed and shared experts, weighted combine and
//      residual -> the next layer's input.
// The flash-moe page runs the same chain per layer on its GPU and feeds the
// combine + norm + residual result straight into the next layer ("Deferred GPU
// Expert Compute" section of "Flash-MoE - Chạy mô hình 397 tỷ tham số trên
// laptop", vi.news.hada.io); here the whole token/layer loop runs inside one
// persistent kernel whose workgroups meet at grid barriers between phases, so no
// host round trip or kernel launch sits between layers (the page's pre-encoded
// command buffers remove a per-layer dispatch gap for the same reason,
// "Optimizaciones Efectivas" section of the autoresearch page).
//
// Dequant mat-vec. The page rewrites (nibble*scale + bias)*x as
// fma(nibble, scale*x, bias*x) ("Kernel dequant tối ưu FMA"). Carried one step
// further, a 64-group contributes scale*sum(q*x) + bias*sum(x); sum(x) per group
// is computed once per vector, so the inner loop is just sum(q*x). That inner
// loop runs on the integer dot-product unit: x is scaled by a power of two to a
// 23-bit integer and split into six signed base-16 digits, the codes are stored
// as signed nibbles (q - 8), and v_dot8_i32_i4 forms eight 4-bit products per
// instruction with exact int32 accumulation. One weight element then costs about
// one VALU operation instead of two and a half for convert + FMA, which keeps the
// 4-bit path under the HBM roofline instead of next to it.
//
// Work split. A block of the packed layout is one wave's worth: lane = (row,
// group). Gate/up items are (expert, block); down items are rows owned by a
// workgroup, with lanes spread over (row, expert, group) so a lane's activation
// digits stay in registers for every row it visits.
#include <algorithm>
#include <cstring>

#include "qmoe_internal.h"

namespace qmoe {

constexpr int kThreads = 256;
constexpr int kNW = kThreads / kWave;  // waves per workgroup
constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23: adding it rounds to an integer in the low mantissa
constexpr int kMaxPass = kMaxK + kMaxShared;
constexpr int kBatch = 4;  // items whose loads are issued before the first is reduced

enum Mode { MODE_LAYER = 0, MODE_ROUTE = 1, MODE_EXPERT = 2 };

struct DecodeArgs {
  Geo geo;
  int E, K, S, flags, mode;
  float eps;
  int L, T;
  const LayerPtrs* layers;
  const uint8_t* single_expert;  // MODE_EXPERT
  const float* x0;               // [T][H]
  float* y;                      // [T][H]
  const uint8_t* boost_mask;     // [T][L][K]
  const float* sel_bias;         // [T][E]
  const int* boosted;            // [T][K]
  int* idx_out;                  // [T][L][K]
  float* w_out;                  // [T][L][K]
  float* logits_out;             // [T][E]
  float* xbuf;                   // [2][H]
  float* logits;                 // [E]
  float* hbuf;                   // [K+S][I]
  int* sel;                      // [2*kMaxK]
  int* prev;                     // [2][L][kMaxK]
  unsigned* sync;                // [0] barrier counter, [1] abort flag
  unsigned* err;
  unsigned long long timeout_ticks;
  unsigned long long* trace;     // optional [T][L][16] wall-clock stamps from workgroup 0
  int nwg;
  int rpw;                       // phase C output rows per workgroup
  int npass;
  int pass_first[kMaxPass], pass_count[kMaxPass];
  int lds_xn, lds_xdig, lds_xsum, lds_hdig, lds_hsum, lds_acc, lds_words;
};

// Small per-workgroup state kept in LDS across phases.
struct Small {
  unsigned long long red64[kNW];
  float redf[kNW][kMaxPass + 2];
  int sel_idx[kMaxK];
  float sel_w[kMaxK];
  int boosted[kMaxK];
  int nboost;
  int ok;
  float xs_x;
  float hsc[kMaxPass];
  float hxs[kMaxPass];
  unsigned long long* tr;  // trace row (workgroup 0, thread 0 only)
};

#define SUBSTAMP(i) \
  if (threadIdx.x == 0 && s.sm->tr) s.sm->tr[i] = wall_clock64();

struct Lds {
  Small* sm;
  float* xn;
  unsigned* xdig;
  float* xsum;
  unsigned* hdig;
  float* hsum;
  float* acc;
};

__device__ inline Lds lds_view(unsigned* raw, const DecodeArgs& a) {
  Lds s;
  s.sm = reinterpret_cast<Small*>(raw);
  s.xn = reinterpret_cast<float*>(raw + a.lds_xn);
  s.xdig = raw + a.lds_xdig;
  s.xsum = reinterpret_cast<float*>(raw + a.lds_xsum);
  s.hdig = raw + a.lds_hdig;
  s.hsum = reinterpret_cast<float*>(raw + a.lds_hsum);
  s.acc = reinterpret_cast<float*>(raw + a.lds_acc);
  return s;
}

// ---------------------------------------------------------------- reductions
__device__ inline float seg_sum(float v, int width) {
  for (int o = width >> 1; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ inline float wave_max(float v) {
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ inline float wave_sum(float v) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ inline unsigned long long wave_max_u64(unsigned long long v) {
  for (int o = 32; o >= 1; o >>= 1) {
    unsigned long long w = __shfl_xor(v, o);
    v = w > v ? w : v;
  }
  return v;
}

// Power-of-two scale that maps |v| <= m into (-2^22, 2^22).
__device__ inline void digit_scale(float m, float* sc, float* xs) {
  if (!(m > 0.f) || !isfinite(m)) {
    *sc = 1.f;
    *xs = 1.f;
    return;
  }
  int e;
  frexpf(m, &e);  // m = f * 2^e, 0.5 <= f < 1, so m < 2^e
  *sc = ldexpf(1.f, 22 - e);
  *xs = ldexpf(1.f, e - 22);
}

// ------------------------------------------------------------ digit encoding
// Values v (scaled by sc, |v*sc| < 2^22) become integers i = rint(v*sc) whose six
// balanced base-16 digits t_d in [-8, 7] satisfy i = sum t_d 16^d. Adding 0x888888
// makes every digit t_d + 8 a plain nibble, so the digits of all values are read
// off the nibbles of one word (then XOR 8 turns t_d + 8 into the signed nibble t_d).
// For the dot product, digit d of eight values is packed into one dword: nibble 2m
// holds value m and nibble 2m+1 holds value 4+m (m = 0..3); the packed codes use
// the same order. The 8x8 nibble transpose is done with byte permutes.
__device__ inline void transpose4(unsigned a, unsigned b, unsigned c, unsigned d, unsigned& t0,
                                  unsigned& t1, unsigned& t2) {
  const unsigned a01l = __builtin_amdgcn_perm(b, a, 0x05010400u);
  const unsigned a01h = __builtin_amdgcn_perm(b, a, 0x0C0C0602u);
  const unsigned a23l = __builtin_amdgcn_perm(d, c, 0x05010400u);
  const unsigned a23h = __builtin_amdgcn_perm(d, c, 0x0C0C0602u);
  t0 = __builtin_amdgcn_perm(a23l, a01l, 0x05040100u);
  t1 = __builtin_amdgcn_perm(a23l, a01l, 0x07060302u);
  t2 = __builtin_amdgcn_perm(a23h, a01h, 0x05040100u);
}

__device__ inline unsigned bfi(unsigned m, unsigned a, unsigned b) { return (m & a) | (~m & b); }

// Encode one chunk of 8 values; writes 6 digit dwords; returns the integer sum.
__device__ inline int encode_chunk(const float v[8], float sc, unsigned out[6]) {
  unsigned D[8];
  int isum = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const unsigned u = __float_as_uint(fmaf(v[i], sc, kMagic));
    isum += (int)(u - 0x4B400000u);
    D[i] = u + 0xB5488888u;  // (i + 0x888888) in the low 24 bits
  }
  unsigned T0, T1, T2, U0, U1, U2;
  transpose4(D[0], D[1], D[2], D[3], T0, T1, T2);
  transpose4(D[4], D[5], D[6], D[7], U0, U1, U2);
  out[0] = bfi(0x0F0F0F0Fu, T0, U0 << 4) ^ 0x88888888u;
  out[1] = bfi(0x0F0F0F0Fu, T0 >> 4, U0) ^ 0x88888888u;
  out[2] = bfi(0x0F0F0F0Fu, T1, U1 << 4) ^ 0x88888888u;
  out[3] = bfi(0x0F0F0F0Fu, T1 >> 4, U1) ^ 0x88888888u;
  out[4] = bfi(0x0F0F0F0Fu, T2, U2 << 4) ^ 0x88888888u;
  out[5] = bfi(0x0F0F0F0Fu, T2 >> 4, U2) ^ 0x88888888u;
  return isum;
}

// Encode nvec vectors of length n (multiple of 64), vector j at src + j*stride,
// with per-vector scales sc[j]. Digits for (vector j, group g) go to
// dig[(j*G + g)*kDigitStride + dw*6 + d]; sums to sum[2*(j*G+g)] = 8*sum(ints),
// sum[2*(j*G+g)+1] = float sum of the values. Whole workgroup participates.
__device__ void encode_vectors(const float* src, size_t stride, int nvec, int n, const float* sc,
                               unsigned* dig, float* sum) {
  const int G = n / kGroup;
  const int chunks_per_vec = n / 8;
  const int total = nvec * chunks_per_vec;
  // total is a multiple of 8 and kThreads is a multiple of 64: the 8 chunks of a
  // group always sit in 8 consecutive lanes of one wave.
  for (int base = 0; base < total; base += kThreads) {
    const int c = base + (int)threadIdx.x;
    int isum = 0;
    float fsum = 0.f;
    const bool active = c < total;
    int j = 0, cc = 0;
    if (active) {
      j = c / chunks_per_vec;
      cc = c % chunks_per_vec;
      const float4* p = reinterpret_cast<const float4*>(src + (size_t)j * stride + (size_t)cc * 8);
      const float4 v0 = p[0], v1 = p[1];
      const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      unsigned o[6];
      isum = encode_chunk(v, sc[j], o);
#pragma unroll
      for (int i = 0; i < 8; ++i) fsum += v[i];
      const int g = cc / 8, dw = cc % 8;
      unsigned* dst = dig + (size_t)(j * G + g) * kDigitStride + dw * 6;
#pragma unroll
      for (int d = 0; d < 6; ++d) dst[d] = o[d];
    }
    for (int o = 1; o < 8; o <<= 1) {
      isum += __shfl_xor(isum, o);
      fsum += __shfl_xor(fsum, o);
    }
    if (active && (cc % 8) == 0) {
      const int g = cc / 8;
      sum[2 * (j * G + g)] = 8.f * (float)isum;
      sum[2 * (j * G + g) + 1] = fsum;
    }
  }
}

// ------------------------------------------------------------ dequant dot
struct Dig {
  unsigned d[48];
  float X8, Xf, xs;
};

__device__ inline void load_dig(Dig& D, const unsigned* dig, const float* sum, int idx, float xs) {
  const uint4* p = reinterpret_cast<const uint4*>(dig + (size_t)idx * kDigitStride);
#pragma unroll
  for (int i = 0; i < 12; ++i) {
    const uint4 v = p[i];
    D.d[4 * i] = v.x;
    D.d[4 * i + 1] = v.y;
    D.d[4 * i + 2] = v.z;
    D.d[4 * i + 3] = v.w;
  }
  D.X8 = sum[2 * idx];
  D.Xf = sum[2 * idx + 1];
  D.xs = xs;
}

struct Slot {
  uint4 c0, c1;
  unsigned sb;
};

template <int BITS>
__device__ inline Slot ld_slot(const uint8_t* blk, int slot) {
  Slot s;
  s.c0 = reinterpret_cast<const uint4*>(blk)[slot];
  if (BITS == 4) {
    s.c1 = reinterpret_cast<const uint4*>(blk + 1024)[slot];
    s.sb = reinterpret_cast<const unsigned*>(blk + 2048)[slot];
  } else {
    s.c1 = make_uint4(0, 0, 0, 0);
    s.sb = reinterpret_cast<const unsigned*>(blk + 1024)[slot];
  }
  return s;
}

// Contribution of one (row, group) slot: scale*sum(q*x) + bias*sum(x).
template <int BITS>
__device__ inline float slot_dot(const Slot& s, const Dig& D) {
  unsigned cw[8];
  if (BITS == 4) {
    cw[0] = s.c0.x; cw[1] = s.c0.y; cw[2] = s.c0.z; cw[3] = s.c0.w;
    cw[4] = s.c1.x; cw[5] = s.c1.y; cw[6] = s.c1.z; cw[7] = s.c1.w;
  } else {
    const unsigned w[4] = {s.c0.x, s.c0.y, s.c0.z, s.c0.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      cw[2 * j] = w[j] & 0x33333333u;
      cw[2 * j + 1] = (w[j] >> 2) & 0x33333333u;
    }
  }
  int S0 = 0, S1 = 0, S2 = 0, S3 = 0, S4 = 0, S5 = 0;
#pragma unroll
  for (int dw = 0; dw < 8; ++dw) {
    const int c = (int)cw[dw];
    S0 = __builtin_amdgcn_sdot8(c, (int)D.d[dw * 6 + 0], S0, false);
    S1 = __builtin_amdgcn_sdot8(c, (int)D.d[dw * 6 + 1], S1, false);
    S2 = __builtin_amdgcn_sdot8(c, (int)D.d[dw * 6 + 2], S2, false);
    S3 = __builtin_amdgcn_sdot8(c, (int)D.d[dw * 6 + 3], S3, false);
    S4 = __builtin_amdgcn_sdot8(c, (int)D.d[dw * 6 + 4], S4, false);
    S5 = __builtin_amdgcn_sdot8(c, (int)D.d[dw * 6 + 5], S5, false);
  }
  const int plo = S0 + (S1 << 4) + (S2 << 8);
  const int phi = S3 + (S4 << 4) + (S5 << 8);
  const float pf = fmaf((float)phi, 4096.f, (float)plo);  // sum((q-8)*i) or sum(q*i)
  const float sc = bf16lo_to_f32(s.sb), bi = bf16hi_to_f32(s.sb);
  if (BITS == 4) return fmaf(sc, (pf + D.X8) * D.xs, bi * D.Xf);
  return fmaf(sc, pf * D.xs, bi * D.Xf);
}

__device__ inline float silu(float z) { return z / (1.f + expf(-z)); }

// ------------------------------------------------------------ grid barrier
__device__ bool grid_sync(const DecodeArgs& a, Small* sm, unsigned index) {
  __syncthreads();
  if (threadIdx.x == 0) {
    int ok = 1;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_fetch_add(a.sync, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned target = index * (unsigned)a.nwg;
    const unsigned long long t0 = wall_clock64();
    unsigned spins = 0;
    while (__hip_atomic_load(a.sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
      __builtin_amdgcn_s_sleep(1);
      if ((++spins & 255u) == 0) {
        if (__hip_atomic_load(a.sync + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
          ok = 0;
          break;
        }
        if (wall_clock64() - t0 > a.timeout_ticks) {
          __hip_atomic_store(a.sync + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          set_dev_err(a.err, DEV_SYNC_TIMEOUT);
          ok = 0;
          break;
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    sm->ok = ok;
  }
  __syncthreads();
  return sm->ok != 0;
}

// ------------------------------------------------------------ phase pieces
__device__ inline const float* token_input(const DecodeArgs& a, int t, int l) {
  return l == 0 ? a.x0 + (size_t)t * a.geo.H : a.xbuf + (size_t)(l & 1) * a.geo.H;
}

// x -> LDS (normalised if requested) -> digits for the gate/up mat-vecs.
__device__ void prepare_x(const DecodeArgs& a, const Lds& s, int t, int l) {
  const int H = a.geo.H;
  const float* x = token_input(a, t, l);
  const float* gamma = a.mode == MODE_EXPERT ? nullptr : a.layers[l].gamma;
  const bool norm = a.mode != MODE_EXPERT && (a.flags & MOE_F_RMSNORM);
  float ss = 0.f, mx = 0.f;
  for (int i = threadIdx.x * 4; i < H; i += kThreads * 4) {
    float4 v = *reinterpret_cast<const float4*>(x + i);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    if (gamma) {
      const float4 gm = *reinterpret_cast<const float4*>(gamma + i);
      v.x *= gm.x; v.y *= gm.y; v.z *= gm.z; v.w *= gm.w;
    }
    *reinterpret_cast<float4*>(s.xn + i) = v;
    mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
  ss = wave_sum(ss);
  mx = wave_max(mx);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x % kWave) == 0) {
    s.sm->redf[w][0] = ss;
    s.sm->redf[w][1] = mx;
  }
  __syncthreads();
  ss = 0.f;
  mx = 0.f;
  for (int i = 0; i < kNW; ++i) {
    ss += s.sm->redf[i][0];
    mx = fmaxf(mx, s.sm->redf[i][1]);
  }
  const float rinv = norm ? 1.f / sqrtf(ss / (float)H + a.eps) : 1.f;
  if (norm) {
    for (int i = threadIdx.x * 4; i < H; i += kThreads * 4) {
      float4 v = *reinterpret_cast<float4*>(s.xn + i);
      v.x *= rinv; v.y *= rinv; v.z *= rinv; v.w *= rinv;
      *reinterpret_cast<float4*>(s.xn + i) = v;
    }
  }
  float sc, xs;
  digit_scale(mx * rinv, &sc, &xs);
  __syncthreads();
  encode_vectors(s.xn, 0, 1, H, &sc, s.xdig, s.xsum);
  if (threadIdx.x == 0) s.sm->xs_x = xs;
  __syncthreads();
}

// Gate/up + SwiGLU over n_items (expert, block) items. Item k runs on global
// wave (rot + k) mod (nwg * kNW), where global wave = blockIdx.x + nwg * wave, so
// consecutive items land on different compute units. item(k, base, hout, blk)
// names the expert, the block and the h vector of item k.
template <int BITS, typename ItemFn>
__device__ void gateup_items(const DecodeArgs& a, const Lds& s, int n_items, int rot,
                             ItemFn item) {
  const Geo& g = a.geo;
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int waves = a.nwg * kNW;
  const int gw = blockIdx.x + a.nwg * w;
  const int k0 = (gw - rot % waves + waves) % waves;
  if (k0 >= n_items) return;
  const int p = lane / g.Gh, grp = lane % g.Gh;
  Dig D;
  load_dig(D, s.xdig, s.xsum, grp, s.sm->xs_x);
  for (int i0 = k0; i0 < n_items; i0 += kBatch * waves) {
    Slot G[kBatch], U[kBatch];
    float* hout[kBatch];
    int row[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int i = i0 + j * waves;
      hout[j] = nullptr;
      row[j] = 0;
      if (i < n_items) {
        const uint8_t* base;
        int blk;
        item(i, base, hout[j], blk);
        G[j] = ld_slot<BITS>(base + (size_t)blk * g.blk, lane);
        U[j] = ld_slot<BITS>(base + g.off_up + (size_t)blk * g.blk, lane);
        row[j] = blk * g.Ph + p;
      }
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (hout[j] == nullptr) continue;
      const float pg = seg_sum(slot_dot<BITS>(G[j], D), g.Gh);
      const float pu = seg_sum(slot_dot<BITS>(U[j], D), g.Gh);
      if (grp == 0 && row[j] < g.I) hout[j][row[j]] = silu(pg) * pu;
    }
  }
}

// Router logits for rows assigned to this wave (items 0..E-1 of phase A).
__device__ void router_items(const DecodeArgs& a, const Lds& s, int t, int l) {
  const int H = a.geo.H, E = a.E;
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int stride = a.nwg * kNW;
  const int my0 = blockIdx.x + a.nwg * w;
  if (my0 >= E) return;
  const float* W = a.layers[l].router;
  const int nq = H / 4;  // float4 columns
  constexpr int kMaxC = kMaxDim / 256;
  float4 xr[kMaxC];
#pragma unroll
  for (int c = 0; c < kMaxC; ++c) {
    const int q = lane + kWave * c;
    xr[c] = q < nq ? reinterpret_cast<const float4*>(s.xn)[q] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int e = my0; e < E; e += stride) {
    const float4* row = reinterpret_cast<const float4*>(W + (size_t)e * H);
    float4 wv[kMaxC];
#pragma unroll
    for (int c = 0; c < kMaxC; ++c) {
      const int q = lane + kWave * c;
      wv[c] = q < nq ? row[q] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < kMaxC; ++c) {
      acc = fmaf(wv[c].x, xr[c].x, acc);
      acc = fmaf(wv[c].y, xr[c].y, acc);
      acc = fmaf(wv[c].z, xr[c].z, acc);
      acc = fmaf(wv[c].w, xr[c].w, acc);
    }
    acc = wave_sum(acc);
    if (lane == 0) {
      a.logits[e] = acc;
      if (a.logits_out) a.logits_out[(size_t)t * E + e] = acc;
    }
  }
}

template <int BITS>
__device__ void phase_a(const DecodeArgs& a, const Lds& s, int t, int l) {
  prepare_x(a, s, t, l);
  SUBSTAMP(8);
  router_items(a, s, t, l);
  SUBSTAMP(9);
  if (a.mode == MODE_LAYER && a.S > 0) {
    const Geo& g = a.geo;
    const uint8_t* shared = a.layers[l].shared;
    // shared items continue the round-robin on the waves after the router rows
    auto fn = [&](int i, const uint8_t*& base, float*& hout, int& blk) {
      const int sh = i / g.nblk_gu;
      blk = i % g.nblk_gu;
      base = shared + (size_t)sh * g.expert_bytes;
      hout = a.hbuf + (size_t)(a.K + sh) * g.I;
    };
    gateup_items<BITS>(a, s, a.S * g.nblk_gu, a.E, fn);
  }
}

__device__ inline unsigned ord_f32(float f) {
  const unsigned u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Top-K with the temporal tier, then softmax over the selected logits.
__device__ void select_topk(const DecodeArgs& a, const Lds& s, int t, int l) {
  const int E = a.E, K = a.K;
  if (threadIdx.x == 0) {
    int nb = 0;
    if (a.mode == MODE_LAYER && a.boost_mask && t > 0) {
      const uint8_t* m = a.boost_mask + ((size_t)t * a.L + l) * K;
      const int* ps = a.prev + ((size_t)((t - 1) & 1) * a.L + l) * kMaxK;
      for (int j = 0; j < K; ++j)
        if (m[j]) s.sm->boosted[nb++] = ps[j];
    } else if (a.boosted) {
      const int* b = a.boosted + (size_t)t * K;
      for (int j = 0; j < K; ++j) {
        const int e = b[j];
        if (e >= 0 && e < E) s.sm->boosted[nb++] = e;
        else if (e >= E || e < -1) set_dev_err(a.err, DEV_BAD_INDEX);
      }
    }
    s.sm->nboost = nb;
  }
  __syncthreads();
  const int nb = s.sm->nboost;
  const bool by_bias = (a.flags & MOE_F_SELECT_BY_BIAS) != 0;
  const float* sb = a.sel_bias ? a.sel_bias + (size_t)t * E : nullptr;
  constexpr int kPer = kMaxE / kThreads;
  unsigned long long key[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int e = threadIdx.x + kThreads * r;
    key[r] = 0;
    if (e < E) {
      const float lg = a.logits[e];
      const float sc = by_bias ? (sb ? sb[e] : 0.f) : lg + (sb ? sb[e] : 0.f);
      unsigned tier = 0;
      for (int j = 0; j < nb; ++j) tier |= (s.sm->boosted[j] == e) ? 1u : 0u;
      key[r] = ((unsigned long long)(tier + 1u) << 42) | ((unsigned long long)ord_f32(sc) << 10) |
               (unsigned long long)(kMaxE - 1 - e);
    }
  }
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  for (int k = 0; k < K; ++k) {
    unsigned long long best = 0;
#pragma unroll
    for (int r = 0; r < kPer; ++r) best = key[r] > best ? key[r] : best;
    best = wave_max_u64(best);
    if (lane == 0) s.sm->red64[w] = best;
    __syncthreads();
    best = 0;
    for (int i = 0; i < kNW; ++i) best = s.sm->red64[i] > best ? s.sm->red64[i] : best;
    const int e = kMaxE - 1 - (int)(best & 1023ull);
#pragma unroll
    for (int r = 0; r < kPer; ++r)
      if (key[r] == best) key[r] = 0;
    if (threadIdx.x == 0) s.sm->sel_idx[k] = e;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    float lg[kMaxK], m = -INFINITY;
    for (int k = 0; k < K; ++k) {
      lg[k] = a.logits[s.sm->sel_idx[k]];
      m = fmaxf(m, lg[k]);
    }
    float z = 0.f;
    for (int k = 0; k < K; ++k) {
      lg[k] = expf(lg[k] - m);
      z += lg[k];
    }
    for (int k = 0; k < K; ++k) s.sm->sel_w[k] = lg[k] / z;
  }
  __syncthreads();
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    // publish for the next phase's launch (phased mode), the outputs, and the
    // sorted set for the next token's temporal tier
    for (int k = 0; k < K; ++k) {
      a.sel[k] = s.sm->sel_idx[k];
      a.sel[kMaxK + k] = __float_as_int(s.sm->sel_w[k]);
    }
    size_t o = ((size_t)t * a.L + l) * K;
    if (a.idx_out)
      for (int k = 0; k < K; ++k) a.idx_out[o + k] = s.sm->sel_idx[k];
    if (a.w_out)
      for (int k = 0; k < K; ++k) a.w_out[o + k] = s.sm->sel_w[k];
    if (a.mode == MODE_LAYER) {
      int srt[kMaxK];
      for (int k = 0; k < K; ++k) srt[k] = s.sm->sel_idx[k];
      for (int i = 1; i < K; ++i)
        for (int j = i; j > 0 && srt[j - 1] > srt[j]; --j) {
          const int tmp = srt[j];
          srt[j] = srt[j - 1];
          srt[j - 1] = tmp;
        }
      int* ps = a.prev + ((size_t)(t & 1) * a.L + l) * kMaxK;
      for (int k = 0; k < K; ++k) ps[k] = srt[k];
    }
  }
}

template <int BITS>
__device__ void phase_b(const DecodeArgs& a, const Lds& s, int t, int l) {
  if (a.mode == MODE_EXPERT) {
    auto fn = [&](int i, const uint8_t*& base, float*& hout, int& blk) {
      base = a.single_expert;
      blk = i;
      hout = a.hbuf;
    };
    gateup_items<BITS>(a, s, a.geo.nblk_gu, 0, fn);
    return;
  }
  select_topk(a, s, t, l);
  SUBSTAMP(10);
  if (a.mode != MODE_LAYER) return;
  const Geo& g = a.geo;
  const uint8_t* experts = a.layers[l].experts;
  auto fn = [&](int i, const uint8_t*& base, float*& hout, int& blk) {
    const int k = i / g.nblk_gu;
    blk = i % g.nblk_gu;
    base = experts + (size_t)s.sm->sel_idx[k] * g.expert_bytes;
    hout = a.hbuf + (size_t)k * g.I;
  };
  gateup_items<BITS>(a, s, a.K * g.nblk_gu, 0, fn);
}

template <int BITS>
__device__ void phase_c(const DecodeArgs& a, const Lds& s, int t, int l) {
  const Geo& g = a.geo;
  const int H = g.H, I = g.I;
  const bool expert_mode = a.mode == MODE_EXPERT;
  const int nlist = expert_mode ? 1 : a.K + a.S;
  // digits of every h vector (each workgroup encodes all of them)
  {
    float mx[kMaxPass];
    for (int j = 0; j < nlist; ++j) mx[j] = 0.f;
    for (int i = threadIdx.x; i < I; i += kThreads)
      for (int j = 0; j < nlist; ++j) mx[j] = fmaxf(mx[j], fabsf(a.hbuf[(size_t)j * I + i]));
    const int w = threadIdx.x / kWave;
    for (int j = 0; j < nlist; ++j) {
      const float m = wave_max(mx[j]);
      if ((threadIdx.x % kWave) == 0) s.sm->redf[w][j] = m;
    }
    __syncthreads();
    if ((int)threadIdx.x < nlist) {
      float m = 0.f;
      for (int i = 0; i < kNW; ++i) m = fmaxf(m, s.sm->redf[i][threadIdx.x]);
      digit_scale(m, &s.sm->hsc[threadIdx.x], &s.sm->hxs[threadIdx.x]);
    }
    __syncthreads();
    encode_vectors(a.hbuf, (size_t)I, nlist, I, s.sm->hsc, s.hdig, s.hsum);
    __syncthreads();
  }
  SUBSTAMP(11);
  const int rpw = a.rpw;
  const int r0 = blockIdx.x * rpw;
  const int r1 = min(H, r0 + rpw);
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int npass = expert_mode ? 1 : a.npass;
  if (r0 < r1) {
    for (int pi = 0; pi < npass; ++pi) {
      const int first = expert_mode ? 0 : a.pass_first[pi];
      const int n = expert_mode ? 1 : a.pass_count[pi];
      const int seg = n * g.Gi;
      const int Pp = kWave / seg;
      const int grp = lane % g.Gi, kl = (lane / g.Gi) % n, p = lane / seg;
      const int li = first + kl;  // index in the expert list
      const uint8_t* ex;
      float wk;
      if (expert_mode) {
        ex = a.single_expert;
        wk = 1.f;
      } else if (li < a.K) {
        ex = a.layers[l].experts + (size_t)s.sm->sel_idx[li] * g.expert_bytes;
        wk = s.sm->sel_w[li];
      } else {
        ex = a.layers[l].shared + (size_t)(li - a.K) * g.expert_bytes;
        wk = 1.f;
      }
      const uint8_t* down = ex + g.off_down;
      const int nchunk = (r1 - r0 + Pp - 1) / Pp;
      if (w >= nchunk) continue;
      Dig D;
      load_dig(D, s.hdig, s.hsum, li * g.Gi + grp, s.sm->hxs[li]);
      for (int c0 = w; c0 < nchunk; c0 += kBatch * kNW) {
        Slot S[kBatch];
        int row[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int c = c0 + j * kNW;
          row[j] = r0 + c * Pp + p;
          if (c < nchunk && row[j] < r1) {
            const int b = row[j] / g.Pi, pd = row[j] % g.Pi;
            S[j] = ld_slot<BITS>(down + (size_t)b * g.blk, pd * g.Gi + grp);
          }
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int c = c0 + j * kNW;
          if (c >= nchunk) continue;
          const bool valid = row[j] < r1;
          float part = valid ? slot_dot<BITS>(S[j], D) * wk : 0.f;
          part = seg_sum(part, seg);
          if (valid && (lane % seg) == 0) s.acc[pi * rpw + (row[j] - r0)] = part;
        }
      }
    }
  }
  __syncthreads();
  SUBSTAMP(12);
  if (r0 < r1) {
    const bool res = !expert_mode && (a.flags & MOE_F_RESIDUAL);
    const float* xin = token_input(a, t, l);
    float* out;
    if (expert_mode || l == a.L - 1) out = a.y + (size_t)t * H;
    else out = a.xbuf + (size_t)((l + 1) & 1) * H;
    for (int r = r0 + threadIdx.x; r < r1; r += kThreads) {
      float v = res ? xin[r] : 0.f;
      for (int pi = 0; pi < npass; ++pi) v += s.acc[pi * rpw + (r - r0)];
      out[r] = v;
    }
  }
}

// only_phase < 0: persistent (all tokens, all layers, grid barriers between phases).
// only_phase = 0/1/2: run that phase for token t_only, layer l_only.
template <int BITS>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a, int only_phase, int t_only,
                                                          int l_only) {
  extern __shared__ __align__(16) unsigned lds_raw[];
  const Lds s = lds_view(lds_raw, a);
  const bool persistent = only_phase < 0;
  const int t0 = persistent ? 0 : t_only, t1 = persistent ? a.T : t_only + 1;
  const int l0 = persistent ? 0 : l_only, l1 = persistent ? a.L : l_only + 1;
  unsigned bar = 0;
  unsigned long long* tr = nullptr;
  for (int t = t0; t < t1; ++t) {
    for (int l = l0; l < l1; ++l) {
      if (a.trace && blockIdx.x == 0 && threadIdx.x == 0) tr = a.trace + ((size_t)t * a.L + l) * 16;
#define QMOE_STAMP(i) \
  if (tr) tr[i] = wall_clock64();
      if (threadIdx.x == 0) s.sm->tr = tr;
      QMOE_STAMP(0);
      bool have_x = false;
      if (a.mode != MODE_EXPERT && (persistent || only_phase == 0)) {
        phase_a<BITS>(a, s, t, l);
        have_x = true;
        QMOE_STAMP(1);
        if (persistent && !grid_sync(a, s.sm, ++bar)) return;
        QMOE_STAMP(2);
      }
      if (persistent || only_phase == 1) {
        if (!have_x && a.mode != MODE_ROUTE) prepare_x(a, s, t, l);
        phase_b<BITS>(a, s, t, l);
        QMOE_STAMP(3);
        if (persistent && !grid_sync(a, s.sm, ++bar)) return;
        QMOE_STAMP(4);
      }
      if (a.mode != MODE_ROUTE && (persistent || only_phase == 2)) {
        if (!persistent && a.mode == MODE_LAYER) {
          if (threadIdx.x < a.K) {
            s.sm->sel_idx[threadIdx.x] = a.sel[threadIdx.x];
            s.sm->sel_w[threadIdx.x] = __int_as_float(a.sel[kMaxK + threadIdx.x]);
          }
          __syncthreads();
        }
        phase_c<BITS>(a, s, t, l);
        QMOE_STAMP(5);
        if (persistent && !grid_sync(a, s.sm, ++bar)) return;
        QMOE_STAMP(6);
      }
#undef QMOE_STAMP
    }
  }
}

__global__ void zero_words(unsigned* p, int n, unsigned* q, int m) {
  if ((int)threadIdx.x < n) p[threadIdx.x] = 0u;
  if ((int)threadIdx.x < m) q[threadIdx.x] = 0u;
}

// ------------------------------------------------------------ host side
static int g_num_cu = -1;
unsigned long long* g_trace = nullptr;  // set only by instrumented builds
static long long g_wall_khz = -1;

static hipError_t device_info() {
  if (g_num_cu > 0) return hipSuccess;
  int dev;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int cu = 0, khz = 0;
  e = hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
  if (e != hipSuccess || khz <= 0) khz = 100000;
  g_num_cu = cu;
  g_wall_khz = khz;
  return hipSuccess;
}

hipError_t launch_decode(const DecodeRequest& r, hipStream_t stream, const char** why) {
  hipError_t e = device_info();
  if (e != hipSuccess) return e;
  const moe_config& c = r.cfg;
  DecodeArgs a;
  memset(&a, 0, sizeof(a));
  a.geo = make_geo(c.hidden, c.inter, c.bits);
  a.E = c.n_experts;
  a.K = c.top_k;
  a.S = c.n_shared;
  a.flags = c.flags;
  a.mode = r.mode;
  a.eps = c.eps;
  a.L = r.L;
  a.T = r.T;
  a.layers = r.layers_dev;
  a.single_expert = r.single_expert;
  a.x0 = r.x0;
  a.y = r.y;
  a.boost_mask = r.boost_mask;
  a.sel_bias = r.sel_bias;
  a.boosted = r.boosted;
  a.idx_out = r.idx_out;
  a.w_out = r.w_out;
  a.logits_out = r.logits_out;
  uint8_t* ws = r.ws;
  a.xbuf = reinterpret_cast<float*>(ws + r.wl.xbuf);
  a.logits = reinterpret_cast<float*>(ws + r.wl.logits);
  a.hbuf = reinterpret_cast<float*>(ws + r.wl.hbuf);
  a.sel = reinterpret_cast<int*>(ws + r.wl.sel);
  a.prev = reinterpret_cast<int*>(ws + r.wl.prev);
  a.sync = reinterpret_cast<unsigned*>(ws + r.wl.sync);
  a.err = reinterpret_cast<unsigned*>(ws + r.wl.err);
  a.timeout_ticks = (unsigned long long)g_wall_khz * 2000ull;  // 2 seconds per barrier wait
  a.trace = g_trace;

  // Expert passes for phase C: routed experts in power-of-two groups that fit a
  // wave (lanes = rows x experts x groups), then the shared experts.
  const int Gi = a.geo.Gi;
  const int maxn = kWave / Gi;
  int np = 0;
  auto add_passes = [&](int first, int count) {
    while (count > 0) {
      int n = 1;
      while (n * 2 <= count && n * 2 <= maxn) n *= 2;
      a.pass_first[np] = first;
      a.pass_count[np] = n;
      ++np;
      first += n;
      count -= n;
    }
  };
  if (r.mode == MODE_EXPERT) {
    a.pass_first[0] = 0;
    a.pass_count[0] = 1;
    np = 1;
  } else {
    add_passes(0, a.K);
    add_passes(a.K, a.S);
  }
  a.npass = np;
  int maxP = 1;
  for (int i = 0; i < np; ++i) maxP = std::max(maxP, kWave / (a.pass_count[i] * Gi));

  // LDS carve-up
  int words = (int)((sizeof(Small) + 15) / 4);
  words = (words + 3) & ~3;
  a.lds_xn = words; words += c.hidden;
  a.lds_xdig = words; words += a.geo.Gh * kDigitStride;
  a.lds_xsum = words; words += 2 * a.geo.Gh;
  words = (words + 3) & ~3;
  a.lds_hdig = words; words += (c.top_k + c.n_shared) * Gi * kDigitStride;
  a.lds_hsum = words; words += 2 * (c.top_k + c.n_shared) * Gi;
  a.lds_acc = words;

  // workgroups: one per CU, capped so that phase C rows per workgroup stay <= 64
  int nwg = g_num_cu;
  int rpw = (c.hidden + nwg - 1) / nwg;
  rpw = ((rpw + maxP - 1) / maxP) * maxP;
  if (rpw > 64) {
    *why = "hidden too large for the phase-C row split";
    return hipErrorInvalidValue;
  }
  a.rpw = rpw;
  words += kMaxPass * rpw;
  a.lds_words = words;
  const size_t lds = (size_t)words * 4;
  a.nwg = nwg;

  auto kern = c.bits == 4 ? decode_kernel<4> : decode_kernel<2>;
  static bool attr_set[2] = {false, false};
  if (lds > 64 * 1024 && !attr_set[c.bits == 4]) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set[c.bits == 4] = true;
  }
  hipLaunchKernelGGL(zero_words, dim3(1), dim3(64), 0, stream, a.sync, 2, a.err, 1);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (r.phased) {
    for (int t = 0; t < r.T; ++t)
      for (int l = 0; l < r.L; ++l)
        for (int ph = 0; ph < 3; ++ph) {
          if (ph == 0 && r.mode == MODE_EXPERT) continue;
          if (ph == 2 && r.mode == MODE_ROUTE) continue;
          hipLaunchKernelGGL(kern, dim3(nwg), dim3(kThreads), lds, stream, a, ph, t, l);
          e = hipGetLastError();
          if (e != hipSuccess) return e;
        }
    return hipSuccess;
  }
  int occ = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(kern),
                                                   kThreads, lds);
  if (e != hipSuccess) return e;
  if (occ < 1) {
    *why = "decode kernel does not fit on a compute unit";
    return hipErrorInvalidConfiguration;
  }
  int only = -1, zero = 0;
  void* args[] = {&a, &only, &zero, &zero};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(kern), dim3(nwg), dim3(kThreads),
                                    args, (unsigned)lds, stream);
}

}  // namespace qmoe
