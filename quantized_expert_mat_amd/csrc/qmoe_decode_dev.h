// qmoe_decode_dev.h -- device code of the decode engine (included by the
// per-code-width kernel files qmoe_decode_k2/k3/k4.hip and by qmoe_decode.hip).
#pragma once
//
// One token through one layer is three phases; each depends on all of the
// previous one:
//   A  RMSNorm of x (every workgroup recomputes it from the 16 KB input), router
//      logits (float32 mat-vec); the general kernel also reduces the shared
//      expert's gate/up + SwiGLU -> h_shared here (the specialised one in B).
//   B  top-K over the logits (every workgroup recomputes it from the logits),
//      routed experts gate/up + SwiGLU -> h_k.
//   C  down projections of the routed and shared experts, weighted combine and
//      residual -> the next layer's input.
// The flash-moe page runs the same chain per layer on its GPU and feeds the
// combine + norm + residual result straight into the next layer ("Deferred GPU
// Expert Compute" section of "Flash-MoE - Chạy mô hình 397 tỷ tham số trên
// laptop", vi.news.hada.io); here the whole token/layer loop runs inside one
// persistent kernel, so no host round trip or kernel launch sits between layers
// (the page's pre-encoded command buffers remove a per-layer dispatch gap for the
// same reason, "Optimizaciones Efectivas" section of the autoresearch page).
//
// Cross-workgroup traffic. The 256 workgroups sit on 8 XCDs with separate L2
// caches, and a grid-wide barrier costs several microseconds there. So there is
// no barrier: every value one phase hands to the next (x, logits, h) is written
// as an 8-byte (value, epoch) pair with a device-coherent store, in kRep
// replicas stored by kRep lanes at once, and each consumer polls exactly the
// values it needs until they carry the current epoch. Each exchanged vector has
// two buffers chosen by the epoch's parity; a workgroup rewrites a buffer only
// after its polls of the next epoch, to which every workgroup contributes, so no
// slot is overwritten before every consumer has read it (the grid is sized so
// that every workgroup publishes logits or h at every epoch).
// Weights never pass through LDS: they are requested into the registers of the
// lanes that reduce them, as early as their addresses are known, so that their
// latency overlaps the exchanges. The vector-memory counter retires loads and
// stores in issue order, and a wave that issues into a full memory pipeline
// stalls; where a poll, a store or a load is issued is chosen with both in mind.
//
// Dequant mat-vec. The page rewrites (nibble*scale + bias)*x as
// fma(nibble, scale*x, bias*x) ("Kernel dequant tối ưu FMA"). Carried one step
// further, a 64-group contributes scale*sum(q*x) + bias*sum(x); sum(x) per group
// is computed once per vector, so the inner loop is just sum(q*x). That inner
// loop runs on the integer dot-product unit: each 64-group of x is scaled by its
// own power of two to 23-bit integers, split into six signed base-16 digits (the
// group's scale comes from the group alone, so encoding needs no vector-wide
// reduction first), the codes are stored
// as signed nibbles (q - 8), and v_dot8_i32_i4 forms eight 4-bit products per
// instruction with exact int32 accumulation. One weight element then costs about
// one VALU operation instead of two and a half for convert + FMA, which keeps the
// 4-bit path under the HBM roofline instead of next to it.

#include <hip/hip_ext.h>

#include "qmoe_internal.h"

namespace qmoe {

constexpr int kThreads = 256;
constexpr int kNW = kThreads / kWave;  // waves per workgroup
constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23: adding it rounds to an integer in the low mantissa
constexpr int kMaxPass = kMaxK + kMaxShared;
constexpr int kBatch = 4;              // items whose loads are issued before the first is reduced
constexpr int kMaxLdsBytes = 160 * 1024;
constexpr int kLdsLayers = 256;        // layer-table entries kept in LDS
// The flash-moe layer shape as compile-time constants (hidden 4096, intermediate
// 1024, 512 experts, top-4 + 1 shared, 256 workgroups): with these the compiler
// folds every index computation and drops the guards the general shapes need.
constexpr int kSpecH = 4096, kSpecI = 1024, kSpecE = 512, kSpecK = 4, kSpecS = 1, kSpecNwg = 256;

enum Mode { MODE_LAYER = 0, MODE_ROUTE = 1, MODE_EXPERT = 2 };

struct DecodeArgs {
  Geo geo;
  int E, K, S, flags, mode;
  float eps;
  int L, T;
  const LayerPtrs* layers;       // [L] in device memory, or NULL: the one layer is layer0
  LayerPtrs layer0;
  const uint8_t* single_expert;  // MODE_EXPERT
  const float* x0;               // [T][H]
  float* y;                      // [T][H]
  const uint8_t* boost_mask;     // [T][L][K]
  const float* sel_bias;         // [T][E]
  const int* boosted;            // [T][K]
  int* idx_out;                  // [T][L][K]
  float* w_out;                  // [T][L][K]
  float* logits_out;             // [T][E]
  unsigned long long* xx;        // [kRep][H] (value, epoch) pairs: next layer's input
  unsigned long long* lx;        // [kRep][E_pad] router logits
  unsigned long long* hx;        // [kRep][(K+S)*I] expert intermediates
  int e_pad;                     // pairs per replica of the logits exchange: kWave * lx_c
  int lx_c;                      // experts per lane in top-K (lx_per_lane(E))
  int* sel;                      // [2*kMaxK]
  unsigned long long* prev;      // [2][L][kMaxK] (expert, epoch) pairs: the sorted set of the
                                 // token before, per layer (temporal tier)
  unsigned* sync;                // [0] abort flag
  unsigned* err;
  unsigned long long timeout_ticks;
  unsigned long long* trace;     // optional [T][L][16] wall-clock stamps from the last workgroup
  unsigned long long* trace_wg;  // optional [L][nwg][4] stamps of every workgroup at token 2
  int nwg;
  int rpw;                       // phase C output rows per workgroup
  int any_sgate;                 // some layer has a shared-expert gate
  int exact_rows;                // nwg * rpw == H: every workgroup owns exactly rpw rows
  int npass;
  int npass_routed;  // passes [0, npass_routed) hold routed experts, the rest shared ones
  int pass_first[kMaxPass], pass_count[kMaxPass];
  int pre_router;                // router rows of a workgroup fit the register prefetch
  int pre_shared;                // shared gate/up items of a workgroup fit it
  int pre_down;                  // phase-C down slots of every wave fit it
  int poll_sleep;                // pause between poll rounds, in units of 64 clocks
  int lds_xn, lds_xdig, lds_xsum, lds_hdig, lds_hsum, lds_acc, lds_xres;
  int lds_layers;  // LDS copy of the layer table (n_lds_layers entries)
  int n_lds_layers;
  int const_pass;  // 1: read the pass table from these arguments (compile-time constants)
  int lds_words;
  // streamed stack: routed experts live in host memory (LayerPtrs::experts) and an
  // HBM cache holds cslots experts per layer ([L][cslots][expert_bytes])
  uint8_t* cache;
  int cslots;
  unsigned long long* ctab;  // [nwg][L][cslots] per-workgroup cache tables
  uint8_t* hit_out;          // [T][L][K] 1 where a routed expert came from the cache
};

// Small per-workgroup state kept in LDS across phases.
struct Small {
  int pass_first[kMaxPass], pass_count[kMaxPass];  // copies of the kernel arguments
  int pass_lgn[kMaxPass];                          // log2(pass_count)
  float redf[kNW][kMaxPass + 2];
  int sel_idx[kMaxK];
  float sel_w[kMaxK];
  int sel_slot[kMaxK];  // streamed stack: cache slot of each selected expert
  int sel_hit[kMaxK];   // and whether the slot already held it
  // specialised kernel: each wave's top-K candidates (key, tier << 16 | expert, logit)
  unsigned cand_key[kNW * kSpecK];
  int cand_te[kNW * kSpecK];
  float cand_lg[kNW * kSpecK];
  int ok;
  float sgc[kMaxShared];       // shared-expert gate factors of the current layer
  float sgp[kNW][kMaxShared];  // their per-wave partial dot products
  unsigned long long* tr;  // trace row (workgroup 0, thread 0 only)
  // Stamps are kept here and written out once per layer, after the layer's last
  // loads are issued: a store in the middle of a phase would be waited for by the
  // next wait on a load (the counter is in issue order), and so distort the phase.
  unsigned long long trl[16];
  unsigned long long twl[4];
};

typedef __attribute__((address_space(1))) unsigned long long gl_u64;
#define SUBSTAMP(i) \
  if (threadIdx.x == 0 && s.sm->tr) s.sm->trl[i] = wall_clock64();

struct Lds {
  Small* sm;
  float* xn;
  unsigned* xdig;
  float* xsum;
  unsigned* hdig;
  float* hsum;
  float* acc;
  float* xres;       // this workgroup's rows of the (pre-norm) layer input
  float* hstage;     // phase C: h vectors (aliases xn and xdig, dead by then)
  unsigned lt;       // LDS byte address of the layer table copy
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
  s.xres = reinterpret_cast<float*>(raw + a.lds_xres);
  s.hstage = reinterpret_cast<float*>(raw + a.lds_xn);
  s.lt = (unsigned)(uintptr_t)(__attribute__((address_space(3))) unsigned*)(raw + a.lds_layers);
  return s;
}

// Layer l's weight pointers. Kept in LDS (copied at kernel start) where they fit:
// reading them there waits only on the LDS counter, whereas a global load of the
// table would make the compiler wait for every load issued before it, prefetches
// included.
__device__ inline LayerPtrs get_layer(const DecodeArgs& a, const Lds& s, int l) {
  LayerPtrs p;
  // the specialised kernel runs only when the whole table is in LDS: no global
  // path to merge with (a merge would make the compiler wait for all loads)
  if (a.const_pass || l < a.n_lds_layers) {
    typedef __attribute__((address_space(3))) const unsigned long long lds_u64;
    lds_u64* q = (lds_u64*)(uintptr_t)(s.lt + (unsigned)l * (unsigned)sizeof(LayerPtrs));
    p.experts = reinterpret_cast<const uint8_t*>(q[0]);
    p.shared = reinterpret_cast<const uint8_t*>(q[1]);
    p.router = reinterpret_cast<const float*>(q[2]);
    p.gamma = reinterpret_cast<const float*>(q[3]);
    p.sgate = reinterpret_cast<const float*>(q[4]);
  } else {
    p = a.layers[l];
  }
  return p;
}

// Pass table entries: constants in the specialised kernel (pass 0 = the K routed
// experts, pass 1 = the shared expert), else the LDS copy.
__device__ inline int pass_first_of(const DecodeArgs& a, const Lds& s, int pi) {
  return a.const_pass ? (pi == 0 ? 0 : kSpecK) : s.sm->pass_first[pi];
}
__device__ inline int pass_count_of(const DecodeArgs& a, const Lds& s, int pi) {
  return a.const_pass ? (pi == 0 ? kSpecK : kSpecS) : s.sm->pass_count[pi];
}
__device__ inline int pass_lgn_of(const DecodeArgs& a, const Lds& s, int pi) {
  return a.const_pass ? (pi == 0 ? log2i(kSpecK) : log2i(kSpecS)) : s.sm->pass_lgn[pi];
}

__device__ inline void split_range(int n, int parts, int p, int& b, int& e) {
  b = (int)((long long)n * p / parts);
  e = (int)((long long)n * (p + 1) / parts);
}

// ------------------------------------------------------------ coherent accesses
__device__ inline void st_coh(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_coh(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float ld_coh(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline int ld_coh(const int* p) {
  return __hip_atomic_load(const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this wave's outstanding memory operations (stores included) are done.
__device__ inline void wait_mem() { __builtin_amdgcn_s_waitcnt(0); }

// A copy of v that the compiler cannot prove equal to v. Values formed from it are
// recomputed where they are used instead of being hoisted out of the layer loop
// and kept live, for the whole loop, in registers that the prefetches need.
template <typename T>
__device__ inline T launder_s(T v) {
  asm volatile("" : "+s"(v));
  return v;
}
template <typename T>
__device__ inline T launder_v(T v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Issue-order point: memory operations are not moved across it by the compiler, so
// prefetches stay where they are written (behind the loads they must not delay, and
// ahead of the waits they should overlap). Emits no instruction.
__device__ inline void issue_order() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

__device__ inline uint4 to_uint4(v4u v) { return make_uint4(v.x, v.y, v.z, v.w); }

// Loads through global-address-space pointers. Weight pointers come from a table in
// memory, so the compiler cannot prove they are global and would emit flat loads,
// which also count against the LDS wait counter: every later LDS wait would then
// wait for them too, and a prefetch would stall the phase it is meant to overlap.
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const v4u gl_v4u;
typedef __attribute__((address_space(1))) const unsigned gl_u32;
typedef __attribute__((address_space(1))) const v4f gl_v4f;
typedef __attribute__((address_space(1))) const v2u gl_v2u;
__device__ inline uint4 ldg_u4(const void* p) { return to_uint4(*(gl_v4u*)(uintptr_t)p); }
__device__ inline uint2 ldg_u2(const void* p) {
  const v2u v = *(gl_v2u*)(uintptr_t)p;
  return make_uint2(v.x, v.y);
}
__device__ inline unsigned ldg_u32(const void* p) { return *(gl_u32*)(uintptr_t)p; }
__device__ inline float4 ldg_f4(const void* p) {
  const v4f v = *(gl_v4f*)(uintptr_t)p;
  return make_float4(v.x, v.y, v.z, v.w);
}

constexpr int kCachePolicySC1 = 16;           // device-coherent (bypasses non-coherent caches)
constexpr int kBufferRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

// 16-byte device-coherent loads through a buffer resource of `bytes` bytes; reads
// past the end return zeros (the hardware range check), so callers may over-read.
__device__ inline __amdgpu_buffer_rsrc_t coh_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kBufferRsrcWord3);
}
__device__ inline v4u ld_coh4(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kCachePolicySC1);
}

// ------------------------------------------------------------ epoch-tagged exchange
// An exchanged vector of n values is kRep replicas of n (value, epoch) pairs; a
// replica holds n_pad = n rounded up to even pairs so it splits into 16-byte chunks.
struct Xv {
  unsigned long long* base;
  int n, n_pad;
};

__device__ inline void xput(const Xv& x, int i, float v, unsigned epoch) {
  const unsigned long long pv = ((unsigned long long)epoch << 32) | __float_as_uint(v);
  // global address space: a store through a generic pointer would be a flat store
  __attribute__((address_space(1))) unsigned long long* base =
      (__attribute__((address_space(1))) unsigned long long*)(uintptr_t)launder_s(x.base);
#pragma unroll
  for (int r = 0; r < kRep; ++r)
    __hip_atomic_store(base + (size_t)r * x.n_pad + i, pv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Replica r of value i, stored by one lane: callers spread the kRep replicas of a
// value over kRep lanes, so a wave stores them with one instruction instead of kRep.
__device__ inline void xput_rep(const Xv& x, int r, int i, float v, unsigned epoch) {
  const unsigned long long pv = ((unsigned long long)epoch << 32) | __float_as_uint(v);
  __attribute__((address_space(1))) unsigned long long* base =
      (__attribute__((address_space(1))) unsigned long long*)(uintptr_t)launder_s(x.base);
  __hip_atomic_store(base + (size_t)r * x.n_pad + i, pv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A value held by all seg lanes of a segment (lane grp of it): with at least kRep
// lanes, lane r < kRep stores replica r; otherwise lane 0 stores all of them.
__device__ inline void xput_seg(const Xv& x, int grp, int seg, int i, float v, unsigned epoch) {
  if (seg >= kRep) {
    if (grp < kRep) xput_rep(x, grp, i, v, epoch);
  } else if (grp == 0) {
    xput(x, i, v, epoch);
  }
}

__device__ __forceinline__ bool poll_abort(const DecodeArgs& a, unsigned long long t0, int lane0);

// Pause between two polls of data that has not arrived: a workgroup that is done
// early would otherwise re-read its inputs back to back and take memory bandwidth
// from the workgroups still streaming weights.
__device__ inline void poll_pause(const DecodeArgs& a) {
  for (int i = 0; i < a.poll_sleep; ++i) __builtin_amdgcn_s_sleep(1);
}

// Request this thread's chunks base + tid + k*kThreads (k < kPer) of this
// workgroup's replica of x.
template <int kPer>
__device__ __forceinline__ void xissue(const Xv& x, int base, v4u (&v)[kPer]) {
  const unsigned long long* src = x.base + (size_t)(blockIdx.x % kRep) * x.n_pad;
  const __amdgpu_buffer_rsrc_t r = coh_rsrc(src, x.n_pad * 8);
#pragma unroll
  for (int k = 0; k < kPer; ++k) v[k] = ld_coh4(r, (base + (int)threadIdx.x + k * kThreads) * 16);
}

// Given the chunks xissue requested, poll until every one of them carries `epoch`
// and copy the values into LDS (dst[i]). Returns false if the kernel is aborting.
template <int kPer>
__device__ __forceinline__ bool xwait(const DecodeArgs& a, const Xv& x, int base, float* dst, unsigned epoch,
                                      v4u (&v)[kPer]) {
  const unsigned long long* src = x.base + (size_t)(blockIdx.x % kRep) * x.n_pad;
  const __amdgpu_buffer_rsrc_t r = coh_rsrc(src, x.n_pad * 8);
  const int nch = (x.n + 1) / 2;  // only the n produced values are awaited
  const unsigned long long t0 = wall_clock64();
  for (unsigned it = 0;; ++it) {
    unsigned pending = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int c = base + (int)threadIdx.x + k * kThreads;
      if (c >= nch) continue;
      const bool ok0 = v[k].y == epoch, ok1 = v[k].w == epoch || 2 * c + 1 >= x.n;
      if (ok0 && ok1) {
        dst[2 * c] = __uint_as_float(v[k].x);
        if (2 * c + 1 < x.n) dst[2 * c + 1] = __uint_as_float(v[k].z);
      } else {
        pending |= 1u << k;
      }
    }
    if (!pending) return true;
    if ((it & 31u) == 31u && !poll_abort(a, t0, 1)) return false;
    poll_pause(a);
#pragma unroll
    for (int k = 0; k < kPer; ++k)
      if (pending & (1u << k)) v[k] = ld_coh4(r, (base + (int)threadIdx.x + k * kThreads) * 16);
  }
}

// Wait until every pair of this workgroup's replica carries `epoch` and copy the
// values into LDS (dst[i]). All threads take part; each polls its own chunks,
// kPer 16-byte chunks per thread in flight at once (a vector of up to
// 2*kPer*kThreads values is awaited in one round trip).
// Returns false if the kernel is aborting.
template <int kPer = 8>
__device__ __forceinline__ bool xget(const DecodeArgs& a, const Xv& x, float* dst, unsigned epoch) {
  const int nch = (x.n + 1) / 2;
  for (int base = 0; base < nch; base += kThreads * kPer) {
    v4u v[kPer];
    xissue<kPer>(x, base, v);
    if (!xwait<kPer>(a, x, base, dst, epoch, v)) return false;
  }
  return true;
}

// ---------------------------------------------------------------- reductions (DPP)
template <int CTRL>
__device__ inline int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ inline float dpp_f(float v) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}
constexpr int kQuad1032 = 0xB1, kQuad2301 = 0x4E, kRowHalfMirror = 0x141, kRowMirror = 0x140;

__device__ inline float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ inline unsigned long long readlane_u64(unsigned long long v, int l) {
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)v, l);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(v >> 32), l);
  return ((unsigned long long)hi << 32) | lo;
}

// Sum over aligned segments of `width` lanes (power of two); every lane of a
// segment receives the segment's total. Within a 16-lane row the steps are DPP
// moves; across rows the four row totals are read out with readlane (a lane
// shuffle would be an LDS permute, a round trip of LDS latency per step).
__device__ inline float seg_sum(float v, int width) {
  if (width >= 2) v += dpp_f<kQuad1032>(v);
  if (width >= 4) v += dpp_f<kQuad2301>(v);
  if (width >= 8) v += dpp_f<kRowHalfMirror>(v);
  if (width >= 16) v += dpp_f<kRowMirror>(v);
  if (width >= 32) {
    const float r0 = readlane_f(v, 0), r1 = readlane_f(v, 16), r2 = readlane_f(v, 32), r3 = readlane_f(v, 48);
    if (width >= 64) v = (r0 + r1) + (r2 + r3);
    else v = (threadIdx.x & 32) ? r2 + r3 : r0 + r1;
  }
  return v;
}
__device__ inline int seg_sum8_i(int v) {
  v += dpp_i<kQuad1032>(v);
  v += dpp_i<kQuad2301>(v);
  v += dpp_i<kRowHalfMirror>(v);
  return v;
}
__device__ inline float seg_max(float v, int width) {
  if (width >= 2) v = fmaxf(v, dpp_f<kQuad1032>(v));
  if (width >= 4) v = fmaxf(v, dpp_f<kQuad2301>(v));
  if (width >= 8) v = fmaxf(v, dpp_f<kRowHalfMirror>(v));
  if (width >= 16) v = fmaxf(v, dpp_f<kRowMirror>(v));
  if (width >= 32) {
    const float r0 = readlane_f(v, 0), r1 = readlane_f(v, 16), r2 = readlane_f(v, 32), r3 = readlane_f(v, 48);
    if (width >= 64) v = fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
    else v = (threadIdx.x & 32) ? fmaxf(r2, r3) : fmaxf(r0, r1);
  }
  return v;
}
// Whole-wave sum, returned uniform (one lane of each 16-lane row read out).
__device__ inline float wave_sum(float v) {
  v = seg_sum(v, 16);
  return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}
__device__ inline float wave_max(float v) { return seg_max(v, 64); }

template <int CTRL>
__device__ inline unsigned long long dpp_max_step(unsigned long long k) {
  const unsigned hi = (unsigned)dpp_i<CTRL>((int)(k >> 32)), lo = (unsigned)dpp_i<CTRL>((int)k);
  const unsigned long long o = ((unsigned long long)hi << 32) | lo;
  return o > k ? o : k;
}
__device__ inline unsigned long long wave_max_u64(unsigned long long k) {
  k = dpp_max_step<kQuad1032>(k);
  k = dpp_max_step<kQuad2301>(k);
  k = dpp_max_step<kRowHalfMirror>(k);
  k = dpp_max_step<kRowMirror>(k);
  const unsigned long long r0 = readlane_u64(k, 0), r1 = readlane_u64(k, 16);
  const unsigned long long r2 = readlane_u64(k, 32), r3 = readlane_u64(k, 48);
  const unsigned long long a = r0 > r1 ? r0 : r1, b = r2 > r3 ? r2 : r3;
  return a > b ? a : b;
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

// One lane's chunk of 8 values (chunk dw of group gi, the 8 chunks of a group in 8
// consecutive lanes of one wave, all active or all inactive) -> its 6 digit dwords
// in dig[gi * kDigitStride + dw * 6 ..], and for dw == 0 the group's sums
// sum[4 * gi + {0, 1, 2}] = 8 * sum(ints), float sum of the values, 1/scale.
__device__ __forceinline__ void encode_chunk8(const float v[8], unsigned* dig, float* sum, int gi, int dw,
                                              bool active) {
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  m = seg_max(m, 8);
  float sc, xs;
  digit_scale(m, &sc, &xs);
  unsigned o[6];
  int isum = encode_chunk(v, sc, o);
  float fsum = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) fsum += v[i];
  if (active) {
    uint2* dst = reinterpret_cast<uint2*>(dig + (size_t)gi * kDigitStride + dw * 6);
    dst[0] = make_uint2(o[0], o[1]);
    dst[1] = make_uint2(o[2], o[3]);
    dst[2] = make_uint2(o[4], o[5]);
  }
  isum = seg_sum8_i(isum);  // |sum of 64 ints| <= 2^28: exact in int32
  fsum = seg_sum(fsum, 8);
  if (active && dw == 0) *reinterpret_cast<float4*>(sum + 4 * gi) = make_float4(8.f * (float)isum, fsum, xs, 0.f);
}

// Encode nvec vectors of length n (multiple of 64) held in LDS at src + j*n, each
// value first multiplied by gamma[i] (if given) and then by mul, the product
// written back when NORM_BACK. Every group of 64
// values gets its own power-of-two scale, from the group's largest magnitude found
// across the 8 lanes that hold the group, so no vector-wide maximum (and no
// barrier) precedes the encoding. Digits for (vector j, group g) go to
// dig[(j*G + g)*kDigitStride + dw*6 + d]; sum[4*(j*G + g) + {0, 1, 2}] = 8*sum(ints),
// float sum of the values, 1/scale. Whole workgroup participates.
template <bool NORM_BACK>
__device__ __forceinline__ void encode_vectors(float* src, int nvec, int n, float mul, const float* gamma,
                                               unsigned* dig, float* sum) {
  const int G = n / kGroup;
  const int chunks_per_vec = n / 8;
  const int total = nvec * chunks_per_vec;
  // total is a multiple of 8 and kThreads a multiple of 64: the 8 chunks of a group
  // always sit in 8 consecutive lanes (one DPP half-row) of one wave, all active or
  // all inactive.
  for (int base = 0; base < total; base += kThreads) {
    const int c = base + (int)threadIdx.x;
    const bool active = c < total;
    const int j = active ? c / chunks_per_vec : 0, cc = active ? c % chunks_per_vec : 0;
    float v[8];
    {
      float4* p = reinterpret_cast<float4*>(src + (size_t)j * n + (size_t)cc * 8);
      float4 v0 = active ? p[0] : make_float4(0.f, 0.f, 0.f, 0.f);
      float4 v1 = active ? p[1] : make_float4(0.f, 0.f, 0.f, 0.f);
      if (NORM_BACK && gamma) {
        const float4 g0 = ldg_f4(gamma + (size_t)cc * 8), g1 = ldg_f4(gamma + (size_t)cc * 8 + 4);
        v0.x *= g0.x; v0.y *= g0.y; v0.z *= g0.z; v0.w *= g0.w;
        v1.x *= g1.x; v1.y *= g1.y; v1.z *= g1.z; v1.w *= g1.w;
      }
      if (NORM_BACK) {
        v0.x *= mul; v0.y *= mul; v0.z *= mul; v0.w *= mul;
        v1.x *= mul; v1.y *= mul; v1.z *= mul; v1.w *= mul;
        if (active) {
          p[0] = v0;
          p[1] = v1;
        }
      }
      v[0] = v0.x; v[1] = v0.y; v[2] = v0.z; v[3] = v0.w;
      v[4] = v1.x; v[5] = v1.y; v[6] = v1.z; v[7] = v1.w;
    }
    encode_chunk8(v, dig, sum, j * G + cc / 8, cc % 8, active);
  }
}

// encode_vectors for the routed h of the specialised shape (K * I = 4096 values, two
// chunks of 8 per thread): both chunks are read from LDS before either is encoded,
// so the two encodings' dependent DPP and conversion chains overlap.
__device__ __forceinline__ void encode_h_spec(const float* src, unsigned* dig, float* sum) {
  constexpr int n = kSpecI, G = n / kGroup, cpv = n / 8;
  static_assert(kSpecK * cpv == 2 * kThreads, "two chunks of the routed h per thread");
  float v[2][8];
  int gi[2], dw[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = h * kThreads + (int)threadIdx.x, j = c / cpv, cc = c % cpv;
    const float4* p = reinterpret_cast<const float4*>(src + (size_t)j * n + (size_t)cc * 8);
    const float4 v0 = p[0], v1 = p[1];
    v[h][0] = v0.x; v[h][1] = v0.y; v[h][2] = v0.z; v[h][3] = v0.w;
    v[h][4] = v1.x; v[h][5] = v1.y; v[h][6] = v1.z; v[h][7] = v1.w;
    gi[h] = j * G + cc / 8;
    dw[h] = cc % 8;
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) encode_chunk8(v[h], dig, sum, gi[h], dw[h], true);
}

// ------------------------------------------------------------ dequant dot
struct Dig {
  unsigned d[48];
  float X8, Xf, xs;
};

__device__ inline void load_dig(Dig& D, const unsigned* dig, const float* sum, int idx) {
  const uint4* p = reinterpret_cast<const uint4*>(dig + (size_t)idx * kDigitStride);
#pragma unroll
  for (int i = 0; i < 12; ++i) {
    const uint4 v = p[i];
    D.d[4 * i] = v.x;
    D.d[4 * i + 1] = v.y;
    D.d[4 * i + 2] = v.z;
    D.d[4 * i + 3] = v.w;
  }
  const float4 sm = *reinterpret_cast<const float4*>(sum + 4 * idx);
  D.X8 = sm.x;
  D.Xf = sm.y;
  D.xs = sm.z;
}

// Codes of one slot: 4-bit c0 and c1; 3-bit c0 and c1.x, c1.y; 2-bit c0.
struct Slot {
  uint4 c0, c1;
  unsigned sb;
};

typedef __attribute__((address_space(3))) const uint8_t lds_u8;

typedef __attribute__((address_space(3))) const v4u lds_v4u;
typedef __attribute__((address_space(3))) const v2u lds_v2u;
typedef __attribute__((address_space(3))) const unsigned lds_u32;


// blk points to global memory, or (in_lds) to an LDS copy of the block.
template <int BITS>
__device__ inline Slot ld_slot(const uint8_t* blk, int slot, bool in_lds) {
  Slot s;
  if (in_lds) {
    const unsigned off = (unsigned)(uintptr_t)(__attribute__((address_space(3))) const uint8_t*)blk;
    lds_v4u* c = (lds_v4u*)(uintptr_t)off;
    s.c0 = to_uint4(c[slot]);
    if (BITS == 4) {
      s.c1 = to_uint4(c[64 + slot]);
    } else if (BITS == 3) {
      const v2u h = ((lds_v2u*)(uintptr_t)(off + kPlane1Offset))[slot];
      s.c1 = make_uint4(h.x, h.y, 0, 0);
    } else {
      s.c1 = make_uint4(0, 0, 0, 0);
    }
    s.sb = ((lds_u32*)(uintptr_t)(off + sb_offset(BITS)))[slot];
    return s;
  }
  s.c0 = ldg_u4(blk + slot * 16);
  if (BITS == 4) {
    s.c1 = ldg_u4(blk + kPlane1Offset + slot * 16);
  } else if (BITS == 3) {
    const uint2 h = ldg_u2(blk + kPlane1Offset + slot * 8);
    s.c1 = make_uint4(h.x, h.y, 0, 0);
  } else {
    s.c1 = make_uint4(0, 0, 0, 0);
  }
  s.sb = ldg_u32(blk + sb_offset(BITS) + slot * 4);
  return s;
}

typedef __attribute__((address_space(1))) v4u gl_v4u_w;
typedef __attribute__((address_space(1))) v2u gl_v2u_w;
typedef __attribute__((address_space(1))) unsigned gl_u32_w;

// Stores one slot into a block laid out like ld_slot's source (vector stores).
template <int BITS>
__device__ inline void st_slot(uint8_t* blk, int slot, const Slot& s) {
  const uintptr_t b = (uintptr_t)blk;
  *(gl_v4u_w*)(b + slot * 16) = v4u{s.c0.x, s.c0.y, s.c0.z, s.c0.w};
  if (BITS == 4) *(gl_v4u_w*)(b + kPlane1Offset + slot * 16) = v4u{s.c1.x, s.c1.y, s.c1.z, s.c1.w};
  if (BITS == 3) *(gl_v2u_w*)(b + kPlane1Offset + slot * 8) = v2u{s.c1.x, s.c1.y};
  *(gl_u32_w*)(b + sb_offset(BITS) + slot * 4) = s.sb;
}

// Contribution of one (row, group) slot: scale*sum(q*x) + bias*sum(x).
template <int BITS>
__device__ inline float slot_dot(const Slot& s, const Dig& D) {
  unsigned cw[8];
  if (BITS == 4) {
    cw[0] = s.c0.x; cw[1] = s.c0.y; cw[2] = s.c0.z; cw[3] = s.c0.w;
    cw[4] = s.c1.x; cw[5] = s.c1.y; cw[6] = s.c1.z; cw[7] = s.c1.w;
  } else if (BITS == 3) {
    const unsigned w[6] = {s.c0.x, s.c0.y, s.c0.z, s.c0.w, s.c1.x, s.c1.y};
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const unsigned a = w[3 * t], b = w[3 * t + 1], c = w[3 * t + 2];
      cw[4 * t] = a & 0x77777777u;
      cw[4 * t + 1] = b & 0x77777777u;
      cw[4 * t + 2] = c & 0x77777777u;
      cw[4 * t + 3] = ((a >> 3) & 0x11111111u) | ((b >> 2) & 0x22222222u) | ((c >> 1) & 0x44444444u);
    }
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
  const float pf = fmaf((float)phi, 4096.f, (float)plo);  // 4-bit sum((q-8)*i), else sum(q*i)
  const float sc = bf16lo_to_f32(s.sb), bi = bf16hi_to_f32(s.sb);
  if (BITS == 4) return fmaf(sc, (pf + D.X8) * D.xs, bi * D.Xf);
  return fmaf(sc, pf * D.xs, bi * D.Xf);
}

__device__ inline float silu(float z) { return z / (1.f + expf(-z)); }

// ------------------------------------------------------------ abort / time-out
// Every wait is bounded: after timeout_ticks a waiter raises the abort flag and the
// device error, and every waiter that sees the flag gives up, so all workgroups
// leave the kernel.
__device__ __forceinline__ bool poll_abort(const DecodeArgs& a, unsigned long long t0, int) {
  if (__hip_atomic_load(a.sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) return false;
  if (wall_clock64() - t0 > a.timeout_ticks) {
    __hip_atomic_store(a.sync, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    set_dev_err(a.err, DEV_SYNC_TIMEOUT);
    return false;
  }
  return true;
}

// Workgroup-wide "all waits succeeded".
__device__ inline bool wg_all(Small* sm, bool ok) {
  if (threadIdx.x == 0) sm->ok = 1;
  __syncthreads();
  if (!ok) sm->ok = 0;
  __syncthreads();
  return sm->ok != 0;
}

// ------------------------------------------------------------ phase pieces
__device__ inline unsigned epoch_of(const DecodeArgs& a, int t, int l) {
  return (unsigned)(t * a.L + l + 1);
}
// Every exchanged vector has two buffers, used by epochs of alternating parity: a
// producer's next write to a buffer (epoch e + 2) comes after its logits or h poll
// of epoch e + 1, and every workgroup produces logits rows or routed h items at
// every epoch only after it has read all of epoch e, so no slot of epoch e is
// overwritten before every workgroup has read it (launch_decode sizes the grid so
// that every workgroup has such rows or items).
__device__ inline unsigned long long* xbuf_of(unsigned long long* base, int n_pad, unsigned epoch) {
  return base + (size_t)(epoch & 1u) * kRep * n_pad;
}
// Position of expert e's (logit, epoch) pair in one replica of the logits
// exchange. The top-K wave holds experts C*lane .. C*lane + C - 1 in each lane (C
// even), so that the lowest expert index among equal scores is the first slot of
// the lowest lane holding them; the pairs are stored as [C/2][64 lanes][2], which
// makes each of a lane's C/2 16-byte loads coalesced across the wave.
__device__ inline int lx_pos(int e, int C) {
  const int lane = e / C, j = e - lane * C;
  return ((j >> 1) * kWave + lane) * 2 + (j & 1);
}

__device__ inline Xv xv_x(const DecodeArgs& a, unsigned epoch) {
  return Xv{xbuf_of(a.xx, a.geo.H, epoch), a.geo.H, a.geo.H};
}
__device__ inline Xv xv_logits(const DecodeArgs& a, unsigned epoch) {
  return Xv{xbuf_of(a.lx, a.e_pad, epoch), a.E, a.e_pad};
}
__device__ inline Xv xv_h(const DecodeArgs& a, unsigned epoch) {
  const int n = (kMaxK + kMaxShared) * a.geo.I;
  return Xv{xbuf_of(a.hx, n, epoch), n, n};
}

// x -> LDS (normalised if requested) -> digits for the gate/up mat-vecs. The raw
// rows this workgroup combines in phase C are kept for the residual.
__device__ __forceinline__ bool prepare_x(const DecodeArgs& a, const Lds& s, int t, int l) {
  const int H = a.geo.H;
  const float* gamma = a.mode == MODE_EXPERT ? nullptr : get_layer(a, s, l).gamma;
  const bool norm = a.mode != MODE_EXPERT && (a.flags & MOE_F_RMSNORM);
  bool ok = true;
  if (a.mode == MODE_LAYER && l > 0) {
    ok = xget(a, xv_x(a, epoch_of(a, t, l)), s.xn, epoch_of(a, t, l));
  } else {
    const float* x = a.x0 + (size_t)t * H;
    for (int i = threadIdx.x * 4; i < H; i += kThreads * 4)
      *reinterpret_cast<float4*>(s.xn + i) = *reinterpret_cast<const float4*>(x + i);
  }
  if (!wg_all(s.sm, ok)) return false;
  SUBSTAMP(14);
  const int r0 = blockIdx.x * a.rpw;
  if ((int)threadIdx.x < a.rpw && r0 + (int)threadIdx.x < H) s.xres[threadIdx.x] = s.xn[r0 + threadIdx.x];
  float ss = 0.f;
  if (norm) {
    for (int i = threadIdx.x * 4; i < H; i += kThreads * 4) {
      const float4 v = *reinterpret_cast<const float4*>(s.xn + i);
      ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    ss = wave_sum(ss);
    if ((threadIdx.x % kWave) == 0) s.sm->redf[threadIdx.x / kWave][0] = ss;
  }
  __syncthreads();
  float rinv = 1.f;
  if (norm) {
    ss = 0.f;
    for (int i = 0; i < kNW; ++i) ss += s.sm->redf[i][0];
    rinv = 1.f / sqrtf(ss / (float)H + a.eps);
  }
  // x_n = (x * gamma) * rinv in place (the router reads it), then its digits; the
  // raw rows were copied to xres before the barrier above
  if (norm || gamma)
    encode_vectors<true>(s.xn, 1, H, rinv, gamma, s.xdig, s.xsum);
  else
    encode_vectors<false>(s.xn, 1, H, 1.f, nullptr, s.xdig, s.xsum);
  __syncthreads();
  return true;
}

// Gate/up + SwiGLU over this workgroup's items [i0, i1); item i runs on wave
// (i - i0) % kNW. src(i, gate, up, hidx, row0) names the gate and up blocks (global
// or LDS) and the index of the item's h vector in the exchange. after_issue() runs
// once, right after the first batch of loads is issued (or at once if the wave has
// no items). WB: src takes two more outputs, blocks that the gate and up slots are
// copied to after use (NULL: none).
template <int BITS, bool WB = false, typename ItemFn, typename Hook>
__device__ __forceinline__ void gateup_items(const DecodeArgs& a, const Lds& s, int i0, int i1, bool in_lds,
                             unsigned epoch, ItemFn src, Hook after_issue) {
  const Geo& g = a.geo;
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  if (i0 + w >= i1) {
    issue_order();
    after_issue();
    issue_order();
    return;
  }
  const Xv hxv = xv_h(a, epoch);
  const int p = lane >> g.lGh, grp = lane & (g.Gh - 1);
  Dig D;
  load_dig(D, s.xdig, s.xsum, grp);
  bool first = true;
  for (int ib = i0 + w; ib < i1; ib += kBatch * kNW) {
    Slot G[kBatch], U[kBatch];
    int hv[kBatch], row[kBatch];
    uint8_t *wg[kBatch], *wu[kBatch];
    // loads are issued unconditionally (items past the range re-read the wave's
    // first item and are not reduced): straight-line loads let the compiler wait
    // for exactly the item it reduces next
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int i = ib + j * kNW;
      const uint8_t *gb, *ub;
      int row0, hvec;
      if constexpr (WB)
        src(i < i1 ? i : i0 + w, gb, ub, hvec, row0, wg[j], wu[j]);
      else
        src(i < i1 ? i : i0 + w, gb, ub, hvec, row0);
      G[j] = ld_slot<BITS>(gb, lane, in_lds);
      U[j] = ld_slot<BITS>(ub, lane, in_lds);
      hv[j] = i < i1 ? hvec : -1;
      row[j] = row0 + p;
    }
    if (first) {
      issue_order();
      after_issue();
      issue_order();
      first = false;
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (hv[j] < 0) continue;
      if constexpr (WB) {
        if (wg[j]) {
          st_slot<BITS>(wg[j], lane, G[j]);
          st_slot<BITS>(wu[j], lane, U[j]);
        }
      }
      const float pg = seg_sum(slot_dot<BITS>(G[j], D), g.Gh);
      const float pu = seg_sum(slot_dot<BITS>(U[j], D), g.Gh);
      if (row[j] < g.I) xput_seg(hxv, grp, g.Gh, hv[j] * g.I + row[j], silu(pg) * pu, epoch);
    }
  }
}

// Router logits for rows [e0, e1) of this workgroup; row e - e0 on wave (e - e0) % kNW.
__device__ __forceinline__ void router_rows(const DecodeArgs& a, const Lds& s, int t, int l, int e0, int e1) {
  const int H = a.geo.H, E = a.E;
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  if (e0 + w >= e1) return;
  const float* W = get_layer(a, s, l).router + (size_t)e0 * H;
  const int nq = H / 4;  // float4 columns
  constexpr int kMaxC = kMaxDim / 256;
  float4 xr[kMaxC];
#pragma unroll
  for (int c = 0; c < kMaxC; ++c) {
    const int q = lane + kWave * c;
    xr[c] = q < nq ? reinterpret_cast<const float4*>(s.xn)[q] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int e = e0 + w; e < e1; e += kNW) {
    const float4* row = reinterpret_cast<const float4*>(W + (size_t)(e - e0) * H);
    float4 wv[kMaxC];
#pragma unroll
    for (int c = 0; c < kMaxC; ++c) {
      const int q = lane + kWave * c;
      wv[c] = q < nq ? ldg_f4(row + q) : make_float4(0.f, 0.f, 0.f, 0.f);
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
    if (lane < kRep) {
      const unsigned ep = epoch_of(a, t, l);
      const unsigned long long pv = ((unsigned long long)ep << 32) | __float_as_uint(acc);
      __hip_atomic_store(xbuf_of(a.lx, a.e_pad, ep) + (size_t)lane * a.e_pad + lx_pos(e, a.lx_c), pv,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (lane == 0 && a.logits_out) a.logits_out[(size_t)t * E + e] = acc;
  }
}

// ------------------------------------------------------------ register prefetch
// Weights a phase needs are requested early, into the registers of the lanes that
// will consume them, so their HBM latency overlaps an exchange wait instead of
// following it: the next layer's router rows right after this layer's combine
// (they land while x is being exchanged; the general kernel also takes its shared
// gate/up slots there, the specialised one right after the x poll), and the down
// slots of phase C at the end of phase B (they land while h is being exchanged;
// the specialised kernel takes the shared expert's down slot in phase A). Plain
// loads keep the compiler's wait counts exact.
constexpr int kRouterPre = 8;  // float4 of router rows per thread
constexpr int kRowsPre = 4;    // router rows per workgroup on the prefetch path
constexpr int kShPre = 1;      // shared gate/up items per wave
constexpr int kDnPre = 5;      // down slots per lane

constexpr int kGatePre = kSpecH / (4 * kThreads);  // float4 of the shared-expert gate per thread

// Column of float4 number q (0..3) of thread t's values in the specialised kernel:
// [8t, 8t + 4), [8t + 4, 8t + 8), [H/2 + 8t, ...), [H/2 + 8t + 4, ...).
__device__ inline int spec_col(int q) {
  return (q >> 1) * (kSpecH / 2) + 8 * (int)threadIdx.x + 4 * (q & 1);
}
static_assert(kSpecH == 16 * kThreads, "16 x values per thread");
static_assert(kRouterPre == 4 * (kSpecE / kSpecNwg), "two router rows of 4 float4 per thread");

struct StaticPre {
  float4 r[kRouterPre];
  Slot g[kShPre], u[kShPre];
  float4 sg[kGatePre];  // specialised kernel with a gate: this thread's share of g_0
};


// chunks per thread that poll the shared and the routed h of the specialised shape
constexpr int kSpecShHPer = kSpecS * kSpecI / 2 / kThreads;
constexpr int kSpecRtHPer = kSpecK * kSpecI / 2 / kThreads;

// Down job k of this lane in phase C (defined with the phase-C code below).
struct DnJob {
  bool on;     // this lane has a slot to read (its row lies inside the workgroup's)
  int pass;    // -1: no job k on this wave
  int li, row, slot;
  const uint8_t* blk;
  uint8_t* wb;  // streamed stack: the cache block the slot is copied to, or NULL
  float wk;
};
template <bool STREAM = false>
__device__ __forceinline__ DnJob down_job(const DecodeArgs& a, const Lds& s, int l, int k);

struct DownPre {
  Slot d[kDnPre];
  v4u shp[kSpecShHPer];  // specialised kernel: the shared expert's h, requested at the end of phase B
};

// Router rows of this workgroup (float4 q = tid + kThreads*i of rows [e0, e1)) and,
// in the general kernel, its shared gate/up items (item i0 + w + kNW*j on wave w)
// for layer l. The specialised kernel takes its share of the two router rows (and
// of the shared-expert gate); its shared gate/up items are requested in phase A.
template <int BITS, bool SPEC = false>
__device__ __forceinline__ void load_static(const DecodeArgs& a, const Lds& s, int l, StaticPre& sp) {
  const Geo& g = a.geo;
  const LayerPtrs lp = get_layer(a, s, l);
  if constexpr (SPEC) {
    // The specialised kernel's layout: thread t takes the columns of the x values
    // it polls and encodes, [8t, 8t + 8) and [H/2 + 8t, H/2 + 8t + 8), of each of
    // its workgroup's two router rows (and of the gate vector), so that phase A
    // forms the dot products in registers.
    if (a.any_sgate) {
      // the gate vector (a layer without one re-reads router row 0, not used)
      const float* G = lp.sgate ? lp.sgate : lp.router;
#pragma unroll
      for (int i = 0; i < kGatePre; ++i) sp.sg[i] = ldg_f4(G + spec_col(i));
    }
    const float* W = lp.router + (size_t)blockIdx.x * (kSpecE / kSpecNwg) * kSpecH;
#pragma unroll
    for (int i = 0; i < kRouterPre; ++i) sp.r[i] = ldg_f4(W + (i >> 2) * kSpecH + spec_col(i & 3));
  } else if (a.pre_router) {
    int e0, e1;
    split_range(a.E, a.nwg, blockIdx.x, e0, e1);
    const int nq = (e1 - e0) * (g.H / 4);
    const float4* W = reinterpret_cast<const float4*>(lp.router + (size_t)e0 * g.H);
#pragma unroll
    for (int i = 0; i < kRouterPre; ++i) {
      const int q = (int)threadIdx.x + kThreads * i;
      sp.r[i] = ldg_f4(W + (q < nq ? q : 0));  // unconditional: exact wait counts
    }
  }
  if (a.pre_shared && !SPEC) {  // the specialised kernel loads them in phase A
    int i0, i1;
    split_range(a.S * g.nblk_gu, a.nwg, blockIdx.x, i0, i1);
    const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    const uint8_t* shared = lp.shared;
#pragma unroll
    for (int j = 0; j < kShPre; ++j) {
      const int i0w = i0 + w + j * kNW;
      const int i = i0w < i1 ? i0w : 0;  // unconditional: exact wait counts
      const uint8_t* gb = shared + (size_t)(i >> g.lnb) * g.expert_bytes +
                          (size_t)(i & (g.nblk_gu - 1)) * g.blk;
      sp.g[j] = ld_slot<BITS>(gb, lane, false);
      sp.u[j] = ld_slot<BITS>(gb + g.off_up, lane, false);
    }
  }
}

// Router logits of rows [e0, e1) from prefetched weights and x_n in LDS.
__device__ __forceinline__ void router_from_regs(const DecodeArgs& a, const Lds& s, int t, int l,
                                                 const StaticPre& sp) {
  const int H = a.geo.H, h4 = H / 4;
  int e0, e1;
  split_range(a.E, a.nwg, blockIdx.x, e0, e1);
  const int nr = e1 - e0;
  float acc[kRowsPre];
#pragma unroll
  for (int j = 0; j < kRowsPre; ++j) acc[j] = 0.f;
#pragma unroll
  for (int i = 0; i < kRouterPre; ++i) {
    const int q = (int)threadIdx.x + kThreads * i;
    if (q < nr * h4) {
      const int row = q / h4;
      const float4 xv = reinterpret_cast<const float4*>(s.xn)[q - row * h4];
      float d = sp.r[i].x * xv.x;
      d = fmaf(sp.r[i].y, xv.y, d);
      d = fmaf(sp.r[i].z, xv.z, d);
      d = fmaf(sp.r[i].w, xv.w, d);
#pragma unroll
      for (int j = 0; j < kRowsPre; ++j) acc[j] += row == j ? d : 0.f;
    }
  }
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
#pragma unroll
  for (int j = 0; j < kRowsPre; ++j) {
    if (j < nr) {
      const float v = wave_sum(acc[j]);
      if (lane == 0) s.sm->redf[w][j] = v;
    }
  }
  __syncthreads();
  const int j = (int)threadIdx.x / kRep, rep = (int)threadIdx.x % kRep;
  if (j < nr) {
    float v = 0.f;
    for (int i = 0; i < kNW; ++i) v += s.sm->redf[i][j];
    const int e = e0 + j;
    const unsigned ep = epoch_of(a, t, l);
    const unsigned long long pv = ((unsigned long long)ep << 32) | __float_as_uint(v);
    __hip_atomic_store(xbuf_of(a.lx, a.e_pad, ep) + (size_t)rep * a.e_pad + lx_pos(e, a.lx_c), pv,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (rep == 0 && a.logits_out) a.logits_out[(size_t)t * a.E + e] = v;
  }
}

// Shared gate/up + SwiGLU from prefetched slots (same items and outputs as the
// direct path in phase A).
template <int BITS>
__device__ __forceinline__ void shared_from_regs(const DecodeArgs& a, const Lds& s, int t, int l,
                                                 const StaticPre& sp) {
  const Geo& g = a.geo;
  int i0, i1;
  split_range(a.S * g.nblk_gu, a.nwg, blockIdx.x, i0, i1);
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  if (i0 + w >= i1) return;
  const unsigned epoch = epoch_of(a, t, l);
  const Xv hxv = xv_h(a, epoch);
  const int p = lane >> g.lGh, grp = lane & (g.Gh - 1);
  Dig D;
  load_dig(D, s.xdig, s.xsum, grp);
#pragma unroll
  for (int j = 0; j < kShPre; ++j) {
    const int i = i0 + w + j * kNW;
    if (i < i1) {
      const float pg = seg_sum(slot_dot<BITS>(sp.g[j], D), g.Gh);
      const float pu = seg_sum(slot_dot<BITS>(sp.u[j], D), g.Gh);
      const int row = ((i & (g.nblk_gu - 1)) << g.lPh) + p;
      if (row < g.I) xput_seg(hxv, grp, g.Gh, (a.K + (i >> g.lnb)) * g.I + row, silu(pg) * pu, epoch);
    }
  }
}

// Shared-expert gate factors c_s = sigmoid(g_s . x_n) of layer l into LDS (x_n in
// LDS); workgroup 0 also publishes them for a following phase launch. Layers
// without a gate keep weight 1 (list_expert reads the factor only when some layer
// has a gate).
__device__ __forceinline__ void shared_gate_factors(const DecodeArgs& a, const Lds& s, int l) {
  const int S = a.S, H = a.geo.H;
  const float* G = a.any_sgate ? get_layer(a, s, l).sgate : nullptr;
  if (G) {
    const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    for (int sh = 0; sh < S; ++sh) {
      float part = 0.f;
      for (int i = threadIdx.x * 4; i < H; i += kThreads * 4) {
        const float4 gv = ldg_f4(G + (size_t)sh * H + i);
        const float4 xv = *reinterpret_cast<const float4*>(s.xn + i);
        part = fmaf(gv.x, xv.x, part);
        part = fmaf(gv.y, xv.y, part);
        part = fmaf(gv.z, xv.z, part);
        part = fmaf(gv.w, xv.w, part);
      }
      part = wave_sum(part);
      if (lane == 0) s.sm->sgp[w][sh] = part;
    }
    __syncthreads();
  }
  if ((int)threadIdx.x < S) {
    float c = 1.f;
    if (G) {
      float z = 0.f;
      for (int i = 0; i < kNW; ++i) z += s.sm->sgp[i][threadIdx.x];
      c = 1.f / (1.f + expf(-z));
    }
    s.sm->sgc[threadIdx.x] = c;
    if (blockIdx.x == 0) st_coh(a.sel + 2 * kMaxK + threadIdx.x, __float_as_int(c));
  }
}

// The shared expert's gate/up item of this wave (the workgroup's four items, one
// per wave), loaded in phase A and reduced in phase B under the routed loads.
struct SharedSpec {
  Slot g, u;
};

template <int BITS>
__device__ __forceinline__ void load_shared_spec(const DecodeArgs& a, const Lds& s, int l, SharedSpec& sh) {
  const Geo& g = a.geo;
  const int w = (int)threadIdx.x / kWave, lane = (int)threadIdx.x % kWave;
  const uint8_t* b = get_layer(a, s, l).shared + ((size_t)blockIdx.x * kNW + w) * g.blk;
  sh.g = ld_slot<BITS>(b, lane, false);
  sh.u = ld_slot<BITS>(b + g.off_up, lane, false);
}

// Phase A of the specialised kernel. Thread t holds the 16 x values [8t, 8t + 8)
// and [H/2 + 8t, H/2 + 8t + 8): polled straight into registers (layer 0: read from
// x0), squared and summed for the RMSNorm and, unnormalised, dotted with its columns
// of the workgroup's two router rows (and of the shared-expert gate); one workgroup
// barrier joins the four sums, the RMSNorm factor scales the dot products into the
// logits, and the normalised values are encoded into digits; the chunks a thread encodes are the
// ones encode_vectors gives it, so the digits and sums land where the general
// path puts them. The logits are published before the digits are formed: the
// encoding then overlaps the logits exchange (nothing reads the digits before
// phase B), and the shared expert's gate/up items are reduced in phase B, under
// the routed experts' loads.
template <int BITS>
__device__ __forceinline__ bool phase_a_spec(const DecodeArgs& a, const Lds& s, int t, int l, const StaticPre& sp,
                                             SharedSpec& sh, DownPre& dp) {
  constexpr int H = kSpecH;
  const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
  const unsigned epoch = epoch_of(a, t, l);
  float v[16];
  bool ok = true;
  if (l == 0) {
    const float* x = a.x0 + (size_t)t * H;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 f = ldg_f4(x + spec_col(q));
      v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
    }
  } else {
    // pairs chunk c = values 2c, 2c + 1; this thread's chunks are 4t .. 4t + 3 and
    // H/4 + 4t .. H/4 + 4t + 3
    const Xv xv = xv_x(a, epoch);
    const __amdgpu_buffer_rsrc_t r = coh_rsrc(xv.base + (size_t)(blockIdx.x % kRep) * xv.n_pad, xv.n_pad * 8);
    v4u raw[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) raw[k] = ld_coh4(r, ((k >> 2) * (H / 4) + 4 * tid + (k & 3)) * 16);
    const unsigned long long t0 = wall_clock64();
    for (unsigned it = 0;; ++it) {
      unsigned pending = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (!(raw[k].y == epoch && raw[k].w == epoch)) pending |= 1u << k;
      if (!pending) break;
      if ((it & 31u) == 31u && !poll_abort(a, t0, 1)) {
        ok = false;
        break;
      }
      poll_pause(a);
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (pending & (1u << k)) raw[k] = ld_coh4(r, ((k >> 2) * (H / 4) + 4 * tid + (k & 3)) * 16);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      v[2 * k] = __uint_as_float(raw[k].x);
      v[2 * k + 1] = __uint_as_float(raw[k].z);
    }
  }
  // this workgroup's rows of the (pre-norm) input, for the residual in phase C
  const int r0 = blockIdx.x * (H / kSpecNwg);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int base = h * (H / 2) + 8 * tid;
    if (base >= r0 && base < r0 + H / kSpecNwg) {
#pragma unroll
      for (int i = 0; i < 8; ++i) s.xres[base - r0 + i] = v[8 * h + i];
    }
  }
  // the shared expert's gate/up slots (phase B) and down slot (phase C), requested as
  // soon as the input has arrived
  load_shared_spec<BITS>(a, s, l, sh);
  {
    // this lane's down slot of the shared expert (the last down job)
    const DnJob j = down_job(a, s, l, kDnPre - 1);
    dp.d[kDnPre - 1] = ld_slot<BITS>(j.on ? j.blk : get_layer(a, s, l).shared, j.on ? j.slot : 0, false);
  }
  const bool norm = (a.flags & MOE_F_RMSNORM) != 0;
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) ss = fmaf(v[i], v[i], ss);
  // x * gamma; the router logits and the shared-expert gate are linear in the
  // normalised input, so their dot products run on x * gamma beside the sum of
  // squares, all four reductions share one barrier, and the RMSNorm factor scales
  // the sums afterwards
  const float* gamma = get_layer(a, s, l).gamma;
  if (gamma) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 g4 = ldg_f4(gamma + spec_col(q));
      v[4 * q] *= g4.x; v[4 * q + 1] *= g4.y; v[4 * q + 2] *= g4.z; v[4 * q + 3] *= g4.w;
    }
  }
  // the router rows (and gate) prefetched at the end of the previous phase C, this
  // thread's columns
  float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 r0 = sp.r[q];
    const float4 r1 = sp.r[4 + q];
    acc0 = fmaf(r0.x, v[4 * q], acc0);
    acc0 = fmaf(r0.y, v[4 * q + 1], acc0);
    acc0 = fmaf(r0.z, v[4 * q + 2], acc0);
    acc0 = fmaf(r0.w, v[4 * q + 3], acc0);
    acc1 = fmaf(r1.x, v[4 * q], acc1);
    acc1 = fmaf(r1.y, v[4 * q + 1], acc1);
    acc1 = fmaf(r1.z, v[4 * q + 2], acc1);
    acc1 = fmaf(r1.w, v[4 * q + 3], acc1);
  }
  ss = wave_sum(ss);
  acc0 = wave_sum(acc0);
  acc1 = wave_sum(acc1);
  if (lane == 0) {
    s.sm->redf[w][0] = ss;
    s.sm->redf[w][1] = acc0;
    s.sm->redf[w][2] = acc1;
  }
  if (a.any_sgate) {
    float part = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 g4 = sp.sg[q];
      part = fmaf(g4.x, v[4 * q], part);
      part = fmaf(g4.y, v[4 * q + 1], part);
      part = fmaf(g4.z, v[4 * q + 2], part);
      part = fmaf(g4.w, v[4 * q + 3], part);
    }
    part = wave_sum(part);
    if (lane == 0) s.sm->sgp[w][0] = part;
  }
  if (!ok) s.sm->ok = 0;
  __syncthreads();
  if (!s.sm->ok) return false;
  SUBSTAMP(14);
  float rinv = 1.f;
  if (norm) {
    ss = 0.f;
    for (int i = 0; i < kNW; ++i) ss += s.sm->redf[i][0];
    rinv = 1.f / sqrtf(ss / (float)H + a.eps);
  }
  // x_n = (x * gamma) * rinv
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] *= rinv;
  SUBSTAMP(8);
  // publish this workgroup's two logits
  if (tid < 2 * kRep) {
    const int j = tid / kRep, rp = tid % kRep;
    float lg = 0.f;
    for (int i = 0; i < kNW; ++i) lg += s.sm->redf[i][1 + j];
    lg *= rinv;
    const int e = blockIdx.x * (kSpecE / kSpecNwg) + j;
    const unsigned long long pv = ((unsigned long long)epoch << 32) | __float_as_uint(lg);
    __hip_atomic_store(xbuf_of(a.lx, a.e_pad, epoch) + (size_t)rp * a.e_pad + lx_pos(e, a.lx_c), pv,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (rp == 0 && a.logits_out) a.logits_out[(size_t)t * a.E + e] = lg;
  }
  if (a.any_sgate && tid == 0) {
    float z = 0.f;
    for (int i = 0; i < kNW; ++i) z += s.sm->sgp[i][0];
    z *= rinv;
    s.sm->sgc[0] = get_layer(a, s, l).sgate ? 1.f / (1.f + expf(-z)) : 1.f;
  }
  SUBSTAMP(9);
  // digits of the two chunks (read in phase B, after the top-K barrier)
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = h * kThreads + tid;  // chunk of 8 values
    encode_chunk8(v + 8 * h, s.xdig, s.xsum, c / 8, c % 8, true);
  }
  return true;
}

template <int BITS, bool SPEC = false>
__device__ __forceinline__ bool phase_a(const DecodeArgs& a, const Lds& s, int t, int l,
                                        StaticPre& sp, bool preloaded) {
  const Geo& g = a.geo;
  if (!preloaded) load_static<BITS>(a, s, l, sp);
  if (!prepare_x(a, s, t, l)) return false;
  SUBSTAMP(8);
  int e0, e1;
  split_range(a.E, a.nwg, blockIdx.x, e0, e1);
  if constexpr (SPEC) {
    if (a.any_sgate) {
      // the specialised kernel's gate: the dot product from the prefetched vector;
      // the router's barrier below publishes the per-wave partials
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < kGatePre; ++i) {
        const float4 xv = reinterpret_cast<const float4*>(s.xn)[(int)threadIdx.x + kThreads * i];
        part = fmaf(sp.sg[i].x, xv.x, part);
        part = fmaf(sp.sg[i].y, xv.y, part);
        part = fmaf(sp.sg[i].z, xv.z, part);
        part = fmaf(sp.sg[i].w, xv.w, part);
      }
      part = wave_sum(part);
      if ((threadIdx.x % kWave) == 0) s.sm->sgp[threadIdx.x / kWave][0] = part;
    }
  }
  if (a.pre_router) router_from_regs(a, s, t, l, sp);
  else router_rows(a, s, t, l, e0, e1);
  if constexpr (SPEC) {
    if (a.any_sgate && threadIdx.x == 0) {
      float z = 0.f;
      for (int i = 0; i < kNW; ++i) z += s.sm->sgp[i][0];
      s.sm->sgc[0] = get_layer(a, s, l).sgate ? 1.f / (1.f + expf(-z)) : 1.f;
    }
  } else if (a.any_sgate && a.mode == MODE_LAYER) {
    shared_gate_factors(a, s, l);
  }
  SUBSTAMP(9);
  if (a.mode == MODE_LAYER && a.S > 0) {
    if (a.pre_shared) {
      shared_from_regs<BITS>(a, s, t, l, sp);
    } else {
      int i0, i1;
      split_range(a.S * g.nblk_gu, a.nwg, blockIdx.x, i0, i1);
      const uint8_t* shared = get_layer(a, s, l).shared;
      auto src = [&](int i, const uint8_t*& gb, const uint8_t*& ub, int& hvec, int& row0) {
        const int sh = i >> g.lnb, b = i & (g.nblk_gu - 1);
        gb = shared + (size_t)sh * g.expert_bytes + (size_t)b * g.blk;
        ub = gb + g.off_up;
        hvec = a.K + sh;
        row0 = b << g.lPh;
      };
      gateup_items<BITS>(a, s, i0, i1, false, epoch_of(a, t, l), src, [] {});
    }
  }
  return true;
}

__device__ inline unsigned ord_f32(float f) {
  const unsigned u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Streamed stack: the HBM expert cache of layer l. Each slot holds one expert;
// its table entry is (last use, expert) with last use = token + 1 (0: empty). A
// selected expert found in a slot is a hit; the misses, taken in increasing expert
// index, each replace the least recently used slot not used at this token (empty
// slots first, then the lowest slot). Every workgroup keeps its own copy of the
// tables and, making the same selections, the same decisions, so no workgroup
// waits for another's; and every byte of a cache slot is written and read by one
// workgroup only (its gate/up blocks and its down rows), so the copy a workgroup
// wrote is the one it reads. Runs on wave 0, lanes 0..K-1 holding the selection.
__device__ __forceinline__ void cache_decide(const DecodeArgs& a, const Lds& s, int t, int l, int my_idx) {
  const int lane = threadIdx.x, K = a.K, C = a.cslots;
  unsigned long long* tab = a.ctab + ((size_t)blockIdx.x * a.L + l) * C;
  unsigned long long ent = lane < C ? tab[lane] : 0ull;
  const unsigned now = (unsigned)t + 1u;
  int rank = 0;  // position of my expert in increasing index order
  for (int j = 0; j < K; ++j) {
    const int other = __builtin_amdgcn_readlane(my_idx, j);
    rank += (j != lane && other < my_idx) ? 1 : 0;
  }
  int my_slot = 0, my_hit = 0;
  for (int k = 0; k < K; ++k) {
    const unsigned e = (unsigned)__builtin_amdgcn_readlane(my_idx, k);
    const unsigned long long m = __ballot(lane < C && (ent >> 32) != 0ull && (unsigned)ent == e);
    if (m) {
      const int sl = __builtin_ctzll(m);  // a slot holds at most one expert, an expert one slot
      if (lane == sl) ent = ((unsigned long long)now << 32) | e;
      if (lane == k) {
        my_slot = sl;
        my_hit = 1;
      }
    }
  }
  for (int r = 0; r < K; ++r) {
    const unsigned long long who = __ballot(lane < K && rank == r);
    if (!who) continue;  // the K selected experts are distinct: every rank is taken
    const int k = __builtin_ctzll(who);
    if (__builtin_amdgcn_readlane(my_hit, k)) continue;
    const unsigned e = (unsigned)__builtin_amdgcn_readlane(my_idx, k);
    const unsigned use = (unsigned)(ent >> 32);
    const unsigned long long key =
        (lane < C && use != now) ? (((unsigned long long)use << 8) | (unsigned)lane) : ~0ull;
    const int sl = (int)(~wave_max_u64(~key) & 255ull);  // C >= K: some slot is free at this token
    if (lane == sl) ent = ((unsigned long long)now << 32) | e;
    if (lane == k) my_slot = sl;
  }
  if (lane < C) tab[lane] = ent;
  if (lane < K) {
    s.sm->sel_slot[lane] = my_slot;
    s.sm->sel_hit[lane] = my_hit;
    if (blockIdx.x == 0 && a.hit_out) a.hit_out[((size_t)t * a.L + l) * K + lane] = (uint8_t)my_hit;
  }
}

// A uniform value moved to a vector register: comparisons against it become
// per-lane selects instead of branches.
__device__ inline int fj_of(int v) { return launder_v(v); }

__device__ inline float ord_to_f32(unsigned u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// Wave-wide maximum of an unsigned value, returned uniform.
__device__ inline unsigned wave_max_u32(unsigned v) {
  v = max(v, (unsigned)dpp_i<kQuad1032>((int)v));
  v = max(v, (unsigned)dpp_i<kQuad2301>((int)v));
  v = max(v, (unsigned)dpp_i<kRowHalfMirror>((int)v));
  v = max(v, (unsigned)dpp_i<kRowMirror>((int)v));
  const unsigned r0 = (unsigned)__builtin_amdgcn_readlane((int)v, 0), r1 = (unsigned)__builtin_amdgcn_readlane((int)v, 16);
  const unsigned r2 = (unsigned)__builtin_amdgcn_readlane((int)v, 32), r3 = (unsigned)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(r0, r1), max(r2, r3));
}

// One selection round over the keys A (larger wins, 0 = none; at least one key is
// non-zero): the winner is the largest key, and among equal keys the lowest
// expert index, i.e. the lowest lane holding it and there its first slot. The
// winner's key is cleared. Returns the expert; *key_out is its key.
template <int kC>
__device__ __forceinline__ int select_round(unsigned (&A)[kC], int C, int lane, unsigned* key_out, int* slot_out,
                                            int* lane_out) {
  unsigned m = 0;
#pragma unroll
  for (int j = 0; j < kC; ++j) m = max(m, A[j]);
  const unsigned W = wave_max_u32(m);
  const int L0 = __builtin_ctzll(__ballot(m == W));
  int fj = 0;
#pragma unroll
  for (int j = kC - 1; j >= 0; --j) fj = A[j] == m ? j : fj;
  const int slot = __builtin_amdgcn_readlane(fj, L0);
  // clear the winner without indexing the register array by a variable: every
  // slot keeps its key unless its bit is set in the winner lane's mask
  const unsigned keep = ~(lane == L0 ? (1u << slot) : 0u);
#pragma unroll
  for (int j = 0; j < kC; ++j) A[j] &= (unsigned)((int)(keep << (31 - j)) >> 31);
  *key_out = W;
  *slot_out = slot;
  *lane_out = L0;
  return C * L0 + slot;
}

// Top-K with the temporal tier, then softmax over the selected logits. Runs on
// wave 0; lane l holds experts C*l .. C*l + C - 1 (C = a.lx_c <= kC). The boosted
// experts (the tier) are selected first, each round taking the largest remaining
// key, then the rest. The result is left in LDS (sel_idx, sel_w, and for the
// streamed stack sel_slot, sel_hit).
template <int kC, bool STREAM = false>
__device__ __forceinline__ void select_topk(const DecodeArgs& a, const Lds& s, int t, int l) {
  if (threadIdx.x >= kWave) return;
  const int E = a.E, K = a.K, lane = threadIdx.x, C = a.lx_c;
  // boosted experts (at most K), uniform across the wave
  int bst[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) bst[j] = -1;
  // The mask bytes and the previous token's set (epoch-tagged pairs written by
  // workgroup 0 a whole token earlier, so the first read normally finds them) are
  // requested together with the logits and checked after the logits poll.
  const bool tier_prev = a.mode == MODE_LAYER && a.boost_mask && t > 0;
  unsigned mk[kMaxK];
  v4u pp[kMaxK / 2];
  const __amdgpu_buffer_rsrc_t rp = coh_rsrc(a.prev + ((size_t)((t + 1) & 1) * a.L + l) * kMaxK, kMaxK * 8);
  if (tier_prev) {
    const uint8_t* m = a.boost_mask + ((size_t)t * a.L + l) * K;
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) mk[j] = m[j < K ? j : 0];
#pragma unroll
    for (int q = 0; q < kMaxK / 2; ++q)
      if (2 * q < K) pp[q] = ld_coh4(rp, 16 * q);
  } else if (a.boosted) {
    const int* b = a.boosted + (size_t)t * K;
    int bv[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) bv[j] = b[j < K ? j : 0];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < K) {
        const int e = bv[j];
        if (e >= 0 && e < E) bst[j] = e;
        else if ((e >= E || e < -1) && lane == 0) set_dev_err(a.err, DEV_BAD_INDEX);
      }
    }
  }
  const bool by_bias = (a.flags & MOE_F_SELECT_BY_BIAS) != 0;
  const float* sb = a.sel_bias ? a.sel_bias + (size_t)t * E : nullptr;
  v4u raw[kC / 2];  // raw[k]: experts C*lane + 2k, C*lane + 2k + 1
  {
    // poll this workgroup's replica of the logits until they carry this epoch
    const unsigned epoch = epoch_of(a, t, l);
    const unsigned long long* src = xbuf_of(a.lx, a.e_pad, epoch) + (size_t)(blockIdx.x % kRep) * a.e_pad;
    const __amdgpu_buffer_rsrc_t r = coh_rsrc(src, a.e_pad * 8);
    const unsigned long long t0 = wall_clock64();
    for (unsigned it = 0;; ++it) {
#pragma unroll
      for (int k = 0; k < kC / 2; ++k)
        if (2 * k < C) raw[k] = ld_coh4(r, (k * kWave + lane) * 16);
      int good = 1;
#pragma unroll
      for (int k = 0; k < kC / 2; ++k) {
        if (2 * k < C) {
          const int e0 = C * lane + 2 * k;
          good &= (e0 >= E || raw[k].y == epoch) && (e0 + 1 >= E || raw[k].w == epoch) ? 1 : 0;
        }
      }
      if (__all(good)) break;
      poll_pause(a);
      if ((it & 31u) == 31u) {
        bool go = true;
        if (lane == 0) go = poll_abort(a, t0, 1);
        if (!__builtin_amdgcn_readlane(go ? 1 : 0, 0)) {
          s.sm->ok = 0;
          return;
        }
      }
    }
  }
  SUBSTAMP(15);
  if (tier_prev) {
    const unsigned pep = epoch_of(a, t - 1, l);
    const unsigned long long t1 = wall_clock64();
    for (unsigned it = 0;; ++it) {
      bool good = true;
#pragma unroll
      for (int q = 0; q < kMaxK / 2; ++q)
        good = good && (2 * q >= K || pp[q].y == pep) && (2 * q + 1 >= K || pp[q].w == pep);
      if (good) break;
      if ((it & 31u) == 31u) {
        bool go = true;
        if (lane == 0) go = poll_abort(a, t1, 1);
        if (!__builtin_amdgcn_readlane(go ? 1 : 0, 0)) {
          s.sm->ok = 0;
          return;
        }
      }
#pragma unroll
      for (int q = 0; q < kMaxK / 2; ++q)
        if (2 * q < K) pp[q] = ld_coh4(rp, 16 * q);
    }
#pragma unroll
    for (int q = 0; q < kMaxK / 2; ++q) {
      if (2 * q < K && mk[2 * q]) bst[2 * q] = (int)pp[q].x;
      if (2 * q + 1 < K && mk[2 * q + 1]) bst[2 * q + 1] = (int)pp[q].z;
    }
  }
  // keys: the score in an order-preserving unsigned form (a NaN ranks as -inf),
  // 0 for slots past E; the boosted slots of this lane move to their own keys
  unsigned key[kC], kb[kC];
  float lgv[kC];
  unsigned bmask = 0;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    const int b = bst[j];
    if (j < K && b >= 0 && b / C == lane) bmask |= 1u << (b - lane * C);
  }
#pragma unroll
  for (int j = 0; j < kC; ++j) {
    const int e = C * lane + j;
    const unsigned bits = (j & 1) ? raw[j >> 1].z : raw[j >> 1].x;
    const float lg = __uint_as_float(bits);
    lgv[j] = lg;
    float sc = lg;
    if (sb) sc = by_bias ? sb[min(e, E - 1)] : lg + sb[min(e, E - 1)];
    if (sc != sc) sc = -INFINITY;
    const unsigned kk = (j < C && e < E) ? ord_f32(sc) : 0u;
    const bool boosted = (bmask >> j) & 1u;
    kb[j] = boosted ? kk : 0u;
    key[j] = boosted ? 0u : kk;
  }
  // distinct boosted experts (every expert sits in exactly one lane and slot)
  int nbd = __popc(bmask);
  nbd += dpp_i<kQuad1032>(nbd);
  nbd += dpp_i<kQuad2301>(nbd);
  nbd += dpp_i<kRowHalfMirror>(nbd);
  nbd += dpp_i<kRowMirror>(nbd);
  nbd = __builtin_amdgcn_readlane(nbd, 0) + __builtin_amdgcn_readlane(nbd, 16) +
        __builtin_amdgcn_readlane(nbd, 32) + __builtin_amdgcn_readlane(nbd, 48);
  SUBSTAMP(6);
  // K rounds; the winner of round k lands in lane k (my_idx, my_lg)
  int my_idx = 0;
  float my_lg = 0.f;
  for (int k = 0; k < K; ++k) {
    unsigned w;
    int slot, wl;
    const int e = k < nbd ? select_round<kC>(kb, C, lane, &w, &slot, &wl) : select_round<kC>(key, C, lane, &w, &slot, &wl);
    float lw;
    if (!sb) {
      lw = ord_to_f32(w);  // the score is the logit
    } else {
      float v = lgv[0];
#pragma unroll
      for (int j = 1; j < kC; ++j) v = j == fj_of(slot) ? lgv[j] : v;
      lw = readlane_f(v, wl);
    }
    if (lane == k) {
      my_idx = e;
      my_lg = lw;
    }
  }
  SUBSTAMP(7);
  // softmax over the K selected logits (lanes 0..K-1, K <= 16: the first row)
  const bool mine = lane < K;
  const float m = readlane_f(seg_max(mine ? my_lg : -INFINITY, 16), 0);
  const float ex = mine ? expf(my_lg - m) : 0.f;
  const float z = readlane_f(seg_sum(ex, 16), 0);
  const float wk = ex / z;
  if (mine) {
    s.sm->sel_idx[lane] = my_idx;
    s.sm->sel_w[lane] = wk;
  }
  if constexpr (STREAM) cache_decide(a, s, t, l, my_idx);
  if (blockIdx.x == 0) {
    // publish for a following phase launch, the outputs, and the sorted set for the
    // next token's temporal tier
    if (mine) {
      st_coh(a.sel + lane, my_idx);
      st_coh(a.sel + kMaxK + lane, __float_as_int(wk));
      const size_t o = ((size_t)t * a.L + l) * K;
      if (a.idx_out) a.idx_out[o + lane] = my_idx;
      if (a.w_out) a.w_out[o + lane] = wk;
    }
    if (a.mode == MODE_LAYER) {
      // rank of my_idx among the selected set = its position in sorted order
      int rank = 0;
      for (int j = 0; j < K; ++j) {
        const int other = __builtin_amdgcn_readlane(my_idx, j);
        rank += (j != lane && other < my_idx) ? 1 : 0;
      }
      unsigned long long* ps = a.prev + ((size_t)(t & 1) * a.L + l) * kMaxK;
      const unsigned long long pv = ((unsigned long long)epoch_of(a, t, l) << 32) | (unsigned)my_idx;
      if (mine) __hip_atomic_store(ps + rank, pv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Top-K of the specialised kernel (512 experts, K = 4), on all four waves. Wave w
// polls the logits of experts [128 w, 128 w + 128), two per lane (the specialised
// logits exchange stores expert e at pair e), and selects its own top K in the
// order (tier, score, lower index); the 16 candidates go through LDS, and every
// wave merges them (a candidate's lane order is its expert order, so the lowest
// lane among equal keys is the lowest expert). Every wave thus knows the set
// without a second barrier and requests its gate/up slots at once; the routing
// weights are formed afterwards (spec_weights). Lanes 0..K-1 return the selected
// expert and its logit. Returns false if the kernel is aborting.
__device__ __forceinline__ bool select_topk_spec(const DecodeArgs& a, const Lds& s, int t, int l, int& my_idx,
                                                 float& my_lg) {
  constexpr int K = kSpecK, E = kSpecE;
  const int lane = (int)threadIdx.x % kWave, w = (int)threadIdx.x / kWave;
  const int e0 = w * (E / kNW) + 2 * lane;  // this lane's two experts
  // boosted experts (at most K), uniform across the workgroup
  int bst[K];
#pragma unroll
  for (int j = 0; j < K; ++j) bst[j] = -1;
  const bool tier_prev = a.boost_mask && t > 0;
  unsigned mk[K];
  v4u pp[K / 2];
  const __amdgpu_buffer_rsrc_t rp = coh_rsrc(a.prev + ((size_t)((t + 1) & 1) * a.L + l) * kMaxK, kMaxK * 8);
  if (tier_prev) {
    const uint8_t* m = a.boost_mask + ((size_t)t * a.L + l) * K;
#pragma unroll
    for (int j = 0; j < K; ++j) mk[j] = m[j];
#pragma unroll
    for (int q = 0; q < K / 2; ++q) pp[q] = ld_coh4(rp, 16 * q);
  } else if (a.boosted) {
    const int* b = a.boosted + (size_t)t * K;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const int e = b[j];
      if (e >= 0 && e < E) bst[j] = e;
      else if ((e >= E || e < -1) && threadIdx.x == 0) set_dev_err(a.err, DEV_BAD_INDEX);
    }
  }
  const bool by_bias = (a.flags & MOE_F_SELECT_BY_BIAS) != 0;
  const float* sb = a.sel_bias ? a.sel_bias + (size_t)t * E : nullptr;
  const unsigned epoch = epoch_of(a, t, l);
  v4u raw;
  bool ok = true;
  {
    const __amdgpu_buffer_rsrc_t r =
        coh_rsrc(xbuf_of(a.lx, a.e_pad, epoch) + (size_t)(blockIdx.x % kRep) * a.e_pad, a.e_pad * 8);
    const unsigned long long t0 = wall_clock64();
    for (unsigned it = 0;; ++it) {
      raw = ld_coh4(r, e0 * 8);
      if (__all(raw.y == epoch && raw.w == epoch)) break;
      poll_pause(a);
      if ((it & 31u) == 31u) {
        bool go = true;
        if (lane == 0) go = poll_abort(a, t0, 1);
        if (!__builtin_amdgcn_readlane(go ? 1 : 0, 0)) {
          ok = false;
          break;
        }
      }
    }
  }
  SUBSTAMP(15);
  if (ok && tier_prev) {
    const unsigned pep = epoch_of(a, t - 1, l);
    const unsigned long long t1 = wall_clock64();
    for (unsigned it = 0;; ++it) {
      bool good = true;
#pragma unroll
      for (int q = 0; q < K / 2; ++q) good = good && pp[q].y == pep && pp[q].w == pep;
      if (good) break;
      if ((it & 31u) == 31u) {
        bool go = true;
        if (lane == 0) go = poll_abort(a, t1, 1);
        if (!__builtin_amdgcn_readlane(go ? 1 : 0, 0)) {
          ok = false;
          break;
        }
      }
#pragma unroll
      for (int q = 0; q < K / 2; ++q) pp[q] = ld_coh4(rp, 16 * q);
    }
#pragma unroll
    for (int q = 0; q < K / 2; ++q) {
      if (mk[2 * q]) bst[2 * q] = (int)pp[q].x;
      if (mk[2 * q + 1]) bst[2 * q + 1] = (int)pp[q].z;
    }
  }
  // keys (order-preserving unsigned form of the score; a NaN ranks as -inf), the
  // boosted experts in their own keys; the distinct boosted count (uniform)
  const float lg0 = __uint_as_float(raw.x), lg1 = __uint_as_float(raw.z);
  float sc0 = lg0, sc1 = lg1;
  if (sb) {
    sc0 = by_bias ? sb[e0] : lg0 + sb[e0];
    sc1 = by_bias ? sb[e0 + 1] : lg1 + sb[e0 + 1];
  }
  if (sc0 != sc0) sc0 = -INFINITY;
  if (sc1 != sc1) sc1 = -INFINITY;
  bool b0 = false, b1 = false;
  int nbd = 0;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int b = bst[j];
    bool dup = false;
#pragma unroll
    for (int i = 0; i < j; ++i) dup = dup || bst[i] == b;
    nbd += (b >= 0 && !dup) ? 1 : 0;
    b0 = b0 || b == e0;
    b1 = b1 || b == e0 + 1;
  }
  unsigned kb0 = b0 ? ord_f32(sc0) : 0u, kb1 = b1 ? ord_f32(sc1) : 0u;
  unsigned kn0 = b0 ? 0u : ord_f32(sc0), kn1 = b1 ? 0u : ord_f32(sc1);
  // this wave's boosted count, then its K local rounds: the winner lands in lane k
  int nbw = __popcll(__ballot(b0)) + __popcll(__ballot(b1));
  unsigned ck = 0u;
  int cte = 0;
  float clg = 0.f;
  // each round: the largest key of the active tier (wave-uniform), its lane and
  // slot, and that key cleared, all with selects (no divergent branch per round)
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const bool tier = k < nbw;
    const unsigned a0 = tier ? kb0 : kn0, a1 = tier ? kb1 : kn1;
    const unsigned m = max(a0, a1);
    const unsigned W = wave_max_u32(m);
    const int L0 = __builtin_ctzll(__ballot(m == W));
    const int slot = __builtin_amdgcn_readlane(a0 == m ? 0 : 1, L0);
    const bool win = lane == L0;
    const bool c0 = win && slot == 0, c1 = win && slot != 0;
    kb0 = tier && c0 ? 0u : kb0;
    kb1 = tier && c1 ? 0u : kb1;
    kn0 = !tier && c0 ? 0u : kn0;
    kn1 = !tier && c1 ? 0u : kn1;
    const float lgw = readlane_f(slot == 0 ? lg0 : lg1, L0);
    const bool mine = lane == k;
    ck = mine ? W : ck;
    cte = mine ? (((tier ? 1 : 0) << 16) | (w * (E / kNW) + 2 * L0 + slot)) : cte;
    clg = mine ? lgw : clg;
  }
  if (lane < K) {
    s.sm->cand_key[w * K + lane] = ck;
    s.sm->cand_te[w * K + lane] = cte;
    s.sm->cand_lg[w * K + lane] = clg;
  }
  if (!ok) s.sm->ok = 0;
  __syncthreads();
  if (!s.sm->ok) return false;
  // merge the 16 candidates (lanes 0..15 of every wave): the nbd boosted ones
  // first, then the rest
  const bool cv = lane < kNW * K;
  const unsigned key = cv ? s.sm->cand_key[lane] : 0u;
  const int te = cv ? s.sm->cand_te[lane] : 0;
  const float lgc = cv ? s.sm->cand_lg[lane] : 0.f;
  unsigned mt = (te >> 16) ? key : 0u, mn = (te >> 16) ? 0u : key;
  my_idx = 0;
  my_lg = 0.f;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const bool tier = k < nbd;  // wave-uniform
    const unsigned A = tier ? mt : mn;
    unsigned v = A;
    v = max(v, (unsigned)dpp_i<kQuad1032>((int)v));
    v = max(v, (unsigned)dpp_i<kQuad2301>((int)v));
    v = max(v, (unsigned)dpp_i<kRowHalfMirror>((int)v));
    v = max(v, (unsigned)dpp_i<kRowMirror>((int)v));
    const unsigned W = (unsigned)__builtin_amdgcn_readlane((int)v, 0);  // the first row's maximum
    const int L0 = __builtin_ctzll(__ballot(A == W && cv));
    const int e = __builtin_amdgcn_readlane(te, L0) & 0xFFFF;
    const float lw = readlane_f(lgc, L0);
    const bool win = lane == L0;
    mt = tier && win ? 0u : mt;
    mn = !tier && win ? 0u : mn;
    const bool mine = lane == k;
    my_idx = mine ? e : my_idx;
    my_lg = mine ? lw : my_lg;
  }
  return true;
}

// The routing weights of the specialised top-K (a softmax over the K selected
// logits in lanes 0..K-1), the LDS selection every wave reads, and (workgroup 0,
// wave 0) the outputs and the sorted set the next token's temporal tier reads.
// Every wave writes the same selection to LDS, so no barrier is needed before a
// wave reads it back.
__device__ __forceinline__ void spec_weights(const DecodeArgs& a, const Lds& s, int t, int l, int my_idx, float my_lg) {
  constexpr int K = kSpecK;
  const int lane = (int)threadIdx.x % kWave;
  const bool mine = lane < K;
  const float m = readlane_f(seg_max(mine ? my_lg : -INFINITY, 16), 0);
  const float ex = mine ? expf(my_lg - m) : 0.f;
  const float z = readlane_f(seg_sum(ex, 16), 0);
  const float wk = ex / z;
  if (mine) {
    s.sm->sel_idx[lane] = my_idx;
    s.sm->sel_w[lane] = wk;
  }
  if (blockIdx.x == 0 && threadIdx.x < kWave) {
    if (mine) {
      st_coh(a.sel + lane, my_idx);
      st_coh(a.sel + kMaxK + lane, __float_as_int(wk));
      const size_t o = ((size_t)t * a.L + l) * K;
      if (a.idx_out) a.idx_out[o + lane] = my_idx;
      if (a.w_out) a.w_out[o + lane] = wk;
    }
    int rank = 0;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const int other = __builtin_amdgcn_readlane(my_idx, j);
      rank += (j != lane && other < my_idx) ? 1 : 0;
    }
    unsigned long long* ps = a.prev + ((size_t)(t & 1) * a.L + l) * kMaxK;
    const unsigned long long pv = ((unsigned long long)epoch_of(a, t, l) << 32) | (unsigned)my_idx;
    if (mine) __hip_atomic_store(ps + rank, pv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The expert-list entry li of phase C: its packed expert and routing weight.
// Streamed stack: routed entry k is read from its cache slot when the slot already
// holds it, else from host memory, and then wb names the slot it is copied into.
__device__ inline const uint8_t* routed_source(const DecodeArgs& a, const Lds& s, int l, int k,
                                               uint8_t*& wb) {
  const size_t eb = a.geo.expert_bytes;
  uint8_t* slot = a.cache + ((size_t)l * a.cslots + s.sm->sel_slot[k]) * eb;
  if (s.sm->sel_hit[k]) {
    wb = nullptr;
    return slot;
  }
  wb = slot;
  return get_layer(a, s, l).experts + (size_t)s.sm->sel_idx[k] * eb;
}

// wb (streamed stack only): where the entry's expert is copied to, or NULL.
template <bool STREAM = false>
__device__ inline const uint8_t* list_expert(const DecodeArgs& a, const Lds& s, int l, int li,
                                             float& wk, uint8_t*& wb) {
  const Geo& g = a.geo;
  wb = nullptr;
  if (a.mode == MODE_EXPERT) {
    wk = 1.f;
    return a.single_expert;
  }
  if (li < a.K) {
    wk = s.sm->sel_w[li];
    if constexpr (STREAM) return routed_source(a, s, l, li, wb);
    return get_layer(a, s, l).experts + (size_t)s.sm->sel_idx[li] * g.expert_bytes;
  }
  wk = a.any_sgate ? s.sm->sgc[li - a.K] : 1.f;
  return get_layer(a, s, l).shared + (size_t)(li - a.K) * g.expert_bytes;
}

__device__ inline const uint8_t* list_expert(const DecodeArgs& a, const Lds& s, int l, int li,
                                             float& wk) {
  uint8_t* wb;
  return list_expert<false>(a, s, l, li, wk, wb);
}

// Job k (0-based) of this lane in phase C's down projection: the k-th (pass, chunk)
// pair that wave w walks, in the order of the direct loop. A pass covers expert-list
// entries [first, first + n); lane (p, kl, grp) handles row r0 + c*Pp + p, entry
// first + kl and group grp of chunk c = w + kNW*m.
template <bool STREAM>
__device__ __forceinline__ DnJob down_job(const DecodeArgs& a, const Lds& s, int l, int k) {
  const Geo& g = a.geo;
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int r0 = blockIdx.x * a.rpw, r1 = a.exact_rows ? r0 + a.rpw : min(g.H, r0 + a.rpw);
  const int npass = a.mode == MODE_EXPERT ? 1 : a.npass;
  DnJob j;
  j.on = false;
  j.pass = -1;
  j.li = 0; j.row = 0; j.slot = 0; j.blk = nullptr; j.wb = nullptr; j.wk = 0.f;
  // all divisors are powers of two: shifts and masks only
  for (int pi = 0; pi < npass; ++pi) {
    const int first = a.mode == MODE_EXPERT ? 0 : pass_first_of(a, s, pi);
    const int lgn = a.mode == MODE_EXPERT ? 0 : pass_lgn_of(a, s, pi);
    const int lseg = lgn + g.lGi, lPp = 6 - lseg;  // seg = n*Gi lanes, Pp = 64/seg rows
    const int nchunk = r0 < r1 ? (r1 - r0 + (1 << lPp) - 1) >> lPp : 0;
    const int cnt = w < nchunk ? (int)((unsigned)(nchunk - w + kNW - 1) / kNW) : 0;
    if (k < cnt) {
      const int c = w + k * kNW;
      const int grp = lane & (g.Gi - 1), kl = (lane >> g.lGi) & ((1 << lgn) - 1), p = lane >> lseg;
      j.pass = pi;
      j.li = first + kl;
      j.row = r0 + (c << lPp) + p;
      j.on = j.row < r1;
      uint8_t* wb;
      const uint8_t* ex = list_expert<STREAM>(a, s, l, j.li, j.wk, wb);
      j.blk = ex + g.off_down + (size_t)(j.row >> g.lPi) * g.blk;
      if constexpr (STREAM) j.wb = wb ? wb + g.off_down + (size_t)(j.row >> g.lPi) * g.blk : nullptr;
      j.slot = ((j.row & (g.Pi - 1)) << g.lGi) + grp;
      return j;
    }
    k -= cnt;
  }
  return j;
}

template <int BITS, bool STREAM = false>
__device__ __forceinline__ void load_down(const DecodeArgs& a, const Lds& s, int l, DownPre& dp) {
  // unconditional loads (a lane without job k re-reads a valid slot it ignores), so
  // the compiler's wait counts stay exact
  const uint8_t* any = a.mode == MODE_EXPERT ? a.single_expert : get_layer(a, s, l).experts;
#pragma unroll
  for (int k = 0; k < kDnPre; ++k) {
    const DnJob j = down_job<STREAM>(a, s, l, k);
    dp.d[k] = ld_slot<BITS>(j.on ? j.blk : any, j.on ? j.slot : 0, false);
  }
}

// Phase C's down projection from prefetched slots; partial sums per (pass, row) go
// to s.acc exactly as in the direct loop; only jobs of passes [p_lo, p_hi).
template <int BITS, bool STREAM = false>
__device__ __forceinline__ void down_from_regs(const DecodeArgs& a, const Lds& s, int l,
                                               const DownPre& dp, int p_lo = 0, int p_hi = kMaxPass) {
  const Geo& g = a.geo;
  const int lane = threadIdx.x % kWave;
  const int r0 = blockIdx.x * a.rpw;
  Dig D;
  int dig_pass = -1;  // the h digits in D are those of this pass's entries
#pragma unroll
  for (int k = 0; k < kDnPre; ++k) {
    const DnJob j = down_job<STREAM>(a, s, l, k);
    if (j.pass < 0) continue;
    if (j.pass < p_lo || j.pass >= p_hi) continue;
    const int n = a.mode == MODE_EXPERT ? 1 : pass_count_of(a, s, j.pass);
    const int seg = n * g.Gi, grp = lane & (g.Gi - 1);
    if (j.pass != dig_pass) {
      load_dig(D, s.hdig, s.hsum, j.li * g.Gi + grp);
      dig_pass = j.pass;
    }
    float part = j.on ? slot_dot<BITS>(dp.d[k], D) * j.wk : 0.f;
    if constexpr (STREAM)
      if (j.on && j.wb) st_slot<BITS>(j.wb, j.slot, dp.d[k]);
    part = seg_sum(part, seg);
    if (j.on && (lane % seg) == 0) s.acc[j.pass * a.rpw + (j.row - r0)] = part;
  }
}

// Phase B of the specialised kernel (hidden 4096, inter 1024, K 4, 256 workgroups):
// a workgroup owns kNW*kBatch consecutive gate/up rows of one routed expert, so
// each wave has exactly one batch. Every address is formed from LDS first; the
// gate/up loads go out in two straight runs (no branch or LDS read among them
// that would make the compiler wait for the loads already issued), with the
// routing weights and the shared item computed between them. The routed down
// slots are requested after the gate/up dot products: phase B then moves only the
// gate/up bytes, and the down slots land while h is being exchanged (measured 2%
// faster than requesting them with the gate/up slots).
static_assert(kSpecK * kSpecI / kSpecNwg == kNW * kBatch, "one batch per wave");
static_assert(kSpecI % (kNW * kBatch) == 0, "a workgroup's rows lie in one expert");
template <int BITS>
__device__ __forceinline__ void gateup_down_spec(const DecodeArgs& a, const Lds& s, int t, int l,
                                                 DownPre& dp, const SharedSpec& sh, int my_idx, float my_lg) {
  const Geo& g = a.geo;
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int i0 = blockIdx.x * (kNW * kBatch);
  const int k = i0 >> g.lnb;  // the routed expert (list entry) of every row here
  const uint8_t* ex = get_layer(a, s, l).experts + (size_t)__builtin_amdgcn_readlane(my_idx, k) * g.expert_bytes;
  const uint8_t* gb[kBatch];
  int row[kBatch];
#pragma unroll
  for (int j = 0; j < kBatch; ++j) {
    const int b = (i0 + w + j * kNW) & (g.nblk_gu - 1);
    gb[j] = ex + (size_t)b * g.blk;
    row[j] = b;  // one row per block in this shape
  }
  Dig D;
  load_dig(D, s.xdig, s.xsum, lane);
  // The gate/up loads go out in two halves. The CU's memory pipeline fills up with
  // the first half of every wave's requests, and a wave that issues more then
  // stalls until some drain; so the routing weights and the shared expert's item
  // are computed between the halves, while the first half streams in.
  constexpr int kFirst = kBatch / 2;
  Slot G[kBatch], U[kBatch];
  issue_order();
#pragma unroll
  for (int j = 0; j < kFirst; ++j) {
    G[j] = ld_slot<BITS>(gb[j], lane, false);
    U[j] = ld_slot<BITS>(gb[j] + g.off_up, lane, false);
  }
  issue_order();
  // the routing weights and the LDS selection (read by the down jobs below and in
  // phase C)
  spec_weights(a, s, t, l, my_idx, my_lg);
  const unsigned epoch = epoch_of(a, t, l);
  const Xv hxv = xv_h(a, epoch);
  {
    // the shared expert's gate/up item of this wave (loaded in phase A); one block
    // of one row per item in this shape
    static_assert(kSpecS * kSpecI / kSpecNwg == kNW, "four shared gate/up items per workgroup");
    const float pg = seg_sum(slot_dot<BITS>(sh.g, D), kWave);
    const float pu = seg_sum(slot_dot<BITS>(sh.u, D), kWave);
    if (lane < kRep) xput_rep(hxv, lane, kSpecK * g.I + blockIdx.x * kNW + w, silu(pg) * pu, epoch);
  }
  issue_order();
#pragma unroll
  for (int j = kFirst; j < kBatch; ++j) {
    G[j] = ld_slot<BITS>(gb[j], lane, false);
    U[j] = ld_slot<BITS>(gb[j] + g.off_up, lane, false);
  }
  issue_order();
  float hj[kBatch];
#pragma unroll
  for (int j = 0; j < kBatch; ++j) {
    const float pg = seg_sum(slot_dot<BITS>(G[j], D), kWave);
    const float pu = seg_sum(slot_dot<BITS>(U[j], D), kWave);
    hj[j] = silu(pg) * pu;
  }
  // A first poll of the shared expert's h (published before the routed dots by
  // every workgroup), then this wave's routed h, then the routed experts' down slots
  // of phase C. The memory counter retires in issue order, stores included, so the
  // poll goes out ahead of the stores and the loads: phase C can use it without
  // waiting for either, and starts on the shared expert at once.
  const uint8_t* db[kDnPre - 1];
  int ds[kDnPre - 1];
#pragma unroll
  for (int q = 0; q < kDnPre - 1; ++q) {
    const DnJob j = down_job(a, s, l, q);
    db[q] = j.on ? j.blk : ex;
    ds[q] = j.on ? j.slot : 0;
  }
  const Xv shx{hxv.base + (size_t)kSpecK * g.I, kSpecS * g.I, hxv.n_pad};
  issue_order();
  xissue<kSpecShHPer>(shx, 0, dp.shp);
  issue_order();
  // lane j*kRep + r stores replica r of row j: all of this wave's h in one instruction
  static_assert(kBatch * kRep <= kWave, "a wave's h replicas fit its lanes");
  if (lane < kBatch * kRep) {
    const int j = lane / kRep;
    float v = hj[0];
    int rj = row[0];
#pragma unroll
    for (int q = 1; q < kBatch; ++q) {
      v = j == q ? hj[q] : v;
      rj = j == q ? row[q] : rj;
    }
    xput_rep(hxv, lane % kRep, k * g.I + rj, v, epoch);
  }
  issue_order();
#pragma unroll
  for (int q = 0; q < kDnPre - 1; ++q) dp.d[q] = ld_slot<BITS>(db[q], ds[q], false);
  issue_order();
}

// Phase B of the specialised kernel: top-K on all four waves (the ok flag is 1
// here: phase A's barrier checked it), then the gate/up work of the routed and
// shared experts.
template <int BITS>
__device__ __forceinline__ bool phase_b_spec(const DecodeArgs& a, const Lds& s, int t, int l, DownPre& dp,
                                             const SharedSpec& sh) {
  int my_idx;
  float my_lg;
  if (!select_topk_spec(a, s, t, l, my_idx, my_lg)) return false;
  SUBSTAMP(10);
  if (a.trace_wg && t == 2 && threadIdx.x == 0) s.sm->twl[1] = wall_clock64();
  gateup_down_spec<BITS>(a, s, t, l, dp, sh, my_idx, my_lg);
  return true;
}

template <int BITS, bool SPEC = false, bool STREAM = false>
__device__ __forceinline__ bool phase_b(const DecodeArgs& a, const Lds& s, int t, int l, DownPre& dp,
                                        bool prefetch) {
  const Geo& g = a.geo;
  if (a.mode == MODE_EXPERT) {
    int i0, i1;
    split_range(g.nblk_gu, a.nwg, blockIdx.x, i0, i1);
    auto src = [&](int i, const uint8_t*& gb, const uint8_t*& ub, int& hvec, int& row0) {
      gb = a.single_expert + (size_t)i * g.blk;
      ub = gb + g.off_up;
      hvec = 0;
      row0 = i << g.lPh;
    };
    auto hook = [&] {
      if (prefetch) load_down<BITS>(a, s, l, dp);
    };
    gateup_items<BITS>(a, s, i0, i1, false, epoch_of(a, t, l), src, hook);
    return true;
  }
  if (threadIdx.x == 0) s.sm->ok = 1;
  __syncthreads();
  if constexpr (SPEC)
    select_topk<kSpecE / kWave>(a, s, t, l);
  else
    select_topk<kMaxE / kWave, STREAM>(a, s, t, l);
  __syncthreads();
  if (!s.sm->ok) return false;
  SUBSTAMP(10);
  if (a.trace_wg && t == 2 && threadIdx.x == 0) s.sm->twl[1] = wall_clock64();
  if (a.mode != MODE_LAYER) return true;

  if constexpr (STREAM) {
    // a workgroup owns whole gate/up blocks (all K entries of each), so a cached
    // expert's block is always read by the workgroup that copied it in
    int b0, b1;
    split_range(g.nblk_gu, a.nwg, blockIdx.x, b0, b1);
    const int K = a.K;
    auto src = [&](int i, const uint8_t*& gb, const uint8_t*& ub, int& hvec, int& row0, uint8_t*& wg,
                   uint8_t*& wu) {
      const int b = i / K, k = i - b * K;
      uint8_t* wb;
      gb = routed_source(a, s, l, k, wb) + (size_t)b * g.blk;
      ub = gb + g.off_up;
      wg = wb ? wb + (size_t)b * g.blk : nullptr;
      wu = wb ? wg + g.off_up : nullptr;
      hvec = k;
      row0 = b << g.lPh;
    };
    auto hook = [&] {
      if (prefetch) load_down<BITS, true>(a, s, l, dp);
    };
    gateup_items<BITS, true>(a, s, b0 * K, b1 * K, false, epoch_of(a, t, l), src, hook);
    return true;
  }
  const uint8_t* experts = get_layer(a, s, l).experts;
  int i0, i1;
  split_range(a.K * g.nblk_gu, a.nwg, blockIdx.x, i0, i1);
  auto src = [&](int i, const uint8_t*& gb, const uint8_t*& ub, int& hvec, int& row0) {
    const int k = i >> g.lnb, b = i & (g.nblk_gu - 1);
    gb = experts + (size_t)s.sm->sel_idx[k] * g.expert_bytes + (size_t)b * g.blk;
    ub = gb + g.off_up;
    hvec = k;
    row0 = b << g.lPh;
  };
  // the down slots of phase C are requested right behind this wave's first gate/up
  // loads, so they arrive while h is being exchanged
  auto hook = [&] {
    if (prefetch) load_down<BITS>(a, s, l, dp);
  };
  gateup_items<BITS>(a, s, i0, i1, false, epoch_of(a, t, l), src, hook);
  return true;
}

template <int BITS, bool SPEC = false, bool STREAM = false>
__device__ __forceinline__ bool phase_c(const DecodeArgs& a, const Lds& s, int t, int l,
                                        bool pre_down, DownPre& dp, bool down_loaded,
                                        StaticPre& sp, bool prefetch_static) {
  const Geo& g = a.geo;
  const int H = g.H, I = g.I;
  const bool expert_mode = a.mode == MODE_EXPERT;
  const int nlist = expert_mode ? 1 : a.K + a.S;
  const int rpw = a.rpw;
  const int r0 = blockIdx.x * rpw;
  const int r1 = a.exact_rows ? r0 + rpw : min(H, r0 + rpw);
  // h vectors of this layer (polled; the down slots prefetched in phase B were
  // requested before these polls, so they have landed when the polls complete)
  float* hs = s.hstage;
  if constexpr (SPEC) {
    // The shared expert's h was published in phase B before the routed dots, and
    // its poll went out at the end of phase B, ahead of the routed down slots; its
    // down slot came in phase A. So its digits and its down pass (pass 1) are done
    // first, while the routed h and the routed down slots are still arriving; then
    // the routed h and pass 0. (The general kernel keeps one poll: there the split
    // measured slower.)
    const Xv hv = xv_h(a, epoch_of(a, t, l));
    const int K = a.K, Gi = g.Gi;
    const Xv sh{hv.base + (size_t)K * I, a.S * I, hv.n_pad};
    static_assert(kSpecS * kSpecI / 2 == kThreads * kSpecShHPer, "the shared h is one round of chunks");
    if (!wg_all(s.sm, xwait<kSpecShHPer>(a, sh, 0, hs + K * I, epoch_of(a, t, l), dp.shp))) return false;
    encode_vectors<false>(hs + K * I, kSpecS, kSpecI, 1.f, nullptr, s.hdig + K * Gi * kDigitStride,
                          s.hsum + 4 * K * Gi);
    __syncthreads();
    // the routed h is requested before the shared pass, so its round trip overlaps
    // that pass; whatever has not arrived by then is polled again
    const Xv rt{hv.base, K * I, hv.n_pad};
    static_assert(kSpecK * kSpecI / 2 == kThreads * kSpecRtHPer, "the routed h is one round of chunks");
    v4u rtp[kSpecRtHPer];
    issue_order();
    xissue<kSpecRtHPer>(rt, 0, rtp);
    issue_order();
    down_from_regs<BITS, STREAM>(a, s, l, dp, a.npass_routed, a.npass);
    if (!wg_all(s.sm, xwait<kSpecRtHPer>(a, rt, 0, hs, epoch_of(a, t, l), rtp))) return false;
    SUBSTAMP(13);
    encode_h_spec(hs, s.hdig, s.hsum);
    __syncthreads();
  } else {
    {
      const Xv hv = xv_h(a, epoch_of(a, t, l));
      const Xv part{hv.base, nlist * I, hv.n_pad};
      if (!wg_all(s.sm, xget(a, part, hs, epoch_of(a, t, l)))) return false;
    }
    SUBSTAMP(13);
    encode_vectors<false>(hs, nlist, I, 1.f, nullptr, s.hdig, s.hsum);
    __syncthreads();
  }
  SUBSTAMP(11);
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int npass = expert_mode ? 1 : a.npass;
  if constexpr (SPEC) {
    down_from_regs<BITS, STREAM>(a, s, l, dp, 0, a.npass_routed);  // the shared pass is done
  } else if (pre_down) {
    if (!down_loaded) load_down<BITS, STREAM>(a, s, l, dp);
    down_from_regs<BITS, STREAM>(a, s, l, dp);
  } else if (r0 < r1) {
    for (int pi = 0; pi < npass; ++pi) {
      const int first = expert_mode ? 0 : pass_first_of(a, s, pi);
      const int n = expert_mode ? 1 : pass_count_of(a, s, pi);
      const int seg = n * g.Gi;
      const int Pp = kWave / seg;
      const int grp = lane % g.Gi, kl = (lane / g.Gi) % n, p = lane / seg;
      const int li = first + kl;  // index in the expert list
      float wk;
      uint8_t* wb;
      const uint8_t* ex = list_expert<STREAM>(a, s, l, li, wk, wb);
      const uint8_t* down = ex + g.off_down;
      uint8_t* down_wb = STREAM && wb ? wb + g.off_down : nullptr;
      const int nchunk = (r1 - r0 + Pp - 1) / Pp;
      if (w >= nchunk) continue;
      Dig D;
      load_dig(D, s.hdig, s.hsum, li * g.Gi + grp);
      for (int c0 = w; c0 < nchunk; c0 += kBatch * kNW) {
        Slot S[kBatch];
        int row[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int c = c0 + j * kNW;
          row[j] = r0 + c * Pp + p;
          if (c < nchunk && row[j] < r1) {
            const int b = row[j] / g.Pi, pd = row[j] % g.Pi;
            S[j] = ld_slot<BITS>(down + (size_t)b * g.blk, pd * g.Gi + grp, false);
          }
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const int c = c0 + j * kNW;
          if (c >= nchunk) continue;
          const bool valid = row[j] < r1;
          if constexpr (STREAM)
            if (valid && down_wb)
              st_slot<BITS>(down_wb + (size_t)(row[j] / g.Pi) * g.blk, (row[j] % g.Pi) * g.Gi + grp, S[j]);
          float part = valid ? slot_dot<BITS>(S[j], D) * wk : 0.f;
          part = seg_sum(part, seg);
          if (valid && (lane % seg) == 0) s.acc[pi * rpw + (row[j] - r0)] = part;
        }
      }
    }
  }
  __syncthreads();
  SUBSTAMP(12);
  const bool res = !expert_mode && (a.flags & MOE_F_RESIDUAL);
  if (expert_mode || l == a.L - 1) {
    const int rr = r0 + (int)threadIdx.x;
    if (rr < r1 && (int)threadIdx.x < rpw) {
      float v = res ? s.xres[threadIdx.x] : 0.f;
      for (int pi = 0; pi < npass; ++pi) v += s.acc[pi * rpw + (rr - r0)];
      a.y[(size_t)t * H + rr] = v;
    }
  } else {
    // thread q stores replica q % kRep of row q / kRep: the replicas of 32 rows per
    // store instruction, each thread forming its row's sum from LDS
    const Xv xo = xv_x(a, epoch_of(a, t, l + 1));
    for (int q = (int)threadIdx.x; q < rpw * kRep; q += kThreads) {
      const int i = q / kRep, rr = r0 + i;
      if (rr >= r1) continue;
      float v = res ? s.xres[i] : 0.f;
      for (int pi = 0; pi < npass; ++pi) v += s.acc[pi * rpw + i];
      xput_rep(xo, q % kRep, rr, v, epoch_of(a, t, l + 1));
    }
  }
  // the next layer's router rows and shared slots land while x is being exchanged;
  // they are requested once the x rows above are out, so that the stores the other
  // workgroups wait for do not queue behind this workgroup's prefetch loads
  if (prefetch_static) {
    __syncthreads();
    issue_order();
    load_static<BITS, SPEC>(a, s, l == a.L - 1 ? 0 : l + 1, sp);
    issue_order();
  }
  return true;
}

// only_phase < 0: persistent (all tokens, all layers; phases wait on their inputs'
// epochs). only_phase = 0/1/2: run that phase for token t_only, layer l_only.
// The layer/stack chain in one persistent launch: every phase runs for every
// (token, layer), so registers prefetched in one phase are handed to the next.
// Used when the router rows and the down slots fit the register prefetch.
template <int BITS, bool SPEC, bool STREAM = false>
__device__ __forceinline__ void decode_chain(const DecodeArgs& a, const Lds& s) {
  StaticPre sp;
  DownPre dp;
  SharedSpec sh;
  load_static<BITS, SPEC>(a, s, 0, sp);
  for (int t = 0; t < a.T; ++t) {
    for (int l = 0; l < a.L; ++l) {
      unsigned long long* tr =
          (a.trace && blockIdx.x == a.nwg - 1 && threadIdx.x == 0) ? a.trace + ((size_t)t * a.L + l) * 16
                                                                    : nullptr;
      if (threadIdx.x == 0) s.sm->tr = tr;
      if (tr) s.sm->trl[0] = wall_clock64();
      unsigned long long* twg = (a.trace_wg && t == 2 && threadIdx.x == 0)
                                    ? a.trace_wg + ((size_t)l * a.nwg + blockIdx.x) * 4
                                    : nullptr;
      if constexpr (SPEC) {
        if (!phase_a_spec<BITS>(a, s, t, l, sp, sh, dp)) return;
      } else {
        if (!phase_a<BITS, SPEC>(a, s, t, l, sp, true)) return;
      }
      if (tr) s.sm->trl[1] = wall_clock64();
      if (twg) s.sm->twl[0] = wall_clock64();
      if constexpr (SPEC) {
        if (!phase_b_spec<BITS>(a, s, t, l, dp, sh)) return;
      } else {
        if (!phase_b<BITS, SPEC, STREAM>(a, s, t, l, dp, true)) return;
      }
      if (tr) s.sm->trl[3] = wall_clock64();
      if (twg) s.sm->twl[2] = wall_clock64();
      const bool more = !(t == a.T - 1 && l == a.L - 1);
      if (!phase_c<BITS, SPEC, STREAM>(a, s, t, l, true, dp, true, sp, more)) return;
      if (tr) {
        s.sm->trl[5] = wall_clock64();
        for (int i = 0; i < 16; ++i) ((gl_u64*)(uintptr_t)tr)[i] = s.sm->trl[i];
      }
      if (twg) {
        s.sm->twl[3] = wall_clock64();
        for (int i = 0; i < 4; ++i) ((gl_u64*)(uintptr_t)twg)[i] = s.sm->twl[i];
      }
    }
  }
}

template <int BITS>
__device__ __forceinline__ void specialise(DecodeArgs& a, bool gate) {
  a.geo = make_geo(kSpecH, kSpecI, BITS);
  a.E = kSpecE;
  a.K = kSpecK;
  a.S = kSpecS;
  a.mode = MODE_LAYER;
  // the specialised logits exchange: expert e at pair e (lx_pos with C = 2 is the
  // identity); the replica holds all 512 pairs
  a.lx_c = 2;
  a.e_pad = kSpecE;
  a.nwg = kSpecNwg;
  a.rpw = kSpecH / kSpecNwg;
  a.exact_rows = 1;
  a.npass = 2;
  a.npass_routed = 1;
  a.pass_first[0] = 0; a.pass_count[0] = kSpecK;
  a.pass_first[1] = kSpecK; a.pass_count[1] = kSpecS;
  a.const_pass = 1;
  a.any_sgate = gate;
  a.pre_router = a.pre_shared = a.pre_down = 1;
}

// only_phase < 0: persistent (all tokens, all layers; phases wait on their inputs'
// epochs). only_phase = 0/1/2: run that phase for token t_only, layer l_only.
// SPEC: the specialised stack kernel (persistent, layer mode, flash-moe shape).
template <int BITS, bool SPEC, bool STREAM = false>
__device__ __forceinline__ void decode_body(const DecodeArgs& a, unsigned* lds_raw, int only_phase,
                                            int t_only, int l_only) {
  const Lds s = lds_view(lds_raw, a);
  const bool persistent = only_phase < 0;
  // LDS copies of the pass table and of the layer table
  if (!a.const_pass && (int)threadIdx.x < kMaxPass) {
    s.sm->pass_first[threadIdx.x] = a.pass_first[threadIdx.x];
    s.sm->pass_count[threadIdx.x] = a.pass_count[threadIdx.x];
    s.sm->pass_lgn[threadIdx.x] = log2i(a.pass_count[threadIdx.x] > 0 ? a.pass_count[threadIdx.x] : 1);
  }
  if (a.layers) {
    const __attribute__((address_space(1))) unsigned long long* src =
        (const __attribute__((address_space(1))) unsigned long long*)(uintptr_t)a.layers;
    unsigned long long* dst = reinterpret_cast<unsigned long long*>(lds_raw + a.lds_layers);
    for (int i = threadIdx.x; i < (int)(sizeof(LayerPtrs) / 8) * a.n_lds_layers; i += kThreads) dst[i] = src[i];
  } else if (a.n_lds_layers == 1 && threadIdx.x == 0) {
    LayerPtrs* dst = reinterpret_cast<LayerPtrs*>(lds_raw + a.lds_layers);
    dst->experts = a.layer0.experts;
    dst->shared = a.layer0.shared;
    dst->router = a.layer0.router;
    dst->gamma = a.layer0.gamma;
    dst->sgate = a.layer0.sgate;
  }
  if (threadIdx.x == 0) s.sm->ok = 1;
  __syncthreads();
  if constexpr (SPEC) {
    decode_chain<BITS, true>(a, s);
    return;
  }
  if (persistent && a.mode == MODE_LAYER && a.pre_router && a.pre_down) {
    decode_chain<BITS, false, STREAM>(a, s);
    return;
  }
  const int t0 = persistent ? 0 : t_only, t1 = persistent ? a.T : t_only + 1;
  const int l0 = persistent ? 0 : l_only, l1 = persistent ? a.L : l_only + 1;
  for (int t = t0; t < t1; ++t) {
    for (int l = l0; l < l1; ++l) {
      if (threadIdx.x == 0) s.sm->tr = nullptr;
      StaticPre sp;
      DownPre dp;
      bool have_x = false;
      if (a.mode != MODE_EXPERT && (persistent || only_phase == 0)) {
        if (!phase_a<BITS>(a, s, t, l, sp, false)) return;
        have_x = true;
      }
      if (persistent || only_phase == 1) {
        if (!have_x && a.mode != MODE_ROUTE && !prepare_x(a, s, t, l)) return;
        if (!phase_b<BITS, false, STREAM>(a, s, t, l, dp, false)) return;
      }
      if (a.mode != MODE_ROUTE && (persistent || only_phase == 2)) {
        if (!persistent && a.mode == MODE_LAYER) {
          // phased launch: the residual rows come straight from memory (the
          // producing launch has completed)
          const int r0 = blockIdx.x * a.rpw;
          if ((int)threadIdx.x < a.rpw && r0 + (int)threadIdx.x < a.geo.H) {
            const int r = r0 + threadIdx.x;
            s.xres[threadIdx.x] = l == 0 ? a.x0[(size_t)t * a.geo.H + r]
                                         : __uint_as_float((unsigned)xv_x(a, epoch_of(a, t, l)).base[r]);
          }
          if ((int)threadIdx.x < a.K) {
            s.sm->sel_idx[threadIdx.x] = ld_coh(a.sel + threadIdx.x);
            s.sm->sel_w[threadIdx.x] = __int_as_float(ld_coh(a.sel + kMaxK + threadIdx.x));
          }
          if ((int)threadIdx.x < a.S)
            s.sm->sgc[threadIdx.x] = __int_as_float(ld_coh(a.sel + 2 * kMaxK + threadIdx.x));
          __syncthreads();
        }
        if (!phase_c<BITS, false, STREAM>(a, s, t, l, a.pre_down, dp, false, sp, false)) return;
      }
    }
  }
}

// GATE (specialised kernel only): some layer has a shared-expert gate.
// STREAM (general kernel only): the streamed stack (routed experts in host memory).
template <int BITS, bool SPEC, bool GATE = false, bool STREAM = false>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a_in, int only_phase, int t_only,
                                                          int l_only) {
  extern __shared__ __align__(16) unsigned lds_raw[];
  if constexpr (SPEC) {
    DecodeArgs a = a_in;
    specialise<BITS>(a, GATE);
    decode_body<BITS, true>(a, lds_raw, only_phase, t_only, l_only);
  } else {
    decode_body<BITS, false, STREAM>(a_in, lds_raw, only_phase, t_only, l_only);
  }
}

// ---------------------------------------------------------------------------
// Fused Q/K/V projection. The three matrices are one packed matrix of R = Rq + Rk +
// Rv rows (the gate-matrix block layout); every workgroup stages, normalises and
// encodes a token's input once and reduces its blocks' rows against it. A wave's
// first kQkvB blocks are requested before the input is staged, the next ones while
// the current ones are reduced.
// ---------------------------------------------------------------------------
struct QkvArgs {
  Geo geo;  // H columns, I = R rows
  int rq, rk, R, T, nwg, norm;
  float eps;
  const uint8_t* w;
  const float* gamma;
  const float* x;
  float *yq, *yk, *yv;
};

constexpr int kQkvB = 4;  // blocks per wave in flight together

template <int BITS>
__global__ __launch_bounds__(kThreads) void qkv_kernel(QkvArgs a) {
  __shared__ __align__(16) unsigned dig[(kMaxDim / kGroup) * kDigitStride];
  __shared__ __align__(16) float sums[4 * (kMaxDim / kGroup)];
  __shared__ float red[kNW];
  const Geo& g = a.geo;
  const int H = g.H;
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int p = lane >> g.lGh, grp = lane & (g.Gh - 1);
  int b0, b1;
  split_range(g.nblk_gu, a.nwg, blockIdx.x, b0, b1);
  if (b0 >= b1) return;  // whole workgroup: no block here
  const int first = b0 + w < b1 ? b0 + w : b0;  // a wave without blocks re-reads a valid one
  auto blk_of = [&](int b) { return a.w + (size_t)(b < b1 ? b : first) * g.blk; };
  for (int t = 0; t < a.T; ++t) {
    Slot S[kQkvB];
#pragma unroll
    for (int j = 0; j < kQkvB; ++j) S[j] = ld_slot<BITS>(blk_of(b0 + w + j * kNW), lane, false);
    issue_order();
    // thread t holds chunks t and t + kThreads of 8 input values (the chunks that
    // encode_chunk8 takes from it), with their gamma, both requested together
    const float* xt = a.x + (size_t)t * H;
    const int nch = H / 8;
    float v[16], gm[16];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = h * kThreads + (int)threadIdx.x;
      float4 v0 = make_float4(0.f, 0.f, 0.f, 0.f), v1 = v0, g0 = make_float4(1.f, 1.f, 1.f, 1.f), g1 = g0;
      if (c < nch) {
        v0 = ldg_f4(xt + 8 * c);
        v1 = ldg_f4(xt + 8 * c + 4);
        if (a.gamma) {
          g0 = ldg_f4(a.gamma + 8 * c);
          g1 = ldg_f4(a.gamma + 8 * c + 4);
        }
      }
      v[8 * h] = v0.x; v[8 * h + 1] = v0.y; v[8 * h + 2] = v0.z; v[8 * h + 3] = v0.w;
      v[8 * h + 4] = v1.x; v[8 * h + 5] = v1.y; v[8 * h + 6] = v1.z; v[8 * h + 7] = v1.w;
      gm[8 * h] = g0.x; gm[8 * h + 1] = g0.y; gm[8 * h + 2] = g0.z; gm[8 * h + 3] = g0.w;
      gm[8 * h + 4] = g1.x; gm[8 * h + 5] = g1.y; gm[8 * h + 6] = g1.z; gm[8 * h + 7] = g1.w;
    }
    float rinv = 1.f;
    if (a.norm) {
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) ss = fmaf(v[i], v[i], ss);
      ss = wave_sum(ss);
      if (lane == 0) red[w] = ss;
      __syncthreads();
      ss = 0.f;
      for (int i = 0; i < kNW; ++i) ss += red[i];
      rinv = 1.f / sqrtf(ss / (float)H + a.eps);
    }
    // x_n = (x * gamma) * rinv, then its digits
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = (v[i] * gm[i]) * rinv;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = h * kThreads + (int)threadIdx.x;
      encode_chunk8(v + 8 * h, dig, sums, c / 8, c % 8, c < nch);
    }
    __syncthreads();
    Dig D;
    load_dig(D, dig, sums, grp);
    for (int ib = b0 + w; ib < b1; ib += kQkvB * kNW) {
      Slot C[kQkvB];
#pragma unroll
      for (int j = 0; j < kQkvB; ++j) C[j] = S[j];
#pragma unroll
      for (int j = 0; j < kQkvB; ++j) S[j] = ld_slot<BITS>(blk_of(ib + (kQkvB + j) * kNW), lane, false);
#pragma unroll
      for (int j = 0; j < kQkvB; ++j) {
        const int b = ib + j * kNW;
        if (b >= b1) continue;
        const float r = seg_sum(slot_dot<BITS>(C[j], D), g.Gh);
        const int row = (b << g.lPh) + p;
        if (grp == 0 && row < a.R) {
          if (row < a.rq) a.yq[(size_t)t * a.rq + row] = r;
          else if (row < a.rq + a.rk) a.yk[(size_t)t * a.rk + (row - a.rq)] = r;
          else a.yv[(size_t)t * (a.R - a.rq - a.rk) + (row - a.rq - a.rk)] = r;
        }
      }
    }
    __syncthreads();  // the next token overwrites the staged input and its digits
  }
}

// Several tokens per call. The single-token kernel above re-reads every slot and
// stages, normalises and encodes one input per pass, with a barrier round trip per
// token. Here a pass takes kQkvTB tokens: their inputs are requested together,
// normalised with one barrier and encoded into kQkvTB digit sets in LDS, and every
// slot, once in registers, is reduced against each token's digits in turn.
constexpr int kQkvTB = 4;

template <int BITS>
__global__ __launch_bounds__(kThreads) void qkv_batched_kernel(QkvArgs a) {
  __shared__ __align__(16) unsigned dig[kQkvTB][(kMaxDim / kGroup) * kDigitStride];
  __shared__ __align__(16) float sums[kQkvTB][4 * (kMaxDim / kGroup)];
  __shared__ float red[kQkvTB][kNW];
  const Geo& g = a.geo;
  const int H = g.H;
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int p = lane >> g.lGh, grp = lane & (g.Gh - 1);
  int b0, b1;
  split_range(g.nblk_gu, a.nwg, blockIdx.x, b0, b1);
  if (b0 >= b1) return;  // whole workgroup: no block here
  const int first = b0 + w < b1 ? b0 + w : b0;  // a wave without blocks re-reads a valid one
  auto blk_of = [&](int b) { return a.w + (size_t)(b < b1 ? b : first) * g.blk; };
  const int nch = H / 8;
  for (int t0 = 0; t0 < a.T; t0 += kQkvTB) {
    const int tb = a.T - t0 < kQkvTB ? a.T - t0 : kQkvTB;
    Slot S[kQkvB];
#pragma unroll
    for (int j = 0; j < kQkvB; ++j) S[j] = ld_slot<BITS>(blk_of(b0 + w + j * kNW), lane, false);
    issue_order();
    // thread t holds chunks t and t + kThreads of 8 values of every token of the
    // pass (tokens past the last are zeros and are never reduced)
    float v[kQkvTB][16], gm[16];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = h * kThreads + (int)threadIdx.x;
      float4 g0 = make_float4(1.f, 1.f, 1.f, 1.f), g1 = g0;
      if (c < nch && a.gamma) {
        g0 = ldg_f4(a.gamma + 8 * c);
        g1 = ldg_f4(a.gamma + 8 * c + 4);
      }
      gm[8 * h] = g0.x; gm[8 * h + 1] = g0.y; gm[8 * h + 2] = g0.z; gm[8 * h + 3] = g0.w;
      gm[8 * h + 4] = g1.x; gm[8 * h + 5] = g1.y; gm[8 * h + 6] = g1.z; gm[8 * h + 7] = g1.w;
#pragma unroll
      for (int tt = 0; tt < kQkvTB; ++tt) {
        float4 v0 = make_float4(0.f, 0.f, 0.f, 0.f), v1 = v0;
        if (c < nch && tt < tb) {
          const float* xt = a.x + (size_t)(t0 + tt) * H;
          v0 = ldg_f4(xt + 8 * c);
          v1 = ldg_f4(xt + 8 * c + 4);
        }
        v[tt][8 * h] = v0.x; v[tt][8 * h + 1] = v0.y; v[tt][8 * h + 2] = v0.z; v[tt][8 * h + 3] = v0.w;
        v[tt][8 * h + 4] = v1.x; v[tt][8 * h + 5] = v1.y; v[tt][8 * h + 6] = v1.z; v[tt][8 * h + 7] = v1.w;
      }
    }
    float rinv[kQkvTB];
#pragma unroll
    for (int tt = 0; tt < kQkvTB; ++tt) rinv[tt] = 1.f;
    if (a.norm) {
#pragma unroll
      for (int tt = 0; tt < kQkvTB; ++tt) {
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) ss = fmaf(v[tt][i], v[tt][i], ss);
        ss = wave_sum(ss);
        if (lane == 0) red[tt][w] = ss;
      }
      __syncthreads();
#pragma unroll
      for (int tt = 0; tt < kQkvTB; ++tt) {
        float ss = 0.f;
        for (int i = 0; i < kNW; ++i) ss += red[tt][i];
        rinv[tt] = 1.f / sqrtf(ss / (float)H + a.eps);
      }
    }
    // x_n = (x * gamma) * rinv, then its digits, one set per token
#pragma unroll
    for (int tt = 0; tt < kQkvTB; ++tt) {
      if (tt >= tb) break;
#pragma unroll
      for (int i = 0; i < 16; ++i) v[tt][i] = (v[tt][i] * gm[i]) * rinv[tt];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = h * kThreads + (int)threadIdx.x;
        encode_chunk8(v[tt] + 8 * h, dig[tt], sums[tt], c / 8, c % 8, c < nch);
      }
    }
    __syncthreads();
    for (int ib = b0 + w; ib < b1; ib += kQkvB * kNW) {
      Slot C[kQkvB];
#pragma unroll
      for (int j = 0; j < kQkvB; ++j) C[j] = S[j];
#pragma unroll
      for (int j = 0; j < kQkvB; ++j) S[j] = ld_slot<BITS>(blk_of(ib + (kQkvB + j) * kNW), lane, false);
      for (int tt = 0; tt < tb; ++tt) {
        Dig D;
        load_dig(D, dig[tt], sums[tt], grp);
        const int t = t0 + tt;
#pragma unroll
        for (int j = 0; j < kQkvB; ++j) {
          const int b = ib + j * kNW;
          if (b >= b1) continue;
          const float r = seg_sum(slot_dot<BITS>(C[j], D), g.Gh);
          const int row = (b << g.lPh) + p;
          if (grp == 0 && row < a.R) {
            if (row < a.rq) a.yq[(size_t)t * a.rq + row] = r;
            else if (row < a.rq + a.rk) a.yk[(size_t)t * a.rk + (row - a.rq)] = r;
            else a.yv[(size_t)t * (a.R - a.rq - a.rk) + (row - a.rq - a.rk)] = r;
          }
        }
      }
    }
    __syncthreads();  // the next pass overwrites the staged inputs and their digits
  }
}

typedef void (*DecodeKernel)(DecodeArgs, int, int, int);
typedef void (*QkvKernel)(QkvArgs);
// Kernel tables, one per code width (each defined in its own file so that the
// three widths compile in parallel). variant: 0 general, 1 specialised,
// 2 specialised with the shared-expert gate, 3 streamed.
DecodeKernel decode_kernel_b2(int variant);
DecodeKernel decode_kernel_b3(int variant);
DecodeKernel decode_kernel_b4(int variant);
QkvKernel qkv_kernel_b2();
QkvKernel qkv_kernel_b3();
QkvKernel qkv_kernel_b4();
QkvKernel qkv_batched_kernel_b2();
QkvKernel qkv_batched_kernel_b3();
QkvKernel qkv_batched_kernel_b4();

}  // namespace qmoe
