// qmoe_internal.h -- packed layout geometry, argument structs and device helpers
// shared by the HIP kernels of libqmoe (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/qmoe.h"

namespace qmoe {

constexpr int kWave = 64;
constexpr int kGroup = 64;
constexpr int kMaxK = 16;  // routed experts per token (the model's native top-k is 10)
constexpr int kMaxE = 1024;
constexpr int kMaxShared = 2;
constexpr int kMaxDim = 4096;
constexpr int kMaxNwg = 1024;     // workgroups a decode launch may use
constexpr int kMaxCacheSlots = 64;  // HBM expert-cache slots per layer (streamed stack)
constexpr int kRep = 4;           // replicas of every exchanged vector (spreads polling)
constexpr int kDigitStride = 52;  // dwords per (vector, group) in LDS: 48 digit dwords + pad

// ---------------------------------------------------------------------------
// Packed expert layout.
//
// Each matrix W[R][C] (R outputs, C inputs, G = C/64 groups per row) is stored as
// blocks of P = 64/G rows. A block has 64 "slots", slot = p*G + g for row p of the
// block and group g, so one wave of 64 lanes reads a whole block with one slot per
// lane (lane-contiguous, fully coalesced 16-byte loads):
//   4-bit: [chunk0: 64 slots x 16 B][chunk1: 64 slots x 16 B][sb: 64 slots x 4 B]
//          = 2304 B; chunk c of a slot holds codes 32c..32c+31 of the group.
//   3-bit: [plane0: 64 slots x 16 B][plane1: 64 slots x 8 B][sb: 64 slots x 4 B]
//          = 1792 B.
//   2-bit: [codes: 64 slots x 16 B][sb: 64 slots x 4 B] = 1280 B.
// sb = (bias_bf16 << 16) | scale_bf16.
// Inside a 4-bit chunk, dword j holds the 8 codes 8j'..8j'+7 of the group
// (j' = 4c + j) in "digit order": nibble 2m <- code 8j'+m, nibble 2m+1 <- code
// 8j'+4+m (m = 0..3), each stored as (q ^ 8), i.e. q - 8 as a signed 4-bit value.
// Inside a 2-bit slot, dword j holds codes 16j..16j+15: bits [4n, 4n+2) hold code
// 16j + d(n) and bits [4n+2, 4n+4) hold code 16j + 8 + d(n), d(2m) = m,
// d(2m+1) = 4 + m, unsigned.
// A 3-bit slot holds six dwords w0..w5 (plane0 = w0..w3, plane1 = w4, w5) in two
// triples (w0, w1, w2) and (w3, w4, w5). Triple t covers codes 32t..32t+31: for
// i = 0, 1, 2, bits [4n, 4n+3) of its i-th dword hold code 32t + 8i + d(n) and
// bit 4n+3 holds bit i of code 32t + 24 + d(n) (d as above, unsigned codes). So
// masking a dword with 0x77777777 gives eight 3-bit codes in nibbles, and the
// fourth octet of a triple is gathered from the three top bits of each nibble.
// An expert is [gate blocks][up blocks][down blocks]; gate/up have R = I, C = H
// and down has R = H, C = I. Blocks are multiples of 256 B, so every block of an
// expert that starts 256-B aligned is 256-B aligned too.
// ---------------------------------------------------------------------------
struct Geo {
  int H, I, bits;
  int Gh, Ph;        // groups per gate/up row, rows per gate/up block
  int Gi, Pi;        // groups per down row, rows per down block
  int blk;           // bytes per block
  int nblk_gu;       // blocks in the gate (and in the up) matrix
  int nblk_d;        // blocks in the down matrix
  size_t off_up;     // byte offset of the up matrix inside an expert
  size_t off_down;   // byte offset of the down matrix
  size_t expert_bytes;
  // log2 of Gh, Ph, Gi, Pi and nblk_gu (all powers of two for the supported shapes)
  int lGh, lPh, lGi, lPi, lnb;
};

__host__ __device__ constexpr int log2i(int v) {
  int r = 0;
  while ((1 << r) < v) ++r;
  return r;
}

__host__ __device__ constexpr bool pow2_dim_ok(int v) {
  return v >= 64 && v <= kMaxDim && (v & (v - 1)) == 0;
}

// Byte offset of the (scale, bias) words inside a block, and of the second code
// plane (4- and 3-bit; its slots are 16 and 8 bytes wide).
__host__ __device__ constexpr int sb_offset(int bits) {
  return bits == 4 ? 2048 : bits == 3 ? 1536 : 1024;
}
constexpr int kPlane1Offset = 1024;

__host__ __device__ constexpr Geo make_geo(int H, int I, int bits) {
  Geo g{};
  g.H = H; g.I = I; g.bits = bits;
  g.Gh = H / kGroup; g.Ph = kWave / g.Gh;
  g.Gi = I / kGroup; g.Pi = kWave / g.Gi;
  g.blk = sb_offset(bits) + 4 * kWave;
  g.nblk_gu = (I + g.Ph - 1) / g.Ph;
  g.nblk_d = (H + g.Pi - 1) / g.Pi;
  g.off_up = (size_t)g.nblk_gu * g.blk;
  g.off_down = 2 * g.off_up;
  g.expert_bytes = g.off_down + (size_t)g.nblk_d * g.blk;
  g.lGh = log2i(g.Gh); g.lPh = log2i(g.Ph); g.lGi = log2i(g.Gi); g.lPi = log2i(g.Pi);
  g.lnb = log2i(g.nblk_gu);
  return g;
}

// Geometry of one packed matrix of R rows and H columns, laid out like an expert's
// gate matrix (blocks of Ph = 64/Gh rows); expert_bytes is the matrix's size.
inline Geo make_matrix_geo(int H, int R, int bits) {
  Geo g{};
  g.H = H; g.I = R; g.bits = bits;
  g.Gh = H / kGroup; g.Ph = kWave / g.Gh;
  g.Gi = 1; g.Pi = 1;
  g.blk = sb_offset(bits) + 4 * kWave;
  g.nblk_gu = (R + g.Ph - 1) / g.Ph;
  g.nblk_d = 0;
  g.expert_bytes = (size_t)g.nblk_gu * g.blk;
  g.off_up = g.off_down = g.expert_bytes;
  g.lGh = log2i(g.Gh); g.lPh = log2i(g.Ph);
  return g;
}

// Device copy of one layer's pointers.
struct LayerPtrs {
  const uint8_t* experts;
  const uint8_t* shared;
  const float* router;
  const float* gamma;
  const float* sgate;  // [n_shared][H] shared-expert gate or NULL
};

// Workspace layout (byte offsets from the workspace base; all 256-B aligned).
struct WsLayout {
  size_t err, sync, xbuf, logits, hbuf, sel, prev, layers, ctab, pack_err, total;
};

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Router logits per lane of the top-K wave: ceil(E / 64) rounded up to even.
__host__ __device__ constexpr int lx_per_lane(int E) { return (((E + kWave - 1) / kWave) + 1) & ~1; }

// with_ctab = false leaves out the streamed stack's cache tables (calls that do
// not stream never touch them)
inline WsLayout ws_layout(const moe_config& c, int T, int L, bool with_ctab = true) {
  (void)T;
  WsLayout w;
  size_t o = 0;
  w.err = o; o += 256;
  w.sync = o; o = align256(o + sizeof(unsigned) * (64 + kMaxNwg));
  w.pack_err = o; o += 256;
  // exchanged vectors: two buffers (epoch parity) of kRep replicas of (value,
  // epoch) pairs
  w.xbuf = o; o = align256(o + 2 * kRep * sizeof(uint64_t) * c.hidden);
  w.logits = o; o = align256(o + 2 * kRep * sizeof(uint64_t) * (size_t)kWave * lx_per_lane(c.n_experts));
  w.hbuf = o; o = align256(o + 2 * kRep * sizeof(uint64_t) * (size_t)(kMaxK + kMaxShared) * c.inter);
  // selection words: [kMaxK] indices, [kMaxK] weights, [kMaxShared] shared-gate factors
  w.sel = o; o = align256(o + sizeof(int) * (2 * kMaxK + kMaxShared));
  w.prev = o; o = align256(o + sizeof(uint64_t) * 2 * (size_t)(L > 0 ? L : 1) * kMaxK);
  w.layers = o; o = align256(o + sizeof(LayerPtrs) * (size_t)(L > 0 ? L : 1));
  // streamed stack: every workgroup's copy of every layer's expert-cache table
  w.ctab = o;
  if (with_ctab) o = align256(o + sizeof(uint64_t) * (size_t)kMaxNwg * (L > 0 ? L : 1) * kMaxCacheSlots);
  w.total = o;
  return w;
}

// One decode-engine call (route, expert forward, layer forward or stack decode).
struct DecodeRequest {
  int mode;  // 0 layer/stack, 1 route only, 2 single expert
  moe_config cfg;
  int L, T;
  const LayerPtrs* layers_host;  // [L] validated layer table in host memory (stack calls), or NULL;
                                 // read during the call only (it travels in kernel arguments)
  const uint8_t* single_expert;
  const float* x0;
  float* y;
  const uint8_t* boost_mask;
  const float* sel_bias;
  const int* boosted;
  int* idx_out;
  float* w_out;
  float* logits_out;
  uint8_t* ws;
  WsLayout wl;
  bool phased;
  bool any_sgate;  // some layer has a shared-expert gate
  // streamed stack: routed experts in host memory, an HBM cache of cslots per layer
  bool stream;
  uint8_t* cache;
  int cslots;
  uint8_t* hit_out;
  // one-layer calls: the layer's pointers travel in the decode kernel's arguments
  // (layers_host == NULL), so no table is written to the workspace
  bool inline_layer;
  LayerPtrs layer0;
};

// mats: 3 (n experts: gate, up, down) or 1 (n matrices of geo.I rows, geo.H columns)
hipError_t launch_pack(const Geo& geo, int n, int mats, const uint8_t* codes, const uint16_t* scales,
                       const uint16_t* biases, void* packed, unsigned* err, hipStream_t stream);
hipError_t launch_qkv(const moe_qkv_config& c, const uint8_t* w, const float* gamma, int T, const float* x,
                      float* q, float* k, float* v, hipStream_t stream);
hipError_t launch_decode(const DecodeRequest& r, hipStream_t stream, const char** why);

// Device error codes (written to the workspace error word; first error wins).
enum DevErr : unsigned {
  DEV_OK = 0,
  DEV_BAD_INDEX = 1,     // an expert index outside [0, E)
  DEV_SYNC_TIMEOUT = 2,  // a wait for another workgroup's data exceeded its time limit
  DEV_BAD_CODE = 3,      // pack: a code >= 2^bits
};

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
__device__ inline float bf16lo_to_f32(unsigned v) { return __uint_as_float(v << 16); }
__device__ inline float bf16hi_to_f32(unsigned v) { return __uint_as_float(v & 0xFFFF0000u); }

__device__ inline void set_dev_err(unsigned* err, unsigned code) {
  unsigned expected = 0;
  __hip_atomic_compare_exchange_strong(err, &expected, code, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace qmoe
