// qmoe_decode.hip -- host side of the decode engine: launch configuration, the
// persistent-grid ordering and the Q/K/V launch. The kernels are in
// qmoe_decode_dev.h (instantiated per code width in qmoe_decode_k*.hip).
#include <hip/hip_ext.h>

#include <algorithm>
#include <mutex>
#include <cstring>

#include "qmoe_decode_dev.h"

namespace qmoe {

__global__ void zero_u64(unsigned long long* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0ull;
}

// Layer-table entries carried in kernel arguments: the table reaches the device
// in the launch itself, so a call never waits for a host-to-device copy.
constexpr int kTableChunk = 64;
struct TableChunk {
  int first, n;
  LayerPtrs p[kTableChunk];
};

// Start of a decode call: clears the abort flag, the error word and every exchange
// slot (epoch 0 never matches a live epoch, which start at 1), and writes the
// first chunk of the layer table.
__global__ void prologue_kernel(unsigned* sync, unsigned* err, unsigned long long* xch, size_t nx,
                                LayerPtrs* table, TableChunk chunk) {
  const size_t i0 = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  if (i0 == 0) {
    sync[0] = 0u;
    err[0] = 0u;
  }
  for (size_t i = i0; i < nx; i += (size_t)gridDim.x * blockDim.x) xch[i] = 0ull;
  if (blockIdx.x == 0 && (int)threadIdx.x < chunk.n) table[chunk.first + threadIdx.x] = chunk.p[threadIdx.x];
}

// Further chunks of the layer table (stacks of more than kTableChunk layers).
__global__ void table_kernel(LayerPtrs* table, TableChunk chunk) {
  if ((int)threadIdx.x < chunk.n) table[chunk.first + threadIdx.x] = chunk.p[threadIdx.x];
}

// ------------------------------------------------------------ host side
// Per-device state, created on first use on a device: its compute-unit count and
// wall-clock rate, which kernel variants have their LDS limit raised, and the
// ordering of persistent launches. This is the library's only state beyond its
// loaded code objects; it holds no device memory.
constexpr int kMaxDevices = 64;
struct DevState {
  std::mutex mu;
  bool ready = false;
  int num_cu = 0;
  long long wall_khz = 0;
  bool lds_attr[3][4] = {};
  // Persistent launches are put in one order on each device: a launch on another
  // stream than the previous one waits for the event that launch signalled on
  // completion (a launch on the same stream is ordered by the stream). So two
  // persistent grids never hold compute units at the same time, however the
  // callers' streams overlap, and a grid launched on a stream allowed to use every
  // unit finds all of them free of this library's persistent work.
  hipEvent_t order_ev = nullptr;
  hipStream_t order_last = nullptr;
  bool order_any = false;
};
static DevState g_dev[kMaxDevices];

// The state of the device `stream` belongs to, initialised on first use.
static hipError_t device_state(hipStream_t stream, DevState** out, const char** why) {
  int dev = 0;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) {
    *why = "device ordinal beyond the library's limit";
    return hipErrorInvalidDevice;
  }
  DevState& d = g_dev[dev];
  std::lock_guard<std::mutex> lock(d.mu);
  if (!d.ready) {
    int cu = 0, khz = 0;
    e = hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
    if (e != hipSuccess || khz <= 0) khz = 100000;
    d.num_cu = cu;
    d.wall_khz = khz;
    d.ready = true;
  }
  *out = &d;
  return hipSuccess;
}

// Compute units a stream may dispatch to (its CU mask); 0 if the mask cannot be read.
static int stream_units(hipStream_t stream) {
  uint32_t mask[32] = {};
  if (hipExtStreamGetCUMask(stream, 32, mask) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  int n = 0;
  for (uint32_t m : mask) n += __builtin_popcount(m);
  return n;
}

// Launches the persistent grid in that order (plain launch when the stream may use
// every unit, else cooperative, whose residency the runtime checks).
static hipError_t launch_ordered(DevState& d, const void* kern, int nwg, size_t lds, hipStream_t stream,
                                 void** args, bool plain) {
  std::lock_guard<std::mutex> lock(d.mu);
  hipError_t e;
  if (!d.order_ev) {
    e = hipEventCreate(&d.order_ev);
    if (e != hipSuccess) {
      d.order_ev = nullptr;
      return e;
    }
  }
  if (d.order_any && stream != d.order_last) {
    e = hipStreamWaitEvent(stream, d.order_ev, 0);
    if (e != hipSuccess) return e;
  }
  if (plain) {
    // the dispatch itself signals the event when the grid completes
    e = hipExtLaunchKernel(kern, dim3(nwg), dim3(kThreads), args, lds, stream, nullptr, d.order_ev, 0);
    if (e != hipSuccess) return e;
  } else {
    e = hipLaunchCooperativeKernel(kern, dim3(nwg), dim3(kThreads), args, (unsigned)lds, stream);
    if (e != hipSuccess) return e;
    e = hipEventRecord(d.order_ev, stream);
    if (e != hipSuccess) return e;
  }
  d.order_last = stream;
  d.order_any = true;
  return hipSuccess;
}

unsigned long long* g_trace = nullptr;     // set only by instrumented builds
unsigned long long* g_trace_wg = nullptr;  // set only by instrumented builds
// Register-prefetch paths in use when a shape allows them: router rows (bit 0),
// shared gate/up slots (bit 1), down slots (bit 2); bit 3 allows the specialised
// kernel. Instrumented builds change it to compare the paths; the results are
// identical either way.
int g_pre_mask = 15;  // bit 3: the specialised kernel
int g_poll_sleep = 0;

hipError_t launch_decode(const DecodeRequest& r, hipStream_t stream, const char** why) {
  DevState* dsp = nullptr;
  hipError_t e = device_state(stream, &dsp, why);
  if (e != hipSuccess) return e;
  DevState& ds = *dsp;
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
  uint8_t* ws = r.ws;
  LayerPtrs* table = r.layers_host ? reinterpret_cast<LayerPtrs*>(ws + r.wl.layers) : nullptr;
  a.layers = table;
  if (r.inline_layer) a.layer0 = r.layer0;
  a.single_expert = r.single_expert;
  a.x0 = r.x0;
  a.y = r.y;
  a.boost_mask = r.boost_mask;
  a.sel_bias = r.sel_bias;
  a.boosted = r.boosted;
  a.idx_out = r.idx_out;
  a.w_out = r.w_out;
  a.logits_out = r.logits_out;
  a.xx = reinterpret_cast<unsigned long long*>(ws + r.wl.xbuf);
  a.lx = reinterpret_cast<unsigned long long*>(ws + r.wl.logits);
  a.hx = reinterpret_cast<unsigned long long*>(ws + r.wl.hbuf);
  a.lx_c = lx_per_lane(a.E);
  a.e_pad = kWave * a.lx_c;
  a.sel = reinterpret_cast<int*>(ws + r.wl.sel);
  a.prev = reinterpret_cast<unsigned long long*>(ws + r.wl.prev);
  a.sync = reinterpret_cast<unsigned*>(ws + r.wl.sync);
  a.err = reinterpret_cast<unsigned*>(ws + r.wl.err);
  a.timeout_ticks = (unsigned long long)ds.wall_khz * 2000ull;  // 2 seconds per wait
  a.poll_sleep = g_poll_sleep;
  a.trace = g_trace;
  a.trace_wg = g_trace_wg;
  if (r.stream) {
    a.cache = r.cache;
    a.cslots = r.cslots;
    a.ctab = reinterpret_cast<unsigned long long*>(ws + r.wl.ctab);
    a.hit_out = r.hit_out;
  }

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
    a.npass_routed = np;
    add_passes(a.K, a.S);
  }
  a.npass = np;
  int maxP = 1;
  for (int i = 0; i < np; ++i) maxP = std::max(maxP, kWave / (a.pass_count[i] * Gi));

  // One workgroup per compute unit, and no more workgroups than there are router
  // rows or routed gate/up items (the mode's exchange work), so that every
  // workgroup produces some of the logits or of the routed h at every epoch: that
  // is what keeps a slot from being rewritten before every workgroup has read it
  // (see the exchange buffers). Phase C rows per workgroup stay <= 64: the routed
  // items alone are at least hidden / 64 for every supported shape.
  const int items = r.mode == MODE_ROUTE    ? a.E
                    : r.mode == MODE_EXPERT ? a.geo.nblk_gu
                                            : std::max(a.E, r.stream ? a.geo.nblk_gu : a.K * a.geo.nblk_gu);
  const int nwg = std::min(ds.num_cu, items);
  if (nwg > kMaxNwg) {
    *why = "more compute units than the decode kernel supports";
    return hipErrorInvalidValue;
  }
  int rpw = (c.hidden + nwg - 1) / nwg;
  rpw = ((rpw + maxP - 1) / maxP) * maxP;
  if (r.mode == MODE_ROUTE) rpw = std::min(rpw, 64);  // no phase C: the rows are not used
  if (rpw > 64) {
    *why = "hidden too large for the phase-C row split";
    return hipErrorInvalidValue;
  }
  a.rpw = rpw;
  a.any_sgate = r.any_sgate ? 1 : 0;
  a.exact_rows = (long long)rpw * nwg == c.hidden;
  a.nwg = nwg;
  const int nlist = r.mode == MODE_EXPERT ? 1 : c.top_k + c.n_shared;

  // LDS carve-up (32-bit words). The h staging area of phase C overlays the x
  // region (x, its digits and sums), which is dead by then.
  auto up4 = [](int v) { return (v + 3) & ~3; };
  const int hstage_words = nlist * c.inter;
  int words = up4((int)((sizeof(Small) + 3) / 4));
  const int xregion = words;
  a.lds_xn = words; words = up4(words + c.hidden);
  a.lds_xdig = words; words = up4(words + a.geo.Gh * kDigitStride);
  a.lds_xsum = words; words = up4(words + 4 * a.geo.Gh);
  words = std::max(words, up4(xregion + hstage_words));
  a.lds_hdig = words; words = up4(words + nlist * Gi * kDigitStride);
  a.lds_hsum = words; words = up4(words + 4 * nlist * Gi);
  a.lds_acc = words; words = up4(words + kMaxPass * rpw);
  a.lds_xres = words; words = up4(words + rpw);
  a.n_lds_layers = r.mode == MODE_EXPERT ? 0
                   : r.inline_layer ? 1
                   : table          ? std::min(r.L, kLdsLayers)
                                    : 0;
  a.lds_layers = (words + 1) & ~1;  // 8-byte aligned
  words = up4(a.lds_layers + a.n_lds_layers * (int)(sizeof(LayerPtrs) / 4));
  // register prefetch eligibility (see load_static / load_down)
  {
    const int rows_pw = (a.E + nwg - 1) / nwg;
    a.pre_router = rows_pw <= kRowsPre && rows_pw * (c.hidden / 4) <= kThreads * kRouterPre;
    const int sh_pw = (a.S * a.geo.nblk_gu + nwg - 1) / nwg;
    a.pre_shared = r.mode == MODE_LAYER && a.S > 0 && sh_pw <= kNW * kShPre;
    // every wave's number of down jobs, for the largest row range a workgroup gets
    int worst = 0;
    for (int w = 0; w < kNW; ++w) {
      int jobs = 0;
      for (int pi = 0; pi < np; ++pi) {
        const int seg = a.pass_count[pi] * Gi, Pp = kWave / seg;
        const int nchunk = (rpw + Pp - 1) / Pp;
        jobs += w < nchunk ? (nchunk - w + kNW - 1) / kNW : 0;
      }
      worst = std::max(worst, jobs);
    }
    a.pre_down = worst <= kDnPre;
    a.pre_router = a.pre_router && (g_pre_mask & 1);
    a.pre_shared = a.pre_shared && (g_pre_mask & 2);
    a.pre_down = a.pre_down && (g_pre_mask & 4);
  }
  // the specialised kernel when the call is exactly the flash-moe stack shape
  const bool spec = !r.stream && r.mode == MODE_LAYER && !r.phased && c.hidden == kSpecH && c.inter == kSpecI &&
                    a.E == kSpecE && a.K == kSpecK && a.S == kSpecS && nwg == kSpecNwg &&
                    a.pre_router && a.pre_shared && a.pre_down && a.n_lds_layers == r.L &&
                    (g_pre_mask & 8);
  const bool gate = spec && r.any_sgate;
  a.lds_words = words;
  const size_t lds = (size_t)words * 4;
  if (lds > (size_t)kMaxLdsBytes) {
    *why = "shape needs more LDS than a workgroup has";
    return hipErrorInvalidValue;
  }
  // variant: general, specialised, specialised with the shared-expert gate, streamed
  const int kv = r.stream ? 3 : spec ? (gate ? 2 : 1) : 0;
  const DecodeKernel kern = c.bits == 4 ? decode_kernel_b4(kv) : c.bits == 3 ? decode_kernel_b3(kv)
                                                                              : decode_kernel_b2(kv);
  {
    std::lock_guard<std::mutex> lock(ds.mu);
    if (lds > 64 * 1024 && !ds.lds_attr[c.bits - 2][kv]) {
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                              hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLdsBytes);
      if (e != hipSuccess) return e;
      ds.lds_attr[c.bits - 2][kv] = true;
    }
  }
  if (!r.phased) {
    int occ = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(kern), kThreads, lds);
    if (e != hipSuccess) return e;
    if (occ < 1) {
      *why = "decode kernel does not fit on a compute unit";
      return hipErrorInvalidConfiguration;
    }
  }
  // Every check is done: from here on the call only enqueues. Every exchange slot,
  // the selection words and the epoch-tagged previous sets start at epoch 0; the
  // layer table travels in the clearing kernel's arguments.
  const size_t nx = (size_t)(r.wl.layers - r.wl.xbuf) / sizeof(unsigned long long);
  TableChunk chunk;
  memset(&chunk, 0, sizeof(chunk));
  const int nt = table ? r.L : 0;
  chunk.n = std::min(nt, kTableChunk);
  for (int i = 0; i < chunk.n; ++i) chunk.p[i] = r.layers_host[i];
  hipLaunchKernelGGL(prologue_kernel, dim3(256), dim3(256), 0, stream, a.sync, a.err, a.xx, nx, table, chunk);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  for (int first = kTableChunk; first < nt; first += kTableChunk) {
    chunk.first = first;
    chunk.n = std::min(nt - first, kTableChunk);
    for (int i = 0; i < chunk.n; ++i) chunk.p[i] = r.layers_host[first + i];
    hipLaunchKernelGGL(table_kernel, dim3(1), dim3(kTableChunk), 0, stream, table, chunk);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (r.stream) {
    // every workgroup's cache tables start empty: nothing cached by an earlier call is used
    hipLaunchKernelGGL(zero_u64, dim3(256), dim3(256), 0, stream, a.ctab, (size_t)nwg * r.L * r.cslots);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
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
  // The grid is at most one workgroup per compute unit and a workgroup fits on a
  // unit (checked above), so on a stream allowed to use every unit all workgroups are
  // resident together under a plain launch, which starts about 18 us sooner than a
  // cooperative one; persistent launches are ordered (launch_ordered), so no other
  // persistent grid of this library competes for the units. A stream restricted to
  // fewer units takes the cooperative launch. If other work holds units, the
  // remaining workgroups start as it retires; every wait is bounded, so the worst
  // outcome is DEV_SYNC_TIMEOUT, never a hang.
  int only = -1, zero = 0;
  void* args[] = {&a, &only, &zero, &zero};
  return launch_ordered(ds, reinterpret_cast<const void*>(kern), nwg, lds, stream, args,
                        stream_units(stream) >= nwg);
}

hipError_t launch_qkv(const moe_qkv_config& c, const uint8_t* w, const float* gamma, int T, const float* x,
                      float* q, float* k, float* v, hipStream_t stream) {
  DevState* dsp = nullptr;
  const char* why = nullptr;
  hipError_t e = device_state(stream, &dsp, &why);
  if (e != hipSuccess) return e;
  const int num_cu = dsp->num_cu;
  QkvArgs a;
  memset(&a, 0, sizeof(a));
  a.R = c.q_rows + c.k_rows + c.v_rows;
  a.geo = make_matrix_geo(c.hidden, a.R, c.bits);
  a.rq = c.q_rows;
  a.rk = c.k_rows;
  a.T = T;
  a.norm = (c.flags & MOE_F_RMSNORM) ? 1 : 0;
  a.eps = c.eps;
  a.w = w;
  a.gamma = gamma;
  a.x = x;
  a.yq = q;
  a.yk = k;
  a.yv = v;
  // two workgroups per compute unit (every unit the same load), at least one block
  // per wave: on 5120 rows of hidden 4096 this beats one block batch per wave (320
  // workgroups, some units holding two and some one) by 5% and 640 workgroups by 25%
  const int per = std::max(kNW, (a.geo.nblk_gu + 2 * num_cu - 1) / (2 * num_cu));
  a.nwg = std::max(1, (a.geo.nblk_gu + per - 1) / per);
  // one token: the single-token kernel; several: kQkvTB tokens per pass
  const QkvKernel kern = T == 1 ? (c.bits == 4 ? qkv_kernel_b4() : c.bits == 3 ? qkv_kernel_b3() : qkv_kernel_b2())
                                : (c.bits == 4   ? qkv_batched_kernel_b4()
                                   : c.bits == 3 ? qkv_batched_kernel_b3()
                                                 : qkv_batched_kernel_b2());
  hipLaunchKernelGGL(kern, dim3(a.nwg), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace qmoe
