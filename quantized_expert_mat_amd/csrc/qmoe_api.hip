// qmoe_api.hip -- the extern "C" entry points of libqmoe: argument validation,
// workspace carve-up and dispatch to the kernels. See include/qmoe.h.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include <vector>

#include "qmoe_internal.h"

namespace qmoe {
size_t prefill_ws_bytes(const moe_config& c, int T);
moe_status prefill_forward(const moe_config& c, const moe_layer_weights* lw, int T,
                           const float* x, float* y, const float* sel_bias, const int32_t* boosted,
                           int32_t* idx_out, float* w_out, uint8_t* ws, size_t ws_bytes,
                           hipStream_t stream, std::string* msg);
}  // namespace qmoe

using namespace qmoe;

// The workspace of moe_stack_decode_noalloc: one fixed array per device, held
// until the process ends. In host code `scratch` names a host-side stand-in, not
// device memory: host code uses only the address hipGetSymbolAddress returns for
// it (looked up once per device, see scratch_of).
constexpr size_t kScratchBytes = size_t(4) << 20;
constexpr int kScratchMaxLayers = 128;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

thread_local std::string g_msg;

moe_status fail(moe_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_msg = buf;
  return s;
}

moe_status hip_fail(hipError_t e, const char* what) {
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr int kKnownFlags =
    MOE_F_RMSNORM | MOE_F_RESIDUAL | MOE_F_SELECT_BY_BIAS | MOE_F_PREFILL_BF16 | MOE_F_PHASED;

moe_status check_config(const moe_config* c) {
  if (!c) return fail(MOE_ERR_ARG, "config is NULL");
  if (!pow2_dim_ok(c->hidden))
    return fail(MOE_ERR_UNSUPPORTED, "hidden=%d: must be 64*2^k, 64..4096", c->hidden);
  if (!pow2_dim_ok(c->inter))
    return fail(MOE_ERR_UNSUPPORTED, "inter=%d: must be 64*2^k, 64..4096", c->inter);
  if (c->group != 64) return fail(MOE_ERR_UNSUPPORTED, "group=%d: only 64", c->group);
  if (c->bits < 2 || c->bits > 4) return fail(MOE_ERR_UNSUPPORTED, "bits=%d: only 2, 3 or 4", c->bits);
  if (c->top_k < 1 || c->top_k > kMaxK)
    return fail(MOE_ERR_UNSUPPORTED, "top_k=%d: must be 1..%d", c->top_k, kMaxK);
  if (c->n_experts < c->top_k || c->n_experts > kMaxE)
    return fail(MOE_ERR_SHAPE, "n_experts=%d: must be top_k..%d", c->n_experts, kMaxE);
  if (c->n_shared < 0 || c->n_shared > kMaxShared)
    return fail(MOE_ERR_UNSUPPORTED, "n_shared=%d: must be 0..%d", c->n_shared, kMaxShared);
  if (c->flags & ~kKnownFlags) return fail(MOE_ERR_ARG, "unknown flags 0x%x", c->flags);
  if ((c->flags & MOE_F_RMSNORM) && !(c->eps > 0.f && c->eps < 1.f))
    return fail(MOE_ERR_ARG, "eps=%g must be in (0, 1)", (double)c->eps);
  return MOE_OK;
}

moe_status check_ws(const moe_config* c, int T, int L, void* ws, size_t ws_bytes) {
  if (!ws) return fail(MOE_ERR_ARG, "workspace is NULL");
  if (!aligned(ws, 256)) return fail(MOE_ERR_ALIGN, "workspace not 256-byte aligned");
  const size_t need = moe_workspace_bytes(c, T, L);
  if (ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  return MOE_OK;
}

#define REQUIRE(cond, status, ...)      \
  do {                                  \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

moe_status check_qkv(const moe_qkv_config* c) {
  if (!c) return fail(MOE_ERR_ARG, "config is NULL");
  if (!pow2_dim_ok(c->hidden))
    return fail(MOE_ERR_UNSUPPORTED, "hidden=%d: must be 64*2^k, 64..4096", c->hidden);
  if (c->q_rows < 1 || c->k_rows < 1 || c->v_rows < 1 ||
      (long long)c->q_rows + c->k_rows + c->v_rows > 65536)
    return fail(MOE_ERR_SHAPE, "rows %d/%d/%d: each >= 1, sum <= 65536", c->q_rows, c->k_rows, c->v_rows);
  if (c->group != 64) return fail(MOE_ERR_UNSUPPORTED, "group=%d: only 64", c->group);
  if (c->bits < 2 || c->bits > 4) return fail(MOE_ERR_UNSUPPORTED, "bits=%d: only 2, 3 or 4", c->bits);
  if (c->flags & ~MOE_F_RMSNORM) return fail(MOE_ERR_ARG, "flags 0x%x: only MOE_F_RMSNORM", c->flags);
  if ((c->flags & MOE_F_RMSNORM) && !(c->eps > 0.f && c->eps < 1.f))
    return fail(MOE_ERR_ARG, "eps=%g must be in (0, 1)", (double)c->eps);
  return MOE_OK;
}

moe_status layer_ptrs(const moe_config& c, const moe_layer_weights& w, int l, LayerPtrs& p) {
  REQUIRE(w.experts && w.router_w, MOE_ERR_ARG, "layer %d: experts/router_w is NULL", l);
  REQUIRE(c.n_shared == 0 || w.shared, MOE_ERR_ARG, "layer %d: shared is NULL", l);
  REQUIRE(aligned(w.experts, 256) && aligned(w.router_w, 256) && (!w.shared || aligned(w.shared, 256)) &&
              (!w.gamma || aligned(w.gamma, 16)) && (!w.shared_gate || aligned(w.shared_gate, 16)),
          MOE_ERR_ALIGN, "layer %d: weight pointers must be 256-byte aligned (gamma, shared_gate 16-byte)", l);
  p.experts = static_cast<const uint8_t*>(w.experts);
  p.shared = static_cast<const uint8_t*>(w.shared);
  p.router = w.router_w;
  p.gamma = w.gamma;
  p.sgate = c.n_shared > 0 ? w.shared_gate : nullptr;
  return MOE_OK;
}

moe_status run_decode(DecodeRequest& r, hipStream_t st) {
  const char* why = nullptr;
  hipError_t e = launch_decode(r, st, &why);
  if (why) return fail(MOE_ERR_UNSUPPORTED, "%s", why);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return MOE_OK;
}

// Validates every layer before anything is enqueued; the table then travels to
// the device in kernel arguments (see launch_decode), so the call never blocks.
moe_status validate_layers(const moe_config& c, int L, const moe_layer_weights* layers, LayerPtrs* out) {
  for (int l = 0; l < L; ++l) {
    const moe_status s = layer_ptrs(c, layers[l], l, out[l]);
    if (s != MOE_OK) return s;
  }
  return MOE_OK;
}

// Device address of this device's `scratch` array: hipGetSymbolAddress once per
// device, with that device current, then kept for the life of the process.
std::mutex g_scratch_mu;
uint8_t* g_scratch[64] = {};

moe_status scratch_of(hipStream_t st, uint8_t*& out) {
  int dev = -1;
  hipError_t e = hipStreamGetDevice(st, &dev);
  if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
  REQUIRE(dev >= 0 && dev < 64, MOE_ERR_UNSUPPORTED, "device %d: at most 64 devices", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e, "hipSetDevice");
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (back != hipSuccess) return hip_fail(back, "hipSetDevice");
    REQUIRE(p && aligned(p, 256), MOE_ERR_HIP, "scratch array at %p is not 256-byte aligned", p);
    g_scratch[dev] = static_cast<uint8_t*>(p);
  }
  out = g_scratch[dev];
  return MOE_OK;
}

// Checks shared by both resident-stack entry points (before any workspace check).
moe_status check_stack(const moe_config* cfg, int L, int T, const moe_layer_weights* layers, const float* x0,
                       const float* y) {
  moe_status s = check_config(cfg);
  if (s != MOE_OK) return s;
  REQUIRE(L >= 1 && T >= 0, MOE_ERR_ARG, "L=%d T=%d", L, T);
  REQUIRE(!(cfg->flags & (MOE_F_PREFILL_BF16 | MOE_F_SELECT_BY_BIAS)), MOE_ERR_ARG,
          "stack decode takes neither MOE_F_PREFILL_BF16 nor MOE_F_SELECT_BY_BIAS");
  if (T == 0) return MOE_OK;
  REQUIRE(layers && x0 && y, MOE_ERR_ARG, "NULL pointer");
  REQUIRE(aligned(x0, 16) && aligned(y, 16), MOE_ERR_ALIGN, "x0/y must be 16-byte aligned");
  return MOE_OK;
}

// Enqueues the resident stack on a validated layer table and a workspace of
// layout wl.
moe_status run_stack(const moe_config* cfg, int L, const moe_layer_weights* layers, const LayerPtrs* table,
                     int T, const float* x0, const uint8_t* boost_mask, float* y, int32_t* idx_trace,
                     float* w_trace, uint8_t* ws, const WsLayout& wl, hipStream_t st) {
  DecodeRequest r = {};
  r.mode = 0;
  r.cfg = *cfg;
  r.L = L;
  r.T = T;
  r.layers_host = table;
  r.x0 = x0;
  r.y = y;
  r.boost_mask = boost_mask;
  r.idx_out = idx_trace;
  r.w_out = w_trace;
  r.ws = ws;
  r.wl = wl;
  r.phased = (cfg->flags & MOE_F_PHASED) != 0;
  r.any_sgate = false;
  for (int l = 0; l < L; ++l) r.any_sgate = r.any_sgate || (cfg->n_shared > 0 && layers[l].shared_gate);
  return run_decode(r, st);
}

}  // namespace

extern "C" {

size_t moe_packed_expert_bytes(const moe_config* cfg) {
  if (check_config(cfg) != MOE_OK) return 0;
  return make_geo(cfg->hidden, cfg->inter, cfg->bits).expert_bytes;
}

size_t moe_workspace_bytes(const moe_config* cfg, int32_t n_tokens, int32_t n_layers) {
  if (check_config(cfg) != MOE_OK || n_tokens < 0 || n_layers < 0) return 0;
  size_t dec = ws_layout(*cfg, n_tokens, n_layers < 1 ? 1 : n_layers).total;
  size_t pre = prefill_ws_bytes(*cfg, n_tokens);
  return dec > pre ? dec : pre;
}

moe_status moe_pack_weights(const moe_config* cfg, int32_t n, const uint8_t* codes,
                            const uint16_t* scales, const uint16_t* biases, void* packed,
                            size_t packed_bytes, void* ws, size_t ws_bytes, void* stream) {
  moe_status s = check_config(cfg);
  if (s != MOE_OK) return s;
  REQUIRE(n >= 0, MOE_ERR_ARG, "n=%d", n);
  if (n == 0) return MOE_OK;
  REQUIRE(codes && scales && biases && packed, MOE_ERR_ARG, "NULL pointer");
  REQUIRE(aligned(codes, 16), MOE_ERR_ALIGN, "codes must be 16-byte aligned");
  REQUIRE(aligned(scales, 2) && aligned(biases, 2), MOE_ERR_ALIGN, "scales/biases misaligned");
  REQUIRE(aligned(packed, 256), MOE_ERR_ALIGN, "packed must be 256-byte aligned");
  s = check_ws(cfg, 0, 1, ws, ws_bytes);
  if (s != MOE_OK) return s;
  const Geo geo = make_geo(cfg->hidden, cfg->inter, cfg->bits);
  REQUIRE(packed_bytes >= geo.expert_bytes * (size_t)n, MOE_ERR_SHAPE,
          "packed_bytes %zu < %d x %zu", packed_bytes, n, geo.expert_bytes);
  const WsLayout wl = ws_layout(*cfg, 0, 1);
  unsigned* err = reinterpret_cast<unsigned*>(static_cast<uint8_t*>(ws) + wl.err);
  hipError_t e = launch_pack(geo, n, 3, codes, scales, biases, packed, err, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "pack launch");
  return MOE_OK;
}

moe_status moe_route(const moe_config* cfg, int32_t T, const float* x, const float* router_w,
                     const float* gamma, const float* sel_bias, const int32_t* boosted,
                     int32_t* idx_out, float* w_out, float* logits_out, void* ws,
                     size_t ws_bytes, void* stream) {
  moe_status s = check_config(cfg);
  if (s != MOE_OK) return s;
  REQUIRE(T >= 0, MOE_ERR_ARG, "T=%d", T);
  if (T == 0) return MOE_OK;
  REQUIRE(x && router_w && idx_out && w_out, MOE_ERR_ARG, "NULL pointer");
  REQUIRE(aligned(x, 16) && aligned(router_w, 256) && (!gamma || aligned(gamma, 16)),
          MOE_ERR_ALIGN, "x/gamma must be 16-byte and router_w 256-byte aligned");
  REQUIRE(!(cfg->flags & MOE_F_SELECT_BY_BIAS) || sel_bias, MOE_ERR_ARG,
          "MOE_F_SELECT_BY_BIAS needs sel_bias");
  s = check_ws(cfg, T, 1, ws, ws_bytes);
  if (s != MOE_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  const WsLayout wl = ws_layout(*cfg, T, 1);
  moe_layer_weights lw = {router_w, nullptr, router_w, gamma, nullptr};  // experts unused when routing
  moe_config c1 = *cfg;
  c1.n_shared = 0;
  DecodeRequest r = {};
  s = layer_ptrs(c1, lw, 0, r.layer0);
  if (s != MOE_OK) return s;
  r.inline_layer = true;
  r.mode = 1;  // MODE_ROUTE
  r.cfg = c1;
  r.L = 1;
  r.T = T;
  r.layers_host = nullptr;
  r.x0 = x;
  r.sel_bias = sel_bias;
  r.boosted = boosted;
  r.idx_out = idx_out;
  r.w_out = w_out;
  r.logits_out = logits_out;
  r.ws = w8;
  r.wl = wl;
  r.phased = (cfg->flags & MOE_F_PHASED) != 0;
  return run_decode(r, st);
}

moe_status moe_expert_forward(const moe_config* cfg, const void* packed_expert, int32_t T,
                              const float* x, float* y, void* ws, size_t ws_bytes, void* stream) {
  moe_status s = check_config(cfg);
  if (s != MOE_OK) return s;
  REQUIRE(T >= 0, MOE_ERR_ARG, "T=%d", T);
  if (T == 0) return MOE_OK;
  REQUIRE(packed_expert && x && y, MOE_ERR_ARG, "NULL pointer");
  REQUIRE(aligned(packed_expert, 256), MOE_ERR_ALIGN, "packed_expert must be 256-byte aligned");
  REQUIRE(aligned(x, 16) && aligned(y, 16), MOE_ERR_ALIGN, "x/y must be 16-byte aligned");
  s = check_ws(cfg, T, 1, ws, ws_bytes);
  if (s != MOE_OK) return s;
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  DecodeRequest r = {};
  r.mode = 2;  // MODE_EXPERT
  r.cfg = *cfg;
  r.cfg.n_shared = 0;
  r.L = 1;
  r.T = T;
  r.single_expert = static_cast<const uint8_t*>(packed_expert);
  r.x0 = x;
  r.y = y;
  r.ws = w8;
  r.wl = ws_layout(*cfg, T, 1);
  r.phased = (cfg->flags & MOE_F_PHASED) != 0;
  return run_decode(r, (hipStream_t)stream);
}

moe_status moe_layer_forward(const moe_config* cfg, const moe_layer_weights* layer, int32_t T,
                             const float* x, float* y, const float* sel_bias,
                             const int32_t* boosted, int32_t* idx_out, float* w_out, void* ws,
                             size_t ws_bytes, void* stream) {
  moe_status s = check_config(cfg);
  if (s != MOE_OK) return s;
  REQUIRE(T >= 0, MOE_ERR_ARG, "T=%d", T);
  if (T == 0) return MOE_OK;
  REQUIRE(layer && x && y, MOE_ERR_ARG, "NULL pointer");
  REQUIRE(aligned(x, 16) && aligned(y, 16), MOE_ERR_ALIGN, "x/y must be 16-byte aligned");
  REQUIRE(!(cfg->flags & MOE_F_SELECT_BY_BIAS) || sel_bias, MOE_ERR_ARG,
          "MOE_F_SELECT_BY_BIAS needs sel_bias");
  s = check_ws(cfg, T, 1, ws, ws_bytes);
  if (s != MOE_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  if (cfg->flags & MOE_F_PREFILL_BF16) {
    REQUIRE(layer->experts && layer->router_w, MOE_ERR_ARG, "experts/router_w is NULL");
    REQUIRE(cfg->n_shared == 0 || layer->shared, MOE_ERR_ARG, "shared is NULL");
    REQUIRE(aligned(layer->experts, 256) && aligned(layer->router_w, 256) &&
                (!layer->shared || aligned(layer->shared, 256)) &&
                (!layer->gamma || aligned(layer->gamma, 16)) &&
                (!layer->shared_gate || aligned(layer->shared_gate, 16)),
            MOE_ERR_ALIGN, "weight pointers must be 256-byte aligned (gamma, shared_gate 16-byte)");
    std::string msg;
    s = prefill_forward(*cfg, layer, T, x, y, sel_bias, boosted, idx_out, w_out, w8, ws_bytes, st,
                        &msg);
    if (s != MOE_OK) g_msg = msg;
    return s;
  }
  const WsLayout wl = ws_layout(*cfg, T, 1);
  DecodeRequest r = {};
  s = layer_ptrs(*cfg, *layer, 0, r.layer0);
  if (s != MOE_OK) return s;
  r.inline_layer = true;
  r.mode = 0;  // MODE_LAYER
  r.cfg = *cfg;
  r.L = 1;
  r.T = T;
  r.layers_host = nullptr;
  r.x0 = x;
  r.y = y;
  r.sel_bias = sel_bias;
  r.boosted = boosted;
  r.idx_out = idx_out;
  r.w_out = w_out;
  r.ws = w8;
  r.wl = wl;
  r.phased = (cfg->flags & MOE_F_PHASED) != 0;
  r.any_sgate = cfg->n_shared > 0 && layer->shared_gate != nullptr;
  return run_decode(r, st);
}

moe_status moe_stack_decode(const moe_config* cfg, int32_t L, const moe_layer_weights* layers,
                            int32_t T, const float* x0, const uint8_t* boost_mask, float* y,
                            int32_t* idx_trace, float* w_trace, void* ws, size_t ws_bytes,
                            void* stream) {
  moe_status s = check_stack(cfg, L, T, layers, x0, y);
  if (s != MOE_OK || T == 0) return s;
  s = check_ws(cfg, T, L, ws, ws_bytes);
  if (s != MOE_OK) return s;
  std::vector<LayerPtrs> table((size_t)L);
  s = validate_layers(*cfg, L, layers, table.data());
  if (s != MOE_OK) return s;
  return run_stack(cfg, L, layers, table.data(), T, x0, boost_mask, y, idx_trace, w_trace,
                   static_cast<uint8_t*>(ws), ws_layout(*cfg, T, L), (hipStream_t)stream);
}

moe_status moe_stack_decode_streamed(const moe_config* cfg, int32_t L, const moe_layer_weights* layers,
                                     int32_t T, const float* x0, const uint8_t* boost_mask, float* y,
                                     int32_t* idx_trace, float* w_trace, uint8_t* hit_trace, void* cache,
                                     size_t cache_bytes, int32_t cache_slots, void* ws, size_t ws_bytes,
                                     void* stream) {
  moe_status s = check_config(cfg);
  if (s != MOE_OK) return s;
  REQUIRE(L >= 1 && T >= 0, MOE_ERR_ARG, "L=%d T=%d", L, T);
  if (T == 0) return MOE_OK;
  REQUIRE(!(cfg->flags & (MOE_F_PREFILL_BF16 | MOE_F_SELECT_BY_BIAS | MOE_F_PHASED)), MOE_ERR_ARG,
          "streamed stack decode takes none of MOE_F_PREFILL_BF16, MOE_F_SELECT_BY_BIAS, MOE_F_PHASED");
  REQUIRE(layers && x0 && y && cache, MOE_ERR_ARG, "NULL pointer");
  REQUIRE(aligned(x0, 16) && aligned(y, 16), MOE_ERR_ALIGN, "x0/y must be 16-byte aligned");
  REQUIRE(aligned(cache, 256), MOE_ERR_ALIGN, "cache must be 256-byte aligned");
  REQUIRE(cache_slots >= cfg->top_k && cache_slots <= kMaxCacheSlots, MOE_ERR_ARG,
          "cache_slots=%d: must be top_k..%d", cache_slots, kMaxCacheSlots);
  const size_t eb = make_geo(cfg->hidden, cfg->inter, cfg->bits).expert_bytes;
  REQUIRE(cache_bytes >= (size_t)L * cache_slots * eb, MOE_ERR_ARG, "cache %zu bytes, need %zu",
          cache_bytes, (size_t)L * cache_slots * eb);
  s = check_ws(cfg, T, L, ws, ws_bytes);
  if (s != MOE_OK) return s;
  // every layer's routed experts must be pinned host memory the device can read:
  // the first and the last byte of the [E][expert_bytes] range are checked
  std::vector<moe_layer_weights> lw(layers, layers + L);
  for (int l = 0; l < L; ++l) {
    const uint8_t* ex = static_cast<const uint8_t*>(layers[l].experts);
    REQUIRE(ex, MOE_ERR_ARG, "layer %d: experts is NULL", l);
    const uint8_t* ends[2] = {ex, ex + (size_t)cfg->n_experts * eb - 1};
    void* dev[2] = {nullptr, nullptr};
    for (int i = 0; i < 2; ++i) {
      hipPointerAttribute_t at;
      hipError_t e = hipPointerGetAttributes(&at, ends[i]);
      if (e != hipSuccess || at.type != hipMemoryTypeHost || !at.devicePointer) {
        (void)hipGetLastError();
        return fail(MOE_ERR_ARG, "layer %d: experts must be pinned host memory (hipHostMalloc) "
                    "covering all %d experts", l, cfg->n_experts);
      }
      dev[i] = at.devicePointer;
    }
    REQUIRE(static_cast<uint8_t*>(dev[1]) - static_cast<uint8_t*>(dev[0]) ==
                (ptrdiff_t)((size_t)cfg->n_experts * eb - 1),
            MOE_ERR_ARG, "layer %d: experts must be one pinned host allocation", l);
    lw[l].experts = dev[0];
  }
  hipStream_t st = (hipStream_t)stream;
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  const WsLayout wl = ws_layout(*cfg, T, L);
  std::vector<LayerPtrs> table((size_t)L);
  s = validate_layers(*cfg, L, lw.data(), table.data());
  if (s != MOE_OK) return s;
  DecodeRequest r = {};
  r.mode = 0;
  r.cfg = *cfg;
  r.L = L;
  r.T = T;
  r.layers_host = table.data();
  r.x0 = x0;
  r.y = y;
  r.boost_mask = boost_mask;
  r.idx_out = idx_trace;
  r.w_out = w_trace;
  r.ws = w8;
  r.wl = wl;
  r.phased = false;
  r.any_sgate = false;
  for (int l = 0; l < L; ++l) r.any_sgate = r.any_sgate || (cfg->n_shared > 0 && layers[l].shared_gate);
  r.stream = true;
  r.cache = static_cast<uint8_t*>(cache);
  r.cslots = cache_slots;
  r.hit_out = hit_trace;
  return run_decode(r, st);
}

moe_status moe_stack_decode_noalloc(const moe_config* cfg, int32_t L, const moe_layer_weights* layers,
                                    int32_t T, const float* x0, const uint8_t* boost_mask, float* y,
                                    int32_t* idx_trace, float* w_trace, uint32_t* dev_err, void* stream) {
  moe_status s = check_stack(cfg, L, T, layers, x0, y);
  if (s != MOE_OK || T == 0) return s;
  REQUIRE(L <= kScratchMaxLayers, MOE_ERR_UNSUPPORTED, "L=%d: at most %d layers", L, kScratchMaxLayers);
  REQUIRE(!dev_err || aligned(dev_err, 4), MOE_ERR_ALIGN, "dev_err must be 4-byte aligned");
  const WsLayout wl = ws_layout(*cfg, T, L, false);
  REQUIRE(wl.total <= kScratchBytes, MOE_ERR_WORKSPACE,
          "this shape needs %zu bytes of scratch; the library's fixed array holds %zu", wl.total,
          kScratchBytes);
  LayerPtrs table[kScratchMaxLayers];
  s = validate_layers(*cfg, L, layers, table);
  if (s != MOE_OK) return s;
  const hipStream_t st = (hipStream_t)stream;
  uint8_t* ws = nullptr;
  s = scratch_of(st, ws);
  if (s != MOE_OK) return s;
  s = run_stack(cfg, L, layers, table, T, x0, boost_mask, y, idx_trace, w_trace, ws, wl, st);
  if (s != MOE_OK) return s;
  if (dev_err) {
    const hipError_t e = hipMemcpyAsync(dev_err, ws + wl.err, sizeof(uint32_t), hipMemcpyDeviceToDevice, st);
    if (e != hipSuccess) return hip_fail(e, "copying the device error word");
  }
  return MOE_OK;
}

size_t moe_qkv_packed_bytes(const moe_qkv_config* cfg) {
  if (check_qkv(cfg) != MOE_OK) return 0;
  return make_matrix_geo(cfg->hidden, cfg->q_rows + cfg->k_rows + cfg->v_rows, cfg->bits).expert_bytes;
}

moe_status moe_qkv_pack(const moe_qkv_config* cfg, const uint8_t* codes, const uint16_t* scales,
                        const uint16_t* biases, void* packed, size_t packed_bytes, void* ws,
                        size_t ws_bytes, void* stream) {
  moe_status s = check_qkv(cfg);
  if (s != MOE_OK) return s;
  REQUIRE(codes && scales && biases && packed && ws, MOE_ERR_ARG, "NULL pointer");
  REQUIRE(aligned(codes, 16) && aligned(packed, 256) && aligned(ws, 256), MOE_ERR_ALIGN,
          "codes must be 16-byte, packed and ws 256-byte aligned");
  REQUIRE(ws_bytes >= 1024, MOE_ERR_WORKSPACE, "workspace %zu bytes, need 1024", ws_bytes);
  const Geo geo = make_matrix_geo(cfg->hidden, cfg->q_rows + cfg->k_rows + cfg->v_rows, cfg->bits);
  REQUIRE(packed_bytes >= geo.expert_bytes, MOE_ERR_SHAPE, "packed %zu bytes, need %zu", packed_bytes,
          geo.expert_bytes);
  unsigned* err = static_cast<unsigned*>(ws);
  hipError_t e = launch_pack(geo, 1, 1, codes, scales, biases, packed, err, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "pack launch");
  return MOE_OK;
}

moe_status moe_qkv_forward(const moe_qkv_config* cfg, const void* packed, const float* gamma, int32_t T,
                           const float* x, float* q, float* k, float* v, void* stream) {
  moe_status s = check_qkv(cfg);
  if (s != MOE_OK) return s;
  REQUIRE(T >= 0, MOE_ERR_ARG, "T=%d", T);
  if (T == 0) return MOE_OK;
  REQUIRE(packed && x && q && k && v, MOE_ERR_ARG, "NULL pointer");
  REQUIRE(aligned(packed, 256) && aligned(x, 16) && (!gamma || aligned(gamma, 16)) && aligned(q, 4) &&
              aligned(k, 4) && aligned(v, 4),
          MOE_ERR_ALIGN, "packed must be 256-byte, x and gamma 16-byte aligned");
  hipError_t e = launch_qkv(*cfg, static_cast<const uint8_t*>(packed), gamma, T, x, q, k, v,
                            (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "qkv launch");
  return MOE_OK;
}

const char* moe_last_error(void) { return g_msg.c_str(); }

moe_status moe_device_status(void* ws, size_t ws_bytes, void* stream) {
  REQUIRE(ws && ws_bytes >= 768, MOE_ERR_ARG, "workspace is NULL or too small");
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "stream synchronize");
  unsigned v = 0;
  e = hipMemcpy(&v, ws, sizeof(v), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "reading the device error word");
  if (v == 0) return MOE_OK;
  const unsigned zero = 0;
  e = hipMemcpy(ws, &zero, sizeof(zero), hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(e, "clearing the device error word");
  switch (v) {
    case DEV_BAD_INDEX: return fail(MOE_ERR_DEVICE, "device: expert index out of range");
    case DEV_SYNC_TIMEOUT: return fail(MOE_ERR_DEVICE, "device: a wait for another workgroup's data timed out");
    case DEV_BAD_CODE: return fail(MOE_ERR_DEVICE, "device: pack input code >= 2^bits");
    default: return fail(MOE_ERR_DEVICE, "device error %u", v);
  }
}

}  // extern "C"
