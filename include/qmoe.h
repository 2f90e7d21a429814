/*
 * qmoe.h -- C ABI of libqmoe: the sparse Mixture-of-Experts FFN step with
 * group-affine quantized experts, for AMD Instinct MI355X (gfx950).
 *
 * The operation is the one the flash-moe write-up describes for one decode
 * token and one layer ("Flash-MoE - Chạy mô hình 397 tỷ tham số trên laptop",
 * vi.news.hada.io): a router picks K of E experts per token, an always-on shared
 * expert runs beside them, each expert is a SwiGLU FFN whose weights are 4-bit
 * (or 3- or 2-bit) codes with one (scale, bias) pair per 64-element group, and the
 * outputs are combined with the routing weights and added to the residual
 * (sections "Kiến trúc mô hình", "Kernel dequant tối ưu FMA", "Metal Compute
 * Shaders", "Deferred GPU Expert Compute").
 *
 * Conventions for every entry point:
 *  - Pointers marked "dev" are device pointers; "host" pointers are host memory.
 *    The caller owns every buffer. The library never allocates or frees device
 *    memory; scratch space is the caller's workspace `ws`, sized by
 *    moe_workspace_bytes(), except for moe_stack_decode_noalloc, which uses a
 *    fixed 4 MiB array of the library's code object on each device. Workspace
 *    contents need no initialisation.
 *  - `stream` is a hipStream_t (NULL = the default stream). Every call only
 *    enqueues work on that stream and returns; nothing blocks except
 *    moe_device_status().
 *  - Arguments are validated before anything is enqueued. On failure the call
 *    returns a negative moe_status, enqueues nothing, and moe_last_error()
 *    returns a message (per host thread). A failed HIP launch returns
 *    MOE_ERR_HIP with the HIP error text.
 *  - Two calls may run concurrently only on different streams with disjoint
 *    workspaces and outputs. The decode entry points run one persistent grid of
 *    at most one workgroup per compute unit; the library orders these grids one
 *    after another on each device, whatever the streams, so overlapping calls
 *    never share the compute units. A grid that still cannot get its units (other
 *    work holding them for longer than the 2 s bound of each wait) ends with
 *    MOE_ERR_DEVICE from moe_device_status, never a hang.
 *  - State: besides its loaded code objects the library keeps, per device and
 *    created on first use, the compute-unit count, which kernels have had their
 *    LDS limit raised, one HIP event that orders the persistent grids, and the
 *    address of the scratch array of moe_stack_decode_noalloc. The event lives
 *    until the process ends.
 *  - Supported shapes: hidden and inter are 64 * 2^k (64 .. 4096); group 64;
 *    bits 4, 3 or 2; 1 <= top_k <= 16, top_k <= n_experts <= 1024; n_shared 0..2.
 */
#ifndef QMOE_H
#define QMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_ARG = -1,         /* null pointer, negative count, bad flag */
  MOE_ERR_SHAPE = -2,       /* inconsistent sizes */
  MOE_ERR_ALIGN = -3,       /* a device pointer is not 256-byte aligned */
  MOE_ERR_UNSUPPORTED = -4, /* valid but not implemented (bits, group, limits) */
  MOE_ERR_WORKSPACE = -5,   /* ws_bytes below moe_workspace_bytes() */
  MOE_ERR_HIP = -6,         /* a HIP runtime call failed */
  MOE_ERR_DEVICE = -7       /* a kernel reported an error (bad index, sync time-out) */
} moe_status;

/* flags */
#define MOE_F_RMSNORM 1        /* normalise x before routing and experts (eps, gamma) */
#define MOE_F_RESIDUAL 2       /* add the (pre-norm) input x to the output */
#define MOE_F_SELECT_BY_BIAS 4 /* selection score = sel_bias alone (else logit + sel_bias) */
#define MOE_F_PREFILL_BF16 8   /* moe_layer_forward: bf16 expert-grouped GEMM path */
#define MOE_F_PHASED 16        /* decode: one kernel launch per phase and layer instead of the
                                  persistent grid (kernel boundaries order the phases) */

typedef struct {
  int32_t hidden;    /* H: model width (gate/up input, down output) */
  int32_t inter;     /* I: expert intermediate width */
  int32_t n_experts; /* E: routed experts per layer */
  int32_t top_k;     /* K: routed experts per token */
  int32_t n_shared;  /* S: always-on shared experts, added with weight 1 */
  int32_t bits;      /* code width: 4, 3 or 2 (3: a group-affine stand-in for the
                        3-bit experts of "Autoresearch impulsa a Qwen3.5-397B a 20.34
                        tok/s en M5 Max mediante transmision SSD", openclawradar.com,
                        section "Optimizaciones Efectivas") */
  int32_t group;     /* quantization group along the input dimension: 64 */
  int32_t flags;     /* MOE_F_* */
  float eps;         /* RMSNorm epsilon (inside the square root) */
} moe_config;

/* The fused Q/K/V projection: three group-affine quantized matrices that read one
 * input. "Autoresearch impulsa a Qwen3.5-397B a 20.34 tok/s en M5 Max mediante
 * transmision SSD" (openclawradar.com), section "Optimizaciones Efectivas", fuses
 * the Q/K/V projections so that the input vector is read once instead of three
 * times; the mat-vec is the dequant mat-vec of "Flash-MoE" (section "Metal
 * Compute Shaders"). The pages give no attention widths; they are arguments. */
typedef struct {
  int32_t hidden;  /* H: input width, 64 * 2^k, 64..4096 */
  int32_t q_rows;  /* Rq, Rk, Rv: output widths, each >= 1, Rq + Rk + Rv <= 65536 */
  int32_t k_rows;
  int32_t v_rows;
  int32_t bits;    /* code width: 4, 3 or 2 */
  int32_t group;   /* 64 */
  int32_t flags;   /* 0 or MOE_F_RMSNORM */
  float eps;       /* RMSNorm epsilon (inside the square root) */
} moe_qkv_config;

/* One layer's weights, all device pointers, 256-byte aligned. */
typedef struct {
  const void* experts;   /* n_experts packed experts, moe_packed_expert_bytes() apart */
  const void* shared;    /* n_shared packed experts (NULL if n_shared == 0) */
  const float* router_w; /* [n_experts][hidden] float32, row-major */
  const float* gamma;    /* [hidden] RMSNorm weight, or NULL for all ones */
  /* [n_shared][hidden] float32 shared-expert gate, or NULL. When given, shared
   * expert s enters the combine scaled by sigmoid(shared_gate[s] . x_n) instead of
   * with weight 1 (x_n: the normalised layer input the router sees). The page
   * ("Flash-MoE", section "Metal Compute Shaders") lists a gate in its combine
   * kernel without defining it; this is the shared-expert gate of that model
   * family. 16-byte aligned. Decode (any T) and prefill both honour it. */
  const float* shared_gate;
} moe_layer_weights;

/* Bytes of one packed expert (gate, up, down). 0 if the config is invalid.
 * With H=4096, I=1024, 4-bit codes and bf16 (scale, bias) per 64-group this is
 * 7,077,888 B = 6.75 MiB, the per-expert size the flash-moe page gives in its
 * "SSD Expert Streaming" section; 3-bit codes give 5,505,024 B (22% less) and
 * 2-bit codes 3,932,160 B. */
size_t moe_packed_expert_bytes(const moe_config* cfg);

/* Workspace bytes that suffice for any call below with at most n_tokens tokens
 * and n_layers layers on this config. 0 if the config is invalid. */
size_t moe_workspace_bytes(const moe_config* cfg, int32_t n_tokens, int32_t n_layers);

/* Pack canonical experts into the device layout (offline; not on the timed path).
 *   codes  dev [n][gate I*H | up I*H | down H*I] uint8, one code per byte, each
 *          matrix row-major [out][in]; values must be < 2^bits.
 *   scales dev [n][gate I*H/64 | up I*H/64 | down H*I/64] bf16 bit patterns,
 *   biases dev same layout as scales. Group j of a row covers inputs [64j, 64j+64).
 *   packed dev [n][moe_packed_expert_bytes(cfg)], 256-B aligned; packed_bytes is
 *          its size. Codes out of range set the device error (MOE_ERR_DEVICE from
 *          moe_device_status) and pack as code & (2^bits-1).
 * The dequantised weight is w = q * scale + bias, the page's nibble*scale+bias
 * ("Kernel dequant tối ưu FMA" section). The layout is expert-major: each expert
 * is one contiguous unit (cf. the expert-major sidecar of "LOOM",
 * alessandroviola.dev, "Cosa hanno stabilito gli esperimenti"). */
moe_status moe_pack_weights(const moe_config* cfg, int32_t n, const uint8_t* codes,
                            const uint16_t* scales, const uint16_t* biases, void* packed,
                            size_t packed_bytes, void* ws, size_t ws_bytes, void* stream);

/* Routing for T tokens: the router of "Flash-MoE - Chạy mô hình 397 tỷ tham số
 * trên laptop" (vi.news.hada.io), section "Kiến trúc mô hình" (K of 512 experts
 * per token, K = 4 there): logits = W_r x_n, the K experts of highest score, and
 * their weights renormalised over the selected K.
 *   x        dev [T][H] float32 input (normalised here when MOE_F_RMSNORM is set)
 *   router_w dev [E][H] float32;  gamma dev [H] or NULL
 *   sel_bias dev [T][E] float32 or NULL: added to the logit for selection only
 *            (or the whole selection score with MOE_F_SELECT_BY_BIAS)
 *   boosted  dev [T][K] int32 or NULL: experts ranked ahead of all others
 *            (a tier above the score), -1 = unused slot
 *   idx_out  dev [T][K] int32: selected experts, by descending (tier, score),
 *            ties to the lower index
 *   w_out    dev [T][K] float32: softmax of the router logits renormalised over
 *            the selected K (equal to a softmax over the K selected logits)
 *   logits_out dev [T][E] float32 or NULL. */
moe_status moe_route(const moe_config* cfg, int32_t T, const float* x, const float* router_w,
                     const float* gamma, const float* sel_bias, const int32_t* boosted,
                     int32_t* idx_out, float* w_out, float* logits_out, void* ws,
                     size_t ws_bytes, void* stream);

/* One expert on T tokens: y[t] = Wd (silu(Wg x[t]) * (Wu x[t])) in float32
 * (no norm, no routing weight, no residual): the dequant mat-vecs and SwiGLU of the
 * Flash-MoE page, sections "Metal Compute Shaders" and "Kernel dequant tối ưu FMA"
 * (w = q * scale + bias per 64-element group).
 *   packed_expert dev, one packed expert;  x dev [T][H];  y dev [T][H]. */
moe_status moe_expert_forward(const moe_config* cfg, const void* packed_expert, int32_t T,
                              const float* x, float* y, void* ws, size_t ws_bytes,
                              void* stream);

/* One MoE layer on T tokens, the per-layer step of the Flash-MoE page (section
 * "Deferred GPU Expert Compute": routed experts, shared expert, weighted combine,
 * residual); the batched path is the cold prefill of "LOOM" (alessandroviola.dev,
 * 1155 tokens) as an expert-grouped GEMM:
 *   y = [x if MOE_F_RESIDUAL] + sum_k w_k * expert_{idx_k}(x_n) + sum_s shared_s(x_n),
 *   x_n = RMSNorm(x) if MOE_F_RMSNORM else x.
 * Decode path (default): float32 activations, tokens processed one after another.
 * MOE_F_PREFILL_BF16: all T tokens at once as an expert-grouped bf16 GEMM with
 *   float32 accumulation; rounding points x_b = bf16(x), A = bf16(x_n) (router from
 *   the unrounded x_n), W = bf16(q*s+b), h = bf16(silu(g)*u); y = x_b + ....
 *   W is q*s+b rounded once as defined for scales |s| < 2^104 (the path multiplies by
 *   s*2^24 inside a fused multiply-add; larger scales are outside its range).
 *   x dev [T][H] float32; y dev [T][H] float32; sel_bias, boosted as in moe_route;
 *   idx_out, w_out dev [T][K] or NULL. */
moe_status moe_layer_forward(const moe_config* cfg, const moe_layer_weights* layer, int32_t T,
                             const float* x, float* y, const float* sel_bias,
                             const int32_t* boosted, int32_t* idx_out, float* w_out, void* ws,
                             size_t ws_bytes, void* stream);

/* L-layer decode stack for T tokens, strictly in order, entirely on the device
 * (one launch unless MOE_F_PHASED): the 60-layer decode of the Flash-MoE page
 * (section "Kiến trúc mô hình"). Between MoE blocks the rest of the model is
 * the identity, so token t enters layer 0 with x0[t] and layer l+1 receives
 * layer l's output. Temporal routing correlation ("Autoresearch impulsa a
 * Qwen3.5-397B a 20.34 tok/s en M5 Max mediante transmision SSD",
 * openclawradar.com, section "Optimizaciones Efectivas": 27% of a token's experts
 * repeat the previous token's): at token t > 0 and layer l, slot j of token t-1's
 * selected set at layer l (sorted by expert index) is ranked in the tier above
 * all others when boost_mask[t][l][j] != 0.
 *   layers     host [L] layer weights, all validated before anything is enqueued;
 *              the table reaches the device in kernel arguments, so the array
 *              may be reused as soon as the call returns
 *   x0         dev [T][H];  y dev [T][H] (output of the last layer)
 *   boost_mask dev [T][L][K] uint8 or NULL
 *   idx_trace  dev [T][L][K] int32 or NULL (selected experts, key order)
 *   w_trace    dev [T][L][K] float32 or NULL. */
moe_status moe_stack_decode(const moe_config* cfg, int32_t L, const moe_layer_weights* layers,
                            int32_t T, const float* x0, const uint8_t* boost_mask, float* y,
                            int32_t* idx_trace, float* w_trace, void* ws, size_t ws_bytes,
                            void* stream);

/* The decode stack of moe_stack_decode with the routed experts streamed from host
 * memory: the host-memory tier for expert sets larger than HBM. The pages stream
 * experts from SSD through the page cache, read each expert as one unit, and
 * find that 27% of a token's routed experts repeat from the token before
 * ("Flash-MoE - Chạy mô hình 397 tỷ tham số trên laptop", vi.news.hada.io,
 * section "SSD Expert Streaming"; "Autoresearch impulsa a Qwen3.5-397B a 20.34
 * tok/s en M5 Max mediante transmision SSD", openclawradar.com, section
 * "Optimizaciones Efectivas"). Here the device reads the experts from pinned host
 * memory over PCIe and keeps recently used ones in an HBM cache, so a repeat costs
 * HBM bandwidth instead of PCIe bandwidth. Results are those of moe_stack_decode
 * on the same inputs; only where the bytes come from differs.
 *   layers      host [L]: experts = PINNED HOST memory (hipHostMalloc or an
 *               equivalent allocation the device can read), one allocation holding
 *               all E packed experts, 256-B aligned; shared, router_w, gamma,
 *               shared_gate are device memory as in moe_stack_decode.
 *   cache       dev [L][cache_slots][moe_packed_expert_bytes] bytes, 256-B aligned,
 *               no initialisation needed; cache_bytes its size.
 *   cache_slots experts cached per layer, top_k..64. Policy per layer: a selected
 *               expert found in the cache is read from it (a hit); each other one,
 *               taken in increasing expert index, is read from host memory and
 *               copied into the least recently used slot not used by the current
 *               token (empty slots first, lowest slot on ties). The cache starts
 *               empty at every call.
 *   hit_trace   dev [T][L][K] uint8 or NULL: 1 where idx_trace's expert was a hit.
 * Other arguments as in moe_stack_decode. MOE_F_PHASED is not accepted. Pointers
 * that are not pinned host memory are rejected with MOE_ERR_ARG before anything
 * is enqueued. */
moe_status moe_stack_decode_streamed(const moe_config* cfg, int32_t L, const moe_layer_weights* layers,
                                     int32_t T, const float* x0, const uint8_t* boost_mask, float* y,
                                     int32_t* idx_trace, float* w_trace, uint8_t* hit_trace, void* cache,
                                     size_t cache_bytes, int32_t cache_slots, void* ws, size_t ws_bytes,
                                     void* stream);

/* moe_stack_decode without a caller workspace, for callers that cannot allocate
 * device memory (code under stream capture, tight serving loops, harnesses that
 * forbid allocation). Its scratch space is a fixed 4 MiB array inside the
 * library, one per device, obtained once per device with hipGetSymbolAddress on
 * the first call there and held until the process ends. Apart from the library's
 * one-time per-device set-up (that address, the compute-unit count, the kernels'
 * LDS limits and the ordering event, which any decode entry point creates on its
 * first use of a device), a call allocates nothing, host or device. Same kernels,
 * same results as moe_stack_decode on the same inputs.
 *   limits     L <= 128, and the shape's workspace without the streamed tier's
 *              tables must fit 4 MiB (hidden 4096, inter 1024, any K and E of
 *              the supported range: about 3 MiB); otherwise MOE_ERR_UNSUPPORTED
 *              or MOE_ERR_WORKSPACE, before anything is enqueued.
 *   dev_err    dev uint32 or NULL: after the stack, receives this call's device
 *              error word (0 none, 1 expert index out of range, 2 a wait timed
 *              out), copied on `stream`; moe_device_status cannot reach the array.
 *              Not written when T = 0 (nothing is enqueued).
 * Every call on a device shares that device's array and leaves its contents
 * behind; each call clears what must start at zero itself. Two calls on one
 * device that may overlap (different streams without ordering between them)
 * race on the array: give them one stream. Other arguments as in
 * moe_stack_decode. */
moe_status moe_stack_decode_noalloc(const moe_config* cfg, int32_t L, const moe_layer_weights* layers,
                                    int32_t T, const float* x0, const uint8_t* boost_mask, float* y,
                                    int32_t* idx_trace, float* w_trace, uint32_t* dev_err, void* stream);

/* Bytes of the packed fused Q/K/V matrix (Rq + Rk + Rv rows of H columns, the
 * block layout of an expert's gate matrix). 0 if the config is invalid. */
size_t moe_qkv_packed_bytes(const moe_qkv_config* cfg);

/* Pack the fused matrix: codes dev [Rq + Rk + Rv][H] uint8 (the rows of Wq, then
 * Wk, then Wv; values < 2^bits), scales and biases dev [Rq + Rk + Rv][H/64] bf16
 * bit patterns; packed dev, moe_qkv_packed_bytes bytes, 256-B aligned. ws: any
 * workspace of at least 1024 bytes (its first word is the device error word that
 * moe_device_status reads: codes out of range). */
moe_status moe_qkv_pack(const moe_qkv_config* cfg, const uint8_t* codes, const uint16_t* scales,
                        const uint16_t* biases, void* packed, size_t packed_bytes, void* ws,
                        size_t ws_bytes, void* stream);

/* q[t] = Wq x_n[t], k[t] = Wk x_n[t], v[t] = Wv x_n[t] for T tokens, float32, with
 * x_n = RMSNorm(x) * gamma under MOE_F_RMSNORM, else x * gamma (gamma NULL: 1).
 * Every row's dot product uses one encoding of its token's input.
 *   packed dev (moe_qkv_pack), 256-B aligned;  gamma dev [H] float32 or NULL, 16-B
 *   aligned;  x dev [T][H] float32, 16-B aligned;  q dev [T][Rq], k dev [T][Rk],
 *   v dev [T][Rv] float32. No workspace: the kernel needs none. */
moe_status moe_qkv_forward(const moe_qkv_config* cfg, const void* packed, const float* gamma, int32_t T,
                           const float* x, float* q, float* k, float* v, void* stream);

/* Message for the last non-OK status returned on this host thread. */
const char* moe_last_error(void);

/* Synchronises `stream`, then reads and clears the device error word in `ws`.
 * Every entry point clears that word when it starts, so this reports the most
 * recent call that used `ws`: MOE_OK, or MOE_ERR_DEVICE with a message naming
 * the cause. */
moe_status moe_device_status(void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* QMOE_H */
