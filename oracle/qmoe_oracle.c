/*
 * qmoe_oracle.c -- plain, slow, single-threaded CPU reference for the sparse
 * Mixture-of-Experts FFN step with group-affine quantized experts.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do. It shares no code with the HIP path.
 *
 * What it computes, and where the pages define it (cited by page title and
 * section; the pages are the flash-moe write-ups listed in the design notes):
 *
 *  - group-affine dequantisation w = q*scale + bias with one (scale, bias) per
 *    64-element group of the input dimension, and the dequant mat-vec that
 *    multiplies by x: "Flash-MoE - Chạy mô hình 397 tỷ tham số trên laptop"
 *    (vi.news.hada.io), section "Kernel dequant tối ưu FMA" (the
 *    (nibble*scale+bias)*x product) and section "Metal Compute Shaders" (4-bit
 *    and 2-bit dequant mat-vec).  The oracle uses the naive form: it never
 *    applies the FMA or group-factored rewrites.  Codes are plain integers, so
 *    the same function serves 2-, 3- and 4-bit experts; 3-bit experts stand in
 *    for the 3-bit ones of "Autoresearch impulsa a Qwen3.5-397B a 20.34 tok/s en
 *    M5 Max mediante transmision SSD" (openclawradar.com), section
 *    "Optimizaciones Efectivas".
 *  - RMS normalisation, SwiGLU, and the MoE combine with residual: same page,
 *    section "Metal Compute Shaders" and section "Deferred GPU Expert Compute"
 *    (combine + norm + residual feed the next layer).
 *  - routing to K of E experts per token plus an always-on shared expert: same
 *    page, section "Kiến trúc mô hình" (512 experts, K=4, hidden 4096).
 *
 * Precision: every dot product is accumulated in float64 in index order.
 * deq(q, s, b) = fp32(fp32(q) * fp32(s) + fp32(b)); q*s is exact in fp32
 * (4-bit times 8-bit significands), so the one rounding is the addition.
 *
 * Built with -O2 -ffp-contract=off so that no operation is fused or reordered.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>

static float bf16_to_f32(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Round a double to bfloat16 precision (8 significant bits, ties to even) and
 * return it as a double. bf16 shares float32's exponent range; the values here
 * are far from overflow and underflow. */
double orc_round_bf16(double d) {
  if (d == 0.0 || !isfinite(d)) return d;
  int e;
  double m = frexp(d, &e);                 /* d = m * 2^e, 0.5 <= |m| < 1 */
  double scaled = ldexp(m, 8);             /* exact: 8 significant bits above the point */
  double r = nearbyint(scaled);            /* default rounding mode: nearest, ties to even */
  return ldexp(r, e - 8);
}

/* deq(q, s, b) = fp32(q*s + b): the page's nibble*scale+bias, rounded once. */
static float deq(uint8_t q, uint16_t s_bits, uint16_t b_bits) {
  volatile float prod = (float)q * bf16_to_f32(s_bits);  /* exact */
  volatile float w = prod + bf16_to_f32(b_bits);        /* one rounding */
  return w;
}

/* RMSNorm: r = sqrt(sum(x^2)/H + eps); out = x / r * gamma (gamma NULL = 1). */
void orc_rmsnorm(int H, const double* x, const float* gamma, double eps, double* out) {
  double ss = 0.0;
  for (int i = 0; i < H; ++i) ss += x[i] * x[i];
  double r = sqrt(ss / (double)H + eps);
  for (int i = 0; i < H; ++i) out[i] = x[i] / r * (gamma ? (double)gamma[i] : 1.0);
}

/* Router logits: logit[e] = sum_i W[e][i] * xn[i]. */
void orc_router(int E, int H, const float* W, const double* xn, double* logits) {
  for (int e = 0; e < E; ++e) {
    double acc = 0.0;
    const float* row = W + (size_t)e * H;
    for (int i = 0; i < H; ++i) acc += (double)row[i] * xn[i];
    logits[e] = acc;
  }
}

/* Top-K selection and renormalised softmax weights.
 *   score[e] = logits[e] + (sel ? sel[e] : 0), or sel[e] alone if by_sel.
 *   tier[e]  = 1 if e is listed in boosted[0..nb-1], else 0.
 *   Order: tier descending, then score descending, then index ascending.
 *   p = softmax(logits) over all E; w_k = p[idx_k] / sum_j p[idx_j].
 * gap_out (nullable) receives score(K-th) - score((K+1)-th) when both are in the
 * same tier, else +inf: the margin that decides the selected set.
 * Returns 0, or -1 on bad arguments. */
int orc_select(int E, int K, const double* logits, const double* sel, int by_sel,
               const int* boosted, int nb, int* idx_out, double* w_out, double* gap_out) {
  if (K < 1 || K > E) return -1;
  double* score = (double*)malloc(sizeof(double) * E);
  int* tier = (int*)calloc(E, sizeof(int));
  char* taken = (char*)calloc(E, 1);
  for (int e = 0; e < E; ++e) score[e] = by_sel ? sel[e] : logits[e] + (sel ? sel[e] : 0.0);
  for (int j = 0; j < nb; ++j)
    if (boosted[j] >= 0 && boosted[j] < E) tier[boosted[j]] = 1;
  int best_e = -1;
  for (int k = 0; k <= K && k < E; ++k) {         /* one extra round finds the runner-up */
    best_e = -1;
    for (int e = 0; e < E; ++e) {
      if (taken[e]) continue;
      if (best_e < 0 || tier[e] > tier[best_e] ||
          (tier[e] == tier[best_e] && score[e] > score[best_e]))
        best_e = e;                                  /* strict '>' keeps the lower index on ties */
    }
    if (k < K) {
      idx_out[k] = best_e;
      taken[best_e] = 1;
    }
  }
  if (gap_out) {
    int last = idx_out[K - 1];
    if (K < E && best_e >= 0 && tier[best_e] == tier[last]) *gap_out = score[last] - score[best_e];
    else *gap_out = INFINITY;
  }
  double m = logits[0];
  for (int e = 1; e < E; ++e) if (logits[e] > m) m = logits[e];
  double z = 0.0;
  for (int e = 0; e < E; ++e) z += exp(logits[e] - m);
  double ps = 0.0;
  for (int k = 0; k < K; ++k) ps += exp(logits[idx_out[k]] - m) / z;
  for (int k = 0; k < K; ++k) w_out[k] = (exp(logits[idx_out[k]] - m) / z) / ps;
  free(score); free(tier); free(taken);
  return 0;
}

/* Dequant mat-vec on canonical inputs: codes [R][C] one per byte, scale/bias
 * [R][C/64] bf16 bits. y[r] = sum_c w[r][c] * x[c] with w = deq(q, s, b), or
 * w = bf16(deq(q, s, b)) when round_w_bf16 is set (the prefill contraction
 * dequantises to bf16). */
void orc_matvec(int R, int C, const uint8_t* q, const uint16_t* s, const uint16_t* b,
                const double* x, int round_w_bf16, double* y) {
  int G = C / 64;
  for (int r = 0; r < R; ++r) {
    double acc = 0.0;
    for (int c = 0; c < C; ++c) {
      size_t gi = (size_t)r * G + c / 64;
      double w = (double)deq(q[(size_t)r * C + c], s[gi], b[gi]);
      if (round_w_bf16) w = orc_round_bf16(w);
      acc += w * x[c];
    }
    y[r] = acc;
  }
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* One expert: g = Wg x, u = Wu x, h = silu(g) * u, o = Wd h.
 * gate/up: [I][H]; down: [H][I]. bf16_points: prefill rounding points (weights
 * rounded to bf16, h rounded to bf16; x is passed already rounded by the caller). */
void orc_expert(int H, int I,
                const uint8_t* qg, const uint16_t* sg, const uint16_t* bg,
                const uint8_t* qu, const uint16_t* su, const uint16_t* bu,
                const uint8_t* qd, const uint16_t* sd, const uint16_t* bd,
                const double* x, int bf16_points, double* o, double* h_out) {
  double* g = (double*)malloc(sizeof(double) * I);
  double* u = (double*)malloc(sizeof(double) * I);
  double* h = (double*)malloc(sizeof(double) * I);
  orc_matvec(I, H, qg, sg, bg, x, bf16_points, g);
  orc_matvec(I, H, qu, su, bu, x, bf16_points, u);
  for (int j = 0; j < I; ++j) {
    h[j] = silu(g[j]) * u[j];
    if (bf16_points) h[j] = orc_round_bf16(h[j]);
  }
  orc_matvec(H, I, qd, sd, bd, h, bf16_points, o);
  if (h_out) memcpy(h_out, h, sizeof(double) * I);
  free(g); free(u); free(h);
}

/* Combine: y = (residual ? x : 0) + sum_k w[k] * o[k] + sum_s c[s] * o_shared[s],
 * with c[s] the shared-expert gate factor (c == NULL: every factor is 1).
 * o: [n_routed][H] then [n_shared][H], contiguous. */
void orc_combine(int H, int n_routed, int n_shared, const double* x, int residual,
                 const double* w, const double* o, const double* c, double* y) {
  for (int i = 0; i < H; ++i) {
    double acc = residual ? x[i] : 0.0;
    for (int k = 0; k < n_routed; ++k) acc += w[k] * o[(size_t)k * H + i];
    for (int s = 0; s < n_shared; ++s) acc += (c ? c[s] : 1.0) * o[(size_t)(n_routed + s) * H + i];
    y[i] = acc;
  }
}
