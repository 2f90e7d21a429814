// qmoe_pack.hip -- canonical experts -> packed expert-major device layout.
//
// One thread writes one slot of one block: the codes of one 64-element group of one
// row (two 16-byte chunks for 4-bit, 16 + 8 bytes for 3-bit, one 16-byte chunk for
// 2-bit) and its (scale, bias) word.
// Consecutive threads write consecutive slots, so the stores are fully coalesced;
// each thread reads its 64 canonical codes as four 16-byte loads.
#include "qmoe_internal.h"

namespace qmoe {

__device__ inline unsigned check_code(unsigned q, unsigned maxq, unsigned* bad) {
  if (q > maxq) *bad = 1u;
  return q & maxq;
}

__global__ __launch_bounds__(256) void pack_kernel(Geo geo, int n, int mats, const uint8_t* __restrict__ codes,
                                                   const uint16_t* __restrict__ scales,
                                                   const uint16_t* __restrict__ biases,
                                                   uint8_t* __restrict__ packed, unsigned* err) {
  const int bpe = mats == 3 ? 2 * geo.nblk_gu + geo.nblk_d : geo.nblk_gu;  // blocks per unit
  const size_t total = (size_t)n * bpe * kWave;
  const size_t codes_per_mat_gu = (size_t)geo.I * geo.H;
  const size_t codes_per_expert = mats * codes_per_mat_gu;
  const size_t groups_per_mat_gu = codes_per_mat_gu / kGroup;
  const size_t groups_per_expert = mats * groups_per_mat_gu;
  const unsigned maxq = (1u << geo.bits) - 1u;
  unsigned bad = 0;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (size_t)gridDim.x * blockDim.x) {
    const int slot = (int)(i % kWave);
    const size_t bidx = i / kWave;
    const int e = (int)(bidx / bpe);
    int b = (int)(bidx % bpe);
    int mat, R, C, G, P;
    size_t mat_off;
    if (b < geo.nblk_gu) {
      mat = 0; mat_off = 0;
    } else if (b < 2 * geo.nblk_gu) {
      mat = 1; b -= geo.nblk_gu; mat_off = geo.off_up;
    } else {
      mat = 2; b -= 2 * geo.nblk_gu; mat_off = geo.off_down;
    }
    if (mat < 2) { R = geo.I; C = geo.H; G = geo.Gh; P = geo.Ph; }
    else { R = geo.H; C = geo.I; G = geo.Gi; P = geo.Pi; }
    const int p = slot / G, g = slot % G;
    const int row = b * P + p;
    uint8_t* blk = packed + (size_t)e * geo.expert_bytes + mat_off + (size_t)b * geo.blk;
    uint4 c0 = make_uint4(0, 0, 0, 0), c1 = make_uint4(0, 0, 0, 0);
    unsigned sb = 0;
    if (p < P && row < R) {
      const size_t cbase = (size_t)e * codes_per_expert + (size_t)mat * codes_per_mat_gu +
                           (size_t)row * C + (size_t)g * kGroup;
      const uint4* src4 = reinterpret_cast<const uint4*>(codes + cbase);
      uint4 q4[4] = {src4[0], src4[1], src4[2], src4[3]};
      const uint8_t* q = reinterpret_cast<const uint8_t*>(q4);
      unsigned w[8];
      if (geo.bits == 4) {
        for (int dw = 0; dw < 8; ++dw) {
          unsigned v = 0;
          for (int m = 0; m < 4; ++m) {
            const unsigned lo = check_code(q[8 * dw + m], maxq, &bad) ^ 8u;
            const unsigned hi = check_code(q[8 * dw + 4 + m], maxq, &bad) ^ 8u;
            v |= (lo << (8 * m)) | (hi << (8 * m + 4));
          }
          w[dw] = v;
        }
        c0 = make_uint4(w[0], w[1], w[2], w[3]);
        c1 = make_uint4(w[4], w[5], w[6], w[7]);
      } else if (geo.bits == 3) {
        for (int t = 0; t < 2; ++t) {
          for (int i = 0; i < 3; ++i) {
            unsigned v = 0;
            for (int nib = 0; nib < 8; ++nib) {
              const int d = (nib & 1) ? 4 + (nib >> 1) : (nib >> 1);
              const unsigned lo = check_code(q[32 * t + 8 * i + d], maxq, &bad);
              const unsigned top = check_code(q[32 * t + 24 + d], maxq, &bad);
              v |= (lo << (4 * nib)) | (((top >> i) & 1u) << (4 * nib + 3));
            }
            w[3 * t + i] = v;
          }
        }
        c0 = make_uint4(w[0], w[1], w[2], w[3]);
        c1 = make_uint4(w[4], w[5], 0, 0);
      } else {
        for (int j = 0; j < 4; ++j) {
          unsigned v = 0;
          for (int nib = 0; nib < 8; ++nib) {
            const int d = (nib & 1) ? 4 + (nib >> 1) : (nib >> 1);
            const unsigned a = check_code(q[16 * j + d], maxq, &bad);
            const unsigned c = check_code(q[16 * j + 8 + d], maxq, &bad);
            v |= (a << (4 * nib)) | (c << (4 * nib + 2));
          }
          w[j] = v;
        }
        c0 = make_uint4(w[0], w[1], w[2], w[3]);
      }
      const size_t gi = (size_t)e * groups_per_expert + (size_t)mat * groups_per_mat_gu +
                        (size_t)row * G + g;
      sb = (unsigned)scales[gi] | ((unsigned)biases[gi] << 16);
    }
    reinterpret_cast<uint4*>(blk)[slot] = c0;
    if (geo.bits == 4) reinterpret_cast<uint4*>(blk + kPlane1Offset)[slot] = c1;
    if (geo.bits == 3) reinterpret_cast<uint2*>(blk + kPlane1Offset)[slot] = make_uint2(c1.x, c1.y);
    reinterpret_cast<unsigned*>(blk + sb_offset(geo.bits))[slot] = sb;
  }
  if (bad) set_dev_err(err, DEV_BAD_CODE);
}

__global__ void zero_err(unsigned* err) {
  if (threadIdx.x == 0) *err = 0u;
}

hipError_t launch_pack(const Geo& geo, int n, int mats, const uint8_t* codes, const uint16_t* scales,
                       const uint16_t* biases, void* packed, unsigned* err, hipStream_t stream) {
  const size_t total = (size_t)n * (mats == 3 ? 2 * geo.nblk_gu + geo.nblk_d : geo.nblk_gu) * kWave;
  size_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_err, dim3(1), dim3(64), 0, stream, err);
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, geo, n, mats, codes,
                     scales, biases, static_cast<uint8_t*>(packed), err);
  return hipGetLastError();
}

}  // namespace qmoe
