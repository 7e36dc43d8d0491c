// Transposed copy of V for the forward kernels (see fwd_vt.hpp).
#include "fwd_vt.hpp"

#include "ffpa_common.hpp"

namespace ffpa {

// One workgroup moves a 64-key x 64-column block of one (b, hk) slice through
// LDS: 16-byte loads along rows of V, 16-byte stores along the d rows of the
// V^T blocks. Keys at or past Nkv are written as zeros.
__global__ __launch_bounds__(256) void fwd_vt_kernel(const uint16_t* __restrict__ v,
                                                     uint16_t* __restrict__ vt, int Nkv,
                                                     int nkv_pad, int D, int kb, int n_ktiles,
                                                     int n_dtiles) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64][72];  // 144-byte rows
  const int t = threadIdx.x;
  int blk = blockIdx.x;
  const int kt = blk % n_ktiles;
  blk /= n_ktiles;
  const int dt = blk % n_dtiles;
  const int bh = blk / n_dtiles;
  const int k0 = kt * 64, d0 = dt * 64;
  const uint16_t* src = v + (size_t)bh * Nkv * D;
  uint16_t* dst = vt + (size_t)bh * D * nkv_pad;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int i = t + 256 * u;  // key i / 8, columns 8 (i % 8) .. +7
    const int key = i >> 3, g = i & 7;
    u32x4 x = {0, 0, 0, 0};
    if (k0 + key < Nkv) x = *(const u32x4*)(src + (size_t)(k0 + key) * D + d0 + 8 * g);
    *(u32x4*)&tile[key][8 * g] = x;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int i = t + 256 * u;  // column i / 8, keys 8 (i % 8) .. +7
    const int d = i >> 3, kg = i & 7;
    u32x4 y;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      y[e] = (uint32_t)tile[vt_key(8 * kg + 2 * e)][d] | ((uint32_t)tile[vt_key(8 * kg + 2 * e + 1)][d] << 16);
    const int pos = k0 + 8 * kg;  // 8 positions, inside one block (kb % 8 == 0)
    *(u32x4*)(dst + (size_t)(pos / kb) * D * kb + (size_t)(d0 + d) * kb + pos % kb) = y;
  }
}

hipError_t launch_fwd_vt(const void* v, void* vt, int BH, int Nkv, int D, int kb, hipStream_t stream) {
  const int nkv_pad = fwd_nkv_pad(Nkv);
  if (kb <= 0 || kb % 32 != 0 || nkv_pad % kb != 0) return hipErrorInvalidValue;
  const int n_ktiles = nkv_pad / 64, n_dtiles = D / 64;
  const int64_t grid = (int64_t)BH * n_ktiles * n_dtiles;
  if (grid >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fwd_vt_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                     (const uint16_t*)v, (uint16_t*)vt, Nkv, nkv_pad, D, kb, n_ktiles, n_dtiles);
  return hipGetLastError();
}

}  // namespace ffpa
