// Small kernels around the projection kernels for gfx950: the exact fp32
// copy of the bias the projection reads, and the two helpers of the backward
// (zero padding of dZ^T's columns, the bias gradient as row sums of dZ^T).
// Each is a plain HBM-bound pass.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bilogp_internal.h"

namespace bilogp {
namespace {

// Zero columns [N, ldz) of every row of dZ^T (the padding the GEMMs read).
__global__ __launch_bounds__(256) void zero_pad_cols_kernel(uint16_t* __restrict__ dzt,
                                                            int64_t rows, int64_t N, int64_t ldz) {
  const int64_t pad = ldz - N;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * pad) return;
  const int64_t r = i / pad;
  dzt[r * ldz + N + (i - r * pad)] = 0;
}

// out[r] = sum over n = 0 .. N-1 of dZ^T[r][n]: one wave per row; lane k adds
// n = k, k + 64, ... in ascending order, then a fixed pairwise tree.
__global__ __launch_bounds__(256) void row_sums_kernel(const uint16_t* __restrict__ dzt,
                                                       int64_t rows, int64_t N, int64_t ldz,
                                                       float* __restrict__ out) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;                    // uniform across the wave
  const uint16_t* row = dzt + r * ldz;
  float s = 0.f;
  for (int64_t n = lane; n < N; n += 64) s += __uint_as_float((uint32_t)row[n] << 16);
#pragma unroll
  for (int d = 1; d <= 32; d <<= 1) s += __shfl_xor(s, d);
  if (lane == 0) out[r] = s;
}

// Exact fp32 copy of the bias (bf16 widens exactly), zero-padded to whole
// vocabulary tiles so the projection kernel reads it in full 16-byte chunks.
__global__ __launch_bounds__(256) void bias_to_f32_kernel(const void* __restrict__ bias,
                                                          int32_t kind, int32_t V,
                                                          int32_t padded, float* __restrict__ out) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= padded) return;
  float v = 0.f;
  if (c < V) {
    v = (kind == kBiasF32) ? ((const float*)bias)[c]
                           : __uint_as_float((uint32_t)((const uint16_t*)bias)[c] << 16);
  }
  out[c] = v;
}

}  // namespace

hipError_t launch_bias_f32(const void* bias, int32_t kind, int32_t V, float* out,
                           hipStream_t stream) {
  const int32_t padded = (V + kVtileCols - 1) / kVtileCols * kVtileCols;
  hipLaunchKernelGGL(bias_to_f32_kernel, dim3((unsigned)(padded / 256)), dim3(256), 0, stream,
                     bias, kind, V, padded, out);
  return hipGetLastError();
}

hipError_t launch_zero_pad_cols(uint16_t* dzt, int64_t rows, int64_t N, int64_t ldz,
                                hipStream_t stream) {
  const int64_t total = rows * (ldz - N);
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_pad_cols_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     stream, dzt, rows, N, ldz);
  return hipGetLastError();
}

hipError_t launch_row_sums(const uint16_t* dzt, int64_t rows, int64_t N, int64_t ldz, float* out,
                           hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(row_sums_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, dzt,
                     rows, N, ldz, out);
  return hipGetLastError();
}

}  // namespace bilogp
