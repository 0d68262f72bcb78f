// Ascending split merge for gfx950: per row, fold the S per-split partial
// online-softmax states into the log-sum-exp and the target log-probability.
//
// RL-Kernel PR #337, "feat(linear-logp): add batch-invariant fused SM90
// operator", description ("What this PR changes": online-softmax partials and
// an ascending combine; the same splits for every N).
//
// One wave64 per row; lane k holds split k (S <= 64 = wave width, the
// invariant policy's split limit).  M = max_k m_k is exact in any order.  The
// terms s_k * exp(m_k - M) are summed by a pairwise tree over ascending split
// index: (s0 + s1), (s2 + s3), ..., then ((s0 + s1) + (s2 + s3)), ... - the
// same tree for every row and every N.  The throughput split policy can give
// up to 1024 splits: lane k then first adds the terms of splits k, k + 64,
// k + 128, ... in ascending order, and the tree combines the 64 lane sums
// (for S <= 64 this is the same computation: 0 + x == x).  With a max-element term of exactly
// 1 the sum is >= 1, so lse >= M >= z_target and logp <= 0 exactly.
//
// logp = (z_target - M) - ln(sum), lse = M + ln(sum).  A target outside
// [0, V) gives logp = NaN (lse is still written).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "bilogp_internal.h"

namespace bilogp {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kRowsPerBlock = 4;   // one wave per row

__global__ __launch_bounds__(64 * kRowsPerBlock) void merge_kernel(
    const float2* __restrict__ part, const float* __restrict__ tlogit,
    const int64_t* __restrict__ target, float* __restrict__ logp, float* __restrict__ lse,
    int64_t N, int32_t S, int32_t V) {
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= N) return;                     // uniform across the wave

  const float2* pr = part + row * S;
  float M = -INFINITY;
  for (int k = lane; k < S; k += 64) M = fmaxf(M, pr[k].x);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) M = fmaxf(M, __shfl_xor(M, d));
  const float mu = (M == -INFINITY) ? 0.f : M;
  float term = 0.f;
  for (int k = lane; k < S; k += 64) {
    const float2 ps = pr[k];
    term += ps.y * __builtin_amdgcn_exp2f((ps.x - mu) * kLog2e);
  }
  // lane k and lane k^d add the same two operands, so every lane of a group
  // carries identical bits after each level
#pragma unroll
  for (int d = 1; d <= 32; d <<= 1) term += __shfl_xor(term, d);

  if (lane == 0) {
    const float ln_sum = __builtin_amdgcn_logf(term) * kLn2;
    lse[row] = M + ln_sum;
    const int64_t t = target[row];
    logp[row] = (t >= 0 && t < V) ? (tlogit[row] - M) - ln_sum : __builtin_nanf("");
  }
}

}  // namespace

hipError_t launch_merge(const float2* part, const float* tlogit, const int64_t* target,
                        float* logp, float* lse, int64_t N, int32_t S, int32_t V,
                        hipStream_t stream) {
  if (N <= 0) return hipSuccess;
  const int64_t blocks = (N + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)blocks), dim3(64 * kRowsPerBlock), 0, stream,
                     part, tlogit, target, logp, lse, N, S, V);
  return hipGetLastError();
}

}  // namespace bilogp
