// Ascending split merge for gfx950: per row, fold the S per-split partial
// online-softmax states into the log-sum-exp and the target log-probability.
//
// RL-Kernel PR #337, "feat(linear-logp): add batch-invariant fused SM90
// operator", description ("What this PR changes": online-softmax partials and
// an ascending combine; the same splits for every N).
//
// One wave64 per row.  M = max_k m_k is exact in any order.  The terms
// s_k * exp(m_k - M) are summed by one perfect pairwise tree over ascending
// split index: (s0 + s1), (s2 + s3), ..., then ((s0 + s1) + (s2 + s3)), ...
// Lane l holds the C consecutive splits [l C, l C + C), C the smallest power
// of two with 64 C >= S (at most 16: the throughput policy's 1024 splits),
// reduces them by the tree's lower levels, and the wave's xor shuffles make
// the upper levels.  Leaves past S are zero and add exactly, so the sum does
// not depend on C beyond S: the same tree for every row and every N.  With
// a max-element term of exactly 1 the sum is >= 1, so lse >= M >= z_target
// and logp <= 0 exactly.
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

template <int C>
__global__ __launch_bounds__(64 * kRowsPerBlock) void merge_kernel(
    const float2* __restrict__ part, const float* __restrict__ tlogit,
    const int64_t* __restrict__ target, float* __restrict__ logp, float* __restrict__ lse,
    int64_t N, int32_t S, int32_t V) {
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= N) return;                     // uniform across the wave

  const float2* pr = part + row * S;
  float2 ps[C];
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int k = lane * C + j;
    ps[j] = (k < S) ? pr[k] : make_float2(-INFINITY, 0.f);
  }
  float M = ps[0].x;
#pragma unroll
  for (int j = 1; j < C; ++j) M = fmaxf(M, ps[j].x);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) M = fmaxf(M, __shfl_xor(M, d));
  const float mu = (M == -INFINITY) ? 0.f : M;
  float t[C];
#pragma unroll
  for (int j = 0; j < C; ++j)
    t[j] = (lane * C + j < S) ? ps[j].y * __builtin_amdgcn_exp2f((ps[j].x - mu) * kLog2e) : 0.f;
  // lower levels of the tree, inside the lane
#pragma unroll
  for (int w = 1; w < C; w <<= 1)
#pragma unroll
    for (int j = 0; j < C; j += 2 * w) t[j] += t[j + w];
  float term = t[0];
  // upper levels: lane l and lane l ^ d add the same two operands, so every
  // lane of a group carries identical bits after each level
#pragma unroll
  for (int d = 1; d <= 32; d <<= 1) term += __shfl_xor(term, d);

  if (lane == 0) {
    // ln(sum) rounded once and shared by both outputs: no multiply-add fused
    // into lse alone
#pragma clang fp contract(off)
    const float ln_sum = __builtin_amdgcn_logf(term) * kLn2;
    lse[row] = M + ln_sum;
    const int64_t tg = target[row];
    logp[row] = (tg >= 0 && tg < V) ? (tlogit[row] - M) - ln_sum : __builtin_nanf("");
  }
}

}  // namespace

hipError_t launch_merge(const float2* part, const float* tlogit, const int64_t* target,
                        float* logp, float* lse, int64_t N, int32_t S, int32_t V,
                        hipStream_t stream) {
  if (N <= 0) return hipSuccess;
  const int64_t blocks = (N + kRowsPerBlock - 1) / kRowsPerBlock;
  const dim3 grid((unsigned)blocks), block(64 * kRowsPerBlock);
  if (S <= 64)
    hipLaunchKernelGGL(merge_kernel<1>, grid, block, 0, stream, part, tlogit, target, logp, lse, N, S, V);
  else if (S <= 128)
    hipLaunchKernelGGL(merge_kernel<2>, grid, block, 0, stream, part, tlogit, target, logp, lse, N, S, V);
  else if (S <= 256)
    hipLaunchKernelGGL(merge_kernel<4>, grid, block, 0, stream, part, tlogit, target, logp, lse, N, S, V);
  else if (S <= 512)
    hipLaunchKernelGGL(merge_kernel<8>, grid, block, 0, stream, part, tlogit, target, logp, lse, N, S, V);
  else if (S <= 1024)
    hipLaunchKernelGGL(merge_kernel<16>, grid, block, 0, stream, part, tlogit, target, logp, lse, N, S, V);
  else
    return hipErrorInvalidValue;            // the split policies never exceed 1024
  return hipGetLastError();
}

}  // namespace bilogp
