// Internal declarations shared by the host library and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bilogp {

// Part of the bit contract: the vocabulary tile width and the largest split
// count decide which columns are reduced together and in which order.
constexpr int kVtileCols = 256;
constexpr int kMaxSplits = 256;

// Cap of the throughput split policy (not part of the invariant contract).
constexpr int kMaxThroughputSplits = 1024;

// Tokens handled by one projection workgroup.  Internal only: a row's
// arithmetic does not depend on it (no reduction mixes rows).
constexpr int kBlockRows = 256;

enum BiasKind : int32_t { kBiasNone = 0, kBiasBf16 = 1, kBiasF32 = 2 };

// What the projection kernels read at ProjParams::bias: fp32 values (the
// caller's fp32 bias, or a zero-padded fp32 copy of any bias) or the caller's
// bf16 values.
enum BiasSrc : int32_t { kBiasSrcNone = 0, kBiasSrcF32 = 1, kBiasSrcBf16 = 2 };

struct ProjParams {
  const void* hidden;      // bf16 [N, H], row-major
  const void* weight;      // bf16 [V, H], row-major
  const int64_t* target;   // [N]
  const void* bias;        // read as bias_src says, addressed by absolute column; or null
  float2* part;            // [N, S]: per (row, split) running max and sum of exp(z - max)
  float* tlogit;           // [N]: logit of each row's target
  int64_t N;
  int32_t H;
  int32_t V;
  int32_t bias_kind;       // the caller's bias dtype (BiasKind)
  int32_t bias_src;        // BiasSrc
  int32_t bias_copy;       // host only: bias is the fp32 copy, filled before the launch
  int32_t T;               // vocabulary tiles, ceil(V / kVtileCols)
  int32_t vps;             // tiles per split
  int32_t S;               // splits
  int32_t rows;            // tokens per row block: 256, or 128 for small batches
  int32_t R;               // row blocks, ceil(N / rows)
  // the launch covers splits [split0, split1) of the S in two phases: per
  // row block, runsA runs of spg consecutive splits over [split0, splitA)
  // (runsA = ceil((splitA - split0) / spg); the last run may be shorter),
  // then single splits over [splitA, split1); R * (runsA + split1 - splitA)
  // workgroups.  A one-phase launch has splitA = split1.  weight and
  // bias are addressed by absolute vocabulary column: for a launch whose
  // weight holds columns from col0 on, the host passes the weight address
  // minus col0 rows (and the bias copy's address minus col0 entries); every
  // address the kernel forms stays inside the slice
  int32_t split0;
  int32_t splitA;
  int32_t split1;
  int32_t spg;
  int32_t runsA;
  // host only: splits [splitT, split1) of the call go to a second launch of
  // 128-token row blocks (splitT = split1: none)
  int32_t splitT;
  int64_t col0;
  // backward only (softmax-gradient kernel): the forward's lse, the upstream
  // gradients of logp and lse, and dZ^T [V, ldz] (bf16) written per tile
  const float* lse;
  const float* g_logp;
  const float* g_lse;
  uint16_t* dzt;
  int64_t ldz;
};

// Enqueue the exact fp32 copy of a bf16 / fp32 bias, zero-padded to whole
// vocabulary tiles (out holds ceil(V / kVtileCols) * kVtileCols floats).
hipError_t launch_bias_f32(const void* bias, int32_t kind, int32_t V, float* out,
                           hipStream_t stream);

// Enqueue the fused projection + per-split online-softmax kernel.
hipError_t launch_proj_lse(const ProjParams& p, hipStream_t stream);

// Enqueue the softmax-gradient kernel: the same projection tiles, and per
// logit dZ = p (g_lse - g_logp) + g_logp [v == target], p = exp(z - lse),
// stored to dZ^T as bf16 (columns of p.dzt past N untouched).
hipError_t launch_softmax_grad(const ProjParams& p, hipStream_t stream);

// Enqueue dZ^T padding: zero columns [N, ldz) of every row of dZ^T.
hipError_t launch_zero_pad_cols(uint16_t* dzt, int64_t rows, int64_t N, int64_t ldz,
                                hipStream_t stream);

// Enqueue grad_bias[v] = sum over n ascending of dZ^T[v][n] (fp32 out).
hipError_t launch_row_sums(const uint16_t* dzt, int64_t rows, int64_t N, int64_t ldz,
                           float* out, hipStream_t stream);

// Enqueue the ascending split merge: lse and logp per row.
hipError_t launch_merge(const float2* part, const float* tlogit, const int64_t* target,
                        float* logp, float* lse, int64_t N, int32_t S, int32_t V,
                        hipStream_t stream);

// Deterministic GEMM: D[p, q] = sum_c X[p, c] * Y[q, c] over ascending c,
// fp32 accumulation, written as out[q][p].  An operand is read either from
// its natural layout (X[p][c] at x + p * ldx + c: contraction contiguous) or
// transposed (stored as [c][p] at x + c * ldx + p).
struct GemmParams {
  const void* x;           // bf16
  const void* y;           // bf16
  void* out;               // out[q][p] at out + q * ldo + p: fp32 or bf16
  int64_t P, Q, C;
  int64_t ldx, ldy, ldo;   // row pitches in elements
  int32_t out_kind;        // GemmOut
  int32_t Pt, Qt;          // tiles along P and Q (set by launch_det_gemm)
  int32_t cu_count;        // compute units of the device (tile-size choice), 0 unknown
};

enum GemmOut : int32_t { kGemmBf16 = 0, kGemmF32 = 1, kGemmF32Accum = 2 };

// Enqueue the GEMM; x_t / y_t select the transposed storage of X / Y.
hipError_t launch_det_gemm(const GemmParams& g, bool x_t, bool y_t, hipStream_t stream);

}  // namespace bilogp
