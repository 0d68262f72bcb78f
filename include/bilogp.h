/*
 * bilogp.h - batch-invariant fused linear log-probability forward for AMD
 * Instinct MI355X (gfx950).  Plain C ABI: device pointers, sizes, a stream.
 *
 * The operation (RL-Kernel PR #337, "feat(linear-logp): add batch-invariant
 * fused SM90 operator": walkthrough, sequence diagram and description):
 *
 *     z[i, v]  = sum_k hidden[i, k] * W[v, k]  (+ bias[v])     v in [0, V)
 *     lse[i]   = log( sum_v exp(z[i, v]) )
 *     logp[i]  = z[i, target[i]] - lse[i]
 *
 * The [N, V] logits are never stored.  The vocabulary is cut into tiles of
 * bilogp_vtile_cols() columns and the tiles into at most bilogp_max_splits()
 * contiguous splits whose count depends on V only (the page's annotation on
 * select_batch_invariant_vocab_splits).  Each split yields a per-row partial
 * online-softmax state (running max, rescaled sum of exponentials); the
 * partials are combined in ascending split order ("What this PR changes"),
 * as one pairwise tree over ascending split index, the same for every N.
 * The bits of row i's outputs depend only on row i's inputs, W, bias, H and
 * V: never on N, on the position of the row in the batch, on the other rows,
 * or on the number of compute units.
 *
 * The page's first contract is forward-only (author's annotation on the
 * requires_grad check: the backward lies outside it).  bilogp_backward, at
 * the end of this header, extends it with a deterministic backward built on
 * the same projection tiles and on the deterministic GEMM below.
 *
 * Conventions for every entry point
 *  - Ownership: the caller owns every buffer.  The library keeps no device
 *    state between calls; bilogp_forward allocates and frees its workspace
 *    stream-ordered on `stream`.
 *  - Asynchrony: all device work is enqueued on `stream` (a hipStream_t;
 *    NULL = the null stream).  No entry point synchronizes; inputs must stay
 *    alive until the stream reaches the work.
 *  - Errors: no entry point throws.  Every argument is checked before any
 *    device work: on BILOGP_E_INVALID_ARG, _UNSUPPORTED or _WORKSPACE nothing
 *    is launched and the outputs are left untouched.  BILOGP_E_HIP reports a
 *    failure of the HIP runtime itself (a launch or allocation the checks
 *    could not foresee); kernels of the same call enqueued before it may
 *    still run.  A status is returned and a thread-local message is
 *    available from bilogp_last_error().
 *  - Grids: a call on any N the checks accept is issued as row chunks whose
 *    grids fit the 32-bit work-item limit; rows are independent, so this
 *    never changes a bit.
 *  - Failing closed (the page's registry maps unsupported platforms to an
 *    explicit error rather than a generic fallback): a device that is not
 *    gfx950 gives BILOGP_E_UNSUPPORTED; there is no other code path.
 *  - Thread safety: entry points are reentrant.  Concurrent calls on
 *    different streams must use different workspaces.
 */
#ifndef BILOGP_H
#define BILOGP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BILOGP_ABI_VERSION 4

/* Version of the bit contract: for given inputs of one row (its hidden row
 * and target, W, bias, H, V), which fp32 bits logp and lse take, and for the
 * deterministic GEMM and backward, which bits their outputs take for given
 * operands.  The page fixes no bits (several fp32 results are equally
 * correct, PR #337 description, "Why this happens"); what this library
 * promises is that the bits of one version never depend on N, the row's
 * position, the other rows, the stream or the compute units (for the
 * weight gradients: on anything but the rows themselves, reduced in
 * ascending order).  A change to anything that orders the arithmetic
 * changes the version:
 *   1  tiles of 256 columns, at most 64 splits; merge tree whose lanes
 *      pre-summed strided splits
 *   2  tiles of 256 columns, at most 256 splits; merge tree whose lanes
 *      pre-sum consecutive splits (a perfect pairwise tree over ascending
 *      split index); K reduced in ascending 16-wide steps of
 *      v_mfma_f32_32x32x16_bf16; per token, each lane sums its 64 values of a
 *      tile in a fixed register order, then the two lane halves and the two
 *      vocabulary-half waves are merged in fixed operand order
 *   3  as 2, but K is reduced in ascending 32-wide steps of
 *      v_mfma_f32_16x16x32_bf16, and per token each lane sums its 32 values
 *      of a tile (8 blocks of 4 vocabulary rows) in a fixed register order,
 *      then the four lane groups (pairs 16 lanes apart, then 32 apart) and
 *      the two vocabulary-half waves are merged in fixed operand order
 *   4  forward as 3; the deterministic GEMM (bilogp_det_gemm_*) and the
 *      backward's two products reduce in ascending 32-wide steps of
 *      v_mfma_f32_16x16x32_bf16 (before: 16-wide steps of
 *      v_mfma_f32_32x32x16_bf16) */
#define BILOGP_BIT_CONTRACT_VERSION 4

typedef enum bilogp_status {
  BILOGP_OK = 0,
  BILOGP_E_INVALID_ARG = 1,   /* null pointer, bad size, aliasing outputs, bad enum */
  BILOGP_E_UNSUPPORTED = 2,   /* not gfx950, pointer not on the current device,
                                 H % 8 != 0, misaligned input */
  BILOGP_E_WORKSPACE = 3,     /* workspace missing or smaller than bilogp_workspace_bytes */
  BILOGP_E_HIP = 4            /* a HIP runtime call or launch failed */
} bilogp_status;

typedef enum bilogp_bias_dtype {
  BILOGP_BIAS_NONE = 0,
  BILOGP_BIAS_BF16 = 1,
  BILOGP_BIAS_F32 = 2
} bilogp_bias_dtype;

/* BILOGP_ABI_VERSION of the built library. */
int bilogp_abi_version(void);

/* BILOGP_BIT_CONTRACT_VERSION of the built library: outputs of two builds
 * with the same value are bit-identical for the same inputs. */
int bilogp_bit_contract_version(void);

/* Width of a vocabulary tile in columns.  Part of the bit contract. */
int bilogp_vtile_cols(void);

/* Largest number of vocabulary splits.  Part of the bit contract. */
int bilogp_max_splits(void);

/* Vocabulary tiles per split for vocabulary size V: with T = ceil(V / tile
 * width), ceil(T / bilogp_max_splits()).  The page gives the policy's
 * constraints (annotation on select_batch_invariant_vocab_splits: at most
 * the maximum number of non-empty contiguous ranges, chosen from V only) but
 * its formula is cut off; this is the plainest reading.  Split k covers
 * tiles [k * per_split, min((k + 1) * per_split, T)).  Returns 0 if V <= 0
 * or V > 2^30.  Takes no N and no device property, by construction. */
int bilogp_vtiles_per_split(int64_t V);

/* Number of splits S = ceil(T / per_split) for vocabulary size V (0 if V is
 * out of range). */
int bilogp_num_vocab_splits(int64_t V);

/* Bytes of device workspace bilogp_forward_ex needs for N rows and vocabulary
 * size V: the [N, S] partial (max, sum-exp) pairs, the [N] target logits and
 * an fp32 copy of the bias padded to whole 256-column tiles (reserved whether
 * or not a call passes a bias; used only for a bias that cannot be read in
 * place, i.e. one not 16-byte aligned or whose V is not a multiple of 4 (fp32)
 * or 8 (bf16)), each 256-byte aligned.  0 for N == 0;
 * (size_t)-1 for invalid N or V. */
size_t bilogp_workspace_bytes(int64_t N, int64_t V);

/* Split policies (RL-Kernel PR #337, description, "Why this happens" and its
 * flowchart: the operator the page starts from has a throughput scheduler
 * that picks the vocabulary split from N, V and the GPU's SM count, so one
 * token row can be reduced as [A][B][C][D] in one batch and [A B][C D] in
 * another; the pull request adds the V-only policy).
 *
 *   BILOGP_SPLITS_INVARIANT   the contract above: splits from V only.  Every
 *                             entry point without a mode argument uses it.
 *   BILOGP_SPLITS_THROUGHPUT  splits from N, V and a compute-unit count, for
 *                             measuring what invariance costs.  The page gives
 *                             no formula; with T tiles and R = ceil(N / 256)
 *                             row blocks: want = min(max(ceil(cu_count / R), 1),
 *                             T, BILOGP_MAX_THROUGHPUT_SPLITS), per_split =
 *                             ceil(T / want), S = ceil(T / per_split) - enough
 *                             splits that R x S approaches cu_count.  A row's
 *                             bits then depend on N and cu_count (the failure
 *                             mode the invariant policy removes); the values
 *                             stay within the same accuracy of the exact ones.
 */
typedef enum bilogp_split_mode {
  BILOGP_SPLITS_INVARIANT = 0,
  BILOGP_SPLITS_THROUGHPUT = 1
} bilogp_split_mode;

#define BILOGP_MAX_THROUGHPUT_SPLITS 1024

/* Tiles per split and split count under `mode` (cu_count is read only by the
 * throughput mode, N only by it and for validity).  0 if N < 1 (throughput),
 * V is out of range, mode is unknown or cu_count < 1 (throughput). */
int bilogp_vtiles_per_split_mode(int64_t N, int64_t V, int mode, int cu_count);
int bilogp_num_vocab_splits_mode(int64_t N, int64_t V, int mode, int cu_count);

/* Workspace bytes for bilogp_forward_mode (as bilogp_workspace_bytes, with
 * the mode's split count).  (size_t)-1 on invalid arguments, 0 for N == 0. */
size_t bilogp_workspace_bytes_mode(int64_t N, int64_t V, int mode, int cu_count);

/* Launch plan of the projection for N rows of H features under `mode`,
 * scheduled for cu_count compute units (what bilogp_forward_mode does with
 * the same arguments): tokens per row block (256, or 128 when 256-token
 * blocks would leave units idle and the 128-token plan has the shorter
 * critical path), consecutive splits per workgroup (of the longest runs),
 * and the workgroup count of all its launches (bilogp_launch_schedule).
 * Scheduling only - in the invariant mode no output bit depends on it.
 * Host-side, no device needed.  Returns 0, or -1 for N < 1, H, V or cu_count
 * out of range, or an unknown mode (outputs untouched).  (ABI 3 added H.) */
int bilogp_launch_plan(int64_t N, int64_t H, int64_t V, int mode, int cu_count,
                       int* rows_per_block, int* splits_per_workgroup, int64_t* workgroups);

/* Split schedule of the same plan, for S splits.  With 256-token row blocks,
 * splits [0, split_a) go in runs of splits_per_workgroup, [split_a, split_t)
 * one per workgroup, both in one launch, and [split_t, S) to a second launch
 * of 128-token row blocks, one split per workgroup: the big launch ends after
 * whole rounds of one workgroup per compute unit and the remainder fills one
 * round of half-height pieces.  It is chosen where a cost model of K stages
 * per compute unit has it ending first; otherwise split_a = split_t = S.
 * Scheduling only, as above.  Returns 0 or -1 as bilogp_launch_plan.
 * (ABI 4.) */
int bilogp_launch_schedule(int64_t N, int64_t H, int64_t V, int mode, int cu_count,
                           int* split_a, int* split_t);

/* Fused forward with an optional fp32 bias and a library-managed workspace
 * (stream-ordered hipMallocAsync / hipFreeAsync on `stream`).
 *
 *   hidden   device, bf16 [N, H] row-major (K contiguous), 16-byte aligned
 *   weight   device, bf16 [V, H] row-major (K contiguous), 16-byte aligned
 *   target   device, int64 [N]; a value outside [0, V) yields logp = NaN for
 *            that row (lse stays valid) - a range check needs a host sync,
 *            which this entry point never does
 *   bias     device, fp32 [V], or NULL for no bias
 *   logp_out device, fp32 [N]   (written)
 *   lse_out  device, fp32 [N]   (written)
 *   0 <= N <= 2^32 (N == 0 is a successful no-op), 8 <= H <= 2^20 with
 *   H % 8 == 0, 1 <= V <= 2^30.  The outputs must not overlap each other, an
 *   input or the workspace; the workspace must not overlap an input.
 */
bilogp_status bilogp_forward(const void* hidden, const void* weight, const int64_t* target,
                             const float* bias, float* logp_out, float* lse_out,
                             int64_t N, int64_t H, int64_t V, void* stream);

/* As bilogp_forward, with the bias dtype given explicitly (bias may be bf16
 * or fp32, [V]; NULL iff bias_dtype == BILOGP_BIAS_NONE) and a caller-owned
 * device workspace of at least bilogp_workspace_bytes(N, V) bytes, 256-byte
 * aligned.  Allocates nothing. */
bilogp_status bilogp_forward_ex(const void* hidden, const void* weight, const int64_t* target,
                                const void* bias, int bias_dtype, float* logp_out,
                                float* lse_out, int64_t N, int64_t H, int64_t V,
                                void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory - code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: the forward
 * of bilogp_forward_ex (same arguments and checks, same bits) with no
 * workspace argument and no allocation of any kind.  The workspace is a
 * library-owned device array of bilogp_noalloc_max_workspace_bytes() bytes
 * (64 MiB), one per GPU, held until the process ends; a call whose
 * bilogp_workspace_bytes(N, V) exceeds it fails with BILOGP_E_WORKSPACE
 * before any device work (at V = 128256: beyond about 33,000 rows).  Every call
 * on one GPU shares that GPU's array, and the array keeps the last call's
 * contents (nothing in it needs to start at zero): calls that may overlap on
 * one GPU - on different streams, or from several threads - race; serialize
 * them, or use bilogp_forward_ex with a workspace per stream. */
size_t bilogp_noalloc_max_workspace_bytes(void);

bilogp_status bilogp_forward_noalloc(const void* hidden, const void* weight,
                                     const int64_t* target, const void* bias, int bias_dtype,
                                     float* logp_out, float* lse_out, int64_t N, int64_t H,
                                     int64_t V, void* stream);

/* bilogp_forward_ex under split policy `mode`, scheduled for `cu_count`
 * compute units.
 *
 * cu_count is the compute-unit count the launch is scheduled for: the row-
 * block height (256 or 128 tokens) and how many consecutive splits one
 * workgroup takes.  0 means the current device's count.  In the invariant
 * mode it is scheduling only: the bits are those of bilogp_forward_ex for
 * every cu_count (that is the contract's "never on the number of compute
 * units", and it lets a test vary the count on one device).  In the
 * throughput mode it is also the count the split policy fills, so it must be
 * >= 1 and the bits then depend on it.
 *
 * The workspace must hold bilogp_workspace_bytes_mode(N, V, mode, cu_count)
 * bytes.  An unknown mode, cu_count outside [0, 65536], or cu_count < 1 in
 * throughput mode gives BILOGP_E_INVALID_ARG.  At most
 * BILOGP_MAX_THROUGHPUT_SPLITS splits are combined, in ascending order. */
bilogp_status bilogp_forward_mode(const void* hidden, const void* weight, const int64_t* target,
                                  const void* bias, int bias_dtype, float* logp_out,
                                  float* lse_out, int64_t N, int64_t H, int64_t V, int mode,
                                  int cu_count, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* The two halves of bilogp_forward_ex, for callers that schedule them
 * separately (a timing harness, or a vocabulary-sharded caller that exchanges
 * partials between the halves).  Same arguments and checks as
 * bilogp_forward_ex; the workspace carries the state between the calls.
 *
 * bilogp_partials: the fused projection and per-split online softmax; writes
 * the workspace's [N, S] (max, sum-exp) partials and the [N] target logits
 * (RL-Kernel PR #337, description: split-V from V only, partial online-
 * softmax states per contiguous split).
 */
bilogp_status bilogp_partials(const void* hidden, const void* weight, const int64_t* target,
                              const void* bias, int bias_dtype, int64_t N, int64_t H, int64_t V,
                              void* workspace, size_t workspace_bytes, void* stream);

/* bilogp_partials_range: one rank's share of a vocabulary-sharded projection.
 * The split boundaries depend on the full V alone (PR #337, description,
 * "What this PR changes", and the annotation on
 * select_batch_invariant_vocab_splits), so every rank of a vocabulary-sharded
 * lm-head agrees on them without communicating.  A rank holding the
 * vocabulary columns of splits [split_begin, split_end) runs the projection
 * and per-split online softmax of those splits only:
 *
 *   weight_slice  bf16 [c1 - c0, H], columns [c0, c1) of the full weight, with
 *                 c0 = split_begin * vps * tile width and
 *                 c1 = min(split_end * vps * tile width, V), vps =
 *                 bilogp_vtiles_per_split(V); 16-byte aligned
 *   bias_slice    the same columns of the bias (bf16 or fp32), or NULL
 *   V             the FULL vocabulary size; 0 <= split_begin < split_end <=
 *                 bilogp_num_vocab_splits(V), else BILOGP_E_INVALID_ARG
 *   workspace     the layout of bilogp_workspace_bytes(N, V) (partials first,
 *                 row-major [N][S] (max, sum) float pairs; then the [N] target
 *                 logits); the call writes its splits' columns of the
 *                 partials and the target logit of each row whose target lies
 *                 in [c0, c1), and nothing else
 *
 * Once every split's columns are present - written by calls on this device,
 * or copied in from the other ranks - bilogp_merge gives bit for bit the
 * result of bilogp_forward_ex on the full weight.  Other arguments and checks
 * as for bilogp_partials.  The exchange between ranks is the caller's. */
bilogp_status bilogp_partials_range(const void* hidden, const void* weight_slice,
                                    const int64_t* target, const void* bias_slice, int bias_dtype,
                                    int64_t N, int64_t H, int64_t V, int split_begin,
                                    int split_end, void* workspace, size_t workspace_bytes,
                                    void* stream);

/* bilogp_merge: the combine, in ascending split order, of the partials left
 * in `workspace` by bilogp_partials (or by bilogp_partials_range over every
 * split) for the same N, V and target (PR #337, description, "What this PR
 * changes"); writes logp_out and lse_out, fp32 [N]. */
bilogp_status bilogp_merge(const int64_t* target, const void* workspace, size_t workspace_bytes,
                           float* logp_out, float* lse_out, int64_t N, int64_t V, void* stream);

/* ------------------------------------------------------------------------
 * Deterministic bf16 GEMM (RL-Kernel PR #395, "feat(musa): add native
 * deterministic gemm kernel", summary: a fixed ascending K-order reduction
 * with fp32 accumulation; [M, K] @ [N, K]^T without materialising the
 * transposed right-hand side; dA; the [N, K] weight gradient).
 *
 * Every output element is one fp32 accumulation over the contraction index
 * in ascending order, started at 0, never split; its bits depend only on the
 * two vectors it contracts (and, for the accumulating output, on its old
 * value): the forward's and dA's rows do not depend on M.  Inputs are bf16,
 * row-major, 16-byte aligned; 8 <= N, K <= 2^20, N % 8 == 0, K % 8 == 0,
 * 0 <= M <= 2^31 (an operand or output of zero bytes may be NULL).  The
 * output must not overlap an operand.  Outputs:
 *   BILOGP_GEMM_OUT_BF16       rounded to bf16 (nearest even)
 *   BILOGP_GEMM_OUT_F32        fp32
 *   BILOGP_GEMM_OUT_F32_ACCUM  fp32, out = out + (the fp32 product), one add
 * Same conventions as above (stream-ordered, no sync, status + message). */
typedef enum bilogp_gemm_out {
  BILOGP_GEMM_OUT_BF16 = 0,
  BILOGP_GEMM_OUT_F32 = 1,
  BILOGP_GEMM_OUT_F32_ACCUM = 2
} bilogp_gemm_out;

/* C[M, N] = A[M, K] . B[N, K]^T (reduction over K).  M == 0 is a no-op. */
bilogp_status bilogp_det_gemm_fwd(const void* a, const void* b, void* c, int64_t M, int64_t N,
                                  int64_t K, int out_kind, void* stream);

/* dA[M, K] = dC[M, N] . B[N, K] (reduction over N): the input gradient of
 * the forward.  M == 0 is a no-op. */
bilogp_status bilogp_det_gemm_da(const void* dc, const void* b, void* da, int64_t M, int64_t N,
                                 int64_t K, int out_kind, void* stream);

/* dB[N, K] = dC[M, N]^T . A[M, K] (reduction over M, ascending): the weight
 * gradient in the forward's [N, K] layout.  M == 0 writes zeros (or leaves an
 * accumulating output unchanged). */
bilogp_status bilogp_det_gemm_db(const void* a, const void* dc, void* db, int64_t M, int64_t N,
                                 int64_t K, int out_kind, void* stream);

/* ------------------------------------------------------------------------
 * Deterministic backward of the fused linear log-probability.
 *
 * The first contract of RL-Kernel PR #337 stops at the forward (author's
 * annotation on the requires_grad check); this extends it with the gradients
 * of the forward's two outputs, reduced in fixed orders with the
 * deterministic GEMM of RL-Kernel PR #395 (summary: dA = dC . B and the
 * weight gradient in the forward's [V, H] layout, fixed ascending
 * contraction, fp32 accumulation).  With P[i, v] = exp(z[i, v] - lse[i])
 * and the upstream gradients g_logp[i] (of logp[i]) and g_lse[i] (of
 * lse[i]):
 *
 *     dZ[i, v]       = g_lse[i] P[i, v] + g_logp[i] ([v == target[i]] - P[i, v])
 *     grad_hidden    = dZ . W            [N, H], reduction over v ascending
 *     grad_weight    = dZ^T . hidden     [V, H], reduction over i ascending
 *     grad_bias[v]   = sum_i dZ[i, v]    [V],    i ascending, fixed tree
 *
 * (g_logp = -1, g_lse = 0 is the cross-entropy gradient softmax - onehot.)
 * z is recomputed tile by tile exactly as the forward computes it; dZ is
 * rounded to bf16 (nearest even), the operand type of the two products, and
 * stored transposed in the workspace ([V, ldz] with ldz = N rounded up to 8);
 * the [N, V] logits are never stored in fp32.  A target outside [0, V)
 * contributes no one-hot term.
 *
 * Bit contract: row i of grad_hidden depends only on hidden[i], target[i],
 * lse[i], g_logp[i], g_lse[i], W, bias, H and V - not on N or on the other
 * rows.  grad_weight and grad_bias sum over the batch in ascending row
 * order: the same bits on every run, stream and device.
 *
 *   hidden, weight, target, bias, bias_dtype   as for bilogp_forward_ex
 *   lse          device, fp32 [N]: the forward's lse for these inputs
 *   grad_logp    device, fp32 [N]
 *   grad_lse     device, fp32 [N]
 *   grad_hidden  device, fp32 [N, H] (written), 16-byte aligned
 *   grad_weight  device, fp32 [V, H] (written), 16-byte aligned
 *   grad_bias    device, fp32 [V] (written), or NULL for no bias gradient
 *   workspace    device, at least bilogp_backward_workspace_bytes(N, V)
 *                bytes, 256-byte aligned; holds dZ^T between the kernels
 *   0 <= N <= 2^21 (N == 0 writes zeros to grad_weight and grad_bias; the
 *   [N] inputs and grad_hidden may then be NULL), H and V as for the
 *   forward.  The gradients must not overlap each other, an input or the
 *   workspace.  Same conventions as above (stream-ordered, no sync, status +
 *   message, nothing launched on an error).
 */
size_t bilogp_backward_workspace_bytes(int64_t N, int64_t V);

bilogp_status bilogp_backward(const void* hidden, const void* weight, const int64_t* target,
                              const void* bias, int bias_dtype, const float* lse,
                              const float* grad_logp, const float* grad_lse, float* grad_hidden,
                              float* grad_weight, float* grad_bias, int64_t N, int64_t H,
                              int64_t V, void* workspace, size_t workspace_bytes, void* stream);

/* Static description of a status code. */
const char* bilogp_status_string(int status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char* bilogp_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BILOGP_H */
