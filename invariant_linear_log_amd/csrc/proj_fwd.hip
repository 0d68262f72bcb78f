// Fused projection + per-split online softmax (the forward) for gfx950 (CDNA4).
//
// Operation (RL-Kernel PR #337, "feat(linear-logp): add batch-invariant fused
// SM90 operator", description): logits z = hidden . W^T (+ bias) are formed
// tile by tile and never stored; every (row block, vocabulary split) pair
// reduces its split's contiguous vocabulary tiles, in ascending order, to a
// per-row online-softmax partial (running max m, sum s of exp(z - m)).  The
// partials are merged by merge.hip.
//
// Workgroup: 512 threads (8 wave64s), one row block of 256 tokens (or 128,
// below) and a run of consecutive splits: their tiles are one contiguous
// range, computed back to back, and a partial is written (and the running
// state restarted) where each split ends.  How many splits a workgroup takes
// only schedules the work: every split's partial is the same either way.
// Per vocabulary tile of 256 columns the workgroup computes the 256 x 256
// product W_tile[256, H] . hidden_block[256, H]^T with
// v_mfma_f32_16x16x32_bf16, W as the A operand (MFMA rows = vocabulary) and
// hidden as the B operand (MFMA columns = tokens).
//
// Why this instruction.  The board runs this kernel at its power cap, so the
// clock - and with it the throughput - is set by energy per flop.  Measured on
// MI355X with random bf16 operands, eight waves per compute unit at the cap,
// the 16 x 16 x 32 form sustains about 13% more flops per joule than
// v_mfma_f32_32x32x16_bf16 (2.0 vs 1.78 PFLOP/s at the same board power); it
// moves half as many accumulator bits per flop.
//
// Waves: w = 2 * wt + wv.  wv in {0, 1} picks vocabulary rows [128 wv, +128)
// of the tile, wt in {0..3} picks tokens [64 wt, +64) of the block (32 with
// 128-token blocks).  A wave holds 8 x kTj MFMA tiles of 16 x 16: tile
// (vi, tj) covers vocabulary rows 16 vi .. 16 vi + 15 of the wave's half and
// tokens 16 tj .. 16 tj + 15 of its quarter.  In an accumulator of that tile,
// lane l holds token column l % 16 and the four vocabulary rows
// 4 (l / 16) + i, i = 0..3 (lane group g = l / 16).  So for each token a lane
// holds 32 of the wave's 128 vocabulary rows, and the per-token max and sum
// over a tile are lane-local loops, then two fixed shuffle levels over the
// four lane groups, then a fixed merge of the two vocabulary halves.
//
// Bit contract.  For a fixed (token, vocabulary column) the K reduction is
// the same chain of MFMA instructions over ascending 32-wide K steps whatever
// N or the token's slot in the block; the per-token reductions over
// vocabulary columns follow the (lane group, register) layout of the tile,
// which is the same for every token column and for both row-block heights;
// the cross-lane and cross-wave merges use fixed operand order.  Nothing
// depends on N, the row block or the number of compute units.
//
// Memory pipeline (unchanged from the 32 x 32 design it replaces).  K is
// staged in 64-wide slices - one whole 128-byte line of every W and hidden
// row - through two LDS buffers (64 KB each: a 256 x 64 W slice and a
// 256 x 64 hidden slice), filled with buffer loads that write LDS directly.
// The W slice of stage g + 2 is requested right after the barrier that
// releases the buffer of stage g; its hidden slice under the first K step of
// stage g + 1.  Out-of-range rows (the vocabulary tail, the last row block)
// and K chunks past H read as zero through the buffer descriptors' range
// check.  Only waves 0-3 (the loader waves) issue these loads and wait for
// them; waves 4-7 run the same MFMA and LDS-read sequence with neither.  Each
// SIMD holds one wave of each half, and its issue arbiter favours the older
// wave, so the waves that carry the memory waits are the ones served first
// (measured: 3.17 ms -> 2.95-3.01 ms at N = H = 4096, V = 128256, against
// every wave issuing an eighth of the loads).
//
// Instruction schedule of a K step (32 wide, two per stage): MFMA (vi, tj) in
// the order vi outer, tj inner.  A fragments are streamed through a ring of
// four registers three vocabulary blocks ahead (A[vi + 3] is read at the
// first MFMA of vi), B fragments of the next step are read during the step,
// and the step's share of direct loads is spread between the MFMAs.  The
// stage barrier sits in the second step right after the last read of the
// current buffer (the MFMAs after it keep the matrix core busy while slower
// waves arrive); the reads of the next stage's first fragments and the refill
// of the released buffer follow it.  Each step is emitted MFMA by MFMA between
// scheduling fences, in this fixed order.
//
// LDS layout.  Each 256 x 64 slice is 256 rows of eight 16-byte chunks,
// chunk c of row r stored at position c ^ f(r), f(r) = (r >> 1) & 7.  An MFMA
// operand read takes 16 rows (lane % 16) at one chunk per lane group; the
// swizzle depends only on the lane, and a pass of 16 lanes touches 16
// distinct (row parity, chunk position) pairs.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "bilogp_internal.h"

namespace bilogp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kThreads = 512;
constexpr int kBK = 64;                            // K per stage
constexpr int kChunks = kBK / 8;                   // 16-byte chunks per slice row
constexpr int kLdsRowBytes = kBK * 2;              // 128 B per slice row
constexpr int kTileBytes = kVtileCols * kLdsRowBytes;         // 32 KB: one operand slice
constexpr int kSlotBytes = 2 * kTileBytes;                    // W, hidden
constexpr int kLoaderWaves = 4;                    // waves 0..3 issue every direct load
constexpr int kLoadsW = kTileBytes / (kLoaderWaves * 64 * 16);  // 8 per loader wave and stage
constexpr int kRowBlockGroup = 4;                  // row blocks per tile-order group
constexpr int kFragStride = 16 * kLdsRowBytes;     // 2 KB: next 16-row MFMA block
constexpr uint32_t kOutOfRange = 0x7ffffff0u;      // any offset past num_records
constexpr int kRsrcWord3 = 0x00020000;             // gfx9 raw buffer, 32-bit data
constexpr float kLog2e = 1.4426950408889634f;

static_assert(kBlockRows == 256 && kVtileCols == 256, "tile geometry is fixed");
static_assert(kLoadsW == 8, "load mapping assumes 8 W instructions per loader wave");

__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits [3:0] and [15:14], expcnt [6:4] and lgkmcnt [11:8] at max).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Merge of two online-softmax states (lo from the lower vocabulary columns).
__device__ __forceinline__ void merge_state(float m_lo, float s_lo, float m_hi, float s_hi,
                                            float& m, float& s) {
  const float M = fmaxf(m_lo, m_hi);
  const float mu = (M == -INFINITY) ? 0.f : M;
  s = s_lo * exp2_hw((m_lo - mu) * kLog2e) + s_hi * exp2_hw((m_hi - mu) * kLog2e);
  m = M;
}

template <int I>
using Slot = std::integral_constant<int, I>;

// fp32 -> bf16 bits, round to nearest even: gfx950's conversion instruction
// (v_cvt_pk_bf16_f32).  fp32 denormals are kept (the kernels run with fp32
// denormal mode on), so every finite value and infinity rounds exactly as
// the IEEE definition; a NaN stays a NaN.
__device__ __forceinline__ uint16_t bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// The kernel body.  kBias: no bias (0), or the bias read as fp32 (1) or as
// bf16 (2) values, widened on reading.  kTj token blocks of 16 per wave: 4
// (256-token row blocks) or 2 (128-token row blocks, for batches too small to
// give every compute unit a 256-token block); kSlots LDS buffers.  With kGrad it is the
// softmax-gradient pass of the backward: the same tiles and the same
// accumulation (z has the forward's bits), and a tile epilogue that writes
// dZ = p (g_lse - g_logp) + g_logp [v == target], p = exp(z - lse), instead
// of reducing it.
template <int kBias, bool kGrad, int kTj, int kSlots>
__device__ __forceinline__ void proj_fwd_body(const ProjParams& p) {
  constexpr bool kHasBias = kBias != 0;
  static_assert(kTj == 4 || kTj == 2, "two or four 16-token blocks per wave");
  static_assert(kSlots == 2 || (kSlots == 3 && kTj == 2), "three buffers fit 128-token blocks");
  constexpr int kRows = 64 * kTj;                  // tokens per row block
  constexpr int kWaveTok = 16 * kTj;               // tokens per wave
  constexpr int kM = 8 * kTj;                      // MFMAs per K step
  // Buffers: each its own variable, so the compiler can tell a read of one
  // from a direct-to-LDS load into another and does not drain the load
  // pipeline before every read.  Layout: W slice (32 KB), hidden slice.
  constexpr int kBuf = kSlots == 2 ? kSlotBytes : kTileBytes + kRows * kLdsRowBytes;
  __shared__ __attribute__((aligned(1024))) uint8_t slot0[kBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t slot1[kBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t slot2[kSlots == 3 ? kBuf : 16];
  __shared__ float2 red[kBlockRows];
  // each token's target (-1 outside [0, V)), read once per tile by the
  // epilogue: kept in LDS rather than in registers through the stage loop
  __shared__ int tgt_lds[kBlockRows];
  // backward: per token the forward's lse, g_lse - g_logp and g_logp
  __shared__ float grad_lds[3][kGrad ? kBlockRows : 1];
  // bias of the current and the next vocabulary tile (bias kernels only)
  __shared__ __attribute__((aligned(16))) float bias_lds[2][kVtileCols];

  auto slot_ptr = [&](auto sc) -> uint8_t* {
    if constexpr (decltype(sc)::value == 0) return slot0;
    else if constexpr (decltype(sc)::value == 1) return slot1;
    else return slot2;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wv = wave & 1;
  const int wt = wave >> 1;
  const int lr = lane & 15;          // token column within a 16-token block
  const int lg = lane >> 4;          // lane group: vocabulary rows 4 lg .. 4 lg + 3

  // Block id -> (split run, row block); a bijection that only orders the
  // work.  A launch has up to two phases, longest work first: workgroups
  // [0, R * runsA) take runs of spg consecutive splits of [split0, splitA),
  // the rest single splits of [splitA, split1), so units that finish a long
  // run early pick up short pieces and the last round ends nearly level.
  // Within a phase, blocks go to the eight XCDs round-robin: first give each
  // XCD a contiguous run of tile indices, then order tiles in groups of
  // kRowBlockGroup row blocks x all split runs (row blocks fastest), so the
  // ~32 tiles an XCD runs at once share a few W slices and a few hidden
  // blocks in its L2.
  const int nA = p.R * p.runsA;
  const bool ph_b = (int)blockIdx.x >= nA;
  const int s_lo = ph_b ? p.splitA : p.split0;
  const int s_hi = ph_b ? p.split1 : p.splitA;
  const int spg = ph_b ? 1 : p.spg;
  const int sg = ph_b ? p.split1 - p.splitA : p.runsA;      // runs per row block
  const int nblk = p.R * sg;
  const int per_xcd = nblk >> 3;
  int u = ph_b ? (int)blockIdx.x - nA : (int)blockIdx.x;
  if (u < (per_xcd << 3)) u = (u & 7) * per_xcd + (u >> 3);
  const int in_group = kRowBlockGroup * sg;
  const int first_rb = (u / in_group) * kRowBlockGroup;
  const int group_rbs = min(p.R - first_rb, kRowBlockGroup);
  const int rb = first_rb + (u % in_group) % group_rbs;
  const int split_first = s_lo + (u % in_group) / group_rbs * spg;
  const int split_last = min(split_first + spg, s_hi);          // exclusive

  const int64_t m0 = (int64_t)rb * kRows;
  const int rows_here = (int)min((int64_t)kRows, p.N - m0);
  const int vt_begin = split_first * p.vps;
  const int nvt = min(split_last * p.vps, p.T) - vt_begin;
  const int H = p.H;
  // K stages per tile, padded to a multiple of the buffer count with stages
  // that read only zeros (they leave the accumulators unchanged), so every
  // tile starts in buffer 0 and ends in the last buffer.
  const int KT = ((H + kBK - 1) / kBK + kSlots - 1) / kSlots * kSlots;
  const int G = nvt * KT;                          // stages in this workgroup

  // ---- per-lane load descriptors ------------------------------------------
  // Waves 0..3 issue every direct-to-LDS load (kLoadsW for the W slice and
  // kLoadsH for the hidden slice per stage); waves 4..7 only compute.  On
  // each SIMD the issue arbiter favours the older of its two waves, so waves
  // 0..3 finish a stage's MFMAs first and would wait at its barrier: the loads
  // and their waits go there, off the critical waves.
  // Instruction j of loader wave w fills chunk slots [(kL w + j) * 64, +64) of
  // its slice (kL = loads per wave): rows r_j = (kL w + j) * 8 + lane / 8, 8
  // rows x 8 chunks of 16 bytes, i.e. eight whole 128-byte lines.  Chunk c of
  // row r sits at c ^ swz(r); swz(r + 16) = swz(r), so the chunk (and with it
  // the in-row byte offset) takes two values over j, one for even and one for
  // odd j: offset_j = base[j & 1] + (j & ~1) * 8 rows * 2H bytes.
  constexpr int kLoadsH = kRows * kLdsRowBytes / (kLoaderWaves * 64 * 16);   // 8 or 4
  const bool loader = wave < kLoaderWaves;
  uint32_t vb_w[2], vb_h[2];
  int kc_w[2], kc_h[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int rw = (wave * kLoadsW + e) * 8 + (lane >> 3);
    const int cw = (lane & 7) ^ swz(rw);
    vb_w[e] = (uint32_t)rw * (uint32_t)H * 2u + (uint32_t)cw * 16u;
    kc_w[e] = cw * 8;
    const int rh = (wave * kLoadsH + e) * 8 + (lane >> 3);
    const int ch = (lane & 7) ^ swz(rh);
    vb_h[e] = (uint32_t)rh * (uint32_t)H * 2u + (uint32_t)ch * 16u;
    kc_h[e] = ch * 8;
  }
  const __amdgpu_buffer_rsrc_t rsrc_h = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint16_t*)p.hidden + m0 * H), (short)0, rows_here * H * 2, kRsrcWord3);

  // ---- per-lane LDS read offsets for the MFMA operands ----------------------
  // A (W) fragment vi of K step u: row wv*128 + 16 vi + lr, K chunk 4 u + lg.
  // B (hidden) fragment tj: row wt*kWaveTok + 16 tj + lr, K chunk 4 u + lg.
  // The swizzle only reads row bits 1-3, which come from lr.
  const int fr = swz(lr);
  int a_off[2], b_off[2];
#pragma unroll
  for (int uu = 0; uu < 2; ++uu) {
    const int c = (4 * uu + lg) ^ fr;
    a_off[uu] = ((wv * 128 + lr) * kChunks + c) * 16;
    b_off[uu] = kTileBytes + ((wt * kWaveTok + lr) * kChunks + c) * 16;
  }

  // ---- targets of the block's tokens (visible after the prologue barrier) --
  if (tid < kRows) {
    const int64_t t = (tid < rows_here) ? p.target[m0 + tid] : (int64_t)-1;
    tgt_lds[tid] = (t >= 0 && t < p.V) ? (int)t : -1;     // V <= 2^30
    if constexpr (kGrad) {
      const bool live = tid < rows_here;
      const float gl = live ? p.g_logp[m0 + tid] : 0.f;
      grad_lds[0][tid] = live ? p.lse[m0 + tid] : 0.f;
      grad_lds[1][tid] = live ? p.g_lse[m0 + tid] - gl : 0.f;
      grad_lds[2][tid] = gl;
    }
  }

  // Direct-to-LDS loads of stage g into buffer SC, one instruction at a
  // time: load j of the W slice (0..kLoadsW-1) or of the hidden slice
  // (0..kLoadsH-1).  A stage past the end (g >= G) reads nothing (empty
  // range) and writes zeros into a buffer that is no longer read; no branch
  // on the stage, so the loads can sit between MFMAs.
  struct LoadCtx {
    __amdgpu_buffer_rsrc_t rsrc;
    uint8_t* dst;
    uint32_t k2;      // byte offset of the stage's K slice
    int kend;         // H, or 0 for a stage past the end
  };
  auto ctx_w = [&](int g, auto sc) {
    const int v = g / KT;
    const int kt = g - v * KT;
    const int vbase = (vt_begin + v) * kVtileCols;
    const int vrows = (g < G) ? min(kVtileCols, p.V - vbase) : 0;
    int dst = wave * kLoadsW * 1024;
    asm volatile("" : "+s"(dst));     // recomputed per stage: LDS addresses stay out of SGPRs
    LoadCtx c;
    c.rsrc = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const uint16_t*)p.weight + (int64_t)(g < G ? vbase : 0) * H), (short)0,
        vrows * H * 2, kRsrcWord3);
    c.dst = slot_ptr(sc) + dst;
    c.k2 = (uint32_t)(kt * kBK) * 2u;
    c.kend = H;
    return c;
  };
  auto ctx_h = [&](int g, auto sc) {
    const int v = g / KT;
    const int kt = g - v * KT;
    int dst = kTileBytes + wave * kLoadsH * 1024;
    asm volatile("" : "+s"(dst));
    LoadCtx c;
    c.rsrc = rsrc_h;
    c.dst = slot_ptr(sc) + dst;
    c.k2 = (uint32_t)(kt * kBK) * 2u;
    c.kend = (g < G) ? H : 0;
    return c;
  };
  // load j of the W slice (is_h false) or of the hidden slice (is_h true);
  // loader waves only
  auto load_one = [&](const LoadCtx& c, int j, auto is_h) {
    int kc;
    uint32_t vb;
    if constexpr (decltype(is_h)::value) {
      kc = kc_h[j & 1];
      vb = vb_h[j & 1];
    } else {
      kc = kc_w[j & 1];
      vb = vb_w[j & 1];
    }
    const bool ok = (int)(c.k2 / 2u) + kc < c.kend;
    const uint32_t voff = ok ? vb + (uint32_t)(j & ~1) * 16u * (uint32_t)H + c.k2 : kOutOfRange;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rsrc, (lds_void*)(c.dst + j * 1024), 16, voff, 0,
                                             0, 0);
  };

  // The pipeline below is instantiated twice, selected by one wave-uniform
  // branch: for the loader waves (with the direct loads and their waits) and
  // for the compute-only waves (without).
  auto run = [&](auto is_loader) {
    constexpr bool kLoader = decltype(is_loader)::value;
    auto ld = [&](const LoadCtx& c, int j, auto is_h) {
      if constexpr (kLoader) load_one(c, j, is_h);
    };

    // acc[vi][tj][i]: vocabulary row wv*128 + 16 vi + 4 lg + i of the tile,
    // token column wt*kWaveTok + 16 tj + lr.
    floatx4 acc[8][kTj];

    // The bias of tile v reaches LDS (bias_lds[v & 1]) by one direct load of
    // 1 KB (fp32) or 512 bytes (bf16, lanes 0-31) from wave 0, issued in the
    // epilogue of tile v - 1 once that tile's bias is consumed (tile 0: in the
    // prologue).  The descriptor covers the tile's columns below V; the host
    // takes this path only where V keeps every 16-byte chunk wholly inside
    // or wholly past it (chunks past V read as zero), else it passes a
    // zero-padded fp32 copy.  A stage barrier of tile v
    // makes it visible: the first one with two buffers (it waits for every
    // load); with three, where a barrier leaves the newest six loads in
    // flight, the first one after six more loads - one or two stages on, long
    // before the epilogue.  Nothing bias-related runs in the stage loop.
    // The descriptor is built per load from the kernel argument, so nothing
    // bias-related stays live in registers through the stage loop.
    auto load_bias = [&](int v) {
      if constexpr (kHasBias) {
        if (wave == 0 && v < nvt) {
          constexpr int kEsz = kBias == 2 ? 2 : 4;
          const int vb = (vt_begin + v) * kVtileCols;
          const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
              (void*)((const uint8_t*)p.bias + (int64_t)vb * kEsz), (short)0,
              min(kVtileCols, p.V - vb) * kEsz, kRsrcWord3);
          const uint32_t off =
              (kEsz == 4 || lane < 32) ? (uint32_t)lane * 16u : kOutOfRange;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)&bias_lds[v & 1][0], 16, off,
                                                   0, 0, 0);
        }
      }
    };
    auto init_acc = [&]() {
#pragma unroll
      for (int vi = 0; vi < 8; ++vi)
#pragma unroll
        for (int tj = 0; tj < kTj; ++tj) acc[vi][tj] = floatx4{};
    };

    // Operand registers.  ar: ring of A fragments, A[vi] of the current step in
    // ar[vi & 3]; bA / bB: B fragments of the even / odd K step of a stage.
    bf16x8 ar[4], bA[kTj], bB[kTj];

    auto rd_a = [&](const uint8_t* st, int uu, int vi) -> bf16x8 {
      return *(const bf16x8*)(st + a_off[uu] + vi * kFragStride);
    };
    auto rd_b = [&](const uint8_t* st, int uu, int tj) -> bf16x8 {
      return *(const bf16x8*)(st + b_off[uu] + tj * kFragStride);
    };

    // Position of each item inside a K step of kM MFMAs, fixed at compile time:
    //  - A[vi + 3] is read right after the first MFMA of vi (for vi + 3 >= 8:
    //    the next step's A[vi - 5], from the next step's buffer);
    //  - B of the next step, fragment t, after MFMA kTj * t + kTj / 2;
    //  - in a step without barrier, direct load j after MFMA kM / nl * (j + 1) - 1;
    //  - in the stage's last step, the barrier after MFMA kBarAt (the MFMA
    //    after the one that carries the read of A[7]); after it the next
    //    stage's reads and the W refill.
    constexpr int kBarAt = 4 * kTj + 1;
    auto kstep = [&](const uint8_t* st, int uu, const uint8_t* nst, int nu,
                     const bf16x8 (&bc)[kTj], bf16x8 (&bn)[kTj], const LoadCtx& lc,
                     auto is_h, auto nloads, auto last, auto sync) {
      constexpr bool kLast = decltype(last)::value;
      constexpr int kNl = decltype(nloads)::value;
#pragma unroll
      for (int i = 0; i < kM; ++i) {
        const int vi = i / kTj, tj = i % kTj;
        acc[vi][tj] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(ar[vi & 3], bc[tj], acc[vi][tj], 0, 0, 0);
        if (tj == 0) {
          if (vi + 3 < 8) ar[(vi + 3) & 3] = rd_a(st, uu, vi + 3);
        }
        if constexpr (!kLast) {
          if (tj == 0 && vi + 3 >= 8) ar[(vi + 3) & 3] = rd_a(nst, nu, vi + 3 - 8);
          if (tj == kTj / 2 && vi < kTj) bn[vi] = rd_b(nst, nu, vi);
          if constexpr (kNl > 0) {
            constexpr int stride = kM / (kNl > 0 ? kNl : 1);
            if (i % stride == stride - 1) ld(lc, i / stride, is_h);
          }
        } else {
          // stage end: the barrier after MFMA kBarAt; after it the next stage's
          // B fragments and first three A fragments, and the W refill of the
          // released buffer spread over the remaining MFMAs
          constexpr int kPost = kM - kBarAt - 1;
          if (i == kBarAt) sync();
          if (i > kBarAt) {
            const int q = i - kBarAt - 1;
            if (tj == 0 && vi + 3 >= 8) ar[(vi + 3) & 3] = rd_a(nst, nu, vi + 3 - 8);
            if (q < kTj) bn[q] = rd_b(nst, nu, q);
#pragma unroll
            for (int j = 0; j < kLoadsW; ++j)
              if (q == j * kPost / kLoadsW) ld(lc, j, std::false_type{});
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // Wait for this wave's loads of the next stage (the only ones in flight)
    // and for its LDS reads, then barrier: afterwards every wave's next-stage
    // data is in LDS and nobody reads the current buffer any more.  The barrier
    // is a bare s_barrier (the compiler-level memory clobber keeps LDS accesses
    // on their side of it); a C++ workgroup fence would also wait for stores.
    auto sync_stage = [&]() {
      if constexpr (kLoader) wait_vmcnt<0>();
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    // Three buffers: at stage g's barrier the loads still allowed in flight are
    // the W and hidden slices of stage g + 2, issued after everything stage
    // g + 1 needs (the load counter completes in order).
    auto sync_stage3 = [&]() {
      if constexpr (kLoader) wait_vmcnt<kLoadsW + kLoadsH>();
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };

    // Stage g from buffer SC; SN holds stage g + 1.  Two buffers: the hidden
    // slice of stage g + 1 goes into SN under the first step, the W slice of
    // stage g + 2 into SC after the barrier.  Three buffers: SP (free since the
    // previous stage's barrier) receives the hidden slice of stage g + 2 under
    // the first step, and SC the W slice of stage g + 3 after the barrier.
    auto stage = [&](int g, auto sc, auto sn, auto sp) {
      const uint8_t* st = slot_ptr(sc);
      if constexpr (kSlots == 2) {
        const LoadCtx lh = ctx_h(g + 1, sn);
        kstep(st, 0, st, 1, bA, bB, lh, std::true_type{}, std::integral_constant<int, kLoadsH>{},
              std::false_type{}, sync_stage);
        const LoadCtx lw = ctx_w(g + 2, sc);
        kstep(st, 1, slot_ptr(sn), 0, bB, bA, lw, std::false_type{},
              std::integral_constant<int, 0>{}, std::true_type{}, sync_stage);
      } else {
        const LoadCtx lh = ctx_h(g + 2, sp);
        kstep(st, 0, st, 1, bA, bB, lh, std::true_type{}, std::integral_constant<int, kLoadsH>{},
              std::false_type{}, sync_stage3);
        const LoadCtx lw = ctx_w(g + 3, sc);
        kstep(st, 1, slot_ptr(sn), 0, bB, bA, lw, std::false_type{},
              std::integral_constant<int, 0>{}, std::true_type{}, sync_stage3);
      }
    };

    float m_run[kTj], s_run[kTj];
#pragma unroll
    for (int tj = 0; tj < kTj; ++tj) {
      m_run[tj] = -INFINITY;
      s_run[tj] = 0.f;
    }

    // A split ends (its last tile is folded into m_run / s_run): merge the four
    // lane groups (lane groups g and g ^ 1, then g and g ^ 2; the lower group
    // is the lower vocabulary rows), then the two vocabulary-half waves
    // (through LDS), write the split's partial and restart the running state.
    // The barrier waits for LDS only: the next stages' loads stay in flight.
    // `red` is free again by the next flush, at least one stage barrier later.
    auto flush = [&](int split) {
      float mm[kTj], ss[kTj];
#pragma unroll
      for (int tj = 0; tj < kTj; ++tj) {
        float m = m_run[tj], s = s_run[tj];
#pragma unroll
        for (int d = 16; d <= 32; d <<= 1) {
          const float om = __shfl_xor(m, d);
          const float os = __shfl_xor(s, d);
          if ((lane & d) == 0)
            merge_state(m, s, om, os, m, s);
          else
            merge_state(om, os, m, s, m, s);
        }
        mm[tj] = m;
        ss[tj] = s;
      }
      if (wv == 1 && lg == 0) {
#pragma unroll
        for (int tj = 0; tj < kTj; ++tj)
          red[wt * kWaveTok + tj * 16 + lr] = make_float2(mm[tj], ss[tj]);
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (wv == 0 && lg == 0) {
#pragma unroll
        for (int tj = 0; tj < kTj; ++tj) {
          const int j = wt * kWaveTok + tj * 16 + lr;
          const float2 hi = red[j];
          float m, s;
          merge_state(mm[tj], ss[tj], hi.x, hi.y, m, s);
          if (j < rows_here) p.part[(m0 + j) * p.S + split] = make_float2(m, s);
        }
      }
#pragma unroll
      for (int tj = 0; tj < kTj; ++tj) {
        m_run[tj] = -INFINITY;
        s_run[tj] = 0.f;
      }
    };

    // Prologue: stage 0 whole and the W slice of stage 1 (its hidden slice is
    // issued in stage 0); with three buffers also the hidden slice of stage 1
    // and the W slice of stage 2.
    {
      const LoadCtx w0 = ctx_w(0, Slot<0>{}), h0 = ctx_h(0, Slot<0>{}), w1 = ctx_w(1, Slot<1>{});
#pragma unroll
      for (int j = 0; j < kLoadsW; ++j) ld(w0, j, std::false_type{});
#pragma unroll
      for (int j = 0; j < kLoadsH; ++j) ld(h0, j, std::true_type{});
#pragma unroll
      for (int j = 0; j < kLoadsW; ++j) ld(w1, j, std::false_type{});
      if constexpr (kSlots == 3) {
        const LoadCtx h1 = ctx_h(1, Slot<1>{}), w2 = ctx_w(2, Slot<2>{});
#pragma unroll
        for (int j = 0; j < kLoadsH; ++j) ld(h1, j, std::true_type{});
#pragma unroll
        for (int j = 0; j < kLoadsW; ++j) ld(w2, j, std::false_type{});
      }
      load_bias(0);
    }
    // Stage 0 has landed once only the loads issued after it (the next
    // stage's W slice, with three buffers also the hidden slice and W slice
    // after it, and wave 0's bias) are outstanding: the counter completes in
    // order.  Those are waited for at stage 0's own barrier.
    if constexpr (kLoader) wait_vmcnt<kSlots == 2 ? kLoadsW : 2 * kLoadsW + kLoadsH>();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    init_acc();
#pragma unroll
    for (int vi = 0; vi < 3; ++vi) ar[vi] = rd_a(slot0, 0, vi);
#pragma unroll
    for (int tj = 0; tj < kTj; ++tj) bA[tj] = rd_b(slot0, 0, tj);

    // G is a multiple of kSlots: stage g lives in buffer g % kSlots.
    for (int g = 0; g < G; g += kSlots) {
      if constexpr (kSlots == 2) {
        stage(g, Slot<0>{}, Slot<1>{}, Slot<0>{});
        stage(g + 1, Slot<1>{}, Slot<0>{}, Slot<1>{});
      } else {
        stage(g, Slot<0>{}, Slot<1>{}, Slot<2>{});
        stage(g + 1, Slot<1>{}, Slot<2>{}, Slot<0>{});
        stage(g + 2, Slot<2>{}, Slot<0>{}, Slot<1>{});
      }

      const int v = g / KT;
      if (g + kSlots != (v + 1) * KT) continue;

      // ---- epilogue of vocabulary tile v -------------------------------------
      const int vbase = (vt_begin + v) * kVtileCols;
      const int vw = vbase + wv * 128;               // first column of this wave
      if constexpr (kHasBias) {
        // z = (the K accumulation) + bias: one fp32 add per logit
        __builtin_amdgcn_sched_barrier(0);
        const int bcol = wv * 128 + 4 * lg;         // + 16 vi: this lane's four columns
#pragma unroll
        for (int vi = 0; vi < 8; ++vi) {
          floatx4 bb;
          if constexpr (kBias == 2) {
            // four bf16 values; bf16 -> fp32 is the bits shifted up 16 (exact)
            const uint2 raw =
                *(const uint2*)((const uint16_t*)&bias_lds[v & 1][0] + bcol + vi * 16);
            bb = floatx4{__uint_as_float(raw.x << 16), __uint_as_float(raw.x & 0xffff0000u),
                         __uint_as_float(raw.y << 16), __uint_as_float(raw.y & 0xffff0000u)};
          } else {
            bb = *(const floatx4*)(&bias_lds[v & 1][bcol + vi * 16]);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int tj = 0; tj < kTj; ++tj) acc[vi][tj][e] += bb[e];
          // in place: without these the compiler gives the sums new registers
          // and spills values that live through the stage loop
#pragma unroll
          for (int tj = 0; tj < kTj; ++tj) asm volatile("" : "+v"(acc[vi][tj]));
          __builtin_amdgcn_sched_barrier(0);        // a few bias values live at a time
        }
        load_bias(v + 1);          // lands during the next tile's first stage
      }
      if constexpr (kGrad) {
        // dZ^T[col][row] = p (g_lse - g_logp) + g_logp [col == target], p =
        // exp(z - lse), rounded to bf16.  One store per (vi, e, tj): each
        // lane group writes 16 consecutive tokens of one vocabulary row, and
        // the kTj stores of an (vi, e) complete the wave's 64 tokens (a whole
        // 128-byte line) of each of its four rows back to back.  The buffer
        // covers the tile's columns below V, so stores past V are dropped.
        const int vrows = min(kVtileCols, p.V - vbase);
        const __amdgpu_buffer_rsrc_t rs_dz = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(p.dzt + (int64_t)vbase * p.ldz), (short)0, vrows * (int)p.ldz * 2,
            kRsrcWord3);
        uint32_t vo[kTj];
        int trel[kTj];
        float lse_r[kTj], coef[kTj], gtg[kTj];
#pragma unroll
        for (int tj = 0; tj < kTj; ++tj) {
          const int jr = wt * kWaveTok + tj * 16 + lr;
          // a token past the batch stores past the resource's end, where the
          // range check drops it: no branch around the stores (kOutOfRange +
          // 127 rows of at most 2^22 bytes stays below 2^32)
          vo[tj] = jr < rows_here
                       ? ((uint32_t)(wv * 128 + 4 * lg) * (uint32_t)p.ldz + (uint32_t)(m0 + jr)) * 2u
                       : kOutOfRange;
          // opaque per tile: the store addresses are formed here, not hoisted
          // out of the stage loop into registers that would then spill
          asm volatile("" : "+v"(vo[tj]));
          trel[tj] = tgt_lds[jr] - vw - 4 * lg;
          lse_r[tj] = grad_lds[0][jr];
          coef[tj] = grad_lds[1][jr];
          gtg[tj] = grad_lds[2][jr];
        }
        uint32_t ld2 = (uint32_t)p.ldz * 2u;
        asm volatile("" : "+s"(ld2));
#pragma unroll
        for (int vi = 0; vi < 8; ++vi) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int k = vi * 16 + e;                // column - vw - 4 lg
#pragma unroll
            for (int tj = 0; tj < kTj; ++tj) {
              float dz = exp2_hw((acc[vi][tj][e] - lse_r[tj]) * kLog2e) * coef[tj];
              if (trel[tj] == k) dz += gtg[tj];
              __builtin_amdgcn_raw_buffer_store_b16(bf16_rne(dz), rs_dz,
                                                    vo[tj] + (uint32_t)k * ld2, 0, 0);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        init_acc();
        continue;
      }
      if (vbase + kVtileCols > p.V) {                // vocabulary tail: mask columns >= V
#pragma unroll
        for (int vi = 0; vi < 8; ++vi)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int col = vw + vi * 16 + 4 * lg + e;
            if (col >= p.V) {
#pragma unroll
              for (int tj = 0; tj < kTj; ++tj) acc[vi][tj][e] = -INFINITY;
            }
          }
      }

#pragma unroll
      for (int tj = 0; tj < kTj; ++tj) {
        // target capture: exactly one (tile, lane, register) in the grid holds it
        const int rel = tgt_lds[wt * kWaveTok + tj * 16 + lr] - vw;
        const bool hit = rel >= 0 && rel < 128 && ((rel >> 2) & 3) == lg;
        if (__any(hit)) {
          const int vi_t = rel >> 4;
          const int e_t = rel & 3;
          float val = 0.f;
#pragma unroll
          for (int vi = 0; vi < 8; ++vi)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (vi == vi_t && e == e_t) val = acc[vi][tj][e];
          if (hit) p.tlogit[m0 + wt * kWaveTok + tj * 16 + lr] = val;
        }

        // online softmax over this lane's 32 values of the tile
        float mx = acc[0][tj][0];
#pragma unroll
        for (int vi = 0; vi < 8; ++vi)
#pragma unroll
          for (int e = 0; e < 4; ++e) mx = fmaxf(mx, acc[vi][tj][e]);
        const float m_new = fmaxf(m_run[tj], mx);
        const float mu = (m_new == -INFINITY) ? 0.f : m_new;
        float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int vi = 0; vi < 8; ++vi)
#pragma unroll
          for (int e = 0; e < 4; ++e) ps[e] += exp2_hw((acc[vi][tj][e] - mu) * kLog2e);
        const float tile_sum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
        s_run[tj] = s_run[tj] * exp2_hw((m_run[tj] - mu) * kLog2e) + tile_sum;
        m_run[tj] = m_new;
      }
      __builtin_amdgcn_sched_barrier(0);      // the tile is consumed before the next one starts
      const int vt = vt_begin + v;
      if (v + 1 == nvt || (vt + 1) % p.vps == 0) flush(vt / p.vps);
      __builtin_amdgcn_sched_barrier(0);
      init_acc();
    }
    // The last stages issued loads past the end (into buffers nobody
    // reads); let them land before the workgroup's LDS is released.
    if constexpr (kLoader) wait_vmcnt<0>();
  };
  if (loader)
    run(std::true_type{});
  else
    run(std::false_type{});
}

__global__ __launch_bounds__(kThreads, 1) void proj_lse_kernel(const ProjParams p) {
  proj_fwd_body<0, false, 4, 2>(p);
}
__global__ __launch_bounds__(kThreads, 1) void proj_lse_bias_kernel(const ProjParams p) {
  proj_fwd_body<1, false, 4, 2>(p);
}
__global__ __launch_bounds__(kThreads, 1) void proj_lse_bias16_kernel(const ProjParams p) {
  proj_fwd_body<2, false, 4, 2>(p);
}
__global__ __launch_bounds__(kThreads, 1) void softmax_grad_kernel(const ProjParams p) {
  proj_fwd_body<0, true, 4, 2>(p);
}
__global__ __launch_bounds__(kThreads, 1) void softmax_grad_bias_kernel(const ProjParams p) {
  proj_fwd_body<1, true, 4, 2>(p);
}
__global__ __launch_bounds__(kThreads, 1) void softmax_grad_bias16_kernel(const ProjParams p) {
  proj_fwd_body<2, true, 4, 2>(p);
}
// 128-token row blocks: twice the workgroups for batches that 256-token
// blocks cannot spread over every compute unit; the same bits
__global__ __launch_bounds__(kThreads, 1) void proj_lse_r128_kernel(const ProjParams p) {
  proj_fwd_body<0, false, 2, 3>(p);
}
__global__ __launch_bounds__(kThreads, 1) void proj_lse_bias_r128_kernel(const ProjParams p) {
  proj_fwd_body<1, false, 2, 3>(p);
}
__global__ __launch_bounds__(kThreads, 1) void proj_lse_bias16_r128_kernel(const ProjParams p) {
  proj_fwd_body<2, false, 2, 3>(p);
}
__global__ __launch_bounds__(kThreads, 1) void softmax_grad_r128_kernel(const ProjParams p) {
  proj_fwd_body<0, true, 2, 3>(p);
}
__global__ __launch_bounds__(kThreads, 1) void softmax_grad_bias_r128_kernel(const ProjParams p) {
  proj_fwd_body<1, true, 2, 3>(p);
}
__global__ __launch_bounds__(kThreads, 1) void softmax_grad_bias16_r128_kernel(const ProjParams p) {
  proj_fwd_body<2, true, 2, 3>(p);
}

}  // namespace

hipError_t launch_softmax_grad(const ProjParams& p, hipStream_t stream) {
  const int64_t blocks = (int64_t)p.R * (p.runsA + p.split1 - p.splitA);
  if (blocks <= 0) return hipSuccess;
  auto k = p.rows == 128 ? (p.bias_src == kBiasSrcBf16  ? softmax_grad_bias16_r128_kernel
                           : p.bias_src == kBiasSrcF32 ? softmax_grad_bias_r128_kernel
                                                       : softmax_grad_r128_kernel)
                         : (p.bias_src == kBiasSrcBf16  ? softmax_grad_bias16_kernel
                           : p.bias_src == kBiasSrcF32 ? softmax_grad_bias_kernel
                                                       : softmax_grad_kernel);
  hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_proj_lse(const ProjParams& p, hipStream_t stream) {
  const int64_t blocks = (int64_t)p.R * (p.runsA + p.split1 - p.splitA);
  if (blocks <= 0) return hipSuccess;
  auto k = p.rows == 128 ? (p.bias_src == kBiasSrcBf16  ? proj_lse_bias16_r128_kernel
                           : p.bias_src == kBiasSrcF32 ? proj_lse_bias_r128_kernel
                                                       : proj_lse_r128_kernel)
                         : (p.bias_src == kBiasSrcBf16  ? proj_lse_bias16_kernel
                           : p.bias_src == kBiasSrcF32 ? proj_lse_bias_kernel
                                                       : proj_lse_kernel);
  hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace bilogp
