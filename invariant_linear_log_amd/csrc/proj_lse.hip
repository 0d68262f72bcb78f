// Fused projection + per-split online softmax for gfx950 (CDNA4).
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
// v_mfma_f32_32x32x16_bf16, W as the A operand (MFMA rows = vocabulary) and
// hidden as the B operand (MFMA columns = tokens).  In that orientation each
// lane's accumulators hold ONE token column and 64 vocabulary rows, so the
// per-token max / sum-exp over a tile is mostly a sequential, lane-local loop
// whose order is fixed by the tile geometry alone.
//
// Waves: w = 2 * wt + wv.  wv in {0, 1} picks vocabulary rows [128 wv, +128)
// of the tile, wt in {0..3} picks tokens [64 wt, +64) of the block.  A wave
// holds 4 x 2 MFMA tiles of 32 x 32 (128 accumulator registers per lane).
// A second instantiation takes 128-token row blocks (tokens [32 wt, +32), 4 x
// 1 MFMA tiles per wave) for batches too small to give every compute unit a
// 256-token block; the vocabulary side, and with it each token's arithmetic,
// is the same in both.
//
// Bit contract.  For a fixed (token, vocabulary column) the K reduction is
// the same chain of MFMA instructions over ascending 16-wide K steps
// whatever N or the token's slot in the block; the per-token reductions over
// vocabulary columns follow the (lane, register) layout of the tile, which
// is the same for every token column; the cross-lane and cross-wave merges
// use fixed operand order.  Nothing depends on N, the row block or the
// number of compute units.
//
// Memory pipeline.  K is staged in 64-wide slices through two LDS buffers
// (64 KB each: a 256 x 64 W slice and a 256 x 64 hidden slice), filled with
// buffer loads that write LDS directly (no VGPR round trip) one stage ahead
// of the MFMAs.  A 64-wide slice is one full 128-byte line of every W and
// hidden row: with row strides of a few KB (H = 4096 gives 8 KB) gfx950's
// L2 serves whole lines several times faster than the two half lines a
// 32-wide slice would need.  Out-of-range rows (the vocabulary tail, the last
// row block) and K chunks past H read as zero through the buffer
// descriptors' range check.
//
// Instruction schedule of a stage (four 16-wide K steps u = 0..3): the
// operand fragments of step u + 1 are read from LDS while the MFMAs of step
// u run (two fragment sets in registers), so LDS latency - which grows while
// the direct loads are writing LDS - stays off the MFMA path.  The stage's
// barrier sits inside step 3, after its first MFMAs (with 256-token blocks
// two; their operands are already in registers, so the matrix core keeps
// working while the wave waits): once every wave has read step 3's operands
// and its loads of the next stage have landed, the buffer is released and
// refilled with stage g + 2 - the W slice under the rest of step 3, the
// hidden slice under the MFMAs of step 0 of stage g + 1.  Each of these steps
// is emitted in a fixed order (MFMA, LDS read, and a direct load after every
// second MFMA): the texture-address unit takes one 1 KB load about every 16
// cycles, so a wave that issued its loads in one burst would sit at the load
// instruction, with its MFMAs queued behind it, until the unit drained.
// Interleaved, the loads drain while the matrix cores work.
//
// Bias.  Each logit is the fp32 K accumulation (started at 0) plus its bias
// value, added once in the tile epilogue (fp32, from the padded copy the host
// library prepares, staged through LDS one tile ahead).
//
// LDS layout.  Each 256 x 64 slice is 256 rows of eight 16-byte chunks,
// chunk c of row r stored at position c ^ f(r), f(r) = (r >> 1) & 7.
// gfx950 serves a 16-byte-per-lane LDS read in four passes of 16 lanes over
// 64 four-byte banks; within each half-wave the two passes take the lane
// quads of even and of odd parity (quads {0,3,5,6} and {1,2,4,7}).  An MFMA
// operand read (32 rows, one chunk per half-wave) then gives the 16 lanes of
// a pass 16 distinct (row parity, chunk position) pairs: no bank conflicts.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "bilogp_internal.h"

namespace bilogp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kThreads = 512;
constexpr int kBK = 64;                            // K per stage
constexpr int kChunks = kBK / 8;                   // 16-byte chunks per slice row
constexpr int kLdsRowBytes = kBK * 2;              // 128 B per slice row
constexpr int kTileBytes = kVtileCols * kLdsRowBytes;         // 32 KB: one operand slice
constexpr int kSlotBytes = 2 * kTileBytes;                    // W, hidden
constexpr int kLoadsPerOperand = kTileBytes / (kThreads * 16);  // 4 per wave and stage
constexpr int kRowBlockGroup = 4;                  // row blocks per tile-order group
constexpr uint32_t kOutOfRange = 0x7ffffff0u;      // any offset past num_records
constexpr int kRsrcWord3 = 0x00020000;             // gfx9 raw buffer, 32-bit data
constexpr float kLog2e = 1.4426950408889634f;

static_assert(kBlockRows == 256 && kVtileCols == 256, "tile geometry is fixed");
static_assert(kLoadsPerOperand == 4, "load mapping assumes 4 instructions per operand");

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

// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// The kernel body, instantiated with and without bias, and (kGrad) as the
// softmax-gradient pass of the backward: the same tiles and the same
// accumulation, with an epilogue that writes dZ instead of reducing it.
template <bool kHasBias, bool kGrad, int kTi, int kSlots = 2>
__device__ __forceinline__ void proj_lse_body(const ProjParams& p) {
  static_assert(kTi == 1 || kTi == 2, "one or two 32-token columns per wave");
  static_assert(kSlots == 2 || (kSlots == 3 && kTi == 1), "three buffers fit 128-token blocks");
  constexpr int kRows = 128 * kTi;                 // tokens per row block
  constexpr int kWaveTok = 32 * kTi;               // tokens per wave
  constexpr int kLoadsH = kRows * kLdsRowBytes / (kThreads * 16);   // hidden loads per stage
  // Two LDS buffers, each its own variable, so the compiler can tell a read
  // of one from a direct-to-LDS load into the other and does not drain the
  // load pipeline before every read.  Buffer layout: W slice (32 KB), hidden
  // slice (32 KB).
  // With three buffers (128-token blocks only) each holds the 32 KB W slice
  // and the 16 KB hidden slice: 144 KB in all.
  constexpr int kBuf = kSlots == 2 ? kSlotBytes : kTileBytes + kRows * kLdsRowBytes;
  __shared__ __attribute__((aligned(1024))) uint8_t slot0[kBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t slot1[kBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t slot2[kSlots == 3 ? kBuf : 16];
  __shared__ float2 red[kBlockRows];
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
  const int half = lane >> 5;

  // Block id -> (split run, row block); a bijection that only orders the
  // work.  Blocks go to the eight XCDs round-robin: first give each XCD a
  // contiguous run of tile indices, then order tiles in groups of
  // kRowBlockGroup row blocks x all split runs (row blocks fastest), so the
  // ~32 tiles an XCD runs at once share a few W slices and a few hidden
  // blocks in its L2.
  const int nblk = p.R * p.S_grid;
  const int per_xcd = nblk >> 3;
  int u = blockIdx.x;
  if (u < (per_xcd << 3)) u = (u & 7) * per_xcd + (u >> 3);
  const int in_group = kRowBlockGroup * p.S_grid;
  const int first_rb = (u / in_group) * kRowBlockGroup;
  const int group_rbs = min(p.R - first_rb, kRowBlockGroup);
  const int rb = first_rb + (u % in_group) % group_rbs;
  const int split_first = p.split0 + (u % in_group) / group_rbs * p.spg;
  const int split_last = min(split_first + p.spg, p.split1);     // exclusive

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

  // ---- per-lane load descriptors: 4 + kLoadsH direct-to-LDS loads per stage --
  // Instruction j of wave `wave` fills chunk slots [(4 wave + j) * 64, +64) of
  // the W slice (and [(kLoadsH wave + j) * 64, +64) of the hidden slice): 8
  // rows x 8 chunks of 16 bytes, i.e. eight whole 128-byte lines.
  uint32_t voff_base[kLoadsPerOperand];
  int kchunk[kLoadsPerOperand];
#pragma unroll
  for (int j = 0; j < kLoadsPerOperand; ++j) {
    const int r = (wave * kLoadsPerOperand + j) * 8 + (lane >> 3);
    const int cc = (lane & 7) ^ swz(r);
    voff_base[j] = (uint32_t)r * (uint32_t)H * 2u + (uint32_t)cc * 16u;
    kchunk[j] = cc * 8;
  }
  // the hidden slice has kRows rows: kLoadsH instructions per wave
  uint32_t voff_h[kLoadsH];
  int kchunk_h[kLoadsH];
#pragma unroll
  for (int j = 0; j < kLoadsH; ++j) {
    const int r = (wave * kLoadsH + j) * 8 + (lane >> 3);
    const int cc = (lane & 7) ^ swz(r);
    voff_h[j] = (uint32_t)r * (uint32_t)H * 2u + (uint32_t)cc * 16u;
    kchunk_h[j] = cc * 8;
  }
  const __amdgpu_buffer_rsrc_t rsrc_h = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const uint16_t*)p.hidden + m0 * H), (short)0, rows_here * H * 2, kRsrcWord3);

  // ---- per-lane LDS read offsets for the MFMA operands ----------------------
  // A (W): row wv*128 + vi*32 + (lane & 31), K chunk 2u + half; vi adds 4 KB.
  // B (hidden): row wt*kWaveTok + ti*32 + (lane & 31); ti adds 4 KB.  The swizzle
  // only reads row bits 1-3, which come from the lane.
  const int fr = swz(lane & 31);
  int a_off[4], b_off[4];
#pragma unroll
  for (int uu = 0; uu < 4; ++uu) {
    const int c = (2 * uu + half) ^ fr;
    a_off[uu] = ((wv * 128 + (lane & 31)) * kChunks + c) * 16;
    b_off[uu] = kTileBytes + ((wt * kWaveTok + (lane & 31)) * kChunks + c) * 16;
  }

  // ---- targets of this lane's token columns (kTi of them) -------------------
  int tgt[kTi];          // the target, or -1 when outside [0, V) (V <= 2^30)
#pragma unroll
  for (int ti = 0; ti < kTi; ++ti) {
    const int j = wt * kWaveTok + ti * 32 + (lane & 31);
    const int64_t t = (j < rows_here) ? p.target[m0 + j] : (int64_t)-1;
    tgt[ti] = (t >= 0 && t < p.V) ? (int)t : -1;
  }
  // backward: the forward's lse and the coefficients of
  // dZ = p (g_lse - g_logp) + g_logp [v == target] for the lane's rows
  float g_lse_row[kTi] = {}, g_coef[kTi] = {}, g_tgt[kTi] = {};
  if constexpr (kGrad) {
#pragma unroll
    for (int ti = 0; ti < kTi; ++ti) {
      const int j = wt * kWaveTok + ti * 32 + (lane & 31);
      if (j < rows_here) {
        const float gl = p.g_logp[m0 + j];
        g_lse_row[ti] = p.lse[m0 + j];
        g_coef[ti] = p.g_lse[m0 + j] - gl;
        g_tgt[ti] = gl;
      }
    }
  }

  // Direct-to-LDS loads of stage g into buffer SC, one instruction at a
  // time: load j of the W slice (0..3) or of the hidden slice (0..kLoadsH-1).  A stage past
  // the end (g >= G) reads nothing (empty range) and writes zeros into a
  // buffer that is no longer read; no branch, so the loads can sit between
  // MFMAs.
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
    int dst = wave * kLoadsPerOperand * 1024;
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
  // load j of the W slice (is_h false) or of the hidden slice (is_h true)
  auto load_one = [&](const LoadCtx& c, int j, auto is_h) {
    int kc;
    uint32_t vb;
    if constexpr (decltype(is_h)::value) {
      kc = kchunk_h[j];
      vb = voff_h[j];
    } else {
      kc = kchunk[j];
      vb = voff_base[j];
    }
    const bool ok = (int)(c.k2 / 2u) + kc < c.kend;
    const uint32_t voff = ok ? vb + c.k2 : kOutOfRange;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rsrc, (lds_void*)(c.dst + j * 1024), 16, voff, 0,
                                             0, 0);
  };

  // acc[vi][ti][r] belongs to vocabulary row wv*128 + vi*32 + 8*(r/4) +
  // 4*half + (r%4) of the tile (for every token column ti).
  floatx16 acc[4][kTi];

  // The bias of tile v reaches LDS (bias_lds[v & 1]) by one direct load of
  // 1 KB from wave 0, issued in the epilogue of tile v - 1 once that tile's
  // bias is consumed (tile 0: in the prologue).  A stage barrier of tile v
  // makes it visible: the first one with two buffers (it waits for every
  // load); with three, where a barrier leaves the newest six loads in
  // flight, the first one after six more loads - one or two stages on, long
  // before the epilogue.  The epilogue of tile v reads it from there: nothing
  // bias-related runs in the stage loop, and no global load whose wait would
  // also wait for the next stages' prefetch (the load counter is in order).
  const __amdgpu_buffer_rsrc_t rsrc_b = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const float*)p.bias + (int64_t)vt_begin * kVtileCols), (short)0,
      kHasBias ? nvt * kVtileCols * 4 : 0, kRsrcWord3);     // unused without bias
  auto load_bias = [&](int v) {
    if constexpr (kHasBias) {
      if (wave == 0 && v < nvt)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_b, (lds_void*)&bias_lds[v & 1][0], 16,
                                                 (uint32_t)v * 1024u + (uint32_t)lane * 16u, 0, 0,
                                                 0);
    }
  };
  // Every tile's accumulators start at 0.
  auto init_acc = [&](int) {
#pragma unroll
    for (int vi = 0; vi < 4; ++vi)
#pragma unroll
      for (int ti = 0; ti < kTi; ++ti) acc[vi][ti] = floatx16{};
  };

  // One K step in a fixed instruction order: MFMA i (tile (i/kTi, i%kTi)) is
  // followed by the next step's LDS reads (two columns: one read after each
  // of the first six MFMAs; one column: b0 and a0 after the first, then one)
  // and, when a load context is given, by its direct loads spread evenly over
  // the step.  The fences keep the compiler from regrouping: reads must not
  // bunch up behind their uses, and loads issued in a burst would stall the
  // wave (the texture-address unit takes one 1 KB load about every 16 cycles)
  // and with it the MFMAs behind them.
  auto step = [&](const bf16x8 (&a)[4], const bf16x8 (&b)[kTi], const uint8_t* nst, int nuu,
                  bf16x8 (&na)[4], bf16x8 (&nb)[kTi], const LoadCtx& lc, auto with_loads,
                  auto is_h) {
#pragma unroll
    for (int i = 0; i < 4 * kTi; ++i) {
      const int vi = i / kTi, ti = i % kTi;
      acc[vi][ti] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[vi], b[ti], acc[vi][ti], 0, 0, 0);
      if constexpr (kTi == 2) {
        // next-step fragments in the order the MFMAs need them: b0 a0 b1 a1 a2 a3
        if (i == 0) nb[0] = *(const bf16x8*)(nst + b_off[nuu]);
        if (i == 1) na[0] = *(const bf16x8*)(nst + a_off[nuu]);
        if (i == 2) nb[1] = *(const bf16x8*)(nst + b_off[nuu] + 32 * kLdsRowBytes);
        if (i >= 3 && i < 6)
          na[i - 2] = *(const bf16x8*)(nst + a_off[nuu] + (i - 2) * 32 * kLdsRowBytes);
      } else {
        if (i == 0) nb[0] = *(const bf16x8*)(nst + b_off[nuu]);
        na[i] = *(const bf16x8*)(nst + a_off[nuu] + i * 32 * kLdsRowBytes);
      }
      if constexpr (decltype(with_loads)::value) {
        constexpr int nl = decltype(is_h)::value ? kLoadsH : kLoadsPerOperand;
        constexpr int stride = 4 * kTi / nl;
        if (i % stride == stride - 1) load_one(lc, i / stride, is_h);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // The last K step of a stage (two token columns per wave) with the stage
  // barrier inside it: the first kPreBarrier MFMAs use fragments already in
  // registers and keep the matrix core busy while the wave waits for the
  // others; after the barrier the remaining six MFMAs each carry one read of
  // the next stage's step-0 fragments (b0 a0 b1 a1 a2 a3), and the W slice of
  // stage g + 2 is loaded into the released buffer after MFMAs 3, 4, 6 and 7.
  // (Two MFMAs ahead of the barrier timed best on MI355X: 3.11 ms at the
  // headline shape against 3.20 ms with one and 3.14 / 3.18 ms with three or
  // four.)
  auto step_bar = [&](const bf16x8 (&a)[4], const bf16x8 (&b)[kTi], const uint8_t* nst,
                      bf16x8 (&na)[4], bf16x8 (&nb)[kTi], const LoadCtx& lc, auto sync) {
    static_assert(kTi == 2, "two token columns per wave");
    constexpr int kPreBarrier = 2;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int vi = i / 2, ti = i % 2;
      acc[vi][ti] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[vi], b[ti], acc[vi][ti], 0, 0, 0);
      if (i == kPreBarrier - 1) sync();
      if (i == 2) nb[0] = *(const bf16x8*)(nst + b_off[0]);
      if (i == 3) na[0] = *(const bf16x8*)(nst + a_off[0]);
      if (i == 4) nb[kTi - 1] = *(const bf16x8*)(nst + b_off[0] + 32 * kLdsRowBytes);
      if (i >= 5) na[i - 4] = *(const bf16x8*)(nst + a_off[0] + (i - 4) * 32 * kLdsRowBytes);
      if (i == 3) load_one(lc, 0, std::false_type{});
      if (i == 4) load_one(lc, 1, std::false_type{});
      if (i == 6) load_one(lc, 2, std::false_type{});
      if (i == 7) load_one(lc, 3, std::false_type{});
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto read_frags = [&](const uint8_t* st, int uu, bf16x8 (&a)[4], bf16x8 (&b)[kTi]) {
    b[0] = *(const bf16x8*)(st + b_off[uu]);
    a[0] = *(const bf16x8*)(st + a_off[uu]);
    if constexpr (kTi == 2) b[1] = *(const bf16x8*)(st + b_off[uu] + 32 * kLdsRowBytes);
#pragma unroll
    for (int vi = 1; vi < 4; ++vi)
      a[vi] = *(const bf16x8*)(st + a_off[uu] + vi * 32 * kLdsRowBytes);
  };

  // Wait for this wave's loads of the next stage (the only ones in flight)
  // and for its LDS reads, then barrier: afterwards every wave's next-stage
  // data is in LDS and nobody reads the current buffer any more.  The barrier
  // is a bare s_barrier (the compiler-level memory clobber keeps LDS accesses
  // on their side of it); a C++ workgroup fence would also wait for stores.
  auto sync_stage = [&]() {
    wait_vmcnt<0>();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  // Three buffers: at stage g's barrier the loads still allowed in flight are
  // the W and hidden slices of stage g + 2, issued after everything stage
  // g + 1 needs (the load counter completes in order).
  auto sync_stage3 = [&]() {
    wait_vmcnt<kLoadsPerOperand + kLoadsH>();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };

  bf16x8 fa0[4], fb0[kTi], fa1[4], fb1[kTi];

  // Stage g, computed from buffer SC; buffer SN holds stage g + 1.  On entry
  // fa0/fb0 hold step 0 of stage g; on exit they hold step 0 of stage g + 1.
  auto stage = [&](int g, auto sc, auto sn) {
    const uint8_t* st = slot_ptr(sc);
    const LoadCtx lh = ctx_h(g + 1, sn);
    step(fa0, fb0, st, 1, fa1, fb1, lh, std::true_type{}, std::true_type{});
    step(fa1, fb1, st, 2, fa0, fb0, lh, std::false_type{}, std::true_type{});
    step(fa0, fb0, st, 3, fa1, fb1, lh, std::false_type{}, std::true_type{});
    const LoadCtx lw = ctx_w(g + 2, sc);
    if constexpr (kTi == 2) {
      step_bar(fa1, fb1, slot_ptr(sn), fa0, fb0, lw, sync_stage);
    } else {
      sync_stage();
      step(fa1, fb1, slot_ptr(sn), 0, fa0, fb0, lw, std::true_type{}, std::false_type{});
    }
  };
  // Stage g with three buffers: SC holds stage g, SN stage g + 1 and SP (free
  // since the previous stage's barrier) receives the hidden slice of stage
  // g + 2 under step 0; after this stage's barrier SC receives the W slice of
  // stage g + 3.  W is requested three stages ahead, hidden two.
  auto stage3 = [&](int g, auto sc, auto sn, auto sp) {
    const uint8_t* st = slot_ptr(sc);
    const LoadCtx lh = ctx_h(g + 2, sp);
    step(fa0, fb0, st, 1, fa1, fb1, lh, std::true_type{}, std::true_type{});
    step(fa1, fb1, st, 2, fa0, fb0, lh, std::false_type{}, std::true_type{});
    step(fa0, fb0, st, 3, fa1, fb1, lh, std::false_type{}, std::true_type{});
    sync_stage3();
    const LoadCtx lw = ctx_w(g + 3, sc);
    step(fa1, fb1, slot_ptr(sn), 0, fa0, fb0, lw, std::true_type{}, std::false_type{});
  };

  float m_run[kTi], s_run[kTi];
#pragma unroll
  for (int ti = 0; ti < kTi; ++ti) {
    m_run[ti] = -INFINITY;
    s_run[ti] = 0.f;
  }

  // A split ends (its last tile is folded into m_run / s_run): merge the
  // lane halves, then the two vocabulary-half waves (through LDS), write the
  // split's partial and restart the running state.  The barrier waits for
  // LDS only: the next stages' loads stay in flight.  `red` is free again by
  // the next flush, at least one stage barrier later.
  auto flush = [&](int split) {
    float mm[kTi], ss[kTi];
#pragma unroll
    for (int ti = 0; ti < kTi; ++ti) {
      const float om = __shfl_xor(m_run[ti], 32);
      const float os = __shfl_xor(s_run[ti], 32);
      if (half == 0)
        merge_state(m_run[ti], s_run[ti], om, os, mm[ti], ss[ti]);
      else
        merge_state(om, os, m_run[ti], s_run[ti], mm[ti], ss[ti]);
    }
    if (wv == 1 && half == 0) {
#pragma unroll
      for (int ti = 0; ti < kTi; ++ti)
        red[wt * kWaveTok + ti * 32 + lane] = make_float2(mm[ti], ss[ti]);
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (wv == 0 && half == 0) {
#pragma unroll
      for (int ti = 0; ti < kTi; ++ti) {
        const int j = wt * kWaveTok + ti * 32 + lane;
        const float2 hi = red[j];
        float m, s;
        merge_state(mm[ti], ss[ti], hi.x, hi.y, m, s);
        if (j < rows_here) p.part[(m0 + j) * p.S + split] = make_float2(m, s);
      }
    }
#pragma unroll
    for (int ti = 0; ti < kTi; ++ti) {
      m_run[ti] = -INFINITY;
      s_run[ti] = 0.f;
    }
  };

  // Prologue: stage 0 whole and the W slice of stage 1 (its hidden slice is
  // issued in stage 0); with three buffers also the hidden slice of stage 1
  // and the W slice of stage 2.
  {
    const LoadCtx w0 = ctx_w(0, Slot<0>{}), h0 = ctx_h(0, Slot<0>{}), w1 = ctx_w(1, Slot<1>{});
#pragma unroll
    for (int j = 0; j < kLoadsPerOperand; ++j) load_one(w0, j, std::false_type{});
#pragma unroll
    for (int j = 0; j < kLoadsH; ++j) load_one(h0, j, std::true_type{});
#pragma unroll
    for (int j = 0; j < kLoadsPerOperand; ++j) load_one(w1, j, std::false_type{});
    if constexpr (kSlots == 3) {
      const LoadCtx h1 = ctx_h(1, Slot<1>{}), w2 = ctx_w(2, Slot<2>{});
#pragma unroll
      for (int j = 0; j < kLoadsH; ++j) load_one(h1, j, std::true_type{});
#pragma unroll
      for (int j = 0; j < kLoadsPerOperand; ++j) load_one(w2, j, std::false_type{});
    }
    load_bias(0);
  }
  wait_vmcnt<0>();
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  init_acc(0);
  read_frags(slot0, 0, fa0, fb0);

  // G is a multiple of kSlots: stage g lives in buffer g % kSlots.
  for (int g = 0; g < G; g += kSlots) {
    if constexpr (kSlots == 2) {
      stage(g, Slot<0>{}, Slot<1>{});
      stage(g + 1, Slot<1>{}, Slot<0>{});
    } else {
      stage3(g, Slot<0>{}, Slot<1>{}, Slot<2>{});
      stage3(g + 1, Slot<1>{}, Slot<2>{}, Slot<0>{});
      stage3(g + 2, Slot<2>{}, Slot<0>{}, Slot<1>{});
    }

    const int v = g / KT;
    if (g + kSlots != (v + 1) * KT) continue;

    // ---- epilogue of vocabulary tile v -------------------------------------
    // acc[vi][ti][r] holds z for token column wt*kWaveTok + ti*32 + (lane & 31) and
    // vocabulary row wv*128 + vi*32 + 8*(r/4) + 4*half + (r%4) of the tile.
    const int vbase = (vt_begin + v) * kVtileCols;
    const int vw = vbase + wv * 128;               // first column of this wave
    if constexpr (kHasBias) {
      // z = (the K accumulation) + bias: one fp32 add per logit
      __builtin_amdgcn_sched_barrier(0);
      const float* bt = &bias_lds[v & 1][wv * 128 + 4 * half];
#pragma unroll
      for (int vi = 0; vi < 4; ++vi) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const floatx4 bb = *(const floatx4*)(bt + vi * 32 + 8 * q);
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int ti = 0; ti < kTi; ++ti) acc[vi][ti][4 * q + e] += bb[e];
        }
        __builtin_amdgcn_sched_barrier(0);        // a few bias values live at a time
      }
      load_bias(v + 1);          // lands during the next tile's first stage
    }
    if constexpr (kGrad) {
      // dZ^T[col][row] = p (g_lse - g_logp) + g_logp [col == target], p =
      // exp(z - lse): 32 consecutive rows per store (coalesced).  The buffer
      // covers the tile's columns below V, so stores past V are dropped.
      const int vrows = min(kVtileCols, p.V - vbase);
      const __amdgpu_buffer_rsrc_t rs_dz = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.dzt + (int64_t)vbase * p.ldz), (short)0, vrows * (int)p.ldz * 2, kRsrcWord3);
      // per token column: its row, whether it exists, the store offset and
      // the target's (vi, r) offset relative to this lane's first column
      uint32_t vo[kTi];
      bool live[kTi];
      int trel[kTi];
#pragma unroll
      for (int ti = 0; ti < kTi; ++ti) {
        const int jr = wt * kWaveTok + ti * 32 + (lane & 31);
        live[ti] = jr < rows_here;
        vo[ti] = ((uint32_t)(wv * 128 + 4 * half) * (uint32_t)p.ldz + (uint32_t)(m0 + jr)) * 2u;
        // opaque per tile: the store addresses are formed here, not hoisted
        // out of the stage loop into registers that would then spill
        asm volatile("" : "+v"(vo[ti]));
        trel[ti] = tgt[ti] - vw - 4 * half;
      }
      uint32_t ld2 = (uint32_t)p.ldz * 2u;
      asm volatile("" : "+s"(ld2));
      // both token columns of a vocabulary row back to back: the two 64-byte
      // halves of each 128-byte line of dZ^T leave together
#pragma unroll
      for (int vi = 0; vi < 4; ++vi) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int k = vi * 32 + 8 * (r >> 2) + (r & 3);      // column - vw - 4 half
#pragma unroll
          for (int ti = 0; ti < kTi; ++ti) {
            float dz = exp2_hw((acc[vi][ti][r] - g_lse_row[ti]) * kLog2e) * g_coef[ti];
            if (trel[ti] == k) dz += g_tgt[ti];
            if (live[ti])
              __builtin_amdgcn_raw_buffer_store_b16(bf16_rne(dz), rs_dz, vo[ti] + (uint32_t)k * ld2,
                                                     0, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      init_acc(v + 1);
      continue;
    }
    if (vbase + kVtileCols > p.V) {                // vocabulary tail: mask columns >= V
#pragma unroll
      for (int vi = 0; vi < 4; ++vi)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int col = vw + vi * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (col >= p.V) {
#pragma unroll
            for (int ti = 0; ti < kTi; ++ti) acc[vi][ti][r] = -INFINITY;
          }
        }
    }

#pragma unroll
    for (int ti = 0; ti < kTi; ++ti) {
      // target capture: exactly one (tile, lane, register) in the grid holds it
      const int rel = tgt[ti] - vw;
      const bool hit = rel >= 0 && rel < 128 && ((rel >> 2) & 1) == half;
      if (__any(hit)) {
        const int vi_t = rel >> 5;
        const int r_t = ((rel >> 3) & 3) * 4 + (rel & 3);
        float val = 0.f;
#pragma unroll
        for (int vi = 0; vi < 4; ++vi)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (vi == vi_t && r == r_t) val = acc[vi][ti][r];
        if (hit) p.tlogit[m0 + wt * kWaveTok + ti * 32 + (lane & 31)] = val;
      }

      // online softmax over this lane's 64 values of the tile
      float mx = acc[0][ti][0];
#pragma unroll
      for (int vi = 0; vi < 4; ++vi)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[vi][ti][r]);
      const float m_new = fmaxf(m_run[ti], mx);
      const float mu = (m_new == -INFINITY) ? 0.f : m_new;
      float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int vi = 0; vi < 4; ++vi)
#pragma unroll
        for (int r = 0; r < 16; ++r) ps[r & 3] += exp2_hw((acc[vi][ti][r] - mu) * kLog2e);
      const float tile_sum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
      s_run[ti] = s_run[ti] * exp2_hw((m_run[ti] - mu) * kLog2e) + tile_sum;
      m_run[ti] = m_new;
    }
    __builtin_amdgcn_sched_barrier(0);      // the tile is consumed before the next one starts
    const int vt = vt_begin + v;
    if (v + 1 == nvt || (vt + 1) % p.vps == 0) flush(vt / p.vps);
    __builtin_amdgcn_sched_barrier(0);
    init_acc(v + 1);
  }

  // The last stages issued loads past the end (into buffers nobody reads);
  // let them land before the workgroup's LDS is released.
  wait_vmcnt<0>();
}

__global__ __launch_bounds__(kThreads, 1) void softmax_grad_kernel(const ProjParams p) {
  proj_lse_body<false, true, 2>(p);
}
__global__ __launch_bounds__(kThreads, 1) void softmax_grad_bias_kernel(const ProjParams p) {
  proj_lse_body<true, true, 2>(p);
}
// 128-token row blocks: twice the workgroups for batches that 256-token
// blocks cannot spread over every compute unit; the same bits
__global__ __launch_bounds__(kThreads, 1) void softmax_grad_r128_kernel(const ProjParams p) {
  proj_lse_body<false, true, 1>(p);
}
__global__ __launch_bounds__(kThreads, 1) void softmax_grad_bias_r128_kernel(const ProjParams p) {
  proj_lse_body<true, true, 1>(p);
}

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

hipError_t launch_softmax_grad(const ProjParams& p, hipStream_t stream) {
  const int64_t blocks = (int64_t)p.R * p.S_grid;
  if (blocks <= 0) return hipSuccess;
  const bool bias = p.bias_kind != kBiasNone;
  auto k = p.rows == 128 ? (bias ? softmax_grad_bias_r128_kernel : softmax_grad_r128_kernel)
                         : (bias ? softmax_grad_bias_kernel : softmax_grad_kernel);
  hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
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
