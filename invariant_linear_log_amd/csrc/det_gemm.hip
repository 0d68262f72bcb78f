// Deterministic bf16 GEMM for gfx950: fixed ascending contraction order,
// fp32 accumulation, 256 x 256 output tiles on v_mfma_f32_16x16x32_bf16.
//
// RL-Kernel PR #395, "feat(musa): add native deterministic gemm kernel",
// summary: a det_gemm whose reduction runs over K in a fixed ascending order
// with fp32 accumulation, providing [M, K] @ [N, K]^T without materialising
// the transposed right-hand side, the input gradient dA = dC . B and the
// weight gradient in the [N, K] layout; the page's kernel computes one output
// per thread and leaves tiling as future work.
//
// One kernel template computes D[p, q] = sum_c X[p, c] * Y[q, c] and writes
// out[q][p]:
//   forward  C[M, N] = A[M, K] . B[N, K]^T : X = B, Y = A (both as stored)
//   dA       dA[M, K] = dC[M, N] . B[N, K] : X = B read transposed, Y = dC
//   dB       dB[N, K] = dC^T . A           : X = A and Y = dC read transposed
// An operand is either contraction-contiguous (X[p][c], the stored layout of
// the forward's operands) or transposed (stored [c][p]: B in dA, A and dC in
// dB).
//
// Bit contract.  Every output element is one chain of MFMA instructions over
// ascending 32-wide contraction steps, started at 0; nothing depends on the
// other outputs, on the number of rows of the batch or on the tile it falls
// in.  So the forward's and dA's rows (M) are batch-invariant; dB reduces
// over M itself, in ascending order.
//
// Workgroup: 512 threads (8 wave64s, two per SIMD), one tile of D of
// 32 kVi rows p x 64 kTj columns q (256 x 256; 128 x 128 for grids too small
// to give every compute unit a 256 x 256 tile).  Waves: w = 2 wt + wv; wv
// picks rows p [16 kVi wv, +16 kVi), wt columns q [16 kTj wt, +16 kTj); a
// wave holds kVi x kTj MFMA tiles of 16 x 16 (128 accumulators per lane in
// the 256-tile), which the register allocator keeps in place in ordinary
// VGPRs.  In an accumulator of tile (vi, tj), lane l holds column q = 16 tj +
// l % 16 and the four rows p = 16 vi + 4 (l / 16) + i, i = 0..3.  The
// 16 x 16 x 32 form does the same work on less energy than 32 x 32 x 16
// (measured on random bf16 data at the board's power limit), and the power
// limit sets the clock of long products.
//
// Pipeline: the one of the fused projection kernel (proj_fwd.hip), with a
// plain store epilogue.  The contraction is staged 64 wide (two MFMA steps of
// 32) through two LDS buffers, each an X slice and a Y slice, filled by
// buffer loads that write LDS directly.  Waves 0..3 issue every load and
// alone wait for them; waves 4..7 only read LDS and run MFMAs (on each SIMD
// the issue arbiter favours the older wave, so the loads go to the waves that
// would otherwise idle at the barrier).  The Y slice of stage s + 1 is loaded
// under the first step of stage s, the X slice of stage s + 2 after the stage
// barrier, which sits in the second step right after the last read of the
// current buffer.  Every step is emitted MFMA by MFMA in a fixed order.
//
// Operand fragments (16 rows or columns x 32 contraction values): lane l
// holds index l % 16 and contraction values 8 (l / 16) .. + 7 of the step.
//
// LDS layouts.  A contraction-contiguous slice is one row of 64 contraction
// values per p (or q): 128-byte rows, 16-byte chunk c at position
// c ^ ((row >> 1) & 7); a fragment is one ds_read_b128 per lane.  A
// transposed slice is 64 contraction rows of 32 kVi (or 64 kTj) values:
// 512- or 256-byte rows, chunk c at position c ^ h(row) with
// h(row) = 2 ((row & 3) | ((row >> 3) & 1) << 2); a fragment is two
// ds_read_b64_tr_b16.  That instruction, per group of 16 lanes, gives lane i
// element j of the 4-element block addressed by lane 4 j + i / 4 at position
// i % 4 (measured on gfx950).  Lane a of group g points at row 8 g + 4 t +
// a / 4 (t = 0, 1 for the two reads) and the 4-column block 4 (a % 4) of the
// fragment's 16 columns, so lane i receives contraction values 8 g + 4 t ..
// + 3 of its own column i.  The 32 lanes of each half of a read then touch 8
// rows whose h values differ: 8 distinct 32-byte bank slots, no conflict.  h
// depends on the row only through lane bits, so every lane's fragment
// offsets are fixed for the whole product.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "bilogp_internal.h"

namespace bilogp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) short4v lds_short4;

constexpr int kThreads = 512;
constexpr int kBK = 64;                             // contraction per stage
constexpr int kTileGroup = 4;                       // q tiles per tile-order group
constexpr int kLoaderWaves = 4;                     // waves 0..3 issue every direct load
constexpr int kFragStride = 16 * 128;               // next 16-row block of a row slice
constexpr uint32_t kOutOfRange = 0x7ffffff0u;       // any offset past num_records
constexpr int kRsrcWord3 = 0x00020000;              // gfx9 raw buffer, 32-bit data

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

template <int I>
using Slot = std::integral_constant<int, I>;

__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// Chunk swizzle of a transposed slice row (see the LDS layouts above).
__device__ __forceinline__ int htr(int row) { return 2 * ((row & 3) | (((row >> 3) & 1) << 2)); }

// fp32 -> bf16 bits, round to nearest even: gfx950's conversion instruction
// (v_cvt_pk_bf16_f32).  fp32 denormals are kept (the kernels run with fp32
// denormal mode on), so every finite value and infinity rounds exactly as
// the IEEE definition; a NaN stays a NaN.
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// A buffer resource over [base, base + bytes), built from values forced into
// scalar registers (the compiler cannot always prove these are uniform, and
// a resource in vector registers turns every load into a per-lane loop).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* base, int bytes) {
  const uint64_t b = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const int n = __builtin_amdgcn_readfirstlane(bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0, n,
                                           kRsrcWord3);
}

// One operand slice of a stage: kRows rows (p or q) of the product.
template <int kRows>
struct Operand {
  static constexpr int kBytes = kRows * kBK * 2;                  // one stage slice
  static constexpr int kL = kBytes / (kLoaderWaves * 64 * 16);    // loads per loader wave
  static constexpr int kRowB = kRows * 2;                         // transposed: bytes per row
  static constexpr int kCpr = kRows / 8;                          // transposed: chunks per row
  static constexpr int kRpl = 1024 / kRowB;                       // transposed: rows per load
};

template <bool kXT, bool kYT, int kVi, int kTj>
__device__ __forceinline__ void det_gemm_body(const GemmParams& g) {
  static_assert((kVi == 8 && kTj == 4) || (kVi == 4 && kTj == 2), "tile shapes");
  constexpr int kTP = 32 * kVi;                     // tile rows p
  constexpr int kTQ = 64 * kTj;                     // tile columns q
  using OX = Operand<kTP>;
  using OY = Operand<kTQ>;
  constexpr int kSlotBytes = OX::kBytes + OY::kBytes;
  constexpr int kM = kVi * kTj;                     // MFMAs per step
  __shared__ __attribute__((aligned(1024))) uint8_t slot0[kSlotBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t slot1[kSlotBytes];

  auto slot_ptr = [&](auto sc) -> uint8_t* {
    if constexpr (decltype(sc)::value == 0) return slot0;
    else return slot1;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wv = wave & 1;
  const int wt = wave >> 1;
  const int lr = lane & 15;          // index within a 16-wide fragment
  const int lg = lane >> 4;          // lane group: contraction values 8 lg .. 8 lg + 7

  // Block id -> (p tile, q tile), XCD-aware and grouped like the projection:
  // each XCD takes a contiguous run of tiles, ordered in groups of kTileGroup
  // q tiles x all p tiles.
  const int nblk = g.Pt * g.Qt;
  const int per_xcd = nblk >> 3;
  int u = blockIdx.x;
  if (u < (per_xcd << 3)) u = (u & 7) * per_xcd + (u >> 3);
  const int in_group = kTileGroup * g.Pt;
  const int first_qt = (u / in_group) * kTileGroup;
  const int group_qts = min(g.Qt - first_qt, kTileGroup);
  const int qt = first_qt + (u % in_group) % group_qts;
  const int pt = (u % in_group) / group_qts;
  const int64_t p0 = (int64_t)pt * kTP;
  const int64_t q0 = (int64_t)qt * kTQ;
  const int64_t C = g.C;
  const int KT = (int)(((C + kBK - 1) / kBK + 1) / 2 * 2);   // even: stage s in buffer s % 2
  const bool loader = wave < kLoaderWaves;

  // ---- load descriptors (used by the loader waves only) -------------------
  // Contraction-contiguous operand: load j of loader wave w fills rows
  // r = (kL w + j) * 8 + lane / 8, 8 chunks each, chunk (lane & 7) ^ swz(r).
  // swz(r) takes two values over j (even and odd j), so the per-lane offset is
  // base[j & 1] + (j & ~1) * 8 rows.  The resource covers the tile's valid
  // rows; the stage adds its contraction offset.
  // Transposed operand: load j of loader wave w fills kRpl LDS rows from
  // kRpl (kL w + j), lane i taking row kRpl (kL w + j) + i / kCpr and chunk
  // (i % kCpr) ^ h(row); columns past the operand's width read nothing.
  struct RowLoads {
    __amdgpu_buffer_rsrc_t rsrc;
    uint32_t base[2];
    int kc[2];
  };
  auto setup_rows = [&](auto opc, const void* ptr, int64_t ld, int64_t row0, int64_t nrows) {
    using O = decltype(opc);
    RowLoads r;
    constexpr int64_t kTileRows = O::kBytes / 128;
    const int64_t valid = nrows - row0 < kTileRows ? nrows - row0 : kTileRows;
    r.rsrc = uniform_rsrc((const uint16_t*)ptr + row0 * ld, (int)(valid > 0 ? valid * ld * 2 : 0));
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int row = (wave * O::kL + e) * 8 + (lane >> 3);
      const int cc = (lane & 7) ^ swz(row);
      r.base[e] = (uint32_t)row * (uint32_t)ld * 2u + (uint32_t)cc * 16u;
      r.kc[e] = cc * 8;
    }
    return r;
  };
  auto setup_cols = [&](auto opc, int64_t ld, int64_t col0, int64_t ncols, uint32_t* off) {
    using O = decltype(opc);
#pragma unroll
    for (int j = 0; j < O::kL; ++j) {
      const int row = O::kRpl * (wave * O::kL + j) + lane / O::kCpr;
      const int chunk = (lane % O::kCpr) ^ htr(row);
      const int64_t col = col0 + chunk * 8;
      off[j] = col < ncols ? (uint32_t)row * (uint32_t)ld * 2u + (uint32_t)col * 2u : kOutOfRange;
    }
  };
  RowLoads xr{}, yr{};
  uint32_t xc[OX::kL], yc[OY::kL];
  if constexpr (!kXT) xr = setup_rows(OX{}, g.x, g.ldx, p0, g.P);
  else setup_cols(OX{}, g.ldx, p0, g.P, xc);
  if constexpr (!kYT) yr = setup_rows(OY{}, g.y, g.ldy, q0, g.Q);
  else setup_cols(OY{}, g.ldy, q0, g.Q, yc);

  struct LoadCtx {
    __amdgpu_buffer_rsrc_t rsrc;
    uint8_t* dst;
    uint32_t k2;      // contraction byte offset of the stage (row operands)
    int64_t kend;     // C, or 0 past the end (row operands)
  };
  // Operand `op` (0 = X, 1 = Y) of stage s into buffer SC.  A stage past the
  // end reads nothing (empty range) into a buffer nobody reads any more.
  auto ctx = [&](int s, auto sc, auto op) {
    constexpr bool is_x = decltype(op)::value == 0;
    constexpr bool tr = is_x ? kXT : kYT;
    const int64_t c0 = (int64_t)s * kBK;
    int dst = (is_x ? 0 : OX::kBytes) + wave * (is_x ? OX::kL : OY::kL) * 1024;
    asm volatile("" : "+s"(dst));     // per stage: LDS addresses stay out of SGPRs
    LoadCtx c;
    c.dst = slot_ptr(sc) + dst;
    if constexpr (tr) {
      const int64_t ld = is_x ? g.ldx : g.ldy;
      // rows c0 .. c0 + 63 clamped to [0, C): an empty range past the end
      const int64_t rows = max((int64_t)0, min(C - c0, (int64_t)kBK));
      c.rsrc = uniform_rsrc((const uint16_t*)(is_x ? g.x : g.y) + min(c0, C) * ld,
                            (int)(rows * ld * 2));
      c.k2 = 0;
      c.kend = 0;
    } else {
      c.rsrc = is_x ? xr.rsrc : yr.rsrc;
      c.k2 = (uint32_t)c0 * 2u;
      c.kend = c0 < C ? C : 0;
    }
    return c;
  };
  auto load_one = [&](const LoadCtx& c, auto op, int j) {
    constexpr bool is_x = decltype(op)::value == 0;
    constexpr bool tr = is_x ? kXT : kYT;
    uint32_t voff;
    if constexpr (tr) {
      voff = is_x ? xc[j] : yc[j];
    } else {
      const RowLoads& r = is_x ? xr : yr;
      const int64_t ld = is_x ? g.ldx : g.ldy;
      const bool ok = (int64_t)(c.k2 / 2u) + r.kc[j & 1] < c.kend;
      voff = ok ? r.base[j & 1] + (uint32_t)(j & ~1) * 16u * (uint32_t)ld + c.k2 : kOutOfRange;
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rsrc, (lds_void*)(c.dst + j * 1024), 16, voff, 0,
                                             0, 0);
  };

  // ---- fragment reads ---------------------------------------------------
  // Row operand: row sub + lr, chunk (4 uu + lg) ^ swz(row) for step uu (swz
  // reads row bits 1-3, which come from lr).  Transposed operand: two
  // ds_read_b64_tr_b16; lane lr of group lg addresses contraction row
  // 32 uu + 8 lg + 4 t + lr / 4 and columns sub + 4 (lr % 4) .. + 3, with
  // h(row) = h(8 lg + lr / 4) for every uu and t.
  const int fr = swz(lr);
  int row_off[2];
#pragma unroll
  for (int uu = 0; uu < 2; ++uu) row_off[uu] = (lr * 8 + ((4 * uu + lg) ^ fr)) * 16;
  const int trow = 8 * lg + (lr >> 2);                 // + 32 uu + 4 t
  auto tr_off = [&](int sub, int rowb) {               // sub: multiple of 16
    const int pos = (sub / 8 + ((lr & 3) >> 1)) ^ htr(trow);
    return trow * rowb + pos * 16 + 8 * (lr & 1);
  };
  int xoff[kXT ? kVi : 1], yoff[kYT ? kTj : 1];
  if constexpr (kXT) {
#pragma unroll
    for (int vi = 0; vi < kVi; ++vi) xoff[vi] = tr_off(wv * 16 * kVi + vi * 16, OX::kRowB);
  } else {
    xoff[0] = wv * 16 * kVi * 128;
  }
  if constexpr (kYT) {
#pragma unroll
    for (int tj = 0; tj < kTj; ++tj)
      yoff[tj] = OX::kBytes + tr_off(wt * 16 * kTj + tj * 16, OY::kRowB);
  } else {
    yoff[0] = OX::kBytes + wt * 16 * kTj * 128;
  }

  auto frag = [&](const uint8_t* st, int uu, int idx, auto op) -> bf16x8 {
    constexpr bool is_x = decltype(op)::value == 0;
    constexpr bool tr = is_x ? kXT : kYT;
    if constexpr (tr) {
      constexpr int rowb = is_x ? OX::kRowB : OY::kRowB;
      const uint8_t* a = st + (is_x ? xoff[idx] : yoff[idx]) + uu * 32 * rowb;
      const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)a);
      const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(a + 4 * rowb));
      const short8v v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      return __builtin_bit_cast(bf16x8, v);
    } else {
      return *(const bf16x8*)(st + (is_x ? xoff[0] : yoff[0]) + row_off[uu] +
                              idx * kFragStride);
    }
  };

  using OpX = std::integral_constant<int, 0>;
  using OpY = std::integral_constant<int, 1>;

  // The pipeline is instantiated twice, selected by one wave-uniform branch:
  // for the loader waves (with the direct loads and their waits) and for the
  // compute-only waves (without).
  auto run = [&](auto is_loader) {
    constexpr bool kLoader = decltype(is_loader)::value;
    auto ld = [&](const LoadCtx& c, auto op, int j) {
      if constexpr (kLoader) load_one(c, op, j);
    };

    // acc[vi][tj][i] = D[p0 + 16 kVi wv + 16 vi + 4 lg + i][q0 + 16 kTj wt + 16 tj + lr]
    floatx4 acc[kVi][kTj];
#pragma unroll
    for (int vi = 0; vi < kVi; ++vi)
#pragma unroll
      for (int tj = 0; tj < kTj; ++tj) acc[vi][tj] = floatx4{};

    // Operand registers.  ar: ring of X fragments, X[vi] of the current step in
    // ar[vi & 3]; bA / bB: Y fragments of the even / odd step of a stage.
    bf16x8 ar[4], bA[kTj], bB[kTj];

    // Position of each item inside a step of kM MFMAs, fixed at compile time:
    //  - X[vi + 3] is read right after the first MFMA of vi (for vi + 3 >= kVi:
    //    the next step's X[vi + 3 - kVi], from the next step's buffer);
    //  - Y fragment t of the next step after MFMA kTj t + kTj / 2;
    //  - in the stage's first step, direct load j of the next stage's Y slice
    //    after MFMA kM / nl (j + 1) - 1;
    //  - in its last step, the barrier after MFMA kBarAt (the MFMA after the
    //    one that carries the read of X[kVi - 1], the last read of the current
    //    buffer); after it the next stage's Y fragments and first X fragments,
    //    and the X refill of the released buffer over the remaining MFMAs.
    constexpr int kBarAt = (kVi - 4) * kTj + 1;
    constexpr int kPost = kM - kBarAt - 1;
    auto sync_stage = [&]() {
      if constexpr (kLoader) wait_vmcnt<0>();
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    auto kstep = [&](const uint8_t* st, int uu, const uint8_t* nst, int nu,
                     const bf16x8 (&bc)[kTj], bf16x8 (&bn)[kTj], const LoadCtx& lc, auto last) {
      constexpr bool kLast = decltype(last)::value;
#pragma unroll
      for (int i = 0; i < kM; ++i) {
        const int vi = i / kTj, tj = i % kTj;
        acc[vi][tj] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(ar[vi & 3], bc[tj], acc[vi][tj], 0, 0, 0);
        if (tj == 0 && vi + 3 < kVi) ar[(vi + 3) & 3] = frag(st, uu, vi + 3, OpX{});
        if constexpr (!kLast) {
          if (tj == 0 && vi + 3 >= kVi) ar[(vi + 3) & 3] = frag(nst, nu, vi + 3 - kVi, OpX{});
          if (tj == kTj / 2 && vi < kTj) bn[vi] = frag(nst, nu, vi, OpY{});
          constexpr int stride = kM / OY::kL;
          if (i % stride == stride - 1) ld(lc, OpY{}, i / stride);
        } else {
          if (i == kBarAt) sync_stage();
          if (i > kBarAt) {
            const int q = i - kBarAt - 1;
            if (tj == 0 && vi + 3 >= kVi) ar[(vi + 3) & 3] = frag(nst, nu, vi + 3 - kVi, OpX{});
            if (q < kTj) bn[q] = frag(nst, nu, q, OpY{});
#pragma unroll
            for (int j = 0; j < OX::kL; ++j)
              if (q == j * kPost / OX::kL) ld(lc, OpX{}, j);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // Stage s from buffer SC (SN holds stage s + 1).
    auto stage = [&](int s, auto sc, auto sn) {
      const uint8_t* st = slot_ptr(sc);
      const LoadCtx ly = ctx(s + 1, sn, OpY{});
      kstep(st, 0, st, 1, bA, bB, ly, std::false_type{});
      const LoadCtx lx = ctx(s + 2, sc, OpX{});
      kstep(st, 1, slot_ptr(sn), 0, bB, bA, lx, std::true_type{});
    };

    // Prologue: stage 0 whole and the X slice of stage 1 (its Y slice is
    // issued in stage 0).
    {
      const LoadCtx x0 = ctx(0, Slot<0>{}, OpX{}), y0 = ctx(0, Slot<0>{}, OpY{}),
                    x1 = ctx(1, Slot<1>{}, OpX{});
#pragma unroll
      for (int j = 0; j < OX::kL; ++j) ld(x0, OpX{}, j);
#pragma unroll
      for (int j = 0; j < OY::kL; ++j) ld(y0, OpY{}, j);
#pragma unroll
      for (int j = 0; j < OX::kL; ++j) ld(x1, OpX{}, j);
    }
    wait_vmcnt<0>();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int vi = 0; vi < 3; ++vi) ar[vi] = frag(slot0, 0, vi, OpX{});
#pragma unroll
    for (int tj = 0; tj < kTj; ++tj) bA[tj] = frag(slot0, 0, tj, OpY{});

    for (int s = 0; s < KT; s += 2) {
      stage(s, Slot<0>{}, Slot<1>{});
      stage(s + 1, Slot<1>{}, Slot<0>{});
    }
    // the last stages issued loads past the end (into buffers nobody reads);
    // let them land before the workgroup's LDS is released
    if constexpr (kLoader) wait_vmcnt<0>();

    // ---- store through LDS.  The stage buffers are free now: the tile is
    // written into them in output order (row q; the 16-byte chunks of a row
    // swizzled by the row), then read back so that consecutive lanes hold
    // consecutive chunks of one row, and stored 16 bytes per lane: every
    // store instruction writes whole tile rows, where writing the
    // accumulators' own layout (16 rows, 32 or 64 bytes each) stalled the
    // load path.  P is a multiple of 8, so a chunk (8 bf16 or 4 fp32) is
    // wholly inside or wholly past P.  fp32 tiles of 256 x 256 go in two
    // passes of 128 rows.
    __syncthreads();        // every wave is done with the stage buffers
    auto epilogue = [&](auto esz_c) {
      constexpr int kEsz = decltype(esz_c)::value;          // bytes per output element
      constexpr int kRowB = kTP * kEsz;                     // bytes per tile row
      constexpr int kC = kRowB / 16;                        // 16-byte chunks per row
      constexpr int kRs = kSlotBytes / kRowB;               // rows per buffer
      constexpr int kPR = 2 * kRs < kTQ ? 2 * kRs : kTQ;    // rows per pass
      constexpr int kPasses = kTQ / kPR;
      constexpr int kWaveRows = 16 * kTj;                   // rows a wave holds
      constexpr int kRpi = 64 / kC;                         // rows per read instruction
      constexpr int kReads = kPR / 8 / kRpi;                // reads per wave and pass
      constexpr int kSwz = kC < 32 ? kC - 1 : 31;
      static_assert(kC <= 64 && 64 % kC == 0 && kPR % kWaveRows == 0 &&
                    kPR % (8 * kRpi) == 0 && kTQ % kPR == 0, "epilogue geometry");
      auto lds_at = [&](int row, int byte) -> uint8_t* {    // row within the pass
        const int r = row % kRs;
        uint8_t* base = row < kRs ? slot0 : slot1;
        return base + r * kRowB + (((byte >> 4) ^ (r & kSwz)) << 4) + (byte & 15);
      };
#pragma unroll
      for (int pass = 0; pass < kPasses; ++pass) {
        const int row_lo = pass * kPR;
        if (wt * kWaveRows >= row_lo && wt * kWaveRows < row_lo + kPR) {
#pragma unroll
          for (int tj = 0; tj < kTj; ++tj)
#pragma unroll
            for (int vi = 0; vi < kVi; ++vi) {
              const int row = wt * kWaveRows + tj * 16 + lr - row_lo;
              const int pb = (wv * 16 * kVi + vi * 16 + 4 * lg) * kEsz;
              const floatx4 v = acc[vi][tj];
              if constexpr (kEsz == 2) {
                const uint2 w2 = {bf16_bits(v[0]) | (bf16_bits(v[1]) << 16),
                                  bf16_bits(v[2]) | (bf16_bits(v[3]) << 16)};
                *(uint2*)lds_at(row, pb) = w2;
              } else {
                *(floatx4*)lds_at(row, pb) = v;
              }
            }
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kReads; ++k) {
          const int row = wave * (kPR / 8) + k * kRpi + lane / kC;
          const int c = lane % kC;
          const uint4 d = *(const uint4*)lds_at(row, c * 16);
          const int64_t q = q0 + row_lo + row;
          const int64_t p = p0 + c * (16 / kEsz);
          if (q < g.Q && p < g.P) {
            uint8_t* o = (uint8_t*)g.out + (q * g.ldo + p) * kEsz;
            if (kEsz == 4 && g.out_kind == kGemmF32Accum)
              *(floatx4*)o = *(const floatx4*)o + __builtin_bit_cast(floatx4, d);
            else
              *(uint4*)o = d;
          }
        }
        if (pass + 1 < kPasses) __syncthreads();
      }
    };
    if (g.out_kind == kGemmBf16)
      epilogue(std::integral_constant<int, 2>{});
    else
      epilogue(std::integral_constant<int, 4>{});
  };
  if (loader)
    run(std::true_type{});
  else
    run(std::false_type{});
}

__global__ __launch_bounds__(kThreads, 1) void det_gemm_nn_kernel(const GemmParams g) {
  det_gemm_body<false, false, 8, 4>(g);
}
__global__ __launch_bounds__(kThreads, 1) void det_gemm_tn_kernel(const GemmParams g) {
  det_gemm_body<true, false, 8, 4>(g);
}
__global__ __launch_bounds__(kThreads, 1) void det_gemm_tt_kernel(const GemmParams g) {
  det_gemm_body<true, true, 8, 4>(g);
}
__global__ __launch_bounds__(kThreads, 1) void det_gemm_nn_t128_kernel(const GemmParams g) {
  det_gemm_body<false, false, 4, 2>(g);
}
__global__ __launch_bounds__(kThreads, 1) void det_gemm_tn_t128_kernel(const GemmParams g) {
  det_gemm_body<true, false, 4, 2>(g);
}
__global__ __launch_bounds__(kThreads, 1) void det_gemm_tt_t128_kernel(const GemmParams g) {
  det_gemm_body<true, true, 4, 2>(g);
}

}  // namespace

// Tile edge: 128 when 256 x 256 tiles would leave compute units idle.  The
// grid is issued in chunks of q tiles so that no launch exceeds 2^32 - 1
// work-items; a tile's arithmetic does not depend on the chunk it is in.
hipError_t launch_det_gemm(const GemmParams& g_in, bool x_t, bool y_t, hipStream_t stream) {
  if (!x_t && y_t) return hipErrorInvalidValue;
  const int64_t tiles256 = ((g_in.P + 255) / 256) * ((g_in.Q + 255) / 256);
  const int kt = (g_in.cu_count > 0 && tiles256 < g_in.cu_count) ? 128 : 256;
  const int64_t Pt = (g_in.P + kt - 1) / kt;
  const int64_t Qt = (g_in.Q + kt - 1) / kt;
  if (Pt <= 0 || Qt <= 0) return hipSuccess;
  void (*k)(const GemmParams);
  if (kt == 128)
    k = !x_t ? det_gemm_nn_t128_kernel : (y_t ? det_gemm_tt_t128_kernel : det_gemm_tn_t128_kernel);
  else
    k = !x_t ? det_gemm_nn_kernel : (y_t ? det_gemm_tt_kernel : det_gemm_tn_kernel);
  const int64_t max_blocks = (int64_t)(UINT32_MAX / (uint32_t)kThreads);
  const int64_t chunk_qt = std::max<int64_t>(1, max_blocks / Pt);
  const size_t out_elem = g_in.out_kind == kGemmBf16 ? 2 : 4;
  for (int64_t qt0 = 0; qt0 < Qt; qt0 += chunk_qt) {
    GemmParams g = g_in;
    const int64_t qs = qt0 * kt;
    g.Q = std::min<int64_t>(g_in.Q - qs, chunk_qt * kt);
    g.Pt = (int32_t)Pt;
    g.Qt = (int32_t)((g.Q + kt - 1) / kt);
    // q selects rows of a contraction-contiguous Y, columns of a transposed one
    g.y = (const uint16_t*)g_in.y + (y_t ? qs : qs * g_in.ldy);
    g.out = (uint8_t*)g_in.out + (size_t)qs * (size_t)g_in.ldo * out_elem;
    hipLaunchKernelGGL(k, dim3((unsigned)((int64_t)g.Pt * g.Qt)), dim3(kThreads), 0, stream, g);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace bilogp
