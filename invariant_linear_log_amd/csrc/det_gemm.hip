// Deterministic bf16 GEMM for gfx950: fixed ascending contraction order,
// fp32 accumulation, 256 x 256 output tiles on v_mfma_f32_32x32x16_bf16.
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
// ascending 16-wide contraction steps, started at 0; nothing depends on the
// other outputs, on the number of rows of the batch or on the tile it falls
// in.  So the forward's and dA's rows (M) are batch-invariant; dB reduces
// over M itself, in ascending order.
//
// Workgroup: 256 threads (4 wave64s, one per SIMD), one 256 x 256 tile of D.
// Waves: w = 2 * wt + wv; wv picks rows p [128 wv, +128), wt columns q
// [128 wt, +128); 4 x 4 MFMA tiles of 32 x 32 per wave, whose 256
// accumulators per lane sit in the matrix (AGPR) half of the wave's 512
// registers.  A 128 x 128 wave tile reads 8 operand fragments per 16 MFMAs,
// a third less LDS traffic than 8 waves of 128 x 64; measured 2-6% faster at
// the backward's shapes, bit for bit the same results.  The contraction is
// staged 64 wide through two 64 KB LDS buffers (an X slice and a Y slice,
// 32 KB each) filled by buffer loads that write LDS directly, one barrier
// per stage and the refill interleaved with the MFMAs (as in the fused
// projection kernel).
//
// LDS layouts.  A contraction-contiguous slice is 256 rows x 64 contraction
// values (128-byte rows, 16-byte chunk c at position c ^ ((row >> 1) & 7));
// operand fragments are one ds_read_b128 per lane.  A transposed slice is 64
// contraction rows x 256 values (512-byte rows, chunk c at position
// c ^ (4 * (row & 3))); a fragment (8 contraction values of one row p per
// lane) is two ds_read_b64_tr_b16.  That instruction, per group of 16 lanes,
// gives lane i element j of the 4-element block addressed by lane 4 j + i / 4
// at position i % 4 (measured on gfx950); lanes pointing at rows c .. c + 3
// and 4-column blocks of 16 consecutive columns hand every lane 4 consecutive
// contraction values of its own column.  Both swizzles keep the reads
// bank-conflict free.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "bilogp_internal.h"

namespace bilogp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) short4v lds_short4;

constexpr int kThreads = 256;
constexpr int kBK = 64;                             // contraction per stage
constexpr int kTileGroup = 4;                       // q tiles per tile-order group
constexpr uint32_t kOutOfRange = 0x7ffffff0u;
constexpr int kRsrcWord3 = 0x00020000;


template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

template <int I>
using Slot = std::integral_constant<int, I>;

// fp32 -> bf16, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
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

// kT: the edge of the square D tile (256, or 128 for grids too small to give
// every compute unit a 256 x 256 tile); each of the 4 waves computes a
// kT/2 x kT/2 quarter.  The tile size orders and groups the work only: every
// output is the same MFMA chain in both.
template <bool kXT, bool kYT, int kT>
__device__ __forceinline__ void det_gemm_body(const GemmParams& g) {
  static_assert(kT == 256 || kT == 128, "tile edge");
  constexpr int kOpBytes = kT * kBK * 2;            // one operand slice: 32 or 16 KB
  constexpr int kSlotBytes = 2 * kOpBytes;          // X slice, Y slice
  constexpr int kLoads = kOpBytes / (kThreads * 16);  // loads per thread and operand: 8 or 4
  constexpr int kHalf = kT / 2;                     // wave tile edge
  constexpr int kNF = kT / 64;                      // 32-wide MFMA tiles per wave edge
  constexpr int kRowB = kT * 2;                     // bytes per row of a transposed slice
  constexpr int kChunksT = kT / 8;                  // 16-byte chunks per transposed row
  constexpr int kRowsPerLoad = 64 / kChunksT;       // transposed rows per load instruction
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
  const int half = lane >> 5;

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
  const int64_t p0 = (int64_t)pt * kT;
  const int64_t q0 = (int64_t)qt * kT;
  const int64_t C = g.C;
  const int KT = (int)(((C + kBK - 1) / kBK + 1) / 2 * 2);   // even: stage g in buffer g % 2

  // ---- loaders ---------------------------------------------------------
  // Contraction-contiguous operand (rows r of the tile, 64 contraction values
  // per stage): load j of wave w fills 8 rows x 8 chunks, row r = (8 w + j) * 8
  // + lane / 8, chunk (lane & 7) ^ ((r >> 1) & 7).  The resource covers the
  // tile's valid rows; the stage adds its contraction offset.
  int rowc_chunk[kLoads];
  uint32_t rowc_off[kLoads];
  auto setup_rows = [&](const void* base, int64_t ld, int64_t row0, int64_t nrows) {
    const int64_t valid = nrows - row0 < kT ? nrows - row0 : kT;
    const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(
        (const uint16_t*)base + row0 * ld, (int)(valid > 0 ? valid * ld * 2 : 0));
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int r = (wave * kLoads + j) * 8 + (lane >> 3);
      const int cc = (lane & 7) ^ ((r >> 1) & 7);
      rowc_chunk[j] = cc * 8;
      rowc_off[j] = (uint32_t)r * (uint32_t)ld * 2u + (uint32_t)cc * 16u;
    }
    return rs;
  };
  // Transposed operand (64 contraction rows x kT columns per stage): load j
  // of wave w fills kRowsPerLoad LDS rows from kRowsPerLoad (kLoads w + j),
  // lane i taking row kRowsPerLoad (kLoads w + j) + i / kChunksT and chunk
  // (i % kChunksT) ^ (4 * (row & 3)).  The resource is rebuilt per stage (rows
  // c0 .. c0 + 63); columns past the operand's width read as zero.
  uint32_t colt_off[kLoads];
  auto setup_cols = [&](int64_t ld, int64_t col0, int64_t ncols) {
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int row = kRowsPerLoad * (wave * kLoads + j) + lane / kChunksT;
      const int chunk = (lane % kChunksT) ^ (4 * (row & 3));
      const int64_t col = col0 + chunk * 8;
      colt_off[j] = col < ncols ? (uint32_t)row * (uint32_t)ld * 2u + (uint32_t)col * 2u
                                : kOutOfRange;
    }
  };

  // X is the p side, Y the q side; each keeps its own tables.
  __amdgpu_buffer_rsrc_t rs_xrows = uniform_rsrc(g.x, 0), rs_yrows = rs_xrows;
  int xrow_chunk[kLoads], yrow_chunk[kLoads];
  uint32_t xrow_off[kLoads], yrow_off[kLoads], xcol_off[kLoads], ycol_off[kLoads];
  if constexpr (!kXT) {
    rs_xrows = setup_rows(g.x, g.ldx, p0, g.P);
#pragma unroll
    for (int j = 0; j < kLoads; ++j) { xrow_chunk[j] = rowc_chunk[j]; xrow_off[j] = rowc_off[j]; }
  } else {
    setup_cols(g.ldx, p0, g.P);
#pragma unroll
    for (int j = 0; j < kLoads; ++j) xcol_off[j] = colt_off[j];
  }
  if constexpr (!kYT) {
    rs_yrows = setup_rows(g.y, g.ldy, q0, g.Q);
#pragma unroll
    for (int j = 0; j < kLoads; ++j) { yrow_chunk[j] = rowc_chunk[j]; yrow_off[j] = rowc_off[j]; }
  } else {
    setup_cols(g.ldy, q0, g.Q);
#pragma unroll
    for (int j = 0; j < kLoads; ++j) ycol_off[j] = colt_off[j];
  }

  struct LoadCtx {
    __amdgpu_buffer_rsrc_t rsrc;
    uint8_t* dst;
    uint32_t k2;      // contraction byte offset of the stage (row operands)
    int64_t kend;     // C, or 0 past the end (row operands)
  };
  // Operand `op` (0 = X, 1 = Y) of stage s into buffer SC.
  auto ctx = [&](int s, auto sc, auto op) {
    constexpr bool is_x = decltype(op)::value == 0;
    constexpr bool tr = is_x ? kXT : kYT;
    const int64_t c0 = (int64_t)s * kBK;
    int dst = (is_x ? 0 : kOpBytes) + wave * kLoads * 1024;
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
      c.rsrc = is_x ? rs_xrows : rs_yrows;
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
      voff = is_x ? xcol_off[j] : ycol_off[j];
    } else {
      const int chunk = is_x ? xrow_chunk[j] : yrow_chunk[j];
      const bool ok = (int64_t)(c.k2 / 2u) + chunk < c.kend;
      voff = ok ? (is_x ? xrow_off[j] : yrow_off[j]) + c.k2 : kOutOfRange;
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rsrc, (lds_void*)(c.dst + j * 1024), 16, voff, 0,
                                             0, 0);
  };

  // ---- fragment reads ---------------------------------------------------
  // Row operand: row sub + (lane & 31), chunk (2 uu + half) ^ f(row).
  // Transposed operand: two ds_read_b64_tr_b16; lane i of 16-lane group gg
  // addresses contraction row 16 uu + 8 (gg >> 1) + 4 t + i / 4 and columns
  // sub + 16 (gg & 1) + 4 (i % 4) .. + 3.
  const int fr = ((lane & 31) >> 1) & 7;
  int row_off[4];
#pragma unroll
  for (int uu = 0; uu < 4; ++uu) row_off[uu] = ((lane & 31) * 8 + ((2 * uu + half) ^ fr)) * 16;
  const int i16 = lane & 15, gg = lane >> 4;
  const int trow = 8 * (gg >> 1) + (i16 >> 2);        // + 16 uu + 4 t (multiples of 4)
  auto tr_off = [&](int sub) {                          // sub: multiple of 32
    const int chunk = (sub + 16 * (gg & 1)) / 8 + ((i16 & 3) >> 1);
    const int pos = chunk ^ (4 * (trow & 3));
    return trow * kRowB + pos * 16 + 8 * (i16 & 1);
  };
  int xoff[kNF], yoff[kNF];
#pragma unroll
  for (int vi = 0; vi < kNF; ++vi)
    xoff[vi] = kXT ? tr_off(wv * kHalf + vi * 32) : ((wv * kHalf + vi * 32) * 8) * 16;
#pragma unroll
  for (int ti = 0; ti < kNF; ++ti)
    yoff[ti] = kOpBytes + (kYT ? tr_off(wt * kHalf + ti * 32) : ((wt * kHalf + ti * 32) * 8) * 16);

  auto frag = [&](const uint8_t* st, int off, int uu, auto trc) -> bf16x8 {
    if constexpr (decltype(trc)::value) {
      const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_short4*)(st + off + uu * 16 * kRowB));
      const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_short4*)(st + off + uu * 16 * kRowB + 4 * kRowB));
      typedef short short8v __attribute__((ext_vector_type(8)));
      const short8v v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      return __builtin_bit_cast(bf16x8, v);
    } else {
      return *(const bf16x8*)(st + off + row_off[uu]);
    }
  };

  floatx16 acc[kNF][kNF];
#pragma unroll
  for (int vi = 0; vi < kNF; ++vi)
#pragma unroll
    for (int ti = 0; ti < kNF; ++ti) acc[vi][ti] = floatx16{};

  // One K step in fixed order: MFMA i = (vi, ti) = (i / kNF, i % kNF), then
  // for i < 2 kNF the next step's fragment (b0 a0 b1 a1 ...), then - with
  // loads - the stage's kLoads direct loads spread evenly over the MFMAs.
  using XT = std::integral_constant<bool, kXT>;
  using YT = std::integral_constant<bool, kYT>;
  auto step = [&](const bf16x8 (&a)[kNF], const bf16x8 (&b)[kNF], const uint8_t* nst, int nuu,
                  bf16x8 (&na)[kNF], bf16x8 (&nb)[kNF], const LoadCtx& lc, auto op,
                  auto with_loads) {
    constexpr int kStride = kNF * kNF / kLoads;     // MFMAs per load
#pragma unroll
    for (int i = 0; i < kNF * kNF; ++i) {
      const int vi = i / kNF, ti = i % kNF;
      acc[vi][ti] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[vi], b[ti], acc[vi][ti], 0, 0, 0);
      if (i < 2 * kNF) {
        if (i & 1) na[i >> 1] = frag(nst, xoff[i >> 1], nuu, XT{});
        else nb[i >> 1] = frag(nst, yoff[i >> 1], nuu, YT{});
      }
      if constexpr (decltype(with_loads)::value) {
        if (i % kStride == kStride - 1) load_one(lc, op, i / kStride);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto read_frags = [&](const uint8_t* st, int uu, bf16x8 (&a)[kNF], bf16x8 (&b)[kNF]) {
#pragma unroll
    for (int i = 0; i < kNF; ++i) {
      b[i] = frag(st, yoff[i], uu, YT{});
      a[i] = frag(st, xoff[i], uu, XT{});
    }
  };
  auto sync_stage = [&]() {
    wait_vmcnt<0>();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };

  bf16x8 fa0[kNF], fb0[kNF], fa1[kNF], fb1[kNF];
  using OpX = std::integral_constant<int, 0>;
  using OpY = std::integral_constant<int, 1>;

  // Stage s from buffer SC (SN holds stage s + 1): the Y slice of stage s + 1
  // is loaded under step 0, the X slice of stage s + 2 under step 3.
  auto stage = [&](int s, auto sc, auto sn) {
    const uint8_t* st = slot_ptr(sc);
    const LoadCtx ly = ctx(s + 1, sn, OpY{});
    step(fa0, fb0, st, 1, fa1, fb1, ly, OpY{}, std::true_type{});
    step(fa1, fb1, st, 2, fa0, fb0, ly, OpY{}, std::false_type{});
    step(fa0, fb0, st, 3, fa1, fb1, ly, OpY{}, std::false_type{});
    sync_stage();
    const LoadCtx lx = ctx(s + 2, sc, OpX{});
    step(fa1, fb1, slot_ptr(sn), 0, fa0, fb0, lx, OpX{}, std::true_type{});
  };

  {
    const LoadCtx x0 = ctx(0, Slot<0>{}, OpX{}), y0 = ctx(0, Slot<0>{}, OpY{}),
                  x1 = ctx(1, Slot<1>{}, OpX{});
#pragma unroll
    for (int j = 0; j < kLoads; ++j) load_one(x0, OpX{}, j);
#pragma unroll
    for (int j = 0; j < kLoads; ++j) load_one(y0, OpY{}, j);
#pragma unroll
    for (int j = 0; j < kLoads; ++j) load_one(x1, OpX{}, j);
  }
  wait_vmcnt<0>();
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  read_frags(slot0, 0, fa0, fb0);

  for (int s = 0; s < KT; s += 2) {
    stage(s, Slot<0>{}, Slot<1>{});
    stage(s + 1, Slot<1>{}, Slot<0>{});
  }
  wait_vmcnt<0>();             // loads past the end must land before LDS is released

  // ---- store: acc[vi][ti][r] = D[p][q] with q = q0 + wt*kHalf + ti*32 + (lane & 31)
  // and p = p0 + wv*kHalf + vi*32 + 8*(r/4) + 4*half + (r%4): four consecutive p
  // per (vi, r / 4), one 16-byte (fp32) or 8-byte (bf16) store.
#pragma unroll
  for (int ti = 0; ti < kNF; ++ti) {
    const int64_t q = q0 + wt * kHalf + ti * 32 + (lane & 31);
    if (q >= g.Q) continue;
#pragma unroll
    for (int vi = 0; vi < kNF; ++vi)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int64_t p = p0 + wv * kHalf + vi * 32 + 8 * r4 + 4 * half;
        if (p >= g.P) continue;
        const floatx4 v = {acc[vi][ti][4 * r4], acc[vi][ti][4 * r4 + 1],
                           acc[vi][ti][4 * r4 + 2], acc[vi][ti][4 * r4 + 3]};
        if (g.out_kind == kGemmBf16) {
          uint16_t* o = (uint16_t*)g.out + q * g.ldo + p;
          const uint2 w2 = {bf16_bits(v[0]) | (bf16_bits(v[1]) << 16),
                            bf16_bits(v[2]) | (bf16_bits(v[3]) << 16)};
          *(uint2*)o = w2;
        } else {
          floatx4* o = (floatx4*)((float*)g.out + q * g.ldo + p);
          *o = g.out_kind == kGemmF32Accum ? *o + v : v;
        }
      }
  }
}

__global__ __launch_bounds__(kThreads, 1) void det_gemm_nn_kernel(const GemmParams g) {
  det_gemm_body<false, false, 256>(g);
}
__global__ __launch_bounds__(kThreads, 1) void det_gemm_tn_kernel(const GemmParams g) {
  det_gemm_body<true, false, 256>(g);
}
__global__ __launch_bounds__(kThreads, 1) void det_gemm_tt_kernel(const GemmParams g) {
  det_gemm_body<true, true, 256>(g);
}
__global__ __launch_bounds__(kThreads, 1) void det_gemm_nn_t128_kernel(const GemmParams g) {
  det_gemm_body<false, false, 128>(g);
}
__global__ __launch_bounds__(kThreads, 1) void det_gemm_tn_t128_kernel(const GemmParams g) {
  det_gemm_body<true, false, 128>(g);
}
__global__ __launch_bounds__(kThreads, 1) void det_gemm_tt_t128_kernel(const GemmParams g) {
  det_gemm_body<true, true, 128>(g);
}

}  // namespace

hipError_t launch_det_gemm(const GemmParams& g_in, bool x_t, bool y_t, hipStream_t stream) {
  if (!x_t && y_t) return hipErrorInvalidValue;
  // 128 x 128 tiles when 256 x 256 tiles would leave compute units idle
  GemmParams g = g_in;
  const int64_t tiles256 = ((g.P + 255) / 256) * ((g.Q + 255) / 256);
  const int kt = (g.cu_count > 0 && tiles256 < g.cu_count) ? 128 : 256;
  g.Pt = (int32_t)((g.P + kt - 1) / kt);
  g.Qt = (int32_t)((g.Q + kt - 1) / kt);
  const int64_t blocks = (int64_t)g.Pt * g.Qt;
  if (blocks <= 0) return hipSuccess;
  void (*k)(const GemmParams);
  if (kt == 128)
    k = !x_t ? det_gemm_nn_t128_kernel : (y_t ? det_gemm_tt_t128_kernel : det_gemm_tn_t128_kernel);
  else
    k = !x_t ? det_gemm_nn_kernel : (y_t ? det_gemm_tt_kernel : det_gemm_tn_kernel);
  hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(kThreads), 0, stream, g);
  return hipGetLastError();
}

}  // namespace bilogp
