// AddressSanitizer / UndefinedBehaviorSanitizer harness for the library's host
// code (bilogp_host.cpp), built with g++ on the CPU (no GPU, no HIP runtime).
//
// The fake runtime below registers ordinary host buffers as "device memory"
// and replaces every kernel launch with a function that reads and writes
// exactly the bytes the kernel would, computed from the launch parameters
// the host code prepared (ProjParams / GemmParams).  Each touched range must
// also lie inside the buffer it belongs to.  So the sanitizers check, on real
// memory, the host code's argument validation, launch planning (row blocks,
// split runs, row chunks), workspace layout, the shifted weight / bias base of
// a vocabulary-range launch, and its error paths.
//
// Build (tests/test_host_asan.py does this): g++ -std=c++17 -g -O1
// -fsanitize=address,undefined -fno-sanitize-recover=all with include paths
// tests/host_asan/fake_hip, include and invariant_linear_log_amd/csrc, on
// bilogp_host.cpp and this file.
//
// Prints "host harness: N cases passed" and exits 0, or reports the first
// failure and exits 1 (a sanitizer report aborts on its own).

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <string>
#include <vector>

#include "bilogp.h"
#include "bilogp_internal.h"

// ------------------------------------------------------------------ fake runtime
namespace {

std::map<uintptr_t, size_t> g_device;   // base -> bytes of "device" allocations
int g_cu_count = 256;
int g_launches = 0;

bool on_device(const void* p) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  auto it = g_device.upper_bound(a);
  if (it == g_device.begin()) return false;
  --it;
  return a >= it->first && a < it->first + it->second;
}

void fail_now(const std::string& msg) {
  fprintf(stderr, "host harness FAILED: %s\n", msg.c_str());
  exit(1);
}

// The buffer a kernel access must stay in: [lo, hi).
struct Span {
  const void* p = nullptr;
  size_t bytes = 0;
};

// Touch [p, p + bytes) as a read (summed into a sink, so the compiler keeps
// it) or a write (a fixed byte pattern), after checking it lies in `in`.
volatile uint32_t g_sink;

void touch(uintptr_t p, size_t bytes, const Span& in, bool write, const char* what) {
  if (bytes == 0) return;
  const uintptr_t lo = reinterpret_cast<uintptr_t>(in.p);
  if (!in.p || p < lo || p + bytes > lo + in.bytes)
    fail_now(std::string("kernel access outside its buffer: ") + what);
  uint8_t* q = reinterpret_cast<uint8_t*>(p);
  if (write) {
    memset(q, 0x3c, bytes);
  } else {
    uint32_t s = 0;
    for (size_t i = 0; i < bytes; i += 64) s += q[i];
    s += q[bytes - 1];
    g_sink = g_sink + s;
  }
}

}  // namespace

hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}

hipError_t hipGetDeviceProperties(hipDeviceProp_t* prop, int) {
  memset(prop, 0, sizeof(*prop));
  strcpy(prop->gcnArchName, "gfx950:sramecc+:xnack-");
  prop->multiProcessorCount = g_cu_count;
  return hipSuccess;
}

hipError_t hipPointerGetAttributes(hipPointerAttribute_t* attr, const void* ptr) {
  if (!on_device(ptr)) return hipErrorInvalidValue;
  attr->type = hipMemoryTypeDevice;
  attr->device = 0;
  return hipSuccess;
}

hipError_t hipGetLastError(void) { return hipSuccess; }

const char* hipGetErrorString(hipError_t) { return "fake runtime error"; }

hipError_t hipMallocAsync(void** ptr, size_t bytes, hipStream_t) {
  void* p = aligned_alloc(256, (bytes + 255) / 256 * 256);
  if (!p) return hipErrorOutOfMemory;
  g_device[reinterpret_cast<uintptr_t>(p)] = bytes;
  *ptr = p;
  return hipSuccess;
}

hipError_t hipFreeAsync(void* ptr, hipStream_t) {
  g_device.erase(reinterpret_cast<uintptr_t>(ptr));
  free(ptr);
  return hipSuccess;
}

hipError_t hipGetSymbolAddress(void** ptr, const void* symbol) {
  *ptr = const_cast<void*>(symbol);
  g_device[reinterpret_cast<uintptr_t>(symbol)] = bilogp_noalloc_max_workspace_bytes();
  return hipSuccess;
}

// ------------------------------------------------------------------ the case's buffers
namespace {

struct CaseBufs {
  Span hidden, weight, target, bias, logp, lse, ws;
  int64_t n_total = 0;     // rows of the whole call (a launch may cover a chunk)
  Span lse_in, g_logp, g_lse, gh, gw, gb;
  Span gx, gy, gout;
} g_bufs;

// The registered allocation that contains p (the workspace, the library's
// scratch array, or a caller buffer); empty if none does.
Span ws_span_for(const void* p) {
  if (on_device(p)) {
    auto it = g_device.upper_bound(reinterpret_cast<uintptr_t>(p));
    --it;
    return Span{reinterpret_cast<const void*>(it->first), it->second};
  }
  return Span{};
}

// Workgroup -> (row block, split run): the projection kernel's block order
// (a phase of runs of spg splits over [split0, splitA), then one of single
// splits over [splitA, split1); in each, blocks round-robin over eight XCDs,
// then groups of four row blocks x all runs), restated here to check that
// every launch visits each (row block, split) of its range exactly once.
struct BlockWork {
  int rb, split_first, split_last;
};

std::vector<BlockWork> block_order(const bilogp::ProjParams& p) {
  if (p.split0 > p.splitA || p.splitA > p.split1) fail_now("phase bounds");
  if (p.runsA != (p.splitA - p.split0 + p.spg - 1) / p.spg) fail_now("phase A run count");
  const int nA = p.R * p.runsA;
  const int nblk_all = nA + p.R * (p.split1 - p.splitA);
  std::vector<BlockWork> out;
  std::vector<uint8_t> seen((size_t)p.R * (p.split1 - p.split0), 0);
  for (int b = 0; b < nblk_all; ++b) {
    const bool ph_b = b >= nA;
    const int s_lo = ph_b ? p.splitA : p.split0;
    const int s_hi = ph_b ? p.split1 : p.splitA;
    const int spg = ph_b ? 1 : p.spg;
    const int sg = ph_b ? p.split1 - p.splitA : p.runsA;
    const int nblk = p.R * sg;
    const int per_xcd = nblk >> 3;
    int u = ph_b ? b - nA : b;
    if (u < (per_xcd << 3)) u = (u & 7) * per_xcd + (u >> 3);
    const int in_group = 4 * sg;
    const int first_rb = (u / in_group) * 4;
    const int group_rbs = std::min(p.R - first_rb, 4);
    const int rb = first_rb + (u % in_group) % group_rbs;
    const int sf = s_lo + (u % in_group) / group_rbs * spg;
    const int sl = std::min(sf + spg, s_hi);
    if (rb < 0 || rb >= p.R || sf < s_lo || sf >= s_hi) fail_now("block order out of range");
    for (int sp = sf; sp < sl; ++sp) {
      uint8_t& v = seen[(size_t)rb * (p.split1 - p.split0) + (sp - p.split0)];
      if (v) fail_now("block order visits a tile twice");
      v = 1;
    }
    out.push_back(BlockWork{rb, sf, sl});
  }
  for (uint8_t v : seen)
    if (!v) fail_now("block order misses a tile");
  return out;
}

// (row, split) pairs whose partial the launches of one call wrote; rows are
// absolute (from the target pointer's offset into the caller's buffer)
std::vector<uint8_t> g_cover;
int64_t g_cover_S = 0;

void cover_begin(int64_t N, int64_t S) {
  g_cover.assign((size_t)(N * S), 0);
  g_cover_S = S;
}

void cover_mark(int64_t row, int split) {
  if (g_cover.empty()) return;
  uint8_t& v = g_cover[(size_t)(row * g_cover_S + split)];
  if (v) fail_now("a partial is written by two workgroups");
  v = 1;
}

// every row's partials of splits [s0, s1) written exactly once, no other
void cover_check(const std::string& tag, int s0, int s1) {
  for (size_t i = 0; i < g_cover.size(); ++i) {
    const int sp = (int)(i % (size_t)g_cover_S);
    if (g_cover[i] != (sp >= s0 && sp < s1 ? 1 : 0))
      fail_now(tag + ": partial coverage differs at row " + std::to_string(i / g_cover_S) +
               ", split " + std::to_string(sp));
  }
  std::fill(g_cover.begin(), g_cover.end(), 0);
}

}  // namespace

// ------------------------------------------------------------------ kernel footprints
namespace bilogp {

hipError_t launch_bias_f32(const void* bias, int32_t kind, int32_t V, float* out, hipStream_t) {
  ++g_launches;
  const size_t esz = kind == kBiasF32 ? 4 : 2;
  const int32_t padded = (V + kVtileCols - 1) / kVtileCols * kVtileCols;
  touch(reinterpret_cast<uintptr_t>(bias), (size_t)V * esz, g_bufs.bias, false, "bias");
  touch(reinterpret_cast<uintptr_t>(out), (size_t)padded * 4, ws_span_for(out), true, "bias copy");
  return hipSuccess;
}

static void proj_footprint(const ProjParams& p, bool grad) {
  ++g_launches;
  if (p.rows != 128 && p.rows != 256) fail_now("row block height");
  if ((int64_t)p.R != (p.N + p.rows - 1) / p.rows) fail_now("row block count");
  if ((uint64_t)p.R * (p.runsA + p.split1 - p.splitA) * 512 > UINT32_MAX)
    fail_now("grid exceeds 32-bit work items");
  const std::vector<BlockWork> blocks = block_order(p);
  const int64_t row_base = reinterpret_cast<const int64_t*>(p.target) -
                           static_cast<const int64_t*>(g_bufs.target.p);
  const uintptr_t H2 = (uintptr_t)p.H * 2;
  touch(reinterpret_cast<uintptr_t>(p.hidden), (size_t)p.N * H2, g_bufs.hidden, false, "hidden");
  touch(reinterpret_cast<uintptr_t>(p.target), (size_t)p.N * 8, g_bufs.target, false, "target");
  // with a caller workspace, partials and target logits must stay in their
  // own regions of its layout ([N, S] pairs first, then [N] floats, each
  // 256-byte aligned); otherwise the containing allocation bounds them
  Span part_span = ws_span_for(p.part), tl_span = ws_span_for(p.tlogit);
  if (g_bufs.ws.p && g_bufs.n_total > 0 && part_span.p == g_bufs.ws.p) {
    const size_t pb = (size_t)g_bufs.n_total * p.S * 8;
    part_span = Span{g_bufs.ws.p, pb};
    tl_span = Span{static_cast<const uint8_t*>(g_bufs.ws.p) + (pb + 255) / 256 * 256,
                   (size_t)g_bufs.n_total * 4};
  }
  // the kernel reads the caller's bias (fp32 or bf16) or the fp32 copy in the
  // workspace; either way from col0 on, addressed by absolute column
  const uintptr_t besz = p.bias_src == kBiasSrcBf16 ? 2 : 4;
  if ((p.bias != nullptr) != (p.bias_src != kBiasSrcNone)) fail_now("bias source");
  if (p.bias_copy && p.bias_src != kBiasSrcF32) fail_now("the bias copy is fp32");
  const Span b_span = !p.bias ? Span{}
                      : p.bias_copy ? ws_span_for(reinterpret_cast<const void*>(
                                          reinterpret_cast<uintptr_t>(p.bias) + p.col0 * besz))
                                    : g_bufs.bias;
  if (p.bias && !p.bias_copy &&
      (reinterpret_cast<uintptr_t>(p.bias) + p.col0 * besz) % 16 != 0)
    fail_now("a direct bias read from a base that is not 16-byte aligned");
  if (p.bias && !p.bias_copy && (p.V * besz) % 16 != 0)
    fail_now("a direct bias read whose last 16-byte chunk is cut by V");
  if (grad) {
    touch(reinterpret_cast<uintptr_t>(p.lse), (size_t)p.N * 4, g_bufs.lse_in, false, "lse");
    touch(reinterpret_cast<uintptr_t>(p.g_logp), (size_t)p.N * 4, g_bufs.g_logp, false, "g_logp");
    touch(reinterpret_cast<uintptr_t>(p.g_lse), (size_t)p.N * 4, g_bufs.g_lse, false, "g_lse");
  }
  const int64_t* tgt = p.target;
  for (const BlockWork& bw : blocks) {
    const int64_t m0 = (int64_t)bw.rb * p.rows;
    const int rows_here = (int)std::min<int64_t>(p.rows, p.N - m0);
    if (rows_here < 1) fail_now("a row block without rows");
    {
      const int split_first = bw.split_first, split_last = bw.split_last;
      for (int j = 0; j < rows_here; ++j)
        for (int sp = split_first; sp < split_last; ++sp) cover_mark(row_base + m0 + j, sp);
      const int vt_begin = split_first * p.vps;
      const int vt_end = std::min(split_last * p.vps, p.T);
      for (int vt = vt_begin; vt < vt_end; ++vt) {
        const int vbase = vt * kVtileCols;
        const int vrows = std::min(kVtileCols, p.V - vbase);
        // weight rows of the tile (absolute column addressing from p.weight)
        touch(reinterpret_cast<uintptr_t>(p.weight) + (uintptr_t)vbase * H2, (size_t)vrows * H2,
              g_bufs.weight, false, "weight");
        if (p.bias)
          touch(reinterpret_cast<uintptr_t>(p.bias) + (uintptr_t)vbase * besz,
                (size_t)vrows * besz, b_span, false, p.bias_copy ? "bias copy (read)" : "bias");
        if (grad)
          for (int j = 0; j < rows_here; ++j)
            for (int c = 0; c < vrows; ++c)
              touch(reinterpret_cast<uintptr_t>(p.dzt + (vbase + c) * p.ldz + m0 + j), 2,
                    ws_span_for(p.dzt), true, "dZ^T");
      }
      if (grad) continue;
      for (int j = 0; j < rows_here; ++j) {
        for (int sp = split_first; sp < split_last; ++sp)
          touch(reinterpret_cast<uintptr_t>(p.part + (m0 + j) * p.S + sp), 8, part_span, true,
                "partials");
        const int64_t t = tgt[m0 + j];
        const int64_t c0 = (int64_t)vt_begin * kVtileCols, c1 = std::min<int64_t>(
                                                                 (int64_t)vt_end * kVtileCols, p.V);
        if (t >= c0 && t < c1)
          touch(reinterpret_cast<uintptr_t>(p.tlogit + m0 + j), 4, tl_span, true, "target logit");
      }
    }
  }
}

// What the projection launches of one call looked like: row-block height and
// splits per workgroup of the first launch, workgroups summed over row chunks.
struct LaunchSeen {
  int rows = 0, spg = 0, launches = 0;
  int64_t workgroups = 0;
} g_seen;

hipError_t launch_proj_lse(const ProjParams& p, hipStream_t) {
  proj_footprint(p, false);
  const bool tail = p.rows == 128 && p.spg == 1 && p.splitA == p.split1 && g_seen.launches > 0 &&
                    g_seen.rows == 256;
  if (g_seen.launches++ == 0) {
    g_seen.rows = p.rows;
    g_seen.spg = p.spg;
  } else if (!tail && (g_seen.rows != p.rows || g_seen.spg != p.spg)) {
    g_seen.rows = -1;     // row chunks of one call must share the plan
  }
  g_seen.workgroups += (int64_t)p.R * (p.runsA + p.split1 - p.splitA);
  return hipSuccess;
}

hipError_t launch_softmax_grad(const ProjParams& p, hipStream_t) {
  proj_footprint(p, true);
  return hipSuccess;
}

hipError_t launch_zero_pad_cols(uint16_t* dzt, int64_t rows, int64_t N, int64_t ldz, hipStream_t) {
  ++g_launches;
  for (int64_t r = 0; r < rows; ++r)
    touch(reinterpret_cast<uintptr_t>(dzt + r * ldz + N), (size_t)(ldz - N) * 2, ws_span_for(dzt),
          true, "dZ^T padding");
  return hipSuccess;
}

hipError_t launch_row_sums(const uint16_t* dzt, int64_t rows, int64_t N, int64_t ldz, float* out,
                           hipStream_t) {
  ++g_launches;
  for (int64_t r = 0; r < rows; ++r)
    touch(reinterpret_cast<uintptr_t>(dzt + r * ldz), (size_t)N * 2, ws_span_for(dzt), false,
          "dZ^T rows");
  touch(reinterpret_cast<uintptr_t>(out), (size_t)rows * 4, g_bufs.gb, true, "grad_bias");
  return hipSuccess;
}

hipError_t launch_merge(const float2* part, const float* tlogit, const int64_t* target,
                        float* logp, float* lse, int64_t N, int32_t S, int32_t, hipStream_t) {
  ++g_launches;
  if (N * 64 > (int64_t)UINT32_MAX) fail_now("merge grid exceeds 32-bit work items");
  Span part_span = ws_span_for(part), tl_span = ws_span_for(tlogit);
  if (g_bufs.ws.p && g_bufs.n_total > 0 && part_span.p == g_bufs.ws.p) {
    const size_t pb = (size_t)g_bufs.n_total * S * 8;
    part_span = Span{g_bufs.ws.p, pb};
    tl_span = Span{static_cast<const uint8_t*>(g_bufs.ws.p) + (pb + 255) / 256 * 256,
                   (size_t)g_bufs.n_total * 4};
  }
  touch(reinterpret_cast<uintptr_t>(part), (size_t)N * S * 8, part_span, false, "partials");
  touch(reinterpret_cast<uintptr_t>(tlogit), (size_t)N * 4, tl_span, false, "tlogit");
  touch(reinterpret_cast<uintptr_t>(target), (size_t)N * 8, g_bufs.target, false, "target");
  touch(reinterpret_cast<uintptr_t>(logp), (size_t)N * 4, g_bufs.logp, true, "logp");
  touch(reinterpret_cast<uintptr_t>(lse), (size_t)N * 4, g_bufs.lse, true, "lse");
  return hipSuccess;
}

hipError_t launch_det_gemm(const GemmParams& g, bool x_t, bool y_t, hipStream_t) {
  ++g_launches;
  const size_t oe = g.out_kind == kGemmBf16 ? 2 : 4;
  // X[p][c] (natural: x + p ldx + c; transposed: x + c ldx + p), likewise Y
  auto operand = [&](const void* base, int64_t rows, int64_t ld, bool tr, const Span& in,
                     const char* what) {
    const uintptr_t b = reinterpret_cast<uintptr_t>(base);
    if (!tr) {
      for (int64_t r = 0; r < rows; ++r) touch(b + (uintptr_t)(r * ld) * 2, (size_t)g.C * 2, in, false, what);
    } else {
      for (int64_t c = 0; c < g.C; ++c) touch(b + (uintptr_t)(c * ld) * 2, (size_t)rows * 2, in, false, what);
    }
  };
  operand(g.x, g.P, g.ldx, x_t, ws_span_for(g.x), "gemm X");
  operand(g.y, g.Q, g.ldy, y_t, ws_span_for(g.y), "gemm Y");
  const Span out_span = ws_span_for(g.out);
  for (int64_t q = 0; q < g.Q; ++q) {
    const uintptr_t o = reinterpret_cast<uintptr_t>(g.out) + (uintptr_t)(q * g.ldo) * oe;
    if (g.out_kind == kGemmF32Accum) touch(o, (size_t)g.P * oe, out_span, false, "gemm out (accumulate)");
    touch(o, (size_t)g.P * oe, out_span, true, "gemm out");
  }
  return hipSuccess;
}

}  // namespace bilogp

// ------------------------------------------------------------------ cases
namespace {

struct Buf {
  void* p = nullptr;
  size_t n = 0;
  explicit Buf(size_t bytes, bool device = true) : n(bytes) {
    p = aligned_alloc(256, (bytes + 255) / 256 * 256 + 256);
    memset(p, 0, (bytes + 255) / 256 * 256 + 256);
    if (device) g_device[reinterpret_cast<uintptr_t>(p)] = bytes;
  }
  ~Buf() {
    g_device.erase(reinterpret_cast<uintptr_t>(p));
    free(p);
  }
  Buf(const Buf&) = delete;
  Buf& operator=(const Buf&) = delete;
  Span span() const { return Span{p, n}; }
};

int g_cases = 0;

void expect(int got, int want, const std::string& what) {
  if (got != want)
    fail_now(what + ": status " + std::to_string(got) + ", expected " + std::to_string(want) +
             " (" + bilogp_last_error() + ")");
  ++g_cases;
}

void fill_targets(Buf& t, int64_t N, int64_t V, uint32_t seed) {
  int64_t* p = static_cast<int64_t*>(t.p);
  uint32_t x = seed * 2654435761u + 1;
  for (int64_t i = 0; i < N; ++i) {
    x = x * 1664525u + 1013904223u;
    p[i] = (int64_t)(x % (uint32_t)V);
  }
  if (N > 0) p[0] = 0;
  if (N > 1) p[N - 1] = V - 1;
}

// One forward through forward_ex / forward_mode / forward / forward_noalloc,
// and the two halves, with exact-size buffers.
void forward_case(int64_t N, int64_t H, int64_t V, int bias_dtype, int mode, int cu) {
  const std::string tag = "forward N=" + std::to_string(N) + " H=" + std::to_string(H) +
                          " V=" + std::to_string(V) + " bias=" + std::to_string(bias_dtype) +
                          " mode=" + std::to_string(mode) + " cu=" + std::to_string(cu);
  Buf h((size_t)N * H * 2), w((size_t)V * H * 2), t((size_t)N * 8), lp((size_t)N * 4),
      ls((size_t)N * 4);
  const size_t besz = bias_dtype == BILOGP_BIAS_F32 ? 4 : 2;
  Buf b(bias_dtype == BILOGP_BIAS_NONE ? 1 : (size_t)V * besz);
  fill_targets(t, N, V, (uint32_t)(N + V));
  const size_t need = bilogp_workspace_bytes_mode(N, V, mode, cu);
  Buf ws(need ? need : 1);
  g_bufs = CaseBufs{};
  g_bufs.hidden = h.span();
  g_bufs.weight = w.span();
  g_bufs.target = t.span();
  g_bufs.bias = b.span();
  g_bufs.logp = lp.span();
  g_bufs.lse = ls.span();
  g_bufs.ws = ws.span();
  g_bufs.n_total = N;
  const void* bias = bias_dtype == BILOGP_BIAS_NONE ? nullptr : b.p;
  bilogp::g_seen = bilogp::LaunchSeen{};
  const int s_mode = N > 0 ? bilogp_num_vocab_splits_mode(N, V, mode, cu) : 0;
  const int s_inv = bilogp_num_vocab_splits(V);
  cover_begin(N, s_mode);
  expect(bilogp_forward_mode(h.p, w.p, (const int64_t*)t.p, bias, bias_dtype, (float*)lp.p, (float*)ls.p, N, H,
                             V, mode, cu, ws.p, need, nullptr),
         BILOGP_OK, tag + " forward_mode");
  cover_check(tag + " forward_mode", 0, s_mode);
  if (N > 0 && cu > 0) {
    // bilogp_launch_plan describes exactly what bilogp_forward_mode launched
    int rows = 0, spg = 0;
    int64_t wgs = 0;
    if (bilogp_launch_plan(N, H, V, mode, cu, &rows, &spg, &wgs) != 0)
      fail_now(tag + ": launch plan refused valid arguments");
    const bilogp::LaunchSeen& seen = bilogp::g_seen;
    if (rows != seen.rows || spg != seen.spg || wgs != seen.workgroups)
      fail_now(tag + ": launch plan (" + std::to_string(rows) + ", " + std::to_string(spg) +
                ", " + std::to_string(wgs) + ") differs from the launch (" +
                std::to_string(seen.rows) + ", " + std::to_string(seen.spg) + ", " +
                std::to_string(seen.workgroups) + ")");
  }
  if (mode == BILOGP_SPLITS_INVARIANT) {
    cover_begin(N, s_inv);
    expect(bilogp_forward_ex(h.p, w.p, (const int64_t*)t.p, bias, bias_dtype, (float*)lp.p, (float*)ls.p, N, H, V,
                             ws.p, need, nullptr),
           BILOGP_OK, tag + " forward_ex");
    cover_check(tag + " forward_ex", 0, s_inv);
    expect(bilogp_partials(h.p, w.p, (const int64_t*)t.p, bias, bias_dtype, N, H, V, ws.p, need, nullptr),
           BILOGP_OK, tag + " partials");
    cover_check(tag + " partials", 0, s_inv);
    expect(bilogp_merge((const int64_t*)t.p, ws.p, need, (float*)lp.p, (float*)ls.p, N, V, nullptr),
           BILOGP_OK, tag + " merge");
    cover_check(tag + " merge", 0, 0);
    g_bufs.ws = Span{};   // library-owned workspaces from here on
    if (bias_dtype != BILOGP_BIAS_BF16) {
      expect(bilogp_forward(h.p, w.p, (const int64_t*)t.p, (const float*)bias, (float*)lp.p,
                            (float*)ls.p, N, H, V, nullptr),
             BILOGP_OK, tag + " forward");
      cover_check(tag + " forward", 0, s_inv);
    }
    if (need <= bilogp_noalloc_max_workspace_bytes()) {
      expect(bilogp_forward_noalloc(h.p, w.p, (const int64_t*)t.p, bias, bias_dtype, (float*)lp.p,
                                    (float*)ls.p, N, H, V, nullptr),
             BILOGP_OK, tag + " forward_noalloc");
      cover_check(tag + " forward_noalloc", 0, s_inv);
    }
  }
  g_cover.clear();
}

// Vocabulary-range partials from an exact-size weight (and bias) slice.
void range_case(int64_t N, int64_t H, int64_t V, int s0, int s1, int bias_dtype) {
  const std::string tag = "range N=" + std::to_string(N) + " V=" + std::to_string(V) + " [" +
                          std::to_string(s0) + "," + std::to_string(s1) + ")";
  const int vps = bilogp_vtiles_per_split(V);
  const int64_t c0 = (int64_t)s0 * vps * 256, c1 = std::min<int64_t>((int64_t)s1 * vps * 256, V);
  Buf h((size_t)N * H * 2), w((size_t)(c1 - c0) * H * 2), t((size_t)N * 8);
  const size_t besz = bias_dtype == BILOGP_BIAS_F32 ? 4 : 2;
  Buf b(bias_dtype == BILOGP_BIAS_NONE ? 1 : (size_t)(c1 - c0) * besz);
  fill_targets(t, N, V, (uint32_t)(s0 * 7 + s1));
  const size_t need = bilogp_workspace_bytes(N, V);
  Buf ws(need);
  g_bufs = CaseBufs{};
  g_bufs.hidden = h.span();
  g_bufs.weight = w.span();
  g_bufs.target = t.span();
  g_bufs.bias = b.span();
  g_bufs.ws = ws.span();
  g_bufs.n_total = N;
  cover_begin(N, bilogp_num_vocab_splits(V));
  expect(bilogp_partials_range(h.p, w.p, (const int64_t*)t.p,
                               bias_dtype == BILOGP_BIAS_NONE ? nullptr : b.p, bias_dtype, N, H,
                               V, s0, s1, ws.p, need, nullptr),
         BILOGP_OK, tag);
  cover_check(tag, s0, s1);
  g_cover.clear();
}

void backward_case(int64_t N, int64_t H, int64_t V, int bias_dtype, bool with_gb) {
  const std::string tag = "backward N=" + std::to_string(N) + " H=" + std::to_string(H) +
                          " V=" + std::to_string(V);
  Buf h((size_t)std::max<int64_t>(N, 1) * H * 2), w((size_t)V * H * 2),
      t((size_t)std::max<int64_t>(N, 1) * 8), l((size_t)std::max<int64_t>(N, 1) * 4),
      gl((size_t)std::max<int64_t>(N, 1) * 4), gs((size_t)std::max<int64_t>(N, 1) * 4),
      gh((size_t)std::max<int64_t>(N, 1) * H * 4), gw((size_t)V * H * 4), gb((size_t)V * 4);
  const size_t besz = bias_dtype == BILOGP_BIAS_F32 ? 4 : 2;
  Buf b(bias_dtype == BILOGP_BIAS_NONE ? 1 : (size_t)V * besz);
  fill_targets(t, N, V, 3);
  const size_t need = bilogp_backward_workspace_bytes(N, V);
  Buf ws(need);
  g_bufs = CaseBufs{};
  g_bufs.hidden = h.span();
  g_bufs.weight = w.span();
  g_bufs.target = t.span();
  g_bufs.bias = b.span();
  g_bufs.lse_in = l.span();
  g_bufs.g_logp = gl.span();
  g_bufs.g_lse = gs.span();
  g_bufs.gb = gb.span();
  g_bufs.ws = ws.span();
  cover_begin(N, bilogp_num_vocab_splits(V));
  expect(bilogp_backward(h.p, w.p, (const int64_t*)t.p,
                         bias_dtype == BILOGP_BIAS_NONE ? nullptr : b.p, bias_dtype,
                         (const float*)l.p, (const float*)gl.p, (const float*)gs.p, (float*)gh.p,
                         (float*)gw.p, with_gb ? (float*)gb.p : nullptr, N, H, V, ws.p, need,
                         nullptr),
         BILOGP_OK, tag);
  cover_check(tag, 0, bilogp_num_vocab_splits(V));
  g_cover.clear();
}

void gemm_case(int64_t M, int64_t N, int64_t K, int kind) {
  const std::string tag = "det_gemm M=" + std::to_string(M) + " N=" + std::to_string(N) +
                          " K=" + std::to_string(K) + " kind=" + std::to_string(kind);
  const size_t oe = kind == BILOGP_GEMM_OUT_BF16 ? 2 : 4;
  const size_t m = (size_t)std::max<int64_t>(M, 1);
  Buf a(m * K * 2), b((size_t)N * K * 2), c(m * N * oe), dc(m * N * 2), da(m * K * oe),
      db((size_t)N * K * oe);
  g_bufs = CaseBufs{};
  expect(bilogp_det_gemm_fwd(a.p, b.p, c.p, M, N, K, kind, nullptr), BILOGP_OK, tag + " fwd");
  expect(bilogp_det_gemm_da(dc.p, b.p, da.p, M, N, K, kind, nullptr), BILOGP_OK, tag + " da");
  expect(bilogp_det_gemm_db(a.p, dc.p, db.p, M, N, K, kind, nullptr), BILOGP_OK, tag + " db");
}

}  // namespace

int main() {
  // The library reads the device's compute-unit count once, at its first
  // call: 256 here.  Other counts reach the plans through forward_mode's
  // explicit count (forward_ex and the rest schedule for the device's).
  g_cu_count = 256;
  forward_case(0, 64, 1000, BILOGP_BIAS_NONE, BILOGP_SPLITS_INVARIANT, 0);
  // forward, all split modes and launch plans (few / many compute units)
  for (int cu : {1, 80, 256, 1024}) {
    forward_case(8, 64, 1000, BILOGP_BIAS_NONE, BILOGP_SPLITS_INVARIANT, cu);
    forward_case(300, 200, 2000, BILOGP_BIAS_F32, BILOGP_SPLITS_INVARIANT, cu);
    forward_case(513, 64, 257, BILOGP_BIAS_BF16, BILOGP_SPLITS_INVARIANT, cu);
    forward_case(1, 16, 128256, BILOGP_BIAS_NONE, BILOGP_SPLITS_INVARIANT, cu);
    forward_case(4096, 8, 151936, BILOGP_BIAS_BF16, BILOGP_SPLITS_INVARIANT, cu);
    forward_case(777, 8, 70001, BILOGP_BIAS_F32, BILOGP_SPLITS_THROUGHPUT, cu);
    forward_case(37, 16, 128256, BILOGP_BIAS_NONE, BILOGP_SPLITS_THROUGHPUT, cu);
    forward_case(5, 8, 1, BILOGP_BIAS_NONE, BILOGP_SPLITS_INVARIANT, cu);
  }
  // vocabulary ranges: exact-size weight and bias slices (the shifted base)
  for (auto r : std::vector<std::pair<int, int>>{{0, 1}, {0, 251}, {7, 9}, {250, 251}, {100, 200}})
    for (int bd : {BILOGP_BIAS_NONE, BILOGP_BIAS_BF16, BILOGP_BIAS_F32})
      range_case(300, 16, 128256, r.first, r.second, bd);
  range_case(1, 8, 16385, 32, 33, BILOGP_BIAS_F32);
  // split schedules with a second, 128-token launch (whole rounds of the big
  // launch, the remainder as half-height pieces), forward and backward
  // bias read directly (V a whole number of 16-byte chunks) or through the copy
  forward_case(40, 16, 1004, BILOGP_BIAS_BF16, BILOGP_SPLITS_INVARIANT, 256);
  forward_case(40, 16, 1004, BILOGP_BIAS_F32, BILOGP_SPLITS_INVARIANT, 256);
  forward_case(4000, 1024, 50257, BILOGP_BIAS_F32, BILOGP_SPLITS_INVARIANT, 256);
  forward_case(4000, 1024, 50257, BILOGP_BIAS_NONE, BILOGP_SPLITS_INVARIANT, 80);
  backward_case(1024, 1024, 20480, BILOGP_BIAS_BF16, true);
  // backward (the softmax-gradient footprint, padding, row sums)
  backward_case(7, 16, 1000, BILOGP_BIAS_NONE, false);
  backward_case(300, 8, 2003, BILOGP_BIAS_BF16, true);
  backward_case(0, 8, 1000, BILOGP_BIAS_F32, true);
  // deterministic GEMM: forward, dA, dB, every output kind
  for (int kind : {BILOGP_GEMM_OUT_BF16, BILOGP_GEMM_OUT_F32, BILOGP_GEMM_OUT_F32_ACCUM}) {
    gemm_case(37, 64, 40, kind);
    gemm_case(300, 264, 520, kind);
    gemm_case(0, 16, 8, kind);
  }
  // fail-closed paths (no launch): a bad size, a missing workspace, an alias
  {
    Buf h(8 * 64 * 2), w(1000 * 64 * 2), t(8 * 8), lp(32), ls(32);
    g_bufs = CaseBufs{};
    expect(bilogp_forward_ex(h.p, w.p, (const int64_t*)t.p, nullptr, 0, (float*)lp.p, (float*)ls.p,
                             8, 60, 1000, nullptr, 0, nullptr),
           BILOGP_E_UNSUPPORTED, "H % 8");
    expect(bilogp_forward_ex(h.p, w.p, (const int64_t*)t.p, nullptr, 0, (float*)lp.p, (float*)ls.p,
                             8, 64, 1000, nullptr, 0, nullptr),
           BILOGP_E_WORKSPACE, "no workspace");
    expect(bilogp_forward_ex(h.p, w.p, (const int64_t*)t.p, nullptr, 0, (float*)lp.p, (float*)lp.p,
                             8, 64, 1000, nullptr, 0, nullptr),
           BILOGP_E_INVALID_ARG, "outputs alias");
    Buf host_only(1 << 20, false);
    expect(bilogp_forward_ex(h.p, w.p, (const int64_t*)t.p, nullptr, 0, (float*)lp.p, (float*)ls.p,
                             8, 64, 1000, host_only.p, 1 << 20, nullptr),
           BILOGP_E_UNSUPPORTED, "host workspace");
  }
  printf("host harness: %d cases passed, %d launches checked\n", g_cases, g_launches);
  return 0;
}
