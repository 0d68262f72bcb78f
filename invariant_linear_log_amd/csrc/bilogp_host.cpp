// C ABI of the batch-invariant fused linear log-probability forward:
// argument validation (fail closed), the gfx950 gate, the V-only split
// policy, workspace layout and the two launches.  Never synchronizes.
//
// RL-Kernel PR #337, "feat(linear-logp): add batch-invariant fused SM90
// operator": the native entry point takes hidden, weight, target and an
// optional bias and returns the log-probability and log-sum-exp (sequence
// diagram); the split count comes from V only (annotation on
// select_batch_invariant_vocab_splits); an unsupported platform is an
// explicit error, never a generic fallback (annotation on the registry entry).

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <string>

#include "../../include/bilogp.h"
#include "bilogp_internal.h"

namespace {

thread_local std::string g_last_error;

bilogp_status fail(bilogp_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

constexpr int64_t kMaxV = int64_t(1) << 30;
constexpr int64_t kMaxH = int64_t(1) << 20;
constexpr int64_t kMaxN = int64_t(1) << 32;
constexpr int kMaxCuCount = 65536;
constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// V rounded up to whole vocabulary tiles.
size_t padded_vocab(int64_t V) {
  return (size_t)((V + bilogp::kVtileCols - 1) / bilogp::kVtileCols) * bilogp::kVtileCols;
}

// Workspace layout: [N, S] float2 partials | [N] float target logits |
// fp32 bias copy padded to whole tiles; each part 256-byte aligned.
struct WsLayout {
  float2* part;
  float* tlogit;
  float* bias32;
};

WsLayout ws_layout(void* ws, int64_t N, int S) {
  char* b = static_cast<char*>(ws);
  const size_t o1 = round_up((size_t)N * S * sizeof(float2));
  const size_t o2 = o1 + round_up((size_t)N * sizeof(float));
  return WsLayout{reinterpret_cast<float2*>(b), reinterpret_cast<float*>(b + o1),
                  reinterpret_cast<float*>(b + o2)};
}

// Per-device result of the architecture check: 0 unknown, 1 gfx950, 2 other;
// and the device's compute-unit count (0 unknown).
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];
std::atomic<int> g_cu_count[kMaxDevices];

bilogp_status check_device(int* dev_out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0)
    return fail(BILOGP_E_UNSUPPORTED, std::string("no usable HIP device: ") + hipGetErrorString(e));
  if (dev >= kMaxDevices) return fail(BILOGP_E_UNSUPPORTED, "device index out of range");
  int st = g_arch_ok[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return fail(BILOGP_E_HIP, std::string("hipGetDeviceProperties: ") + hipGetErrorString(e));
    st = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_cu_count[dev].store(prop.multiProcessorCount, std::memory_order_release);
    g_arch_ok[dev].store(st, std::memory_order_release);
    if (st != 1)
      return fail(BILOGP_E_UNSUPPORTED,
                  std::string("device architecture is ") + prop.gcnArchName + ", need gfx950");
  }
  if (st != 1) return fail(BILOGP_E_UNSUPPORTED, "device architecture is not gfx950");
  *dev_out = dev;
  return BILOGP_OK;
}

// Consecutive splits per projection workgroup.  It only schedules the work:
// each split's partial is written by the same arithmetic however the splits
// are grouped.  Candidates are 1 .. about kTilesPerRun tiles' worth of
// splits; the host takes the one whose grid, run in whole rounds of one
// workgroup per compute unit, ends first: ceil(R * runs / cu) rounds of that
// many splits each (a grid that leaves units idle scores its idle share too);
// ties go to the longer run (fewer workgroup starts).  (Measured on MI355X
// at H = 4096, V = 128256: runs of 4 tiles beat runs of 2, 8, 16 or 32 from
// N = 256 up, or tie within 1%, where the rounds come out even; with 3 row
// blocks, runs of 2 splits left half of the second round idle and took
// 0.80 ms where runs of 1 split, 3 full rounds, take 0.66 ms.)
constexpr int kTilesPerRun = 4;

int32_t splits_per_run(int64_t R, int nsplits, int vps, int cu) {
  if (nsplits <= 1) return 1;
  const int32_t cap = std::min(std::max(1, kTilesPerRun / std::max(vps, 1)), nsplits);
  if (cu <= 0) return cap;
  int32_t best = 1;
  int64_t best_len = INT64_MAX;
  for (int32_t spg = 1; spg <= cap; ++spg) {
    const int64_t wgs = R * ((nsplits + spg - 1) / spg);
    const int64_t len = (wgs + cu - 1) / cu * spg;
    if (len <= best_len) {
      best_len = len;
      best = spg;
    }
  }
  return best;
}

// K stages a compute unit runs for R row blocks: whole rounds of one
// workgroup per unit, each workgroup a run of splits of vps tiles of kt
// stages (the run length as splits_per_run chooses it).
int64_t plan_stages(int64_t R, int nsplits, int vps, int cu, int64_t kt) {
  const int32_t spg = splits_per_run(R, nsplits, vps, cu);
  const int64_t wgs = R * ((nsplits + spg - 1) / spg);
  return (wgs + cu - 1) / cu * spg * vps * kt;
}

// Row-block height of a projection launch: 256 tokens, or 128 when 256-token
// blocks give fewer workgroups than `cu` compute units and the 128-token
// plan's K stages per compute unit, at 15/32 of the cost of a 256-token stage
// (half the MFMA work and a deeper load pipeline), come out fewer.  K stages
// per tile are ceil(H / 64) rounded up to the buffer count: 2 for 256-token
// blocks, slots128 for 128-token blocks.  (Measured on MI355X: at H = 1024,
// V = 32000, N = 512, one 256-token tile per workgroup, 250 workgroups,
// takes 0.0386 ms against 0.042 ms for two 128-token tiles; at H = 4096,
// V = 128256, 128-token blocks win for N <= 256, e.g. 0.184 against
// 0.225 ms at N = 64.)  A row's arithmetic is the same in either (row blocking
// never changes bits), so the choice may follow N, H and the device.
int32_t row_block_rows(int64_t N, int64_t H, int64_t splits, int vps, int cu, int slots128) {
  const int64_t r256 = (N + 255) / 256;
  if (cu <= 0 || r256 * splits >= cu) return 256;
  const int64_t k = (H + 63) / 64;
  const int64_t kt256 = (k + 1) / 2 * 2;
  const int64_t kt128 = (k + slots128 - 1) / slots128 * slots128;
  const int64_t c256 = plan_stages(r256, (int)splits, vps, cu, kt256);
  const int64_t c128 = plan_stages((N + 127) / 128, (int)splits, vps, cu, kt128);
  return c128 * 15 < c256 * 32 ? 128 : 256;
}

// Schedule of a launch of 256-token row blocks over ns splits of vps tiles:
// splits [0, sa) in runs of spg, [sa, sb) one per workgroup, and [sb, ns) in
// a second launch of 128-token row blocks.  The last round of one workgroup
// per compute unit is what it improves: with R * ns = q * cu + r splits,
// q whole rounds plus r left over, the plain launch (sb = sa = ns) pays a
// whole round for the r; here the big launch stops after whole rounds and
// the r splits, cut in two halves of 128 tokens, fill one round of half
// pieces.  A row's arithmetic is the same in either row-block height, so
// the schedule never changes a bit.  Cost model, in 256-token K stages per
// compute unit: kt256 per tile, 19/32 of one per 128-token stage (measured on
// MI355X with every unit busy: 3.56 ms for 128-token blocks against 2.95 ms
// for 256-token blocks at N = H = 4096, V = 128256, one tile per split), one
// stage per workgroup start (measured: runs of 1 tile instead of 4 cost
// 1.2% there) and three for the second launch.  Runs of single splits
// between the long runs and the short pieces (at least three rounds of
// them) level the end of the big launch.
struct Schedule {
  int32_t spg, sa, sb;
};

Schedule schedule_256(int64_t R, int ns, int vps, int cu, int64_t kt256, int64_t kt128) {
  const int32_t spg = splits_per_run(R, ns, vps, cu);
  Schedule best{spg, ns, ns};
  if (cu <= 0 || R * ns <= cu) return best;
  auto cdiv = [](int64_t a, int64_t b) { return (a + b - 1) / b; };
  const int64_t wgs = R * cdiv(ns, spg);
  int64_t best_cost = 32 * (cdiv(wgs, cu) * spg * vps * kt256 + cdiv(wgs, cu));
  const int32_t cap = std::min(std::max(1, kTilesPerRun / std::max(vps, 1)), ns);
  const int64_t b_min = cdiv(3 * (int64_t)cu, R);       // splits per row block in phase B
  for (int64_t ts = 1; ts < ns && 2 * R * ts <= cu; ++ts) {
    const int64_t sb = ns - ts;
    const int64_t sa = std::max<int64_t>(0, sb - b_min) / cap * cap;
    const int64_t starts = cdiv(R * (sa / cap), cu) + cdiv(R * (sb - sa), cu) + 1;
    const int64_t cost = 32 * (cdiv(R * sb, cu) * vps * kt256 + starts + 3) + 19 * vps * kt128;
    if (cost < best_cost) {
      best_cost = cost;
      best = Schedule{sa > 0 ? cap : 1, (int32_t)sa, (int32_t)sb};
    }
  }
  return best;
}

int device_cus(int dev) { return g_cu_count[dev].load(std::memory_order_acquire); }

// Whether the projection reads the caller's bias directly: 16-byte aligned
// and V a whole number of 16-byte chunks of it, so that the kernel's
// per-tile descriptor (the tile's columns below V) never cuts a chunk.
// Otherwise the host first writes a zero-padded fp32 copy into the
// workspace.  Either way the kernel adds the same fp32 value.
bool bias_direct(int bias_dtype, int64_t V, const void* bias) {
  if (!bias || reinterpret_cast<uintptr_t>(bias) % 16 != 0) return false;
  if (bias_dtype == BILOGP_BIAS_F32) return V % 4 == 0;
  if (bias_dtype == BILOGP_BIAS_BF16) return V % 8 == 0;
  return false;
}

// The kernel's view of a bias: its source kind and base address, shifted back
// by col0 columns (absolute-column addressing), reading the caller's values
// where bias_direct allows, else the fp32 copy at bias32.
void set_bias(bilogp::ProjParams& p, const void* bias, int bias_dtype, int64_t V, int64_t col0,
              float* bias32) {
  p.bias_kind = bias_dtype == BILOGP_BIAS_BF16 ? bilogp::kBiasBf16
                : bias_dtype == BILOGP_BIAS_F32 ? bilogp::kBiasF32
                                                : bilogp::kBiasNone;
  if (!bias) {
    p.bias = nullptr;
    p.bias_src = bilogp::kBiasSrcNone;
    p.bias_copy = 0;
  } else if (bias_direct(bias_dtype, V, bias)) {
    const uintptr_t esz = bias_dtype == BILOGP_BIAS_F32 ? 4 : 2;
    p.bias = reinterpret_cast<const void*>(reinterpret_cast<uintptr_t>(bias) - (uintptr_t)col0 * esz);
    p.bias_src = bias_dtype == BILOGP_BIAS_F32 ? bilogp::kBiasSrcF32 : bilogp::kBiasSrcBf16;
    p.bias_copy = 0;
  } else {
    p.bias = reinterpret_cast<const void*>(reinterpret_cast<uintptr_t>(bias32) -
                                           (uintptr_t)col0 * sizeof(float));
    p.bias_src = bilogp::kBiasSrcF32;
    p.bias_copy = 1;
  }
}

// Workgroups a launch may have (the grid stays within 32-bit work-item
// counts); a call with more row blocks x splits keeps the one-phase schedule
// and is issued in row chunks.
constexpr int64_t kMaxLaunchBlocks = (int64_t)(UINT32_MAX / 512u);

// Row blocking and schedule of a projection over splits [p.split0, p.split1)
// of p.vps tiles each (p.N and p.H set).
void plan_projection(bilogp::ProjParams& p, int cu, int slots128) {
  const int ns = p.split1 - p.split0;
  p.rows = row_block_rows(p.N, p.H, ns, p.vps, cu, slots128);
  p.R = (int32_t)((p.N + p.rows - 1) / p.rows);
  Schedule sc{splits_per_run(p.R, ns, p.vps, cu), ns, ns};
  if (p.rows == 256 && (int64_t)p.R * ns <= kMaxLaunchBlocks) {
    const int64_t k = ((int64_t)p.H + 63) / 64;
    sc = schedule_256(p.R, ns, p.vps, cu, (k + 1) / 2 * 2, (k + 2) / 3 * 3);
  }
  p.spg = sc.spg;
  p.splitA = p.split0 + sc.sa;
  p.splitT = p.split0 + sc.sb;
  p.runsA = (sc.sa + sc.spg - 1) / sc.spg;
}

// The launches of a planned projection: the 256-token (or 128-token) launch
// over [split0, splitT) and, if splitT < split1, the 128-token launch over
// [splitT, split1), single splits.
bilogp::ProjParams main_launch(const bilogp::ProjParams& p) {
  bilogp::ProjParams q = p;
  q.split1 = p.splitT;
  return q;
}
bilogp::ProjParams tail_launch(const bilogp::ProjParams& p) {
  bilogp::ProjParams q = p;
  q.rows = 128;
  q.R = (int32_t)((p.N + 127) / 128);
  q.split0 = p.splitT;
  q.splitA = p.split1;
  q.splitT = p.split1;
  q.spg = 1;
  q.runsA = p.split1 - p.splitT;
  return q;
}

// The plan bilogp_forward_mode makes for these arguments (no device needed);
// false for arguments it would refuse.
bool plan_for(int64_t N, int64_t H, int64_t V, int mode, int cu_count, bilogp::ProjParams* out) {
  if (N < 1 || N > kMaxN || H < 1 || H > kMaxH || V <= 0 || V > kMaxV || cu_count < 1 ||
      cu_count > kMaxCuCount)
    return false;
  const int S = bilogp_num_vocab_splits_mode(N, V, mode, cu_count);
  const int vps = bilogp_vtiles_per_split_mode(N, V, mode, cu_count);
  if (S == 0 || vps == 0) return false;
  bilogp::ProjParams& p = *out;
  p.N = N;
  p.H = (int32_t)H;
  p.V = (int32_t)V;
  p.vps = vps;
  p.S = S;
  p.split0 = 0;
  p.split1 = S;
  plan_projection(p, cu_count, 3);
  return true;
}


bilogp_status check_on_device(const void* ptr, int dev, const char* name) {
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, ptr);
  if (e != hipSuccess) {
    (void)hipGetLastError();   // clear the sticky error left by a host pointer
    return fail(BILOGP_E_UNSUPPORTED, std::string(name) + " is not device memory");
  }
  if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)
    return fail(BILOGP_E_UNSUPPORTED, std::string(name) + " is not device memory");
  if (attr.device != dev)
    return fail(BILOGP_E_UNSUPPORTED, std::string(name) + " is on another device");
  return BILOGP_OK;
}

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

Range range_of(const void* p, size_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + bytes};
}

}  // namespace

extern "C" {

int bilogp_abi_version(void) { return BILOGP_ABI_VERSION; }

int bilogp_bit_contract_version(void) { return BILOGP_BIT_CONTRACT_VERSION; }

int bilogp_vtile_cols(void) { return bilogp::kVtileCols; }

int bilogp_max_splits(void) { return bilogp::kMaxSplits; }

int bilogp_vtiles_per_split(int64_t V) {
  if (V <= 0 || V > kMaxV) return 0;
  const int64_t tiles = (V + bilogp::kVtileCols - 1) / bilogp::kVtileCols;
  return (int)((tiles + bilogp::kMaxSplits - 1) / bilogp::kMaxSplits);
}

int bilogp_num_vocab_splits(int64_t V) {
  const int per_split = bilogp_vtiles_per_split(V);
  if (per_split == 0) return 0;
  const int64_t tiles = (V + bilogp::kVtileCols - 1) / bilogp::kVtileCols;
  return (int)((tiles + per_split - 1) / per_split);
}

size_t bilogp_workspace_bytes(int64_t N, int64_t V) {
  return bilogp_workspace_bytes_mode(N, V, BILOGP_SPLITS_INVARIANT, 0);
}

int bilogp_vtiles_per_split_mode(int64_t N, int64_t V, int mode, int cu_count) {
  if (mode == BILOGP_SPLITS_INVARIANT) return bilogp_vtiles_per_split(V);
  if (mode != BILOGP_SPLITS_THROUGHPUT) return 0;
  if (N < 1 || N > kMaxN || V <= 0 || V > kMaxV || cu_count < 1) return 0;
  // want = min(max(ceil(cu / R), 1), T, cap); per_split = ceil(T / want)
  const int64_t tiles = (V + bilogp::kVtileCols - 1) / bilogp::kVtileCols;
  const int64_t row_blocks = (N + bilogp::kBlockRows - 1) / bilogp::kBlockRows;
  int64_t want = ((int64_t)cu_count + row_blocks - 1) / row_blocks;
  want = std::min(std::max<int64_t>(want, 1), std::min<int64_t>(tiles, bilogp::kMaxThroughputSplits));
  return (int)((tiles + want - 1) / want);
}

int bilogp_num_vocab_splits_mode(int64_t N, int64_t V, int mode, int cu_count) {
  const int per_split = bilogp_vtiles_per_split_mode(N, V, mode, cu_count);
  if (per_split == 0) return 0;
  const int64_t tiles = (V + bilogp::kVtileCols - 1) / bilogp::kVtileCols;
  return (int)((tiles + per_split - 1) / per_split);
}

size_t bilogp_workspace_bytes_mode(int64_t N, int64_t V, int mode, int cu_count) {
  if (N < 0 || N > kMaxN) return (size_t)-1;
  if (mode != BILOGP_SPLITS_INVARIANT && mode != BILOGP_SPLITS_THROUGHPUT) return (size_t)-1;
  if (N == 0) return (V > 0 && V <= kMaxV) ? 0 : (size_t)-1;
  const int S = bilogp_num_vocab_splits_mode(N, V, mode, cu_count);
  if (S == 0) return (size_t)-1;
  return round_up((size_t)N * (size_t)S * sizeof(float2)) + round_up((size_t)N * sizeof(float)) +
         round_up(padded_vocab(V) * sizeof(float));
}

const char* bilogp_status_string(int status) {
  switch (status) {
    case BILOGP_OK: return "ok";
    case BILOGP_E_INVALID_ARG: return "invalid argument";
    case BILOGP_E_UNSUPPORTED: return "unsupported request";
    case BILOGP_E_WORKSPACE: return "workspace missing or too small";
    case BILOGP_E_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* bilogp_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

namespace {

// Which parts of the call are present: the projection needs the inputs, the
// merge needs the outputs; both need target and the workspace.
enum Part : int { kProj = 1, kMerge = 2 };

struct Call {
  const void* hidden;
  const void* weight;
  const int64_t* target;
  const void* bias;
  int bias_dtype;
  float* logp;
  float* lse;
  int64_t N, H, V;
  void* ws;
  size_t ws_bytes;
  int mode = BILOGP_SPLITS_INVARIANT;
  int cu_count = 0;
  // projection over splits [split_begin, split_end) only (split_end < 0: all);
  // weight and bias then hold just those splits' vocabulary columns
  int split_begin = 0;
  int split_end = -1;
  // the workspace is the library's own per-device scratch array (known to be
  // device memory of the current device; not checked by pointer attributes)
  bool ws_is_scratch = false;
};

// Full argument validation (fail closed) and the launch parameters.  Pure
// host checks come first, then the device checks; nothing is launched here.
bilogp_status validate(const Call& c, int parts, bilogp::ProjParams* out) {
  const bool proj = parts & kProj, merge = parts & kMerge;
  if (!c.target || (proj && (!c.hidden || !c.weight)) || (merge && (!c.logp || !c.lse)))
    return fail(BILOGP_E_INVALID_ARG, "a required pointer is null");
  if (c.N < 0 || c.N > kMaxN) return fail(BILOGP_E_INVALID_ARG, "N out of range [0, 2^32]");
  if (proj && (c.H <= 0 || c.H > kMaxH))
    return fail(BILOGP_E_INVALID_ARG, "H out of range [1, 2^20]");
  if (c.V <= 0 || c.V > kMaxV) return fail(BILOGP_E_INVALID_ARG, "V out of range [1, 2^30]");
  if (c.mode != BILOGP_SPLITS_INVARIANT && c.mode != BILOGP_SPLITS_THROUGHPUT)
    return fail(BILOGP_E_INVALID_ARG, "unknown split mode");
  if (c.mode == BILOGP_SPLITS_THROUGHPUT && c.cu_count < 1)
    return fail(BILOGP_E_INVALID_ARG, "the throughput split mode needs cu_count >= 1");
  if (c.cu_count < 0 || c.cu_count > kMaxCuCount)
    return fail(BILOGP_E_INVALID_ARG, "cu_count out of range [0, 65536]");
  size_t bias_esz = 0;
  if (proj) {
    if (c.bias_dtype != BILOGP_BIAS_NONE && c.bias_dtype != BILOGP_BIAS_BF16 &&
        c.bias_dtype != BILOGP_BIAS_F32)
      return fail(BILOGP_E_UNSUPPORTED, "unknown bias dtype");
    if ((c.bias_dtype == BILOGP_BIAS_NONE) != (c.bias == nullptr))
      return fail(BILOGP_E_INVALID_ARG, "bias must be null exactly when bias_dtype is NONE");
    if (c.H % 8 != 0) return fail(BILOGP_E_UNSUPPORTED, "H must be a multiple of 8");
    if ((reinterpret_cast<uintptr_t>(c.hidden) | reinterpret_cast<uintptr_t>(c.weight)) % 16)
      return fail(BILOGP_E_UNSUPPORTED, "hidden and weight must be 16-byte aligned");
    bias_esz = c.bias_dtype == BILOGP_BIAS_F32 ? 4 : 2;
    if (c.bias && reinterpret_cast<uintptr_t>(c.bias) % bias_esz != 0)
      return fail(BILOGP_E_UNSUPPORTED, "bias is misaligned for its dtype");
  }
  if (reinterpret_cast<uintptr_t>(c.target) % 8 != 0)
    return fail(BILOGP_E_UNSUPPORTED, "target must be 8-byte aligned");
  if (merge && (reinterpret_cast<uintptr_t>(c.logp) | reinterpret_cast<uintptr_t>(c.lse)) % 4)
    return fail(BILOGP_E_UNSUPPORTED, "outputs must be 4-byte aligned");
  if (c.split_end >= 0) {      // split ranges exist for the V-only policy alone
    const int S_inv = bilogp_num_vocab_splits(c.V);
    if (c.mode != BILOGP_SPLITS_INVARIANT || c.split_begin < 0 ||
        c.split_begin >= c.split_end || c.split_end > S_inv)
      return fail(BILOGP_E_INVALID_ARG, "split range must satisfy 0 <= begin < end <= " +
                                            std::to_string(S_inv));
  }
  if (c.N == 0) return BILOGP_OK;

  const int S = bilogp_num_vocab_splits_mode(c.N, c.V, c.mode, c.cu_count);
  const int vps = bilogp_vtiles_per_split_mode(c.N, c.V, c.mode, c.cu_count);
  // vocabulary columns [col0, col1) that weight and bias hold
  const bool ranged = c.split_end >= 0;
  const int64_t col0 = ranged ? (int64_t)c.split_begin * vps * bilogp::kVtileCols : 0;
  const int64_t col1 =
      ranged ? std::min<int64_t>((int64_t)c.split_end * vps * bilogp::kVtileCols, c.V) : c.V;

  if (merge) {
    const Range r_logp = range_of(c.logp, (size_t)c.N * 4), r_lse = range_of(c.lse, (size_t)c.N * 4);
    const Range others[] = {
        proj ? range_of(c.hidden, (size_t)c.N * c.H * 2) : Range{0, 0},
        proj ? range_of(c.weight, (size_t)(col1 - col0) * c.H * 2) : Range{0, 0},
        range_of(c.target, (size_t)c.N * 8),
        (proj && c.bias) ? range_of(c.bias, (size_t)(col1 - col0) * bias_esz) : Range{0, 0},
        c.ws ? range_of(c.ws, c.ws_bytes) : Range{0, 0}};
    if (overlap(r_logp, r_lse)) return fail(BILOGP_E_INVALID_ARG, "logp_out and lse_out overlap");
    for (const Range& in : others)
      if (overlap(r_logp, in) || overlap(r_lse, in))
        return fail(BILOGP_E_INVALID_ARG, "an output overlaps an input or the workspace");
  }

  const size_t need = bilogp_workspace_bytes_mode(c.N, c.V, c.mode, c.cu_count);
  if (!c.ws || c.ws_bytes < need)
    return fail(BILOGP_E_WORKSPACE, "workspace needs " + std::to_string(need) + " bytes");
  if (reinterpret_cast<uintptr_t>(c.ws) % kAlign != 0)
    return fail(BILOGP_E_WORKSPACE, "workspace must be 256-byte aligned");
  {
    // the projection writes the workspace while it reads the inputs: they
    // must not share a byte (checked for every part, so a workspace is never
    // an input of any call)
    const Range r_ws = range_of(c.ws, c.ws_bytes);
    const Range ins[] = {
        proj ? range_of(c.hidden, (size_t)c.N * c.H * 2) : Range{0, 0},
        proj ? range_of(c.weight, (size_t)(col1 - col0) * c.H * 2) : Range{0, 0},
        range_of(c.target, (size_t)c.N * 8),
        (proj && c.bias) ? range_of(c.bias, (size_t)(col1 - col0) * bias_esz) : Range{0, 0}};
    for (const Range& in : ins)
      if (overlap(r_ws, in))
        return fail(BILOGP_E_INVALID_ARG, "the workspace overlaps an input");
  }

  int dev = -1;
  bilogp_status st = check_device(&dev);
  if (st != BILOGP_OK) return st;
  const void* ptrs[] = {proj ? c.hidden : nullptr, proj ? c.weight : nullptr, c.target,
                        proj ? c.bias : nullptr, merge ? c.logp : nullptr,
                        merge ? c.lse : nullptr, c.ws_is_scratch ? nullptr : c.ws};
  const char* names[] = {"hidden", "weight", "target", "bias", "logp_out", "lse_out", "workspace"};
  for (int i = 0; i < 7; ++i) {
    if (!ptrs[i]) continue;
    st = check_on_device(ptrs[i], dev, names[i]);
    if (st != BILOGP_OK) return st;
  }

  const WsLayout L = ws_layout(c.ws, c.N, S);
  bilogp::ProjParams& p = *out;
  // compute units the launch is scheduled for: the caller's count, else the
  // device's (row blocking and split runs never change a bit)
  const int cu = c.cu_count > 0 ? c.cu_count : device_cus(dev);
  p.hidden = c.hidden;
  // absolute-column addressing: shift the slice's base back by col0 columns
  // (unsigned arithmetic; the kernel adds them again before any access)
  p.weight = reinterpret_cast<const void*>(reinterpret_cast<uintptr_t>(c.weight) -
                                           (uintptr_t)col0 * (uintptr_t)c.H * 2u);
  p.target = c.target;
  set_bias(p, c.bias, c.bias_dtype, c.V, col0, L.bias32);
  p.part = L.part;
  p.tlogit = L.tlogit;
  p.N = c.N;
  p.H = (int32_t)c.H;
  p.V = (int32_t)c.V;
  p.T = (int32_t)((c.V + bilogp::kVtileCols - 1) / bilogp::kVtileCols);
  p.vps = vps;
  p.S = S;
  p.split0 = ranged ? c.split_begin : 0;
  p.split1 = ranged ? c.split_end : S;
  plan_projection(p, cu, 3);
  p.col0 = col0;
  return BILOGP_OK;
}

// Every grid stays within 32-bit work-item counts: the projection and the
// merge are issued in row chunks.  Rows are independent and a row's
// arithmetic does not depend on the rows around it, so chunking never changes
// a bit.  Projection: 512 work-items per workgroup, runsA + split1 - splitA
// workgroups per row block.  Merge: 64 work-items per row.
int64_t proj_chunk_rows(const bilogp::ProjParams& p) {
  const int64_t per_rb = p.runsA + p.split1 - p.splitA;
  return std::max<int64_t>(1, kMaxLaunchBlocks / std::max<int64_t>(per_rb, 1)) * p.rows;
}
constexpr int64_t kMergeChunkRows = int64_t(1) << 25;

bilogp_status launch(const bilogp::ProjParams& p, const Call& c, int parts, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((parts & kProj) && p.bias_copy) {
    // the padded fp32 copy of the bias columns the launch reads, from col0
    const int64_t cols = c.split_end >= 0
        ? std::min<int64_t>((int64_t)p.split1 * p.vps * bilogp::kVtileCols, p.V) -
              p.col0
        : p.V;
    float* bias32 = reinterpret_cast<float*>(reinterpret_cast<uintptr_t>(p.bias) +
                                             (uintptr_t)p.col0 * sizeof(float));
    hipError_t e = bilogp::launch_bias_f32(c.bias, p.bias_kind, (int32_t)cols, bias32, s);
    if (e != hipSuccess)
      return fail(BILOGP_E_HIP, std::string("bias copy launch: ") + hipGetErrorString(e));
  }
  if (parts & kProj) {
    const bilogp::ProjParams m = main_launch(p);
    const int64_t chunk = proj_chunk_rows(m);
    for (int64_t r0 = 0; r0 < p.N && m.split1 > m.split0; r0 += chunk) {
      bilogp::ProjParams q = m;
      q.N = std::min(chunk, p.N - r0);
      q.R = (int32_t)((q.N + p.rows - 1) / p.rows);
      q.hidden = static_cast<const uint16_t*>(p.hidden) + r0 * p.H;
      q.target = p.target + r0;
      q.part = p.part + r0 * p.S;
      q.tlogit = p.tlogit + r0;
      hipError_t e = bilogp::launch_proj_lse(q, s);
      if (e != hipSuccess)
        return fail(BILOGP_E_HIP, std::string("projection launch: ") + hipGetErrorString(e));
    }
    if (p.splitT < p.split1) {
      // the planner only makes a second launch when one launch holds the first
      hipError_t e = bilogp::launch_proj_lse(tail_launch(p), s);
      if (e != hipSuccess)
        return fail(BILOGP_E_HIP, std::string("projection launch: ") + hipGetErrorString(e));
    }
  }
  if (parts & kMerge) {
    for (int64_t r0 = 0; r0 < p.N; r0 += kMergeChunkRows) {
      const int64_t n = std::min(kMergeChunkRows, p.N - r0);
      hipError_t e = bilogp::launch_merge(p.part + r0 * p.S, p.tlogit + r0, p.target + r0,
                                          c.logp + r0, c.lse + r0, n, p.S, p.V, s);
      if (e != hipSuccess)
        return fail(BILOGP_E_HIP, std::string("merge launch: ") + hipGetErrorString(e));
    }
  }
  return BILOGP_OK;
}

bilogp_status run(const Call& c, int parts, void* stream) {
  g_last_error.clear();
  bilogp::ProjParams p;
  bilogp_status st = validate(c, parts, &p);
  if (st != BILOGP_OK || c.N == 0) return st;
  return launch(p, c, parts, stream);
}

}  // namespace

extern "C" {

int bilogp_launch_plan(int64_t N, int64_t H, int64_t V, int mode, int cu_count,
                       int* rows_per_block, int* splits_per_workgroup, int64_t* workgroups) {
  bilogp::ProjParams p{};
  if (!plan_for(N, H, V, mode, cu_count, &p)) return -1;
  if (rows_per_block) *rows_per_block = p.rows;
  if (splits_per_workgroup) *splits_per_workgroup = p.spg;
  if (workgroups) {
    const bilogp::ProjParams m = main_launch(p);
    *workgroups = (int64_t)m.R * (m.runsA + m.split1 - m.splitA);
    if (p.splitT < p.split1) {
      const bilogp::ProjParams t = tail_launch(p);
      *workgroups += (int64_t)t.R * (t.runsA + t.split1 - t.splitA);
    }
  }
  return 0;
}

int bilogp_launch_schedule(int64_t N, int64_t H, int64_t V, int mode, int cu_count,
                           int* split_a, int* split_t) {
  bilogp::ProjParams p{};
  if (!plan_for(N, H, V, mode, cu_count, &p)) return -1;
  if (split_a) *split_a = p.splitA;
  if (split_t) *split_t = p.splitT;
  return 0;
}

bilogp_status bilogp_forward_ex(const void* hidden, const void* weight, const int64_t* target,
                                const void* bias, int bias_dtype, float* logp_out,
                                float* lse_out, int64_t N, int64_t H, int64_t V,
                                void* workspace, size_t workspace_bytes, void* stream) {
  const Call c{hidden, weight, target, bias, bias_dtype, logp_out, lse_out,
               N,      H,      V,      workspace, workspace_bytes};
  return run(c, kProj | kMerge, stream);
}

bilogp_status bilogp_forward_mode(const void* hidden, const void* weight, const int64_t* target,
                                  const void* bias, int bias_dtype, float* logp_out,
                                  float* lse_out, int64_t N, int64_t H, int64_t V, int mode,
                                  int cu_count, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  Call c{hidden, weight, target, bias, bias_dtype, logp_out, lse_out,
         N,      H,      V,      workspace, workspace_bytes};
  c.mode = mode;
  c.cu_count = cu_count;
  return run(c, kProj | kMerge, stream);
}

bilogp_status bilogp_partials(const void* hidden, const void* weight, const int64_t* target,
                              const void* bias, int bias_dtype, int64_t N, int64_t H, int64_t V,
                              void* workspace, size_t workspace_bytes, void* stream) {
  const Call c{hidden, weight, target, bias, bias_dtype, nullptr, nullptr,
               N,      H,      V,      workspace, workspace_bytes};
  return run(c, kProj, stream);
}

bilogp_status bilogp_partials_range(const void* hidden, const void* weight_slice,
                                    const int64_t* target, const void* bias_slice, int bias_dtype,
                                    int64_t N, int64_t H, int64_t V, int split_begin,
                                    int split_end, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  Call c{hidden, weight_slice, target, bias_slice, bias_dtype, nullptr, nullptr,
         N,      H,            V,      workspace,  workspace_bytes};
  c.split_begin = split_begin;
  c.split_end = split_end < 0 ? 0 : split_end;   // a negative end is an empty (invalid) range
  return run(c, kProj, stream);
}

bilogp_status bilogp_merge(const int64_t* target, const void* workspace, size_t workspace_bytes,
                           float* logp_out, float* lse_out, int64_t N, int64_t V, void* stream) {
  const Call c{nullptr, nullptr, target, nullptr, BILOGP_BIAS_NONE, logp_out, lse_out,
               N,       8,       V,      const_cast<void*>(workspace), workspace_bytes};
  return run(c, kMerge, stream);
}

bilogp_status bilogp_forward(const void* hidden, const void* weight, const int64_t* target,
                             const float* bias, float* logp_out, float* lse_out, int64_t N,
                             int64_t H, int64_t V, void* stream) {
  g_last_error.clear();
  const size_t need = bilogp_workspace_bytes(N, V);
  if (need == (size_t)-1) {
    // let the full validation report the precise reason
    return bilogp_forward_ex(hidden, weight, target, bias,
                             bias ? BILOGP_BIAS_F32 : BILOGP_BIAS_NONE, logp_out, lse_out, N, H,
                             V, nullptr, 0, stream);
  }
  if (need == 0)
    return bilogp_forward_ex(hidden, weight, target, bias,
                             bias ? BILOGP_BIAS_F32 : BILOGP_BIAS_NONE, logp_out, lse_out, N, H,
                             V, nullptr, 0, stream);
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  hipError_t e = hipMallocAsync(&ws, need, s);
  if (e != hipSuccess)
    return fail(BILOGP_E_HIP, std::string("hipMallocAsync: ") + hipGetErrorString(e));
  bilogp_status st = bilogp_forward_ex(hidden, weight, target, bias,
                                       bias ? BILOGP_BIAS_F32 : BILOGP_BIAS_NONE, logp_out,
                                       lse_out, N, H, V, ws, need, stream);
  std::string keep = g_last_error;
  e = hipFreeAsync(ws, s);
  if (st != BILOGP_OK) return fail(st, keep);
  if (e != hipSuccess)
    return fail(BILOGP_E_HIP, std::string("hipFreeAsync: ") + hipGetErrorString(e));
  return BILOGP_OK;
}


}  // extern "C"

// ---------------------------------------------------------------------------
// Forward with no allocation at all: the workspace is a file-scope device
// array of a fixed size, one copy per GPU, for callers that cannot allocate.
// Its address is looked up once per device (hipGetSymbolAddress, with that
// device current) and kept; host code never uses the array's name as an
// address.
namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::atomic<void*> g_scratch_ptr[kMaxDevices];

bilogp_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0)
    return fail(BILOGP_E_UNSUPPORTED, std::string("no usable HIP device: ") + hipGetErrorString(e));
  if (dev >= kMaxDevices) return fail(BILOGP_E_UNSUPPORTED, "device index out of range");
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!ptr) {
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(BILOGP_E_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev].store(ptr, std::memory_order_release);
  }
  *out = ptr;
  return BILOGP_OK;
}

}  // namespace

extern "C" {

size_t bilogp_noalloc_max_workspace_bytes(void) { return kScratchBytes; }

bilogp_status bilogp_forward_noalloc(const void* hidden, const void* weight,
                                     const int64_t* target, const void* bias, int bias_dtype,
                                     float* logp_out, float* lse_out, int64_t N, int64_t H,
                                     int64_t V, void* stream) {
  g_last_error.clear();
  const size_t need = bilogp_workspace_bytes(N, V);
  if (need != (size_t)-1 && need > kScratchBytes)
    return fail(BILOGP_E_WORKSPACE, "the no-allocation forward holds at most " +
                                        std::to_string(kScratchBytes) + " workspace bytes; N = " +
                                        std::to_string(N) + ", V = " + std::to_string(V) +
                                        " needs " + std::to_string(need));
  Call c{hidden, weight, target, bias, bias_dtype, logp_out, lse_out, N, H, V, nullptr, 0};
  if (need == (size_t)-1 || need == 0) return run(c, kProj | kMerge, stream);  // checks report it
  void* ws = nullptr;
  bilogp_status st = scratch_address(&ws);
  if (st != BILOGP_OK) return st;
  c.ws = ws;
  c.ws_bytes = kScratchBytes;
  c.ws_is_scratch = true;
  return run(c, kProj | kMerge, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Deterministic GEMM (RL-Kernel PR #395): forward, dA, dB.
namespace {

constexpr int64_t kMaxGemmNK = int64_t(1) << 20;
constexpr int64_t kMaxGemmM = int64_t(1) << 31;

struct GemmCall {
  const void* x;
  const void* y;
  void* out;
  bool xt, yt;
  int64_t P, Q, C, ldx, ldy, ldo;
  int out_kind;
  size_t x_bytes, y_bytes, out_bytes;
};

bilogp_status gemm_run(const GemmCall& c, int64_t M, int64_t N, int64_t K, void* stream) {
  g_last_error.clear();
  // an operand or output of zero bytes is never touched and may be null
  if ((!c.x && c.x_bytes) || (!c.y && c.y_bytes) || (!c.out && c.out_bytes))
    return fail(BILOGP_E_INVALID_ARG, "a required pointer is null");
  if (M < 0 || M > kMaxGemmM) return fail(BILOGP_E_INVALID_ARG, "M out of range [0, 2^31]");
  if (N < 8 || N > kMaxGemmNK || K < 8 || K > kMaxGemmNK)
    return fail(BILOGP_E_INVALID_ARG, "N and K must lie in [8, 2^20]");
  if (c.out_kind != BILOGP_GEMM_OUT_BF16 && c.out_kind != BILOGP_GEMM_OUT_F32 &&
      c.out_kind != BILOGP_GEMM_OUT_F32_ACCUM)
    return fail(BILOGP_E_INVALID_ARG, "unknown output kind");
  if (N % 8 != 0 || K % 8 != 0) return fail(BILOGP_E_UNSUPPORTED, "N and K must be multiples of 8");
  if ((reinterpret_cast<uintptr_t>(c.x) | reinterpret_cast<uintptr_t>(c.y) |
       reinterpret_cast<uintptr_t>(c.out)) % 16)
    return fail(BILOGP_E_UNSUPPORTED, "operands and output must be 16-byte aligned");
  if (c.out_bytes == 0) return BILOGP_OK;        // empty output: nothing to write
  const Range ro = range_of(c.out, c.out_bytes);
  if (overlap(ro, range_of(c.x, c.x_bytes)) || overlap(ro, range_of(c.y, c.y_bytes)))
    return fail(BILOGP_E_INVALID_ARG, "the output overlaps an operand");
  int dev = -1;
  bilogp_status st = check_device(&dev);
  if (st != BILOGP_OK) return st;
  const void* ptrs[] = {c.x_bytes ? c.x : nullptr, c.y_bytes ? c.y : nullptr, c.out};
  const char* names[] = {"operand", "operand", "output"};
  for (int i = 0; i < 3; ++i) {
    if (!ptrs[i]) continue;
    st = check_on_device(ptrs[i], dev, names[i]);
    if (st != BILOGP_OK) return st;
  }
  bilogp::GemmParams g;
  g.x = c.x;
  g.y = c.y;
  g.out = c.out;
  g.P = c.P;
  g.Q = c.Q;
  g.C = c.C;
  g.ldx = c.ldx;
  g.ldy = c.ldy;
  g.ldo = c.ldo;
  g.out_kind = c.out_kind;
  g.Pt = (int32_t)((c.P + 255) / 256);
  g.Qt = (int32_t)((c.Q + 255) / 256);
  g.cu_count = device_cus(dev);
  if ((int64_t)g.Pt * g.Qt > INT32_MAX) return fail(BILOGP_E_INVALID_ARG, "too many tiles");
  hipError_t e = bilogp::launch_det_gemm(g, c.xt, c.yt, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(BILOGP_E_HIP, std::string("gemm launch: ") + hipGetErrorString(e));
  return BILOGP_OK;
}

size_t out_elem(int kind) { return kind == BILOGP_GEMM_OUT_BF16 ? 2 : 4; }

}  // namespace

extern "C" {

bilogp_status bilogp_det_gemm_fwd(const void* a, const void* b, void* c, int64_t M, int64_t N,
                                  int64_t K, int out_kind, void* stream) {
  // C[M, N] = A[M, K] . B[N, K]^T: p = n (X = B), q = m (Y = A), contraction k
  const GemmCall g{b, a, c, false, false, N, M, K, K, K, N, out_kind,
                   (size_t)N * K * 2, (size_t)(M > 0 ? M : 0) * K * 2,
                   (size_t)(M > 0 ? M : 0) * N * out_elem(out_kind)};
  return gemm_run(g, M, N, K, stream);
}

bilogp_status bilogp_det_gemm_da(const void* dc, const void* b, void* da, int64_t M, int64_t N,
                                 int64_t K, int out_kind, void* stream) {
  // dA[M, K] = dC[M, N] . B[N, K]: p = k (X = B, stored [n][k]), q = m (Y = dC)
  const GemmCall g{b, dc, da, true, false, K, M, N, K, N, K, out_kind,
                   (size_t)N * K * 2, (size_t)(M > 0 ? M : 0) * N * 2,
                   (size_t)(M > 0 ? M : 0) * K * out_elem(out_kind)};
  return gemm_run(g, M, N, K, stream);
}

bilogp_status bilogp_det_gemm_db(const void* a, const void* dc, void* db, int64_t M, int64_t N,
                                 int64_t K, int out_kind, void* stream) {
  // dB[N, K] = dC[M, N]^T . A[M, K]: p = k (X = A, stored [m][k]), q = n (Y = dC,
  // stored [m][n]), contraction m
  const GemmCall g{a, dc, db, true, true, K, N, M, K, N, K, out_kind,
                   (size_t)(M > 0 ? M : 0) * K * 2, (size_t)(M > 0 ? M : 0) * N * 2,
                   (size_t)N * K * out_elem(out_kind)};
  return gemm_run(g, M, N, K, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Backward of the fused linear log-probability (row f2).
namespace {

constexpr int64_t kMaxBwdN = int64_t(1) << 21;

int64_t dz_ld(int64_t N) { return (N + 7) / 8 * 8; }

}  // namespace

extern "C" {

size_t bilogp_backward_workspace_bytes(int64_t N, int64_t V) {
  if (N < 0 || N > kMaxBwdN || V <= 0 || V > kMaxV) return (size_t)-1;
  return round_up((size_t)V * (size_t)dz_ld(N) * 2) + round_up(padded_vocab(V) * sizeof(float));
}

bilogp_status bilogp_backward(const void* hidden, const void* weight, const int64_t* target,
                              const void* bias, int bias_dtype, const float* lse,
                              const float* grad_logp, const float* grad_lse, float* grad_hidden,
                              float* grad_weight, float* grad_bias, int64_t N, int64_t H,
                              int64_t V, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (!weight || !grad_weight || (N > 0 && (!hidden || !target || !lse || !grad_logp ||
                                            !grad_lse || !grad_hidden)))
    return fail(BILOGP_E_INVALID_ARG, "a required pointer is null");
  if (N < 0 || N > kMaxBwdN) return fail(BILOGP_E_INVALID_ARG, "N out of range [0, 2^21]");
  if (H <= 0 || H > kMaxH) return fail(BILOGP_E_INVALID_ARG, "H out of range [1, 2^20]");
  if (V <= 0 || V > kMaxV) return fail(BILOGP_E_INVALID_ARG, "V out of range [1, 2^30]");
  if (bias_dtype != BILOGP_BIAS_NONE && bias_dtype != BILOGP_BIAS_BF16 &&
      bias_dtype != BILOGP_BIAS_F32)
    return fail(BILOGP_E_UNSUPPORTED, "unknown bias dtype");
  if ((bias_dtype == BILOGP_BIAS_NONE) != (bias == nullptr))
    return fail(BILOGP_E_INVALID_ARG, "bias must be null exactly when bias_dtype is NONE");
  if (H % 8 != 0) return fail(BILOGP_E_UNSUPPORTED, "H must be a multiple of 8");
  if ((reinterpret_cast<uintptr_t>(hidden) | reinterpret_cast<uintptr_t>(weight) |
       reinterpret_cast<uintptr_t>(grad_hidden) | reinterpret_cast<uintptr_t>(grad_weight)) % 16)
    return fail(BILOGP_E_UNSUPPORTED, "hidden, weight and the gradients must be 16-byte aligned");
  const size_t bias_esz = bias_dtype == BILOGP_BIAS_F32 ? 4 : 2;
  if (bias && reinterpret_cast<uintptr_t>(bias) % bias_esz != 0)
    return fail(BILOGP_E_UNSUPPORTED, "bias is misaligned for its dtype");
  if ((reinterpret_cast<uintptr_t>(target) % 8) ||
      ((reinterpret_cast<uintptr_t>(lse) | reinterpret_cast<uintptr_t>(grad_logp) |
        reinterpret_cast<uintptr_t>(grad_lse) | reinterpret_cast<uintptr_t>(grad_bias)) % 4))
    return fail(BILOGP_E_UNSUPPORTED, "target, lse, grad_logp, grad_lse or grad_bias misaligned");
  const size_t need = bilogp_backward_workspace_bytes(N, V);
  if (!workspace || workspace_bytes < need)
    return fail(BILOGP_E_WORKSPACE, "workspace needs " + std::to_string(need) + " bytes");
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
    return fail(BILOGP_E_WORKSPACE, "workspace must be 256-byte aligned");
  // outputs must not overlap each other, the inputs or the workspace
  const Range outs[] = {range_of(grad_hidden, (size_t)N * H * 4),
                        range_of(grad_weight, (size_t)V * H * 4),
                        grad_bias ? range_of(grad_bias, (size_t)V * 4) : Range{0, 0}};
  const Range ins[] = {range_of(hidden, (size_t)N * H * 2), range_of(weight, (size_t)V * H * 2),
                       range_of(target, (size_t)N * 8),
                       bias ? range_of(bias, (size_t)V * bias_esz) : Range{0, 0},
                       range_of(lse, (size_t)N * 4), range_of(grad_logp, (size_t)N * 4),
                       range_of(grad_lse, (size_t)N * 4), range_of(workspace, workspace_bytes)};
  for (int i = 0; i < 3; ++i) {
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outs[j])) return fail(BILOGP_E_INVALID_ARG, "gradients overlap");
    for (const Range& in : ins)
      if (overlap(outs[i], in))
        return fail(BILOGP_E_INVALID_ARG, "a gradient overlaps an input or the workspace");
  }

  int dev = -1;
  bilogp_status st = check_device(&dev);
  if (st != BILOGP_OK) return st;
  const void* ptrs[] = {hidden, weight, target, bias, lse, grad_logp, grad_lse, grad_hidden,
                        grad_weight, grad_bias, workspace};
  for (const void* q : ptrs) {
    if (!q) continue;
    st = check_on_device(q, dev, "an argument");
    if (st != BILOGP_OK) return st;
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t ldz = dz_ld(N);
  uint16_t* dzt = static_cast<uint16_t*>(workspace);
  float* bias32 = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                           round_up((size_t)V * (size_t)ldz * 2));
  const int32_t kind = bias_dtype == BILOGP_BIAS_BF16 ? bilogp::kBiasBf16
                       : bias_dtype == BILOGP_BIAS_F32 ? bilogp::kBiasF32
                                                       : bilogp::kBiasNone;
  hipError_t e = hipSuccess;
  if (N > 0) {
    bilogp::ProjParams p{};
    set_bias(p, bias, bias_dtype, V, 0, bias32);
    if (p.bias_copy) e = bilogp::launch_bias_f32(bias, kind, (int32_t)V, bias32, s);
    if (e == hipSuccess) e = bilogp::launch_zero_pad_cols(dzt, V, N, ldz, s);
    if (e == hipSuccess) {
      p.hidden = hidden;
      p.weight = weight;
      p.target = target;
      p.N = N;
      p.H = (int32_t)H;
      p.V = (int32_t)V;
      p.T = (int32_t)((V + bilogp::kVtileCols - 1) / bilogp::kVtileCols);
      p.vps = bilogp_vtiles_per_split(V);
      p.S = bilogp_num_vocab_splits(V);
      p.split0 = 0;
      p.split1 = p.S;
      plan_projection(p, device_cus(dev), 3);
      p.col0 = 0;
      p.lse = lse;
      p.g_logp = grad_logp;
      p.g_lse = grad_lse;
      p.dzt = dzt;
      p.ldz = ldz;
      e = bilogp::launch_softmax_grad(main_launch(p), s);
      if (e == hipSuccess && p.splitT < p.split1)
        e = bilogp::launch_softmax_grad(tail_launch(p), s);
    }
    if (e == hipSuccess) {
      // grad_hidden[n][h] = sum over v ascending of dZ^T[v][n] W[v][h]
      bilogp::GemmParams g{};
      g.x = weight; g.y = dzt; g.out = grad_hidden;
      g.P = H; g.Q = N; g.C = V; g.ldx = H; g.ldy = ldz; g.ldo = H;
      g.out_kind = bilogp::kGemmF32;
      g.cu_count = device_cus(dev);
      g.Pt = (int32_t)((H + 255) / 256);
      g.Qt = (int32_t)((N + 255) / 256);
      e = bilogp::launch_det_gemm(g, true, true, s);
    }
  }
  if (e == hipSuccess) {
    // grad_W[v][h] = sum over n ascending of dZ^T[v][n] hidden[n][h] (zero if N == 0)
    bilogp::GemmParams g{};
    g.x = hidden; g.y = dzt; g.out = grad_weight;
    g.P = H; g.Q = V; g.C = N; g.ldx = H; g.ldy = ldz; g.ldo = H;
    g.out_kind = bilogp::kGemmF32;
    g.cu_count = device_cus(dev);
    g.Pt = (int32_t)((H + 255) / 256);
    g.Qt = (int32_t)((V + 255) / 256);
    e = bilogp::launch_det_gemm(g, true, false, s);
  }
  if (e == hipSuccess && grad_bias) e = bilogp::launch_row_sums(dzt, V, N, ldz, grad_bias, s);
  if (e != hipSuccess) return fail(BILOGP_E_HIP, std::string("backward launch: ") + hipGetErrorString(e));
  return BILOGP_OK;
}

}  // extern "C"
