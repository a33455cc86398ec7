// dg_api.hip -- the C ABI (include/dg.h): host-side validation, the per-shape
// tile heuristic and kernel dispatch.  Validation runs before any HIP call, so
// every error path can be exercised on a machine without a GPU.
#include <dlfcn.h>

#include <atomic>
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/dg.h"
#include "dg_kernel.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];  // 0 = not queried yet

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Compute units of the current device (cached per device).
int device_cus(int* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (dev >= 0 && dev < kMaxDevices) {
    int v = g_cu_count[dev].load(std::memory_order_relaxed);
    if (v > 0) {
      *out = v;
      return 0;
    }
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return -1;
  if (dev >= 0 && dev < kMaxDevices) g_cu_count[dev].store(cus, std::memory_order_relaxed);
  *out = cus;
  return 0;
}

// Workgroups per CU an instance can keep resident: LDS-limited (160 KB per
// CU), at most two 4-wave or one 8-wave workgroup (register file).
int occupancy(int kind, const dg::TileShape& s) {
  const int lds = dg::lds_bytes_of(kind, s);
  int occ = lds > 0 ? (160 * 1024) / lds : 1;
  const int cap = dg::threads_of(s) >= 512 ? 1 : 2;
  if (occ > cap) occ = cap;
  return occ < 1 ? 1 : occ;
}

// Dense kinds (C [M,N] bf16, one group, K may be split): FP8 with fp32 or
// power-of-two scales, and BF16.
bool dense_like(int kind) {
  return kind == DG_KIND_DENSE || kind == DG_KIND_DENSE_POW2 || kind == DG_KIND_BF16;
}

bool parse_forced(dg::TileShape* s) {
  const char* e = std::getenv("DG_FORCE_TILE");
  if (!e || !*e) return false;
  int bm, bn, wm, wn;
  if (std::sscanf(e, "%dx%dx%dx%d", &bm, &bn, &wm, &wn) != 4) return false;
  *s = dg::TileShape{bm, bn, wm, wn};
  return true;
}

// Split K (dense and masked): when a shape's output tiles cannot occupy the
// CUs and K is long, kSplitTarget workgroups share each tile, each covering
// at least kSplitMinBlocks K blocks -- fewer or shorter splits lose more to
// the extra reduction pass than they gain (measured).
constexpr int kMaxSplits = 16;
constexpr int kSplitTarget = 4;
constexpr int kSplitMinBlocks = 12;
// The masked layout's tall tiles read each B column block once per group, so
// a few-group decode has few tiles: up to 8 splits of at least 6 K blocks
// (G=1, N=4096, K=7168: 26 us at 8 splits against 31 us at 4, cold).
constexpr int kMaskedSplitTarget = 8;
constexpr int kMaskedSplitMinBlocks = 6;
constexpr size_t kMaxWorkspaceBytes = size_t(256) << 20;  // split-K partials per call

int choose_splits(int kind, int rows, long tiles, int num_cus, int kbs) {
  const bool masked = dg::layout_of(kind) == DG_KIND_MASKED;
  if (!masked && !dense_like(kind)) return 1;
  if (rows > 256) return 1;  // large M: the extra pass costs more than the idle CUs (measured)
  if (tiles * 10 >= num_cus * 7L) return 1;  // enough tiles already
  if (masked && kbs < 3 * kSplitMinBlocks) return 1;  // short K: the reduction pass costs more (measured)
  const long target = masked ? kMaskedSplitTarget : kSplitTarget;
  const long most = kbs / (masked ? kMaskedSplitMinBlocks : kSplitMinBlocks);
  long s = (num_cus + tiles - 1) / tiles;
  if (s > target) s = target;
  if (s > most) s = most;
  return s < 2 ? 1 : (int)s;
}

struct Candidate {
  dg::TileShape s;
  double eff;  // relative matrix-unit efficiency of the tile shape
};

// Per-shape tile choice (DeepGEMM pages: block sizes and wave counts are
// selected per shape; small M underuses the matrix units).  `rows` is the
// output rows per group, `groups` the number of groups whose tiles share the
// launch (masked: an upper bound from M_max).  `allow_split`: K may be split
// over workgroups (choose_splits).  Thresholds are from measured sweeps on
// MI355X:
//   * masked layout: tall 256-row tiles (B read once per group, the waves
//     skip the row quarters past masked_m): 256 columns when the groups give
//     1.5 tiles per CU, else 128 columns on 4 waves (long K split to fill the
//     CUs), or 64 when even those are too few for a short K;
//   * few rows (<= 128 per group): the largest tile that still leaves enough
//     tiles -- about 0.7 of the CUs, or a quarter of that when a long K is
//     split four ways -- since such shapes stream B from HBM;
//   * otherwise: minimise (full waves of tiles over the CUs) x (workgroups
//     per CU) x (tile area / tile efficiency), so a large tile wins unless
//     it leaves CUs idle.
dg::TileShape heuristic(int kind, int rows, int n, int k, int groups, int num_cus, bool allow_split) {
  // the fused SwiGLU epilogue's tile: 128 gate + 128 up columns on 2x4 waves
  // (3-4% faster than 1x8, like the plain contiguous GEMM)
  if (kind == DG_KIND_CONTIGUOUS_SWIGLU) return dg::TileShape{256, 256, 2, 4};
  const int kbs = k / 128;
  const bool long_k = allow_split && kbs >= 3 * kSplitMinBlocks;
  const int layout = dg::layout_of(kind);  // the power-of-two kinds plan as their fp32-scale kind
  if (layout == DG_KIND_MASKED && rows <= 256) {
    // 256 columns on 2x4 waves: 3-4% faster than 1x8 for 16 groups (cold)
    const dg::TileShape tall256{256, 256, 2, 4}, tall128{256, 128, 1, 4}, tall64{256, 64, 1, 4};
    const dg::TileShape tall32{256, 32, 4, 1};
    const long cols128 = (long)groups * ceil_div(n, 128);
    if (cols128 * 2 >= 3L * num_cus) return tall256;   // enough tiles at 256 columns
    if (long_k) return tall128;
    // without a split (short K, or a call being captured): 32 columns per
    // tile when that still gives at most one tile per CU -- each tile then
    // streams a quarter of a 128-column tile's B; G=1, N=4096, K=7168 51 us
    // against 67 us on 64 columns, G=1, N=7168, K=2048 19.5 against 22.4 us
    // (cold); with more groups the extra A re-reads cost more (G=4: 95 vs 69 us)
    if ((long)groups * ceil_div(n, 32) <= num_cus) return tall32;
    return cols128 * 4 >= 3L * num_cus ? tall128 : tall64;
  }
  if (rows <= 128 || layout == DG_KIND_MASKED) {
    const int bm = rows <= 64 ? 64 : 128;
    const dg::TileShape wide = bm == 64 ? dg::TileShape{64, 128, 1, 4} : dg::TileShape{128, 128, 2, 2};
    const dg::TileShape mid = bm == 64 ? dg::TileShape{64, 64, 1, 4} : dg::TileShape{128, 64, 2, 2};
    const dg::TileShape cands[5] = {wide, mid, {64, 128, 1, 4}, {64, 64, 1, 4}, {64, 32, 2, 2}};
    const long need = long_k && dense_like(kind)
                          ? (num_cus * 7L) / (10L * kSplitTarget)
                                                         : (num_cus * 7L) / 10L;
    // a long K split four ways: the 64-column tile when the wide one leaves
    // too few tiles, even if it gives fewer tiles than `need` -- narrower
    // tiles re-read A once more per column tile (M=64, N=2112, K=7168:
    // 64x64 tiles 17.2 us against 19.7 us on 64x32, cold)
    if (long_k && dense_like(kind)) {
      const long wide_tiles = (long)groups * ceil_div(rows, wide.bm) * ceil_div(n, wide.bn);
      if (wide_tiles < need && dg::has_instance(kind, mid)) return mid;
    }
    for (const auto& c : cands) {
      if (!dg::has_instance(kind, c)) continue;
      const long tiles = (long)groups * ceil_div(rows, c.bm) * ceil_div(n, c.bn);
      if (tiles >= need) return c;
    }
    return dg::TileShape{64, 32, 2, 2};
  }
  static const Candidate cands[] = {
      // efficiencies measured relative to the 256x256 tile on full waves
      // (the 256x224 tile, 4x2 waves, balances N=7168 over the CUs but ran
      // slower per tile than 256x256 by more than it gains: not a candidate;
      // nor are 256x144 and 256x176 on 8x1 waves, fitted to N=2112, measured
      // at half the per-tile rate; the 192-row tile gives M=4096, N=2112 198
      // tiles instead of 144 on 256 CUs, 10% faster)
      {{256, 256, 2, 4}, 1.00}, {{256, 256, 1, 8}, 0.98}, {{224, 256, 1, 8}, 0.92}, {{192, 256, 2, 4}, 0.80},
      {{256, 128, 2, 2}, 0.85},
      {{128, 128, 2, 2}, 0.70},
      {{128, 64, 2, 2}, 0.50},  {{64, 128, 1, 4}, 0.50},  {{64, 64, 1, 4}, 0.35},
  };
  double best = 1e300;
  dg::TileShape pick{128, 128, 2, 2};
  for (const auto& c : cands) {
    if (!dg::has_instance(kind, c.s)) continue;
    const long tiles = (long)groups * ceil_div(rows, c.s.bm) * ceil_div(n, c.s.bn);
    const long slots = (long)num_cus * occupancy(kind, c.s);
    const long waves = (tiles + slots - 1) / slots;
    // occ workgroups share a CU, so each full wave of tiles takes occ times a
    // tile's own time
    const double cost = (double)waves * occupancy(kind, c.s) * c.s.bm * c.s.bn / c.eff;
    if (cost < best * 0.999) {
      best = cost;
      pick = c.s;
    }
  }
  return pick;
}

struct Launch {
  dg::TileShape shape;
  int grid;
};

// `allow_split`: split-K needs a temporary workspace, so it is planned only
// for calls that may allocate (not under stream capture).
dg_status plan(int kind, int rows, int n, int k, int groups, int num_cus, bool allow_split, dg::Params& p,
               Launch& l) {
  dg::TileShape s;
  const bool forced = parse_forced(&s);
  if (!forced) s = heuristic(kind, rows, n, k, groups, num_cus, allow_split);
  if (!dg::has_instance(kind, s)) return DG_ERROR_UNSUPPORTED;
  p.tiles_m = ceil_div(rows, s.bm);
  p.tiles_n = ceil_div(n, s.bn);
  const long tiles = (long)groups * p.tiles_m * p.tiles_n;
  if (tiles > 0x7fffffffL / kMaxSplits) return DG_ERROR_UNSUPPORTED;
  p.tiles = (int)tiles;
  const long slots = (long)num_cus * occupancy(kind, s);
  const int kbs = k / 128;
  int splits = allow_split ? choose_splits(kind, rows, tiles, num_cus, kbs) : 1;
  if (const char* e = std::getenv("DG_FORCE_SPLITS"))
    if (allow_split && (dense_like(kind) || dg::layout_of(kind) == DG_KIND_MASKED))
      splits = std::atoi(e);
  if (splits < 1) splits = 1;
  if (splits > kMaxSplits) splits = kMaxSplits;
  if (splits > kbs) splits = kbs;
  const double split_bytes = 4.0 * groups * rows * (double)n;  // one fp32 partial of every output
  while (splits > 1 && splits * split_bytes > (double)kMaxWorkspaceBytes) --splits;
  // equal chunks with no empty split: every partial the reduction reads is written
  int chunk = ceil_div(kbs, splits);
  splits = ceil_div(kbs, chunk);
  p.splits = splits;
  p.kchunk = chunk;
  const long work = tiles * splits;
  // a multiple of 8 workgroups keeps the workgroup -> XCD round robin
  // aligned with the kernel's per-XCD item ranges: rounded up when the work
  // fits in one pass (the extra workgroups find no item), so no workgroup
  // takes a second item while others idle; else the largest multiple of 8
  // that fits on the CUs
  long grid = work < slots ? (work + 7) / 8 * 8 : slots;
  if (grid > slots && slots >= 8) grid = slots - slots % 8;
  if (grid > 8 && grid == slots) grid -= grid % 8;
  if (grid < 1) grid = 1;
  l.shape = s;
  l.grid = (int)grid;
  if (std::getenv("DG_LOG"))
    std::fprintf(stderr, "[dg] kind=%d rows=%d n=%d k=%d G=%d -> tile %dx%d waves %dx%d tiles=%ld splits=%d grid=%ld\n",
                 kind, rows, n, k, groups, s.bm, s.bn, s.wm, s.wn, tiles, splits, grid);
  return DG_SUCCESS;
}

// Split-K partials live in a workspace cached per stream: calls on one stream
// run in order, so they share it.  A stream is identified by its unique id
// where the HIP runtime in the process provides one (hipStreamGetId, looked up
// at run time: the runtime that torch loads may predate it), so a stream
// created after another was destroyed never inherits that one's buffer; with
// an older runtime the stream handle is the key, and a caller that destroys a
// stream while a split-K call on it is still running must not start calls on
// a new stream before that work ends (the new stream may receive the same
// handle).  A workspace grows when a call needs more: the new buffer comes
// from a memory pool the library owns per device and the old one goes back to
// it, both in the stream's order (no device synchronisation).  At most
// kMaxCachedStreams streams keep a workspace; a call on any other stream takes
// a buffer from the pool for itself and returns it after its two kernels, in
// stream order.  The pool keeps freed blocks for reuse until the process
// ends.  If no buffer can be had, the call runs without a split.  (An event
// recorded after each call to order a reused handle behind the old work
// would cost about 4 us of GPU time per call: measured, not used.)
constexpr int kMaxCachedStreams = 64;

struct StreamWorkspace {
  int dev;
  unsigned long long key;  // stream id, or the handle's bits
  void* ptr;
  size_t bytes;
};

std::mutex g_ws_mutex;
hipMemPool_t g_pool[kMaxDevices];
StreamWorkspace g_ws[kMaxCachedStreams];
int g_ws_count = 0;

// The cache key of `stream`: its id if the loaded runtime has hipStreamGetId.
unsigned long long stream_key(hipStream_t stream) {
  using GetId = hipError_t (*)(hipStream_t, unsigned long long*);
  static const GetId get_id = reinterpret_cast<GetId>(dlsym(RTLD_DEFAULT, "hipStreamGetId"));
  unsigned long long id = 0;
  if (get_id && get_id(stream, &id) == hipSuccess) return id | (1ull << 63);
  (void)hipGetLastError();
  return reinterpret_cast<uintptr_t>(stream);
}

hipMemPool_t device_pool(int dev) {  // caller holds g_ws_mutex
  if (!g_pool[dev]) {
    hipMemPoolProps props;
    std::memset(&props, 0, sizeof(props));
    props.allocType = hipMemAllocationTypePinned;
    props.handleTypes = hipMemHandleTypeNone;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t pool = nullptr;
    if (hipMemPoolCreate(&pool, &props) != hipSuccess) return nullptr;
    uint64_t keep = UINT64_MAX;
    (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
    g_pool[dev] = pool;
  }
  return g_pool[dev];
}

// A split-K buffer of at least `bytes` usable in the order of `stream`, or
// null.  *owned: the buffer is the call's own (return it with hipFreeAsync
// after the kernels).
void* stream_workspace(hipStream_t stream, size_t bytes, bool* owned) {
  *owned = false;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  const unsigned long long key = stream_key(stream);
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  hipMemPool_t pool = device_pool(dev);
  if (!pool) return nullptr;
  StreamWorkspace* w = nullptr;
  for (int i = 0; i < g_ws_count; ++i)
    if (g_ws[i].dev == dev && g_ws[i].key == key) w = &g_ws[i];
  if (w && w->bytes >= bytes) return w->ptr;
  if (!w && g_ws_count < kMaxCachedStreams) {
    w = &g_ws[g_ws_count++];
    *w = StreamWorkspace{dev, key, nullptr, 0};
  }
  if (!w) {  // not cached: a buffer for this call only
    void* p = nullptr;
    if (hipMallocFromPoolAsync(&p, bytes, pool, stream) != hipSuccess) return nullptr;
    *owned = true;
    return p;
  }
  // grow geometrically so a sequence of slightly larger calls allocates rarely
  size_t want = w->bytes * 2 > bytes ? w->bytes * 2 : bytes;
  if (want > kMaxWorkspaceBytes) want = bytes;
  void* p = nullptr;
  if (hipMallocFromPoolAsync(&p, want, pool, stream) != hipSuccess) return nullptr;
  if (w->ptr) (void)hipFreeAsync(w->ptr, stream);  // after the calls that used it
  w->ptr = p;
  w->bytes = want;
  return p;
}

bool stream_capturing(hipStream_t stream) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return true;  // unknown: do not allocate
  return cs != hipStreamCaptureStatusNone;
}

// Where split-K partials come from: the pool (scratch == nullptr; not while
// the stream is being captured, then K is not split), or a device buffer of
// scratch_floats floats that needs no allocation, which scratch() returns
// (asked only once K is split; split K also under capture; a call whose
// partials do not fit is rejected).
dg_status run(int kind, dg::Params& p, int rows, int n, int k, int groups, hipStream_t stream,
              float* (*scratch)() = nullptr, size_t scratch_floats = 0) {
  int cus = 0;
  if (device_cus(&cus) != 0) return DG_ERROR_LAUNCH;
  (void)hipGetLastError();  // clear a stale error from unrelated work
  if (p.sks == 0) p.sks = p.kbs;  // one fp32 scale per K block unless packed
  const bool splittable = dense_like(kind) || dg::layout_of(kind) == DG_KIND_MASKED;
  const bool may_split = splittable && (scratch != nullptr || !stream_capturing(stream));
  Launch l;
  dg_status st = plan(kind, rows, n, k, groups, cus, may_split, p, l);
  if (st != DG_SUCCESS) return st;
  auto launch_gemm = [&]() {
    return dg::launch(kind, l.shape, p, l.grid, stream);
  };
  if (p.splits <= 1) return launch_gemm() == hipSuccess ? DG_SUCCESS : DG_ERROR_LAUNCH;
  p.ws_stride = (int64_t)groups * rows * n;
  const size_t bytes = (size_t)p.splits * p.ws_stride * sizeof(float);
  if (scratch) {
    if (bytes > scratch_floats * sizeof(float)) return DG_ERROR_WORKSPACE;
    p.ws = scratch();
    if (!p.ws) return DG_ERROR_LAUNCH;
    if (launch_gemm() != hipSuccess) return DG_ERROR_LAUNCH;
    return dg::launch_splitk_reduce(kind, p, stream) == hipSuccess ? DG_SUCCESS : DG_ERROR_LAUNCH;
  }
  bool owned = false;
  void* ws = stream_workspace(stream, bytes, &owned);
  if (!ws) {
    // no workspace to be had (out of memory): the same call without a split
    (void)hipGetLastError();
    st = plan(kind, rows, n, k, groups, cus, false, p, l);
    if (st != DG_SUCCESS) return st;
    return launch_gemm() == hipSuccess ? DG_SUCCESS : DG_ERROR_LAUNCH;
  }
  p.ws = static_cast<float*>(ws);
  const bool ok = launch_gemm() == hipSuccess && dg::launch_splitk_reduce(kind, p, stream) == hipSuccess;
  // the call's own buffer goes back to the pool after both kernels, in stream order
  const bool freed = !owned || hipFreeAsync(ws, stream) == hipSuccess;
  return ok && freed ? DG_SUCCESS : DG_ERROR_LAUNCH;
}

dg_status quantize(int mode, const float* x, void* q, float* s, int rows, int cols, hipStream_t stream) {
  int cus = 0;
  if (device_cus(&cus) != 0) return DG_ERROR_LAUNCH;
  (void)hipGetLastError();  // clear a stale error from unrelated work
  if (dg::launch_quantize(mode, x, static_cast<uint8_t*>(q), s, rows, cols, cus, stream) != hipSuccess)
    return DG_ERROR_LAUNCH;
  return DG_SUCCESS;
}

dg::Params base_params() {
  dg::Params p;
  std::memset(&p, 0, sizeof(p));
  return p;
}

}  // namespace

namespace dg {
// The masked-layout call with split-K partials from the pool (scratch ==
// nullptr) or from the buffer scratch() returns (scratch_floats floats, no
// allocation).
dg_status grouped_masked(const void* a, const float* sa, const void* b, const float* sb, void* c,
                         const int32_t* masked_m, int num_groups, int m_max, int n, int k, hipStream_t stream,
                         float* (*scratch)(), size_t scratch_floats) {
  if (!a || !sa || !b || !sb || !c || !masked_m) return DG_ERROR_INVALID_VALUE;
  if (num_groups <= 0 || m_max <= 0 || n <= 0 || k <= 0) return DG_ERROR_INVALID_VALUE;
  if (k % 128 != 0) return DG_ERROR_UNSUPPORTED;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(sa, 4) || !aligned(sb, 4) || !aligned(c, 2) ||
      !aligned(masked_m, 4))
    return DG_ERROR_UNSUPPORTED;
  Params p = base_params();
  p.a = static_cast<const uint8_t*>(a);
  p.sa = sa;
  p.b = static_cast<const uint8_t*>(b);
  p.sb = sb;
  p.out = c;
  p.ctrl = masked_m;
  p.m = m_max;
  p.n = n;
  p.lda = k;
  p.kbs = k / 128;
  p.groups = num_groups;
  p.vec_out = (n % 4 == 0) && aligned(c, 8);
  return run(KIND_MASKED, p, m_max, n, k, num_groups, stream, scratch, scratch_floats);
}
}  // namespace dg

extern "C" {

dg_status dg_gemm_fp8_nt(const void* a, const float* sa, const void* b, const float* sb, void* c,
                         int m, int n, int k, hipStream_t stream) {
  if (!a || !sa || !b || !sb || !c) return DG_ERROR_INVALID_VALUE;
  if (m <= 0 || n <= 0 || k <= 0) return DG_ERROR_INVALID_VALUE;
  if (k % 128 != 0) return DG_ERROR_UNSUPPORTED;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(sa, 4) || !aligned(sb, 4) || !aligned(c, 2))
    return DG_ERROR_UNSUPPORTED;
  dg::Params p = base_params();
  p.a = static_cast<const uint8_t*>(a);
  p.sa = sa;
  p.b = static_cast<const uint8_t*>(b);
  p.sb = sb;
  p.out = c;
  p.m = m;
  p.n = n;
  p.lda = k;
  p.kbs = k / 128;
  p.groups = 1;
  p.vec_out = (n % 4 == 0) && aligned(c, 8);
  return run(dg::KIND_DENSE, p, m, n, k, 1, stream);
}

dg_status dg_gemm_fp8_nt_ue8m0(const void* a, const float* sa, const void* b, const float* sb, void* c,
                               int m, int n, int k, hipStream_t stream) {
  if (!a || !sa || !b || !sb || !c) return DG_ERROR_INVALID_VALUE;
  if (m <= 0 || n <= 0 || k <= 0) return DG_ERROR_INVALID_VALUE;
  if (k % 128 != 0) return DG_ERROR_UNSUPPORTED;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(sa, 4) || !aligned(sb, 4) || !aligned(c, 2))
    return DG_ERROR_UNSUPPORTED;
  dg::Params p = base_params();
  p.a = static_cast<const uint8_t*>(a);
  p.sa = sa;
  p.b = static_cast<const uint8_t*>(b);
  p.sb = sb;
  p.out = c;
  p.m = m;
  p.n = n;
  p.lda = k;
  p.kbs = k / 128;
  p.groups = 1;
  p.vec_out = (n % 4 == 0) && aligned(c, 8);
  return run(dg::KIND_DENSE_POW2, p, m, n, k, 1, stream);
}

dg_status dg_gemm_fp8_nt_ue8m0_packed(const void* a, const int32_t* sa, const void* b, const int32_t* sb, void* c,
                                      int m, int n, int k, hipStream_t stream) {
  if (!a || !sa || !b || !sb || !c) return DG_ERROR_INVALID_VALUE;
  if (m <= 0 || n <= 0 || k <= 0) return DG_ERROR_INVALID_VALUE;
  if (k % 128 != 0) return DG_ERROR_UNSUPPORTED;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(sa, 4) || !aligned(sb, 4) || !aligned(c, 2))
    return DG_ERROR_UNSUPPORTED;
  dg::Params p = base_params();
  p.a = static_cast<const uint8_t*>(a);
  p.sa = reinterpret_cast<const float*>(sa);  // the kernel copies the words and reads their bytes
  p.b = static_cast<const uint8_t*>(b);
  p.sb = reinterpret_cast<const float*>(sb);
  p.out = c;
  p.m = m;
  p.n = n;
  p.lda = k;
  p.kbs = k / 128;
  p.sks = (p.kbs + 3) / 4;
  p.spk = 2;
  p.groups = 1;
  p.vec_out = (n % 4 == 0) && aligned(c, 8);
  return run(dg::KIND_DENSE_POW2, p, m, n, k, 1, stream);
}

dg_status dg_gemm_bf16_nt(const void* a, const void* b, void* c, int m, int n, int k, hipStream_t stream) {
  if (!a || !b || !c) return DG_ERROR_INVALID_VALUE;
  if (m <= 0 || n <= 0 || k <= 0) return DG_ERROR_INVALID_VALUE;
  if (k % 64 != 0 || k > (1 << 22)) return DG_ERROR_UNSUPPORTED;  // 32-bit byte ranges per tile
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(c, 2)) return DG_ERROR_UNSUPPORTED;
  dg::Params p = base_params();
  p.a = static_cast<const uint8_t*>(a);
  p.b = static_cast<const uint8_t*>(b);
  p.out = c;
  p.m = m;
  p.n = n;
  p.lda = 2 * k;    // bytes per row
  p.kbs = k / 64;   // 128-byte K blocks
  p.groups = 1;
  p.vec_out = (n % 4 == 0) && aligned(c, 8);
  // the planner counts K in bytes / 128: pass the row length in bytes
  return run(dg::KIND_BF16, p, m, n, 2 * k, 1, stream);
}

dg_status dg_grouped_bf16_contiguous(const void* a, const void* b, void* c, const int32_t* m_indices, int m_total,
                                     int n, int k, int num_groups, hipStream_t stream) {
  if (!a || !b || !c || !m_indices) return DG_ERROR_INVALID_VALUE;
  if (m_total <= 0 || n <= 0 || k <= 0 || num_groups <= 0) return DG_ERROR_INVALID_VALUE;
  if (k % 64 != 0 || k > (1 << 22) || m_total % 128 != 0) return DG_ERROR_UNSUPPORTED;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(c, 2) || !aligned(m_indices, 4)) return DG_ERROR_UNSUPPORTED;
  dg::Params p = base_params();
  p.a = static_cast<const uint8_t*>(a);
  p.b = static_cast<const uint8_t*>(b);
  p.out = c;
  p.ctrl = m_indices;
  p.m = m_total;
  p.n = n;
  p.lda = 2 * k;    // bytes per row
  p.kbs = k / 64;   // 128-byte K blocks
  p.groups = num_groups;
  p.vec_out = (n % 4 == 0) && aligned(c, 8);
  return run(dg::KIND_CONTIG_BF16, p, m_total, n, 2 * k, 1, stream);
}

dg_status dg_grouped_bf16_masked(const void* a, const void* b, void* c, const int32_t* masked_m, int num_groups,
                                 int m_max, int n, int k, hipStream_t stream) {
  if (!a || !b || !c || !masked_m) return DG_ERROR_INVALID_VALUE;
  if (num_groups <= 0 || m_max <= 0 || n <= 0 || k <= 0) return DG_ERROR_INVALID_VALUE;
  if (k % 64 != 0 || k > (1 << 22)) return DG_ERROR_UNSUPPORTED;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(c, 2) || !aligned(masked_m, 4)) return DG_ERROR_UNSUPPORTED;
  dg::Params p = base_params();
  p.a = static_cast<const uint8_t*>(a);
  p.b = static_cast<const uint8_t*>(b);
  p.out = c;
  p.ctrl = masked_m;
  p.m = m_max;
  p.n = n;
  p.lda = 2 * k;
  p.kbs = k / 64;
  p.groups = num_groups;
  p.vec_out = (n % 4 == 0) && aligned(c, 8);
  return run(dg::KIND_MASKED_BF16, p, m_max, n, 2 * k, num_groups, stream);
}

dg_status dg_grouped_fp8_contiguous(const void* a, const float* sa, const void* b, const float* sb,
                                    void* c, const int32_t* m_indices, int m_total, int n, int k,
                                    int num_groups, hipStream_t stream) {
  if (!a || !sa || !b || !sb || !c || !m_indices) return DG_ERROR_INVALID_VALUE;
  if (m_total <= 0 || n <= 0 || k <= 0 || num_groups <= 0) return DG_ERROR_INVALID_VALUE;
  if (k % 128 != 0 || m_total % 128 != 0) return DG_ERROR_UNSUPPORTED;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(sa, 4) || !aligned(sb, 4) || !aligned(c, 2) ||
      !aligned(m_indices, 4))
    return DG_ERROR_UNSUPPORTED;
  dg::Params p = base_params();
  p.a = static_cast<const uint8_t*>(a);
  p.sa = sa;
  p.b = static_cast<const uint8_t*>(b);
  p.sb = sb;
  p.out = c;
  p.ctrl = m_indices;
  p.m = m_total;
  p.n = n;
  p.lda = k;
  p.kbs = k / 128;
  p.groups = num_groups;
  p.vec_out = (n % 4 == 0) && aligned(c, 8);
  return run(dg::KIND_CONTIGUOUS, p, m_total, n, k, 1, stream);
}

dg_status dg_grouped_fp8_contiguous_ue8m0_packed(const void* a, const int32_t* sa, const void* b, const int32_t* sb,
                                                 void* c, const int32_t* m_indices, int m_total, int n, int k,
                                                 int num_groups, hipStream_t stream) {
  if (!a || !sa || !b || !sb || !c || !m_indices) return DG_ERROR_INVALID_VALUE;
  if (m_total <= 0 || n <= 0 || k <= 0 || num_groups <= 0) return DG_ERROR_INVALID_VALUE;
  if (k % 128 != 0 || m_total % 128 != 0) return DG_ERROR_UNSUPPORTED;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(sa, 4) || !aligned(sb, 4) || !aligned(c, 2) ||
      !aligned(m_indices, 4))
    return DG_ERROR_UNSUPPORTED;
  dg::Params p = base_params();
  p.a = static_cast<const uint8_t*>(a);
  p.sa = reinterpret_cast<const float*>(sa);  // the kernel copies the words and reads their bytes
  p.b = static_cast<const uint8_t*>(b);
  p.sb = reinterpret_cast<const float*>(sb);
  p.out = c;
  p.ctrl = m_indices;
  p.m = m_total;
  p.n = n;
  p.lda = k;
  p.kbs = k / 128;
  p.sks = (p.kbs + 3) / 4;
  p.spk = 2;
  p.groups = num_groups;
  p.vec_out = (n % 4 == 0) && aligned(c, 8);
  return run(dg::KIND_CONTIG_POW2, p, m_total, n, k, 1, stream);
}

dg_status dg_grouped_fp8_masked_ue8m0_packed(const void* a, const int32_t* sa, const void* b, const int32_t* sb,
                                             void* c, const int32_t* masked_m, int num_groups, int m_max, int n,
                                             int k, hipStream_t stream) {
  if (!a || !sa || !b || !sb || !c || !masked_m) return DG_ERROR_INVALID_VALUE;
  if (num_groups <= 0 || m_max <= 0 || n <= 0 || k <= 0) return DG_ERROR_INVALID_VALUE;
  if (k % 128 != 0) return DG_ERROR_UNSUPPORTED;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(sa, 4) || !aligned(sb, 4) || !aligned(c, 2) ||
      !aligned(masked_m, 4))
    return DG_ERROR_UNSUPPORTED;
  dg::Params p = base_params();
  p.a = static_cast<const uint8_t*>(a);
  p.sa = reinterpret_cast<const float*>(sa);
  p.b = static_cast<const uint8_t*>(b);
  p.sb = reinterpret_cast<const float*>(sb);
  p.out = c;
  p.ctrl = masked_m;
  p.m = m_max;
  p.n = n;
  p.lda = k;
  p.kbs = k / 128;
  p.sks = (p.kbs + 3) / 4;
  p.spk = 2;
  p.groups = num_groups;
  p.vec_out = (n % 4 == 0) && aligned(c, 8);
  return run(dg::KIND_MASKED_POW2, p, m_max, n, k, num_groups, stream);
}

dg_status dg_grouped_fp8_contiguous_swiglu(const void* a, const float* sa, const void* b, const float* sb,
                                           void* q, float* s, const int32_t* m_indices, int m_total, int n, int k,
                                           int num_groups, hipStream_t stream) {
  if (!a || !sa || !b || !sb || !q || !s || !m_indices) return DG_ERROR_INVALID_VALUE;
  if (m_total <= 0 || n <= 0 || k <= 0 || num_groups <= 0) return DG_ERROR_INVALID_VALUE;
  if (k % 128 != 0 || m_total % 128 != 0 || n % 256 != 0) return DG_ERROR_UNSUPPORTED;
  // one B range spans the tile's gate and up rows: (N/2 + 128) * K bytes
  if ((int64_t)(n / 2 + 128) * k > (int64_t)0xffffffffLL) return DG_ERROR_UNSUPPORTED;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(sa, 4) || !aligned(sb, 4) || !aligned(q, 4) ||
      !aligned(s, 4) || !aligned(m_indices, 4))
    return DG_ERROR_UNSUPPORTED;
  dg::Params p = base_params();
  p.a = static_cast<const uint8_t*>(a);
  p.sa = sa;
  p.b = static_cast<const uint8_t*>(b);
  p.sb = sb;
  p.out = q;
  p.out_scale = s;
  p.ctrl = m_indices;
  p.m = m_total;
  p.n = n;
  p.lda = k;
  p.kbs = k / 128;
  p.groups = num_groups;
  return run(dg::KIND_CONTIG_SWIGLU, p, m_total, n, k, 1, stream);
}

dg_status dg_grouped_fp8_masked(const void* a, const float* sa, const void* b, const float* sb,
                                void* c, const int32_t* masked_m, int num_groups, int m_max, int n,
                                int k, hipStream_t stream) {
  return dg::grouped_masked(a, sa, b, sb, c, masked_m, num_groups, m_max, n, k, stream, nullptr, 0);
}

dg_status dg_wgrad_fp8_nt(const void* a, const float* sa, const void* b, const float* sb, float* d,
                          int m, int n, int k, hipStream_t stream) {
  if (!a || !sa || !b || !sb || !d) return DG_ERROR_INVALID_VALUE;
  if (m <= 0 || n <= 0 || k <= 0) return DG_ERROR_INVALID_VALUE;
  if (k % 128 != 0) return DG_ERROR_UNSUPPORTED;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(sa, 4) || !aligned(sb, 4) || !aligned(d, 4))
    return DG_ERROR_UNSUPPORTED;
  dg::Params p = base_params();
  p.a = static_cast<const uint8_t*>(a);
  p.sa = sa;
  p.b = static_cast<const uint8_t*>(b);
  p.sb = sb;
  p.out = d;
  p.m = m;
  p.n = n;
  p.lda = k;
  p.kbs = k / 128;
  p.groups = 1;
  p.vec_out = (n % 4 == 0) && aligned(d, 16);
  return run(dg::KIND_WGRAD, p, m, n, k, 1, stream);
}

dg_status dg_k_grouped_wgrad_fp8_nt(const void* a, const float* sa, const void* b, const float* sb,
                                    float* d, const int32_t* ks_host, int num_groups, int m, int n,
                                    hipStream_t stream) {
  if (!a || !sa || !b || !sb || !d || !ks_host) return DG_ERROR_INVALID_VALUE;
  if (num_groups <= 0 || m <= 0 || n <= 0) return DG_ERROR_INVALID_VALUE;
  if (num_groups > dg::kMaxKGroups) return DG_ERROR_UNSUPPORTED;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(sa, 4) || !aligned(sb, 4) || !aligned(d, 4))
    return DG_ERROR_UNSUPPORTED;
  dg::Params p = base_params();
  long total = 0;
  int min_blocks = 0x7fffffff;
  for (int g = 0; g < num_groups; ++g) {
    if (ks_host[g] < 0) return DG_ERROR_INVALID_VALUE;
    if (ks_host[g] % 128 != 0) return DG_ERROR_UNSUPPORTED;
    p.kb_begin[g] = (int)(total / 128);
    total += ks_host[g];
    if (ks_host[g] > 0 && ks_host[g] / 128 < min_blocks) min_blocks = ks_host[g] / 128;
  }
  p.kg_min_blocks = min_blocks;
  if (total > 0x7fffffffL) return DG_ERROR_UNSUPPORTED;
  p.kb_begin[num_groups] = (int)(total / 128);
  if (total == 0) return DG_SUCCESS;  // no tokens: every D[g] stays as it is
  p.a = static_cast<const uint8_t*>(a);
  p.sa = sa;
  p.b = static_cast<const uint8_t*>(b);
  p.sb = sb;
  p.out = d;
  p.m = m;
  p.n = n;
  p.lda = (int)total;
  p.kbs = (int)(total / 128);
  p.groups = num_groups;
  p.vec_out = (n % 4 == 0) && aligned(d, 16);
  return run(dg::KIND_KGROUPED, p, m, n, (int)total, num_groups, stream);
}

const char* dg_status_string(dg_status s) {
  switch (s) {
    case DG_SUCCESS: return "success";
    case DG_ERROR_INVALID_VALUE: return "invalid value (null pointer or a size <= 0)";
    case DG_ERROR_UNSUPPORTED: return "unsupported (K or row count not a multiple of 128, misaligned pointer, or layout limit)";
    case DG_ERROR_LAUNCH: return "kernel launch failed";
    case DG_ERROR_WORKSPACE:
      return "the call's split-K partials exceed the fixed scratch of the allocation-free entry point";
  }
  return "unknown status";
}

dg_status dg_select_config(int kind, int m, int n, int k, int num_groups, int num_cus,
                           dg_tile_config* out) {
  if (!out) return DG_ERROR_INVALID_VALUE;
  if (kind < DG_KIND_DENSE || kind > DG_KIND_MASKED_BF16) return DG_ERROR_INVALID_VALUE;
  if (kind == DG_KIND_CONTIGUOUS_SWIGLU && (n % 256 != 0 || m % 128 != 0)) return DG_ERROR_UNSUPPORTED;
  if (m <= 0 || n <= 0 || k <= 0 || num_groups <= 0 || num_cus <= 0) return DG_ERROR_INVALID_VALUE;
  if (dg::bf16_kind(kind) && k > (1 << 22)) return DG_ERROR_UNSUPPORTED;
  dg::Params p = base_params();
  Launch l;
  const int groups =
      (dg::layout_of(kind) == DG_KIND_MASKED || kind == DG_KIND_K_GROUPED_WGRAD) ? num_groups : 1;
  // the planner counts K in 128-byte blocks: BF16 rows are 2K bytes long
  dg_status st = plan(kind, m, n, dg::bf16_kind(kind) ? 2 * k : k, groups, num_cus, true, p, l);
  if (st != DG_SUCCESS) return st;
  out->block_m = l.shape.bm;
  out->block_n = l.shape.bn;
  out->waves_m = l.shape.wm;
  out->waves_n = l.shape.wn;
  out->tiles = p.tiles;
  out->grid = l.grid;
  out->k_splits = p.splits;
  out->kernel = 0;
  return DG_SUCCESS;
}

dg_status dg_quantize_fp8_1x128(const float* x, void* q, float* s, int m, int k, hipStream_t stream) {
  if (!x || !q || !s) return DG_ERROR_INVALID_VALUE;
  if (m <= 0 || k <= 0) return DG_ERROR_INVALID_VALUE;
  if (k % 128 != 0) return DG_ERROR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(q, 4) || !aligned(s, 4)) return DG_ERROR_UNSUPPORTED;
  return quantize(0, x, q, s, m, k, stream);
}

dg_status dg_quantize_fp8_128x128(const float* x, void* q, float* s, int n, int k, hipStream_t stream) {
  if (!x || !q || !s) return DG_ERROR_INVALID_VALUE;
  if (n <= 0 || k <= 0) return DG_ERROR_INVALID_VALUE;
  if (k % 128 != 0) return DG_ERROR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(q, 4) || !aligned(s, 4)) return DG_ERROR_UNSUPPORTED;
  return quantize(1, x, q, s, n, k, stream);
}

dg_status dg_quantize_fp8_1x128_ue8m0(const float* x, void* q, int32_t* s, int m, int k, hipStream_t stream) {
  if (!x || !q || !s) return DG_ERROR_INVALID_VALUE;
  if (m <= 0 || k <= 0) return DG_ERROR_INVALID_VALUE;
  if (k % 128 != 0) return DG_ERROR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(q, 4) || !aligned(s, 4)) return DG_ERROR_UNSUPPORTED;
  return quantize(3, x, q, reinterpret_cast<float*>(s), m, k, stream);
}

dg_status dg_quantize_fp8_128x128_ue8m0(const float* x, void* q, int32_t* s, int n, int k, hipStream_t stream) {
  if (!x || !q || !s) return DG_ERROR_INVALID_VALUE;
  if (n <= 0 || k <= 0) return DG_ERROR_INVALID_VALUE;
  if (k % 128 != 0) return DG_ERROR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(q, 4) || !aligned(s, 4)) return DG_ERROR_UNSUPPORTED;
  return quantize(4, x, q, reinterpret_cast<float*>(s), n, k, stream);
}

dg_status dg_quantize_fp8_1x128_transposed(const float* x, void* q, float* s, int t, int f,
                                           hipStream_t stream) {
  if (!x || !q || !s) return DG_ERROR_INVALID_VALUE;
  if (t <= 0 || f <= 0) return DG_ERROR_INVALID_VALUE;
  if (t % 128 != 0 || f % 4 != 0) return DG_ERROR_UNSUPPORTED;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(s, 4)) return DG_ERROR_UNSUPPORTED;
  return quantize(2, x, q, s, t, f, stream);
}

dg_status dg_swiglu_quantize_fp8_1x128(const void* c, void* q, float* s, int m, int i, hipStream_t stream) {
  if (!c || !q || !s) return DG_ERROR_INVALID_VALUE;
  if (m <= 0 || i <= 0) return DG_ERROR_INVALID_VALUE;
  if (i % 128 != 0 || i > INT_MAX / 2) return DG_ERROR_UNSUPPORTED;
  if (!aligned(c, 16) || !aligned(q, 8) || !aligned(s, 4)) return DG_ERROR_UNSUPPORTED;
  int cus = 0;
  if (device_cus(&cus) != 0) return DG_ERROR_LAUNCH;
  (void)hipGetLastError();  // clear a stale error from unrelated work
  if (dg::launch_swiglu_quantize(static_cast<const uint16_t*>(c), static_cast<uint8_t*>(q), s, m, i, cus, stream) !=
      hipSuccess)
    return DG_ERROR_LAUNCH;
  return DG_SUCCESS;
}

int dg_version(void) { return 100; }

}  // extern "C"
