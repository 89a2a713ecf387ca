// C ABI of the Stream-K GEMM library: argument checks, the Stream-K planner,
// per-(device, stream) scratch, and the launch.
//
// The scratch (fp32 partial tiles P, lock flags, an error word) is owned here
// and cached per device *and* stream, never shared between devices: a single
// global buffer on the default device breaks calls made on another GPU
// ("Stream-k mxfp4 kernel", Copilot comment on the global Stream-K scratch
// buffers).  The flags carry a per-launch epoch, so their old contents never
// matter (freshly allocated lock buffers may hold anything).

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "../../include/sk_gemm.h"
#include "sk_common.h"

namespace {

using sk::KArgs;
using sk::Variant;

using sk::kMaxIters;
using sk::kMaxK;
using sk::kMaxM;
using sk::kMaxN;
constexpr uint64_t kDefaultSpin = 200000000ull;  // 2 s of the 100 MHz device clock

struct DeviceInfo {
  bool ok = false;
  bool gfx950 = false;
  int cus = 0;
};

struct Workspace {
  int device = -1;
  hipStream_t stream = nullptr;
  float* P = nullptr;
  size_t p_bytes = 0;
  uint8_t* S = nullptr;       // MXFP4 scales of A and B, k-step-major
  size_t s_bytes = 0;
  uint8_t* T = nullptr;       // bf16 backward: transposed operands, dbias partial sums
  size_t t_bytes = 0;
  uint32_t* flags = nullptr;  // kMaxGrid locks, then the error word
  uint32_t epoch = 0;         // last epoch used
};

std::mutex g_mu;
std::map<std::pair<int, uintptr_t>, Workspace*> g_ws;
std::map<int, DeviceInfo> g_dev;
// Compute units a stream's kernels may use, read once per (device, stream).
std::map<std::pair<int, uintptr_t>, int> g_stream_cus;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool dtype_ok(int d) { return d >= SK_MXFP4 && d <= SK_MXFP8_MXFP4; }

// Block-scaled (MX) input types: one E8M0 scale byte per 32 K elements.
bool is_mx(int d) { return dtype_ok(d) && d != SK_BF16 && d != SK_FP8_E4M3; }

// Bytes of one row of A (b: of B) for K elements: E2M1 4 bits, E2M3 / E3M2 6,
// E4M3 8, bf16 16 per element.
int64_t row_bytes(int dtype, int64_t K, bool b = false) {
  switch (dtype) {
    case SK_MXFP4: return K / 2;
    case SK_BF16: return 2 * K;
    case SK_MXFP6_E2M3:
    case SK_MXFP6_E3M2: return 3 * K / 4;
    case SK_MXFP4_MXFP8: return b ? K : K / 2;
    case SK_MXFP8_MXFP4: return b ? K / 2 : K;
    default: return K;
  }
}

sk_status device_info(int* dev_out, DeviceInfo* info) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SK_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_dev.find(dev);
  if (it == g_dev.end()) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return SK_ERR_HIP;
    DeviceInfo d;
    d.ok = true;
    d.gfx950 = std::strncmp(p.gcnArchName, "gfx950", 6) == 0;
    d.cus = p.multiProcessorCount;
    it = g_dev.emplace(dev, d).first;
  }
  *dev_out = dev;
  *info = it->second;
  return SK_OK;
}

// Number of set bits among the first `cus` bits of a CU mask.
int mask_count(const uint32_t* mask, int words, int cus) {
  int n = 0;
  for (int i = 0; i < words; ++i) {
    uint32_t w = mask[i];
    if (32 * i + 32 > cus) w &= (32 * i >= cus) ? 0u : ((1u << (cus - 32 * i)) - 1u);
    n += __builtin_popcount(w);
  }
  return n;
}

// Compute units that kernels launched on `stream` may use: the size of its
// CU mask (every CU for the null stream or when the mask cannot be read).
int stream_cus(int dev, hipStream_t stream, int device_cus) {
  if (!stream) return device_cus;
  const auto key = std::make_pair(dev, (uintptr_t)stream);
  {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_stream_cus.find(key);
    if (it != g_stream_cus.end()) return it->second;
  }
  const int words = (device_cus + 31) / 32;
  std::vector<uint32_t> mask((size_t)words, 0u);
  int n = device_cus;
  if (hipExtStreamGetCUMask(stream, (uint32_t)words, mask.data()) == hipSuccess) {
    const int m = mask_count(mask.data(), words, device_cus);
    if (m > 0) n = m;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  g_stream_cus[key] = n;
  return n;
}

// Measured choices for SK_POLICY_AUTO: the fastest (kernel, policy) at each
// swept shape (written by persistent_gemm_amd/tune.py).  An entry is used
// only while the kernel at its index still has the tile and thread count it
// was measured with.
struct TuneEntry {
  int dtype;
  int64_t M, N, K;
  int variant, policy;
  int bm, bn, threads;
};
#include "sk_tuning_table.inc"

// The tuned (variant, policy) of the measured shape nearest to (M, N, K)
// in log scale; false if the table has no usable entry for the dtype.  The
// entries' logarithms are taken once, and each host thread remembers its last
// answer, so a repeated call costs one comparison (the scan alone took about
// 8 us per call, as long as a small kernel).
bool tuned_choice(int dtype, int64_t M, int64_t N, int64_t K, int* variant, int* policy) {
  constexpr int kEntries = (int)(sizeof(kTuneTable) / sizeof(kTuneTable[0]));
  struct Logs {
    double m[kEntries], n[kEntries], k[kEntries];
    bool usable[kEntries];
  };
  static const Logs logs = [] {
    Logs l;
    for (int i = 0; i < kEntries; ++i) {
      const TuneEntry& e = kTuneTable[i];
      const Variant* v = sk::variant(e.variant);
      l.usable[i] = v && v->dtype == e.dtype && v->bm == e.bm && v->bn == e.bn && v->threads == e.threads;
      l.m[i] = std::log2((double)e.M);
      l.n[i] = std::log2((double)e.N);
      l.k[i] = std::log2((double)e.K);
    }
    return l;
  }();
  struct Last {
    int dtype = -1;
    int64_t M = 0, N = 0, K = 0;
    bool found = false;
    int variant = 0, policy = 0;
  };
  thread_local Last last;
  if (last.dtype == dtype && last.M == M && last.N == N && last.K == K) {
    *variant = last.variant;
    *policy = last.policy;
    return last.found;
  }
  const double lm = std::log2((double)M), ln = std::log2((double)N), lk = std::log2((double)K);
  double best = 1e300;
  bool found = false;
  for (int i = 0; i < kEntries; ++i) {
    if (kTuneTable[i].dtype != dtype || !logs.usable[i]) continue;
    const double d = std::fabs(lm - logs.m[i]) + std::fabs(ln - logs.n[i]) + std::fabs(lk - logs.k[i]);
    if (d < best) {
      best = d;
      *variant = kTuneTable[i].variant;
      *policy = kTuneTable[i].policy;
      found = true;
    }
  }
  last.dtype = dtype;
  last.M = M;
  last.N = N;
  last.K = K;
  last.found = found;
  last.variant = found ? *variant : 0;
  last.policy = found ? *policy : 0;
  return found;
}

// Kernel shape: an explicit (tile_m, tile_n), else a choice by problem shape.
int pick_variant(int dtype, int64_t M, int64_t N, int tile_m, int tile_n, int forced) {
  const int nv = sk::num_variants();
  if (forced > 0) {
    const Variant* v = sk::variant(forced - 1);
    return (v && v->dtype == dtype) ? forced - 1 : -1;
  }
  // (kernels that read only the caller's scales are taken from the tuned table, or by index)
  auto find = [&](int bm, int bn) {
    for (int i = 0; i < nv; ++i) {
      const Variant* v = sk::variant(i);
      if (v->dtype == dtype && v->bm == bm && v->bn == bn && v->launch) return i;
    }
    return -1;
  };
  if (tile_m > 0 || tile_n > 0) return find(tile_m, tile_n);
  if (M <= 16) {
    int i = find(16, 256);
    if (i >= 0) return i;
  }
  if (M <= 64 && N <= 64) {
    int i = find(64, 64);
    if (i >= 0) return i;
  }
  if (M * N <= (int64_t)2048 * 2048) {
    int i = find(128, 128);
    if (i >= 0) return i;
  }
  return find(256, 256);
}

// Whether a call can read the MX scales straight from the caller's arrays
// with variant v: K a whole number of the kernel's k-steps (no k-step reads
// past a row's last scale byte), and the scale arrays aligned for the
// kernel's loads (4 bytes; 16 for the k-split kernels, whose loads take 16
// bytes of a row at a time).  `align`: the alignment both scale arrays share
// (a power of two up to 16), 0 when the caller asked for the re-laid copy.
bool direct_fits(const Variant* v, int64_t K, int align) {
  if (!v->launch_direct || align < (v->wk > 1 ? 16 : 4)) return false;
  const int64_t spr = v->dtype == SK_MXFP4 ? v->kb / 16 : v->kb / 32;   // scale bytes per row per k-step
  return (K / 32) % spr == 0;
}

int scale_alignment(const sk_gemm_args& g) {
  if (g.debug_flags & SK_DEBUG_RELAYOUT) return 0;
  const uintptr_t x = (uintptr_t)g.A_scale | (uintptr_t)g.B_scale;
  int a = 1;
  while (a < 16 && !(x & (uintptr_t)a)) a *= 2;
  return a;
}

// `scale_align`: direct_fits' `align` for the call (a plan query assumes 16).
// A kernel that reads only the caller's scales (no re-layout launcher) is
// used only where direct_fits; the tuned table's choice is then skipped, and
// an explicitly chosen kernel is SK_ERR_UNSUPPORTED.
sk_status make_plan(int dtype, int policy, int64_t M, int64_t N, int64_t K, int grid_cap, int tile_m, int tile_n,
                    int forced, int num_cus, sk_plan_info* p, int scale_align = 16) {
  if (!dtype_ok(dtype)) return SK_ERR_ARG;
  if (policy < SK_POLICY_HYBRID || policy > SK_POLICY_AUTO) return SK_ERR_ARG;
  if (M < 1 || N < 1 || K < 1 || M >= kMaxM || N > kMaxN || K > kMaxK) return SK_ERR_ARG;
  if (num_cus < 1) return SK_ERR_ARG;
  if (forced < 0) return SK_ERR_ARG;
  auto usable = [&](const Variant* v) { return v->launch || direct_fits(v, K, scale_align); };
  if (policy == SK_POLICY_AUTO) {
    // measured (kernel, policy) unless the caller fixed the kernel; else HYBRID
    int tv = -1, tp = SK_POLICY_HYBRID;
    if (forced == 0 && tile_m <= 0 && tile_n <= 0 && tuned_choice(dtype, M, N, K, &tv, &tp)) {
      if (usable(sk::variant(tv))) forced = tv + 1;
      else tp = SK_POLICY_HYBRID;
    }
    policy = tp;
  }
  const int vi = pick_variant(dtype, M, N, tile_m, tile_n, forced);
  if (vi < 0) return SK_ERR_UNSUPPORTED;
  const Variant* v = sk::variant(vi);
  if (!usable(v)) return SK_ERR_UNSUPPORTED;
  std::memset(p, 0, sizeof(*p));
  p->tile_m = v->bm;
  p->tile_n = v->bn;
  p->tile_k = v->bk;
  p->tiles_m = (int32_t)cdiv(M, v->bm);
  p->tiles_n = (int32_t)cdiv(N, v->bn);
  p->tiles = (int64_t)p->tiles_m * p->tiles_n;
  p->iters_per_tile = (int32_t)cdiv(K, v->bk);
  p->policy = policy;
  p->variant = vi;
  p->threads = v->threads;
  p->lds_bytes = v->lds;
  int64_t cap = grid_cap <= 0 ? num_cus : (grid_cap < num_cus ? grid_cap : num_cus);
  if (cap > sk::kMaxGrid) cap = sk::kMaxGrid;
  const int64_t T = p->tiles, I = p->iters_per_tile;
  if (T * I > kMaxIters) return SK_ERR_ARG;
  int64_t G, sk_tiles;
  if (policy == SK_POLICY_PURE_DP) {
    G = cap < T ? cap : T;
    sk_tiles = 0;
  } else if (policy == SK_POLICY_PURE_SK) {
    G = cap < T * I ? cap : T * I;
    sk_tiles = T;
  } else {
    if (T >= cap) {
      G = cap;
      const int64_t rem = T % G;
      sk_tiles = rem == 0 ? 0 : rem + G;
      if (sk_tiles > T) sk_tiles = T;
    } else {
      G = cap < T * I ? cap : T * I;
      sk_tiles = T;
    }
  }
  p->grid = (int32_t)G;
  p->sk_tiles = sk_tiles;
  p->sk_iters = sk_tiles * I;
  p->iters_per_wg = p->sk_iters / G;
  p->iters_extra = p->sk_iters % G;
  p->scratch_bytes = sk_tiles > 0 ? G * (int64_t)v->bm * v->bn * (int64_t)sizeof(float) : 0;
  return SK_OK;
}

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  if (!a || !b || na <= 0 || nb <= 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

sk_status validate(const sk_gemm_args& g) {
  if (!dtype_ok(g.dtype)) return SK_ERR_ARG;
  if (g.policy < SK_POLICY_HYBRID || g.policy > SK_POLICY_AUTO) return SK_ERR_ARG;
  if (!g.A || !g.B || !g.C) return SK_ERR_ARG;
  if (g.M < 1 || g.N < 1 || g.K < 1 || g.M >= kMaxM || g.N > kMaxN || g.K > kMaxK) return SK_ERR_ARG;
  if (is_mx(g.dtype) && (!g.A_scale || !g.B_scale)) return SK_ERR_ARG;
  if (g.dtype == SK_BF16 && (g.A_scale || g.B_scale)) return SK_ERR_ARG;
  if (is_mx(g.dtype) && g.K % 32) return SK_ERR_ALIGN;
  if (g.dtype == SK_FP8_E4M3 && g.K % 16) return SK_ERR_ALIGN;
  if (g.dtype == SK_BF16 && g.K % 8) return SK_ERR_ALIGN;
  if (((uintptr_t)g.A | (uintptr_t)g.B | (uintptr_t)g.C) & 15) return SK_ERR_ALIGN;
  if (g.bias && ((uintptr_t)g.bias & 1)) return SK_ERR_ALIGN;
  if (g.dtype == SK_FP8_E4M3 && (((uintptr_t)g.A_scale | (uintptr_t)g.B_scale) & 3)) return SK_ERR_ALIGN;
  const int64_t rb = row_bytes(g.dtype, g.K), rbb = row_bytes(g.dtype, g.K, true);
  const int64_t c_bytes = g.M * g.N * 2;
  const int64_t sbytes = is_mx(g.dtype) ? g.K / 32 : (g.dtype == SK_FP8_E4M3 ? 4 : 0);
  if (overlaps(g.C, c_bytes, g.A, g.M * rb) || overlaps(g.C, c_bytes, g.B, g.N * rbb) ||
      overlaps(g.C, c_bytes, g.bias, g.N * 2) ||
      overlaps(g.C, c_bytes, g.A_scale, is_mx(g.dtype) ? g.M * sbytes : sbytes) ||
      overlaps(g.C, c_bytes, g.B_scale, is_mx(g.dtype) ? g.N * sbytes : sbytes))
    return SK_ERR_ARG;
  return SK_OK;
}

// Grows one workspace buffer; work queued on the stream may still read the old one.
template <class T>
sk_status grow(hipStream_t stream, T** buf, size_t* have, size_t want) {
  if (want <= *have) return SK_OK;
  if (*buf) {
    if (hipStreamSynchronize(stream) != hipSuccess) return SK_ERR_HIP;
    hipFree(*buf);
    *buf = nullptr;
    *have = 0;
  }
  if (hipMalloc((void**)buf, want) != hipSuccess) {
    *buf = nullptr;
    return SK_ERR_NOMEM;
  }
  *have = want;
  return SK_OK;
}

// Scratch of (device, stream), grown to p_bytes of partial tiles and s_bytes
// of re-laid scales; called with g_mu unlocked.
sk_status get_workspace(int dev, hipStream_t stream, size_t p_bytes, size_t s_bytes, Workspace** out) {
  std::lock_guard<std::mutex> lk(g_mu);
  const auto key = std::make_pair(dev, (uintptr_t)stream);
  Workspace*& ws = g_ws[key];
  if (!ws) {
    Workspace* w = new Workspace();
    w->device = dev;
    w->stream = stream;
    if (hipMalloc((void**)&w->flags, sk::kFlagWords * sizeof(uint32_t)) != hipSuccess) {
      delete w;
      g_ws.erase(key);
      return SK_ERR_NOMEM;
    }
    if (hipMemset(w->flags, 0, sk::kFlagWords * sizeof(uint32_t)) != hipSuccess) {
      hipFree(w->flags);
      delete w;
      g_ws.erase(key);
      return SK_ERR_HIP;
    }
    ws = w;
  }
  sk_status st = grow(stream, &ws->P, &ws->p_bytes, p_bytes);
  if (st != SK_OK) return st;
  st = grow(stream, &ws->S, &ws->s_bytes, s_bytes);
  if (st != SK_OK) return st;
  *out = ws;
  return SK_OK;
}

// The backward pass's buffer of (device, stream), grown to t_bytes; called
// with g_mu unlocked.
sk_status get_aux(int dev, hipStream_t stream, size_t t_bytes, uint8_t** out) {
  Workspace* ws = nullptr;
  sk_status st = get_workspace(dev, stream, 0, 0, &ws);
  if (st != SK_OK) return st;
  std::lock_guard<std::mutex> lk(g_mu);
  st = grow(stream, &ws->T, &ws->t_bytes, t_bytes);
  if (st != SK_OK) return st;
  *out = ws->T;
  return SK_OK;
}

// Next epoch of a workspace; restarts the flags when the counter would wrap.
sk_status next_epoch(Workspace* ws, uint32_t* epoch) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (ws->epoch == 0xFFFFFFFFu) {
    if (hipMemsetAsync(ws->flags, 0, sk::kMaxGrid * sizeof(uint32_t), ws->stream) != hipSuccess) return SK_ERR_HIP;
    ws->epoch = 0;
  }
  *epoch = ++ws->epoch;
  return SK_OK;
}

// ---------------------------------------------------------------- fixed scratch (no allocation)
//
// sk_gemm_mxfp4_noalloc runs the same kernels with their scratch (lock flags
// and the error word, fp32 partial tiles, the re-laid MX scales) taken from
// this file-scope device array instead of the per-(device, stream)
// workspace, for callers that cannot allocate device memory.  Each device the
// library runs on holds its own copy until the process ends.  Host code never
// uses the array's name as an address: its device address is read once per
// device (static_scratch) and only that pointer is passed on.
constexpr size_t kStaticFlagBytes = 8192;               // the flag words, rounded up
constexpr size_t kStaticDataBytes = (size_t)32 << 20;   // partial tiles and re-laid scales
static_assert(sk::kFlagWords * sizeof(uint32_t) <= kStaticFlagBytes, "flag words fit");
static __device__ __align__(256) uint8_t scratch[kStaticFlagBytes + kStaticDataBytes];

constexpr int kMaxDevices = 64;
struct StaticScratch {
  uint8_t* ptr = nullptr;   // device address of `scratch` on this device
  uint32_t epoch = 0;       // last epoch used on it
};
StaticScratch g_static[kMaxDevices];   // guarded by g_mu

// The device address of this device's copy of `scratch`, set up on the first
// call: the address comes from the runtime (the array's name is only a
// host-side stand-in), and the flag words are cleared once, on `stream`,
// before any kernel reads them.  Called with g_mu unlocked.
sk_status static_scratch(int dev, hipStream_t stream, uint8_t** out) {
  if (dev < 0 || dev >= kMaxDevices) return SK_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_mu);
  StaticScratch& st = g_static[dev];
  if (!st.ptr) {
    uint8_t* ptr = nullptr;
    if (hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SK_ERR_HIP;
    if (hipMemsetAsync(ptr, 0, kStaticFlagBytes, stream) != hipSuccess) return SK_ERR_HIP;
    if (hipStreamSynchronize(stream) != hipSuccess) return SK_ERR_HIP;
    st.ptr = ptr;
  }
  *out = st.ptr;
  return SK_OK;
}

// A stream being captured into a HIP graph is refused before anything is
// enqueued: the fixup compares lock flags with an epoch passed as a kernel
// argument, so a replayed launch would reuse one epoch and an owner could
// accept the flags (and read the partials) of the previous replay; growing
// the scratch would also need a synchronisation that capture forbids.
sk_status refuse_capture(hipStream_t stream) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return SK_ERR_HIP;
  return cs == hipStreamCaptureStatusNone ? SK_OK : SK_ERR_UNSUPPORTED;
}

// The scratch one launch uses: partial tiles, re-laid scales, the flag words
// (locks, then the error word) and this launch's epoch.
struct Scratch {
  float* P = nullptr;
  uint8_t* S = nullptr;
  uint32_t* flags = nullptr;
  uint32_t epoch = 0;
};

// fixed: take the scratch from this device's `scratch` array (nothing is
// allocated); a plan whose partial tiles do not fit there runs data-parallel
// instead, and one whose re-laid scales do not fit is refused (SK_ERR_SCRATCH).
sk_status run(const sk_gemm_args& g, bool fixed = false) {
  sk_status st = validate(g);
  if (st != SK_OK) return st;
  st = refuse_capture((hipStream_t)g.stream);
  if (st != SK_OK) return st;
  int dev = 0;
  DeviceInfo info;
  st = device_info(&dev, &info);
  if (st != SK_OK) return st;
  if (!info.gfx950) return SK_ERR_UNSUPPORTED;
  sk_plan_info p;
  // The grid is sized to the compute units the stream may use, so on a
  // CU-masked stream the cap is a partition of the device, not a count.
  const int cus = stream_cus(dev, (hipStream_t)g.stream, info.cus);
  const int scale_align = scale_alignment(g);
  st = make_plan(g.dtype, g.policy, g.M, g.N, g.K, g.grid_cap, g.tile_m, g.tile_n, g.variant, cus, &p, scale_align);
  if (st != SK_OK) return st;
  if (fixed && (uint64_t)p.scratch_bytes > kStaticDataBytes) {
    // The same kernel over whole tiles needs no partial tiles.  Only MXFP4 takes
    // this path, whose fp32 sums are exact in any order: the bits are the same.
    st = make_plan(g.dtype, SK_POLICY_PURE_DP, g.M, g.N, g.K, g.grid_cap, 0, 0, p.variant + 1, cus, &p, scale_align);
    if (st != SK_OK) return st;
  }
  hipStream_t stream = (hipStream_t)g.stream;
  const Variant* v = sk::variant(p.variant);
  // MX scales are read from a k-step-major copy in the kernel's lane order:
  // one k-step's scales of a tile are one contiguous block (row-major scales
  // would put each row's 2 to 8 bytes in a different cache line), and each
  // lane finds the bytes of all its MFMA blocks together.  The copy holds
  // whole tiles.  Every offset into it must fit in 32 bits.  A k-step holds
  // kb bytes of a row's LDS image: 2 * kb E2M1 elements for MXFP4, kb elements
  // for the other MX types (one byte per element there), so kb / 16 or kb / 32
  // scale bytes.
  const int64_t spr = g.dtype == SK_MXFP4 ? v->kb / 16 : v->kb / 32, ksteps = p.iters_per_tile;
  // Kernels of at most 128-row tiles instead gather the scales straight from the caller's
  // arrays, saving the re-layout launch, where direct_fits.
  const bool direct = is_mx(g.dtype) && direct_fits(v, g.K, scale_align);
  if (!direct && !v->launch) return SK_ERR_UNSUPPORTED;   // (make_plan has ruled this out)
  int64_t sa_bytes = 0, sb_bytes = 0, rows_a = 0, rows_b = 0;
  if (is_mx(g.dtype) && !direct) {
    rows_a = cdiv(g.M, v->bm) * v->bm;
    rows_b = cdiv(g.N, v->bn) * v->bn;
    sa_bytes = ksteps * rows_a * spr;
    sb_bytes = ksteps * rows_b * spr;
    if (sa_bytes >= ((int64_t)1 << 31) || sb_bytes >= ((int64_t)1 << 31)) return SK_ERR_ARG;
  }
  const int64_t sb_at = (sa_bytes + 255) / 256 * 256;
  const size_t s_need = is_mx(g.dtype) && !direct ? (size_t)(sb_at + sb_bytes) : 0;
  Scratch sc;
  if (fixed) {
    const size_t p_at = ((size_t)p.scratch_bytes + 255) / 256 * 256;
    if (p_at + s_need > kStaticDataBytes) return SK_ERR_SCRATCH;
    uint8_t* base = nullptr;
    st = static_scratch(dev, stream, &base);
    if (st != SK_OK) return st;
    sc.flags = (uint32_t*)base;
    sc.P = (float*)(base + kStaticFlagBytes);
    sc.S = base + kStaticFlagBytes + p_at;
    std::lock_guard<std::mutex> lk(g_mu);
    StaticScratch& ss = g_static[dev];
    if (ss.epoch == 0xFFFFFFFFu) {
      if (hipMemsetAsync(sc.flags, 0, sk::kMaxGrid * sizeof(uint32_t), stream) != hipSuccess) return SK_ERR_HIP;
      ss.epoch = 0;
    }
    sc.epoch = ++ss.epoch;
  } else {
    Workspace* ws = nullptr;
    st = get_workspace(dev, stream, (size_t)p.scratch_bytes, s_need, &ws);
    if (st != SK_OK) return st;
    st = next_epoch(ws, &sc.epoch);
    if (st != SK_OK) return st;
    sc.P = ws->P;
    sc.S = ws->S;
    sc.flags = ws->flags;
  }

  KArgs a;
  std::memset(&a, 0, sizeof(a));
  a.A = (const uint8_t*)g.A;
  a.B = (const uint8_t*)g.B;
  if (direct) {
    a.SA = (const uint8_t*)g.A_scale;
    a.SB = (const uint8_t*)g.B_scale;
    a.sa_kstride = (uint32_t)spr;
    a.sb_kstride = (uint32_t)spr;
    a.s_pitch = (int32_t)(g.K / 32);
  } else if (is_mx(g.dtype)) {
    const sk::ScaleLayout la{(int)g.M, v->bm, v->mfma, v->ng, v->bm / v->wm / v->mfma, v->nu};
    const sk::ScaleLayout lb{(int)g.N, v->bn, v->mfma, v->ng, v->bn / v->wn / v->mfma, v->nu};
    if (sk::launch_scale_relayout((const uint8_t*)g.A_scale, sc.S, la, (const uint8_t*)g.B_scale, sc.S + sb_at, lb,
                                  (int)(g.K / 32), (int)ksteps, (int)spr, stream) != hipSuccess)
      return SK_ERR_HIP;
    a.SA = sc.S;
    a.SB = sc.S + sb_at;
    a.sa_kstride = (uint32_t)(rows_a * spr);
    a.sb_kstride = (uint32_t)(rows_b * spr);
  } else if (g.dtype == SK_FP8_E4M3) {
    a.fsa = (const float*)g.A_scale;
    a.fsb = (const float*)g.B_scale;
  }
  a.bias = (const uint16_t*)g.bias;
  a.C = (uint16_t*)g.C;
  a.P = sc.P;
  a.locks = sc.flags;
  a.err = sc.flags + sk::kErrIndex;
  a.M = (int32_t)g.M;
  a.N = (int32_t)g.N;
  a.K = (int32_t)g.K;
  a.row_bytes = (int32_t)row_bytes(g.dtype, g.K);
  a.row_bytes_b = (int32_t)row_bytes(g.dtype, g.K, true);
  a.tiles = (int32_t)p.tiles;
  a.sk_tiles = (int32_t)p.sk_tiles;
  a.q = (int32_t)p.iters_per_wg;
  a.r = (int32_t)p.iters_extra;
  a.tiles_m = p.tiles_m;
  a.tiles_n = p.tiles_n;
  a.iters = p.iters_per_tile;
  a.G = p.grid;
  a.epoch = sc.epoch;
  a.spin_limit = g.spin_limit_ticks ? g.spin_limit_ticks : kDefaultSpin;
  a.trace = g.trace;
  a.drop_wg = (g.debug_flags & SK_DEBUG_DROP_SIGNAL) ? g.drop_signal_wg : -1;
  a.delay_seed = (g.debug_flags & SK_DEBUG_DELAY) ? (g.delay_seed ? g.delay_seed : 1u) : 0u;
  if ((direct ? v->launch_direct : v->launch)(p.grid, a, stream) != hipSuccess) return SK_ERR_HIP;
  return SK_OK;
}

sk_gemm_args base_args(int dtype, const void* A, const void* B, const void* sa, const void* sb, const void* bias,
                       void* C, int64_t M, int64_t N, int64_t K, int grid_cap, void* stream) {
  sk_gemm_args g;
  std::memset(&g, 0, sizeof(g));
  g.dtype = dtype;
  g.policy = SK_POLICY_AUTO;
  g.A = A;
  g.B = B;
  g.A_scale = sa;
  g.B_scale = sb;
  g.bias = bias;
  g.C = C;
  g.M = M;
  g.N = N;
  g.K = K;
  g.grid_cap = grid_cap;
  g.stream = stream;
  g.drop_signal_wg = -1;
  return g;
}

}  // namespace

extern "C" {

sk_status sk_gemm_mxfp4(const uint8_t* A, const uint8_t* B, const uint8_t* A_scale, const uint8_t* B_scale,
                        const void* bias, void* C, int64_t M, int64_t N, int64_t K, int grid_cap, void* stream) {
  return run(base_args(SK_MXFP4, A, B, A_scale, B_scale, bias, C, M, N, K, grid_cap, stream));
}

sk_status sk_gemm_mxfp4_noalloc(const uint8_t* A, const uint8_t* B, const uint8_t* A_scale, const uint8_t* B_scale,
                                const void* bias, void* C, int64_t M, int64_t N, int64_t K, int grid_cap,
                                void* stream) {
  return run(base_args(SK_MXFP4, A, B, A_scale, B_scale, bias, C, M, N, K, grid_cap, stream), true);
}

sk_status sk_gemm_bf16(const void* A, const void* B, const void* bias, void* C, int64_t M, int64_t N, int64_t K,
                       int grid_cap, void* stream) {
  return run(base_args(SK_BF16, A, B, nullptr, nullptr, bias, C, M, N, K, grid_cap, stream));
}

sk_status sk_gemm_fp8(const uint8_t* A, const uint8_t* B, const float* A_scale, const float* B_scale,
                      const void* bias, void* C, int64_t M, int64_t N, int64_t K, int grid_cap, void* stream) {
  return run(base_args(SK_FP8_E4M3, A, B, A_scale, B_scale, bias, C, M, N, K, grid_cap, stream));
}

sk_status sk_gemm_mxfp8(const uint8_t* A, const uint8_t* B, const uint8_t* A_scale, const uint8_t* B_scale,
                        const void* bias, void* C, int64_t M, int64_t N, int64_t K, int grid_cap, void* stream) {
  return run(base_args(SK_MXFP8, A, B, A_scale, B_scale, bias, C, M, N, K, grid_cap, stream));
}

sk_status sk_addmm(sk_dtype dtype, const void* bias, const void* A, const void* B, const void* A_scale,
                   const void* B_scale, void* C, int64_t M, int64_t N, int64_t K, int grid_cap, void* stream) {
  if (!bias) return SK_ERR_ARG;
  return run(base_args((int)dtype, A, B, A_scale, B_scale, bias, C, M, N, K, grid_cap, stream));
}

sk_status sk_gemm_bf16_backward(const void* dC, const void* A, const void* B, void* dA, void* dB, void* dbias,
                                int64_t M, int64_t N, int64_t K, int grid_cap, void* stream) {
  if (!dC || (!dA && !dB && !dbias)) return SK_ERR_ARG;
  if ((dA && !B) || (dB && !A)) return SK_ERR_ARG;
  if (M < 1 || N < 1 || K < 1 || K > kMaxN) return SK_ERR_ARG;
  if ((dA && (N > kMaxK || M >= kMaxM)) || (dB && (M > kMaxK || N >= kMaxM))) return SK_ERR_ARG;
  if (M % 8 || N % 8 || K % 8) return SK_ERR_ALIGN;
  if (((uintptr_t)dC | (uintptr_t)A | (uintptr_t)B | (uintptr_t)dA | (uintptr_t)dB) & 15) return SK_ERR_ALIGN;
  if (dbias && ((uintptr_t)dbias & 1)) return SK_ERR_ALIGN;
  const int64_t bc = M * N * 2, ba = M * K * 2, bb = N * K * 2;
  for (const void* out : {(const void*)dA, (const void*)dB, (const void*)dbias}) {
    const int64_t n = out == dA ? ba : (out == dB ? bb : N * 2);
    if (out && (overlaps(out, n, dC, bc) || overlaps(out, n, A, ba) || overlaps(out, n, B, bb))) return SK_ERR_ARG;
  }
  if ((dA && dB && overlaps(dA, ba, dB, bb)) || (dA && dbias && overlaps(dA, ba, dbias, N * 2)) ||
      (dB && dbias && overlaps(dB, bb, dbias, N * 2)))
    return SK_ERR_ARG;
  int dev = 0;
  DeviceInfo info;
  sk_status st = refuse_capture((hipStream_t)stream);
  if (st != SK_OK) return st;
  st = device_info(&dev, &info);
  if (st != SK_OK) return st;
  if (!info.gfx950) return SK_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  // transposed operands, each 256-byte aligned: B^T [K][N]; dC^T [N][M]; A^T [K][M]; dbias partials
  auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
  const int64_t at_bt = 0, at_dct = up(dA ? bb : 0), at_at = at_dct + up(dB ? bc : 0), at_part = at_at + up(dB ? ba : 0);
  const int64_t total = at_part + (dbias ? sk::colsum_scratch_bytes((int)M, (int)N) : 0);
  uint8_t* T = nullptr;
  st = get_aux(dev, s, (size_t)total, &T);
  if (st != SK_OK) return st;
  if (dA) {
    // dA[m][k] = sum_n dC[m][n] B[n][k]: A' = dC (K' = N contiguous), B' = B^T [K][N]
    if (sk::launch_transpose_bf16((const uint16_t*)B, (uint16_t*)(T + at_bt), (int)N, (int)K, s) != hipSuccess)
      return SK_ERR_HIP;
    st = run(base_args(SK_BF16, dC, T + at_bt, nullptr, nullptr, nullptr, dA, M, K, N, grid_cap, stream));
    if (st != SK_OK) return st;
  }
  if (dB) {
    // dB[n][k] = sum_m dC[m][n] A[m][k]: A' = dC^T [N][M], B' = A^T [K][M] (K' = M)
    if (sk::launch_transpose_bf16((const uint16_t*)dC, (uint16_t*)(T + at_dct), (int)M, (int)N, s) != hipSuccess ||
        sk::launch_transpose_bf16((const uint16_t*)A, (uint16_t*)(T + at_at), (int)M, (int)K, s) != hipSuccess)
      return SK_ERR_HIP;
    st = run(base_args(SK_BF16, T + at_dct, T + at_at, nullptr, nullptr, nullptr, dB, N, K, M, grid_cap, stream));
    if (st != SK_OK) return st;
  }
  if (dbias && sk::launch_colsum_bf16((const uint16_t*)dC, (float*)(T + at_part), (uint16_t*)dbias, (int)M, (int)N,
                                      s) != hipSuccess)
    return SK_ERR_HIP;
  return SK_OK;
}

sk_status sk_gemm_mx(sk_dtype a_fmt, sk_dtype b_fmt, const uint8_t* A, const uint8_t* B, const uint8_t* A_scale,
                     const uint8_t* B_scale, const void* bias, void* C, int64_t M, int64_t N, int64_t K, int grid_cap,
                     void* stream) {
  // the same format for both operands: that type's kernels; one MXFP4 and one
  // MXFP8 operand: the mixed kernels, in which the scaled MFMA takes each in its
  // own format; other pairs are not compiled
  auto element_format = [](int d) { return is_mx(d) && d != SK_MXFP4_MXFP8 && d != SK_MXFP8_MXFP4; };
  if (!element_format(a_fmt) || !element_format(b_fmt)) return SK_ERR_ARG;
  int dtype = -1;
  if (a_fmt == b_fmt) dtype = a_fmt;
  else if (a_fmt == SK_MXFP4 && b_fmt == SK_MXFP8) dtype = SK_MXFP4_MXFP8;
  else if (a_fmt == SK_MXFP8 && b_fmt == SK_MXFP4) dtype = SK_MXFP8_MXFP4;
  if (dtype < 0) return SK_ERR_UNSUPPORTED;
  return run(base_args(dtype, A, B, A_scale, B_scale, bias, C, M, N, K, grid_cap, stream));
}

sk_status sk_gemm_ex(const sk_gemm_args* args) {
  if (!args) return SK_ERR_ARG;
  return run(*args);
}

sk_status sk_plan(const sk_plan_query* q, sk_plan_info* out) {
  if (!q || !out) return SK_ERR_ARG;
  int cus = q->num_cus;
  if (cus <= 0) {
    int dev = 0;
    DeviceInfo info;
    sk_status st = device_info(&dev, &info);
    if (st != SK_OK) return st;
    cus = info.cus;
  }
  return make_plan(q->dtype, q->policy, q->M, q->N, q->K, q->grid_cap, q->tile_m, q->tile_n, q->variant, cus, out);
}

sk_status sk_plan_wg_range(const sk_plan_info* p, int32_t wg, int64_t* begin, int64_t* end) {
  if (!p || !begin || !end || wg < 0 || wg >= p->grid) return SK_ERR_ARG;
  if (p->sk_tiles == 0) {
    *begin = *end = 0;
    return SK_OK;
  }
  *begin = sk::sk_begin(wg, (int32_t)p->iters_per_wg, (int32_t)p->iters_extra);
  *end = sk::sk_begin(wg + 1, (int32_t)p->iters_per_wg, (int32_t)p->iters_extra);
  return SK_OK;
}

sk_status sk_plan_wg_work(const sk_plan_info* p, int32_t wg, sk_work_item* items, int32_t max_items,
                          int32_t* count) {
  if (!p || !count || wg < 0 || wg >= p->grid || max_items < 0 || (max_items > 0 && !items)) return SK_ERR_ARG;
  sk::WorkIter work(wg, (int32_t)p->sk_tiles, (int32_t)p->tiles, p->iters_per_tile, (int32_t)p->iters_per_wg,
                    (int32_t)p->iters_extra, p->grid);
  sk::WorkItem it;
  int32_t n = 0;
  while (work.next(it)) {
    if (n < max_items) {
      items[n].tile = it.tile;
      items[n].k0 = it.k0;
      items[n].k1 = it.k1;
      items[n].mode = it.mode;
      items[n].first = it.first;
    }
    ++n;
  }
  *count = n;
  return SK_OK;
}

sk_status sk_check(void* stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SK_ERR_HIP;
  const sk_status cap = refuse_capture((hipStream_t)stream);
  if (cap != SK_OK) return cap;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return SK_ERR_HIP;
  // the error words this stream's launches may have set: its workspace's,
  // and the fixed scratch's of this device (sk_gemm_mxfp4_noalloc)
  uint32_t* words[2] = {nullptr, nullptr};
  {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_ws.find(std::make_pair(dev, (uintptr_t)stream));
    if (it != g_ws.end() && it->second) words[0] = it->second->flags + sk::kErrIndex;
    if (dev >= 0 && dev < kMaxDevices && g_static[dev].ptr) words[1] = (uint32_t*)g_static[dev].ptr + sk::kErrIndex;
  }
  bool timed_out = false;
  for (uint32_t* wp : words) {
    if (!wp) continue;
    uint32_t err = 0;
    if (hipMemcpy(&err, wp, sizeof(err), hipMemcpyDeviceToHost) != hipSuccess) return SK_ERR_HIP;
    if (err) {
      if (hipMemset(wp, 0, sizeof(uint32_t)) != hipSuccess) return SK_ERR_HIP;
      timed_out = true;
    }
  }
  return timed_out ? SK_ERR_TIMEOUT : SK_OK;
}

void sk_release_workspace(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  int cur = 0;
  const bool have_cur = hipGetDevice(&cur) == hipSuccess;
  for (auto& kv : g_ws) {
    Workspace* ws = kv.second;
    if (!ws) continue;
    hipSetDevice(ws->device);
    hipStreamSynchronize(ws->stream);
    if (ws->P) hipFree(ws->P);
    if (ws->S) hipFree(ws->S);
    if (ws->T) hipFree(ws->T);
    if (ws->flags) hipFree(ws->flags);
    delete ws;
  }
  g_ws.clear();
  if (have_cur) hipSetDevice(cur);
}

sk_status sk_debug_poison_workspace(void* stream, int64_t scratch_bytes) {
  int dev = 0;
  DeviceInfo info;
  sk_status st = refuse_capture((hipStream_t)stream);
  if (st != SK_OK) return st;
  st = device_info(&dev, &info);
  if (st != SK_OK) return st;
  Workspace* ws = nullptr;
  st = get_workspace(dev, (hipStream_t)stream, scratch_bytes > 0 ? (size_t)scratch_bytes : 0, 0, &ws);
  if (st != SK_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (ws->P && hipMemsetAsync(ws->P, 0xFF, ws->p_bytes, s) != hipSuccess) return SK_ERR_HIP;  // all-ones = NaN
  // Stale flags: the current epoch, which the next launch (epoch + 1) must not accept.
  std::vector<uint32_t> stale(sk::kMaxGrid, ws->epoch);
  if (hipMemcpyAsync(ws->flags, stale.data(), stale.size() * sizeof(uint32_t), hipMemcpyHostToDevice, s) != hipSuccess)
    return SK_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return SK_ERR_HIP;
  return SK_OK;
}

int32_t sk_num_variants(void) { return sk::num_variants(); }

sk_status sk_variant_info(int32_t index, int32_t* dtype, int32_t* tile_m, int32_t* tile_n, int32_t* tile_k,
                          int32_t* threads, int32_t* lds_bytes) {
  const Variant* v = sk::variant(index);
  if (!v) return SK_ERR_ARG;
  if (dtype) *dtype = v->dtype;
  if (tile_m) *tile_m = v->bm;
  if (tile_n) *tile_n = v->bn;
  if (tile_k) *tile_k = v->bk;
  if (threads) *threads = v->threads;
  if (lds_bytes) *lds_bytes = v->lds;
  return SK_OK;
}

sk_status sk_variant_k_split(int32_t index, int32_t* k_slices, int32_t* direct_only) {
  const Variant* v = sk::variant(index);
  if (!v) return SK_ERR_ARG;
  if (k_slices) *k_slices = v->wk;
  if (direct_only) *direct_only = v->launch == nullptr;
  return SK_OK;
}

sk_status sk_stream_create_cu_masked(const uint32_t* cu_mask, int32_t words, void** stream) {
  if (!cu_mask || !stream || words < 1 || words > 64) return SK_ERR_ARG;
  int dev = 0;
  DeviceInfo info;
  sk_status st = device_info(&dev, &info);
  if (st != SK_OK) return st;
  const int n = mask_count(cu_mask, words, info.cus);
  if (n < 1) return SK_ERR_ARG;
  hipStream_t s = nullptr;
  if (hipExtStreamCreateWithCUMask(&s, (uint32_t)words, cu_mask) != hipSuccess) return SK_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_mu);
  g_stream_cus[std::make_pair(dev, (uintptr_t)s)] = n;
  *stream = (void*)s;
  return SK_OK;
}

sk_status sk_stream_destroy(void* stream) {
  if (!stream) return SK_ERR_ARG;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SK_ERR_HIP;
  hipStream_t s = (hipStream_t)stream;
  if (hipStreamSynchronize(s) != hipSuccess) return SK_ERR_HIP;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    const auto key = std::make_pair(dev, (uintptr_t)s);
    auto it = g_ws.find(key);
    if (it != g_ws.end()) {
      Workspace* ws = it->second;
      if (ws) {
        if (ws->P) hipFree(ws->P);
        if (ws->S) hipFree(ws->S);
        if (ws->T) hipFree(ws->T);
        if (ws->flags) hipFree(ws->flags);
        delete ws;
      }
      g_ws.erase(it);
    }
    g_stream_cus.erase(key);
  }
  return hipStreamDestroy(s) == hipSuccess ? SK_OK : SK_ERR_HIP;
}

sk_status sk_stream_cu_count(void* stream, int32_t* count) {
  if (!count) return SK_ERR_ARG;
  int dev = 0;
  DeviceInfo info;
  sk_status st = device_info(&dev, &info);
  if (st != SK_OK) return st;
  *count = stream_cus(dev, (hipStream_t)stream, info.cus);
  return SK_OK;
}

const char* sk_status_string(sk_status s) {
  switch (s) {
    case SK_OK: return "ok";
    case SK_ERR_ARG: return "invalid argument";
    case SK_ERR_ALIGN: return "misaligned size or pointer";
    case SK_ERR_UNSUPPORTED: return "unsupported device or tile";
    case SK_ERR_HIP: return "HIP runtime error";
    case SK_ERR_NOMEM: return "out of device memory";
    case SK_ERR_TIMEOUT: return "a workgroup timed out waiting for a partial tile";
    case SK_ERR_SCRATCH: return "the call needs more device scratch than the fixed no-allocation buffer holds";
  }
  return "unknown status";
}

}  // extern "C"
