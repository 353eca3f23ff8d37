// mhc.hip -- host side of libmhc: argument validation, launch planning and
// the C ABI declared in include/mhc.h.  Everything is checked before anything
// is enqueued; every launch goes to the caller's stream; nothing allocates.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "mhc.h"
#include "mhc_kernels.hpp"

namespace {

using namespace mhc;

// Few tokens: the 4C row of a 16-token tile is split over workgroups, which
// spreads the (L2/HBM-resident) projection weight over the chip; the last
// split to arrive sums the partials.  More splits shorten the weight reads and
// lengthen that sum.  Split counts per tile count, measured on MI355X (C =
// 5120, graph replay, the delayed pre): 32 splits for 1-2 tiles (T = 1:
// 8.6 us against 9.1 us with 16), 16 up to 16 tiles (T = 64: 9.9 us against
// 10.2 with 32; T = 128: 10.7 us against 12.1 with 8), 8 up to 64 tiles (T =
// 1024: 20.7 us), 4 up to 128 (T = 2048: 34.5 us against 36.1 with 8) and 2 up
// to 256 tiles (T = 4096: 63.9 us).  The forms that collapse with their own
// pre-mix (mhc_pre, the entry seam) stop splitting past 128 tiles, where each
// tile's own workgroup collapses its tokens (T = 4096: 72 us unsplit against
// 82 us with 2 splits).
constexpr int kMaxSplitTiles = 256;     // tiles beyond which the row is never split
constexpr int kMaxSplitTilesOwn = 128;  // the same for the forms with their own pre-mix
int splits_for(int ntile, bool delayed) {
  if (ntile > (delayed ? kMaxSplitTiles : kMaxSplitTilesOwn)) return 1;
  return ntile <= 2 ? 32 : ntile <= 16 ? 16 : ntile <= 64 ? 8 : ntile <= 128 ? 4 : 2;
}
constexpr int kMinKBPerSplit = 8;   // two 32-k steps per wave at least
constexpr size_t kStreamBytes = (size_t)256 << 20;   // the memory-side cache (MALL) of MI355X
constexpr int kMaxC = 16384;
// The persistent kernels keep a tile's collapsed rows on chip and split each
// 64-token tile over a group of workgroups; they win once the split form's
// per-tile weight reads and duplicate residual reads (projection and collapse
// workgroups) outweigh its parallelism.  Measured (eager, back to back, split
// vs persistent, microseconds):
//   C = 5120  delayed  T = 4096: 62.9 vs 67.5, 4608: 84.5 vs 68.3, 8192: 172.6 vs 117.0
//             own      T = 4096: 78.3 vs 91.2, 4608: 116.2 vs 95.5, 16384: 355.7 vs 283.4
//             fused    T = 3072: 81.8 vs 88.3, 3584: 125.3 vs 99.0 (two launches vs one)
//   C = 4096  delayed  T = 4096: 59.9 vs 63.9, 4608: 72.9 vs 63.3
//             own      T = 4096: 72.9 vs 81.0, 4608: 102.5 vs 84.4
//             fused    T = 3072: 64.4 vs 71.4, 3584: 99.7 vs 81.4
//   C = 7168  delayed  T = 3584: 76.0 vs 83.6, 4096: 98.3 vs 99.5, 4608: 131.3 vs 107.2
//             own      T = 2048: 95.0 vs 77.1, 3072: 108.4 vs 101.6
//             fused    T = 2048: 79.1 vs 81.8, 3072: 144.7 vs 121.3
// The own-pre-mix persistent form is the gates-only pass, then the collapse
// kernel with the seam's pre-mix (a second pass over x, which this form needs
// anyway); its split form is one workgroup per 16-token tile collapsing its
// tokens after the gates.
// Hidden sizes with a persistent form, and the workgroups of one group (the
// member count: each member's weight slice must fit in LDS).
int persist_pg(int C) {
  switch (C) {
    case 4096: return PersistGeom<4096>::kPG;
    case 5120: return PersistGeom<5120>::kPG;
    case 7168: return PersistGeom<7168>::kPG;
    default: return 0;
  }
}
// The largest token counts that run the split form; persistent beyond.
constexpr int kDelayedSplitMaxT = 4096;
int own_split_max_t(int C) { return C >= 7168 ? 2048 : 4096; }
int fused_group_split_max_t(int C) { return C >= 7168 ? 2048 : 3072; }
// Fused seam below the persistent form: the split kernel's fused mode (one
// launch) against the post kernel followed by the delayed split kernel, T =
// 16: 10.8 vs 11.9 us, T = 128: 14.5 vs 18.0 us, T = 1024: 32.1 vs 41.7 us.
// At other hidden sizes the fused mode runs up to the same token count and
// the two launches beyond it.
constexpr int kFusedSplitMaxT = 3072;

struct Plan {
  int ntile, nsplit, nproj;
  bool persist;  // persistent form (C with a persistent geometry, many tokens)
  int pg;        // its group size
};

// form: kModePre / kModeEntry (own pre-mix), kModeDelayed or kModeFused;
// C: the hidden size; pg: group size of the persistent kernels for this hidden size (0: none).
Plan make_plan(int T, int C, int KB, int form, int pg) {
  Plan pl;
  const bool persist_ok = pg > 0;
  pl.pg = pg;
  pl.ntile = (T + kTileT - 1) / kTileT;
  const bool delayed = form == kModeDelayed || form == kModeFused;
  pl.persist = persist_ok && ((form == kModeDelayed && T > kDelayedSplitMaxT) ||
                              (form == kModeFused && T > fused_group_split_max_t(C)) ||
                              (form == kModePre && T > own_split_max_t(C)));
  int ns = pl.persist ? 1 : splits_for(pl.ntile, delayed);
  int maxs = KB / kMinKBPerSplit;
  if (maxs < 1) maxs = 1;
  if (ns > maxs) ns = maxs;
  pl.nsplit = ns;
  pl.nproj = pl.ntile * ns;
  return pl;
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Workspace layout.  Counters must read zero when a call starts, and one
// workspace serves calls of both forms, so the two forms' counters live in
// disjoint places that nothing else writes; their data (rewritten before it is
// read in every call) share the region from 192 KiB.
//   [0, 256)            persistent form: word 0 finished waves, word 2 wait-budget flag
//   [256, 82176)        persistent form: arrival counters [group][wave][5], 256 B apart
//   [96 KiB, +1028)     split form: tile counters [ntile] u32 (ntile <= 256 whenever split),
//                       then the wait-ran-out word
//   [100 KiB, +32 KiB)  split form: own-pre-mix records [T <= 2048][4] u32 (pre-mix bits
//                       with the sign bit set; zero when empty)
//   [192 KiB, ...)      split form: partials [ntile][nsplit][16][25] f32, or
//                       persistent form: records [group][wave][4] (1 KB + 32 KB each)
constexpr size_t kSplitCntOffset = 96 * 1024;
static_assert(kMaxSplitTiles <= kSplitFlagStride, "split tile counters overlap the wait word");
static_assert((kSplitFlagStride + 1) * sizeof(unsigned) <= (size_t)kSplitRecBytes,
              "split counters overlap the own-pre-mix records");
static_assert(kMaxSplitTilesOwn * kTileT <= kOwnMaxTokens, "own-pre-mix records too few for a split call");
static_assert(kSplitCntOffset + kSplitBytes <= kPPartOffset, "split counters and records overlap the data region");
static_assert(kPCntBase * 4 + (size_t)kPMaxGroups * kPW * kPSlots * kPCntStride * 4 <= kSplitCntOffset,
              "persistent counters overlap the split counters");
size_t plan_ws_bytes(const Plan& pl) {
  if (pl.persist) return persist_ws_bytes(pl.pg);
  if (pl.nsplit <= 1) return 0;
  return kPPartOffset + (size_t)pl.ntile * pl.nsplit * kTileT * kPartStride * sizeof(float);
}
static_assert(MHC_WS_WAIT_ERROR_PERSIST == 2 * 4, "persistent wait-error word");
static_assert(MHC_WS_WAIT_ERROR_SPLIT == kSplitCntOffset + kSplitWaitErr * 4, "split wait-error word");
static_assert(MHC_WS_FLAG_BYTES == kPPartOffset, "flag region");

// Bounds of the kernels' waits, set by mhc_debug_force_wait_timeouts (a
// non-zero bias puts every wait target out of reach).
unsigned g_wait_bias = 0;
int g_wait_budget = kWaitBudget;

void set_split_ws(PreParams& p, void* ws) {
  p.cnt = reinterpret_cast<unsigned*>(static_cast<char*>(ws) + kSplitCntOffset);
  p.part = reinterpret_cast<float*>(static_cast<char*>(ws) + kPPartOffset);
}

// Groups of the persistent kernel: one workgroup per CU at most (its LDS use
// guarantees that), never more groups than tiles.  The CU count is that of the
// device the launch stream belongs to (not the calling thread's current
// device), cached per device; a race between threads only stores the same
// value twice.  -1: the device could not be queried (nothing is launched);
// 0: fewer CUs than one group needs.
int persist_groups(int T, int pg, hipStream_t stream) {
  static std::atomic<int> cus[64];
  hipDevice_t dev = 0;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return -1;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  const int tiles = (T + kPT - 1) / kPT;
  int ng = n / pg;
  if (ng > kPMaxGroups) ng = kPMaxGroups;
  if (ng > tiles) ng = tiles;
  return ng;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  const void* p;
  size_t n;
};
bool overlap(Range a, Range b) {
  if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
  uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.n && b0 < a0 + a.n;
}

// Outputs must not overlap each other or any input.
bool any_alias(const Range* outs, int nout, const Range* ins, int nin) {
  for (int i = 0; i < nout; ++i) {
    for (int j = i + 1; j < nout; ++j)
      if (overlap(outs[i], outs[j])) return true;
    for (int j = 0; j < nin; ++j)
      if (overlap(outs[i], ins[j])) return true;
  }
  return false;
}

mhc_status check_common(int T, int n, int C) {
  if (n != MHC_HC_MULT) return MHC_ERR_UNSUPPORTED;
  if (C < 256 || C > kMaxC || C % 256 != 0) return MHC_ERR_UNSUPPORTED;
  if (T < 0 || T > MHC_MAX_TOKENS) return MHC_ERR_SHAPE;
  return MHC_OK;
}

mhc_status check_scalars(float eps, int iters) {
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return MHC_ERR_SHAPE;
  if (iters < 1 || iters > MHC_MAX_SINKHORN_ITERS) return MHC_ERR_SHAPE;
  return MHC_OK;
}

mhc_status launched() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? MHC_OK : MHC_ERR_HIP;
}

// The persistent kernel of hidden size kC in the form `mode` (fused seam,
// delayed pre, or the gates-only pass of the own-pre-mix form).
template <int kC>
void launch_persist(int mode, const PreParams& p, int ng, hipStream_t s) {
  const dim3 grid(ng * PersistGeom<kC>::kPG), block(kPThreads);
  if (mode == kModeFused)
    hipLaunchKernelGGL((mhc_persist_kernel<kC, true>), grid, block, 0, s, p, ng);
  else if (mode == kModeDelayed)
    hipLaunchKernelGGL((mhc_persist_kernel<kC, false>), grid, block, 0, s, p, ng);
  else
    hipLaunchKernelGGL((mhc_persist_kernel<kC, false, true>), grid, block, 0, s, p, ng);
}

// the post kernel: one thread per (token, 8 hidden elements); when a wave's 64
// threads always share one token (C / 8 a multiple of 64), the wave-token form
void launch_post(const uint4* y, const uint4* x, const float* post, const float* comb, uint4* out, int T, int C8,
                 hipStream_t s) {
  const long long total = (long long)T * C8;
  const unsigned grid = (unsigned)((total + kThreads - 1) / kThreads);
  if (C8 % kWave == 0)
    hipLaunchKernelGGL(mhc_post_kernel<true>, dim3(grid), dim3(kThreads), 0, s, y, x, post, comb, out, T, C8);
  else
    hipLaunchKernelGGL(mhc_post_kernel<false>, dim3(grid), dim3(kThreads), 0, s, y, x, post, comb, out, T, C8);
}

// ------------------------------------------------------------------ no-allocation variant
// A workspace in device memory the library owns: one per GPU (each device
// holds its own copy of the array), used by mhc_post_pre_delayed_noalloc for
// callers that cannot allocate.  Its size covers every plan of the fused seam
// (the persistent kernels' records at the largest group, the split form's
// partial sums at the most tiles x splits a plan has).
constexpr size_t kScratchBytes = MHC_NOALLOC_SCRATCH_BYTES;
static_assert(kPPartOffset + (size_t)kPMaxGroups * kPW * kPRing * persist_rec_floats(kPMaxPG) * sizeof(float) <=
                  kScratchBytes,
              "scratch too small for the persistent records");
static_assert(kPPartOffset + (size_t)kMaxSplitTiles * 2 * kTileT * kPartStride * sizeof(float) <= kScratchBytes,
              "scratch too small for the split partial sums");
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of `scratch` per device (the array's name is a host-side
// stand-in, not a device address), taken once with that device current, and
// whether its flag region has been cleared since (not under graph capture: a
// captured clear runs only on replay).
std::mutex g_scratch_mu;
void* g_scratch_ptr[64];
bool g_scratch_clear[64];

__global__ __launch_bounds__(256) void mhc_clear_kernel(uint4* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

mhc_status scratch_of(hipStream_t s, void** out) {
  hipDevice_t dev = 0;
  if (hipStreamGetDevice(s, &dev) != hipSuccess || dev < 0 || dev >= 64) return MHC_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return MHC_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return MHC_ERR_HIP;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return MHC_ERR_HIP;
    if (e != hipSuccess || ptr == nullptr) return MHC_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  if (!g_scratch_clear[dev]) {
    // the words calls read before they write start at zero (every call leaves them so)
    const int n = (int)(kPPartOffset / 16);
    hipLaunchKernelGGL(mhc_clear_kernel, dim3((n + 255) / 256), dim3(256), 0, s,
                       static_cast<uint4*>(g_scratch_ptr[dev]), n);
    if (hipGetLastError() != hipSuccess) return MHC_ERR_HIP;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) return MHC_ERR_HIP;
    if (cs == hipStreamCaptureStatusNone) g_scratch_clear[dev] = true;
  }
  *out = g_scratch_ptr[dev];
  return MHC_OK;
}

// The previous seam's post-stage inputs of the fused form.
struct PostIn {
  const uint16_t* y;
  const float* post;
  const float* comb;
};

// Shared by the pre-stage entry points.
mhc_status pre_common(int mode, const uint16_t* x, const float* pre_in, int T, int n, int C,
                      mhc_weights w, const uint16_t* norm_weight, float eps, int iters,
                      uint16_t* x_out, float* pre, float* post, float* comb, uint16_t* li,
                      void* ws, size_t ws_bytes, void* stream, PostIn pi = {nullptr, nullptr, nullptr},
                      bool noalloc = false) {
  mhc_status st = check_common(T, n, C);
  if (st != MHC_OK) return st;
  if ((st = check_scalars(eps, iters)) != MHC_OK) return st;
  const bool entry = mode == kModeEntry;
  const bool fused = mode == kModeFused;
  const bool delayed = mode == kModeDelayed || fused;
  if (!x || !w.fn_packed || !w.bias || !w.alpha || !pre || !post || !comb) return MHC_ERR_NULL;
  if (delayed && !pre_in) return MHC_ERR_NULL;
  if ((entry || fused) && !x_out) return MHC_ERR_NULL;
  if (fused && (!pi.y || !pi.post || !pi.comb)) return MHC_ERR_NULL;
  if (!entry && !li) return MHC_ERR_NULL;
  const void* ptrs[] = {x, pre_in, w.fn_packed, w.bias, w.alpha, norm_weight, x_out,
                        pre, post, comb, li, ws, pi.y, pi.post, pi.comb};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return MHC_ERR_ALIGN;

  const int K = entry ? C : n * C;
  const int KB = K / kKB;
  const size_t Tz = (size_t)T;
  const Range ins[] = {{x, Tz * K * 2},
                       {pre_in, delayed ? Tz * 16 : 0},
                       {w.fn_packed, mhc_fn_packed_bytes(K)},
                       {w.bias, 96},
                       {w.alpha, 12},
                       {norm_weight, norm_weight ? (size_t)C * 2 : 0},
                       {pi.y, fused ? Tz * C * 2 : 0},
                       {pi.post, fused ? Tz * 16 : 0},
                       {pi.comb, fused ? Tz * 64 : 0}};
  const Range outs[] = {{pre, Tz * 16},
                        {post, Tz * 16},
                        {comb, Tz * 64},
                        {li, li ? Tz * C * 2 : 0},
                        {x_out, (entry || fused) ? Tz * n * C * 2 : 0},
                        {ws, ws ? ws_bytes : 0}};
  if (any_alias(outs, 6, ins, 9)) return MHC_ERR_ALIAS;

  if (T == 0) return MHC_OK;
  if (noalloc) {
    // the library's own buffer instead of a workspace, once the arguments are known good
    if ((st = scratch_of(static_cast<hipStream_t>(stream), &ws)) != MHC_OK) return st;
    ws_bytes = kScratchBytes;
  }
  Plan pl = make_plan(T, C, KB, mode, entry ? 0 : persist_pg(C));
  const size_t need = plan_ws_bytes(pl);
  if (need > 0 && (!ws || ws_bytes < need)) return MHC_ERR_WORKSPACE;

  PreParams p{};
  p.x = x;
  p.pre_in = pre_in;
  p.fnp = static_cast<const uint4*>(w.fn_packed);
  p.bias = w.bias;
  p.alpha = w.alpha;
  p.nw = norm_weight;
  p.pre = pre;
  p.post = post;
  p.comb = comb;
  p.li = li;
  p.xout = x_out;
  p.ysub = pi.y;
  p.post_in = pi.post;
  p.comb_in = pi.comb;
  p.cnt = nullptr;
  p.part = nullptr;
  if (need && pl.persist) {
    p.cnt = static_cast<unsigned*>(ws);
    p.part = reinterpret_cast<float*>(static_cast<char*>(ws) + kPPartOffset);
  } else if (need) {
    set_split_ws(p, ws);
  }
  p.eps = eps;
  p.iters = iters;
  p.T = T;
  p.C = C;
  p.K = K;
  p.KB = KB;
  p.ntile = pl.ntile;
  p.nsplit = pl.nsplit;
  p.nproj = pl.nproj;
  // own pre-mix, split projection: one collapse workgroup per token, waiting
  // for its tile's pre-mix (instead of the tile's last arriver collapsing all
  // of its tokens after the gates)
  p.own_wgs = (!delayed && pl.nsplit > 1 && C <= kWaveCollapseMaxC && T <= kOwnMaxTokens) ? 1 : 0;
  p.wait_bias = noalloc ? 0u : g_wait_bias;
  p.wait_budget = noalloc ? kWaitBudget : g_wait_budget;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 block(kThreads);
  if (fused && !pl.persist && T > kFusedSplitMaxT) {
    // two launches: the post stage writes x_out, the delayed pre reads it
    const int C8 = C / 8;
    const long long total = (long long)T * C8;
    launch_post(reinterpret_cast<const uint4*>(pi.y), reinterpret_cast<const uint4*>(x), pi.post, pi.comb,
                reinterpret_cast<uint4*>(x_out), T, C8, s);
    p.x = x_out;
    mode = kModeDelayed;
  }
  if (pl.persist) {
    const int ng = persist_groups(T, pl.pg, s);
    if (ng < 0) return MHC_ERR_HIP;
    if (ng > 0) {
      switch (C) {
        case 4096: launch_persist<4096>(mode, p, ng, s); break;
        case 5120: launch_persist<5120>(mode, p, ng, s); break;
        default: launch_persist<7168>(mode, p, ng, s); break;
      }
      if (mode == kModePre) {
        // own pre-mix: the gates above, then the collapse with them (and the folded norm)
        PreParams c{};
        c.x = x;
        c.pre_in = pre;
        c.nw = norm_weight;
        c.li = li;
        c.eps = eps;
        c.T = T;
        c.C = C;
        c.K = K;
        if (Tz * (size_t)(n + 1) * C * 2 > kStreamBytes)
          hipLaunchKernelGGL(mhc_collapse_kernel<true>, dim3(T), block, 0, s, c);
        else
          hipLaunchKernelGGL(mhc_collapse_kernel<false>, dim3(T), block, 0, s, c);
      }
      return launched();
    }
    // a device too small for one group: the split form (its workspace need is covered)
    pl = make_plan(T, C, KB, mode, 0);
    p.ntile = pl.ntile;
    p.nsplit = pl.nsplit;
    p.nproj = pl.nproj;
    if (pl.nsplit > 1) set_split_ws(p, ws);
  }
  switch (mode) {
    case kModePre:
      hipLaunchKernelGGL(mhc_pre_split_kernel<kModePre>, dim3(pl.nproj + (p.own_wgs ? T : 0)), block, 0, s, p);
      break;
    case kModeDelayed:
      hipLaunchKernelGGL(mhc_pre_split_kernel<kModeDelayed>, dim3(pl.nproj + T), block, 0, s, p);
      break;
    case kModeFused:
      hipLaunchKernelGGL(mhc_pre_split_kernel<kModeFused>, dim3(pl.nproj + T), block, 0, s, p);
      break;
    default:
      hipLaunchKernelGGL(mhc_pre_split_kernel<kModeEntry>, dim3(pl.nproj + (p.own_wgs ? T : 0)), block, 0, s,
                         p);
      break;
  }
  return launched();
}

}  // namespace

extern "C" {

size_t mhc_fn_packed_bytes(int K) {
  if (K <= 0) return 0;
  return (size_t)K * kNL * 4;  // two bf16 per weight
}

mhc_status mhc_pack_fn(const float* fn, int K, void* fn_packed, void* stream) {
  if (!fn || !fn_packed) return MHC_ERR_NULL;
  if (K <= 0 || K % kKB != 0 || K > MHC_HC_MULT * kMaxC) return MHC_ERR_SHAPE;
  if (!aligned16(fn) || !aligned16(fn_packed)) return MHC_ERR_ALIGN;
  if (overlap({fn, (size_t)K * kNL * 4}, {fn_packed, mhc_fn_packed_bytes(K)})) return MHC_ERR_ALIAS;
  const int KB = K / kKB;
  const int total = KB * kFragPerKB * kWave;
  hipLaunchKernelGGL(mhc_pack_fn_kernel, dim3((total + 255) / 256), dim3(256), 0,
                     static_cast<hipStream_t>(stream), fn, KB, static_cast<uint4*>(fn_packed));
  return launched();
}

size_t mhc_workspace_bytes(int T_max, int n, int C) {
  if (n != MHC_HC_MULT || C < 256 || C > kMaxC || C % 256 != 0 || T_max <= 0) return 0;
  if (T_max > MHC_MAX_TOKENS) T_max = MHC_MAX_TOKENS;
  size_t best = 0;
  // the entry seam (K = C) and the 4-stream seams (K = 4C) may plan differently
  const int KBs[2] = {C / kKB, MHC_HC_MULT * C / kKB};
  const int ntile_max = (T_max + kTileT - 1) / kTileT;
  for (int KB : KBs) {
    for (int nt = 1; nt <= ntile_max && nt <= kMaxSplitTiles; ++nt) {
      for (int form : {kModePre, kModeDelayed, kModeFused}) {
        const Plan pl = make_plan(nt * kTileT, C, KB, form, 0);
        const size_t b = plan_ws_bytes(pl);
        if (b > best) best = b;
      }
    }
  }
  // the persistent forms: fixed size
  const int persist_min_t = std::min(std::min(fused_group_split_max_t(C), kDelayedSplitMaxT), own_split_max_t(C)) + 1;
  const int pg = persist_pg(C);
  if (pg > 0 && T_max >= persist_min_t && persist_ws_bytes(pg) > best) best = persist_ws_bytes(pg);
  return best;
}

mhc_status mhc_pre(const uint16_t* x, int T, int n, int C, mhc_weights w,
                   const uint16_t* norm_weight, float eps, int sinkhorn_iters, float* pre,
                   float* post, float* comb, uint16_t* layer_input, void* workspace,
                   size_t workspace_bytes, void* stream) {
  return pre_common(kModePre, x, nullptr, T, n, C, w, norm_weight, eps, sinkhorn_iters, nullptr,
                    pre, post, comb, layer_input, workspace, workspace_bytes, stream);
}

mhc_status mhc_pre_delayed(const uint16_t* x, const float* pre_in, int T, int n, int C,
                           mhc_weights w, const uint16_t* norm_weight, float eps,
                           int sinkhorn_iters, float* pre_out, float* post, float* comb,
                           uint16_t* layer_input, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return pre_common(kModeDelayed, x, pre_in, T, n, C, w, norm_weight, eps, sinkhorn_iters,
                    nullptr, pre_out, post, comb, layer_input, workspace, workspace_bytes, stream);
}

mhc_status mhc_broadcast_entry(const uint16_t* h, int T, int n, int C, mhc_weights w_entry,
                               const uint16_t* norm_weight, float eps, int sinkhorn_iters,
                               uint16_t* x_out, float* pre, float* post, float* comb,
                               uint16_t* layer_input, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return pre_common(kModeEntry, h, nullptr, T, n, C, w_entry, norm_weight, eps, sinkhorn_iters,
                    x_out, pre, post, comb, layer_input, workspace, workspace_bytes, stream);
}

mhc_status mhc_post_pre_delayed(const uint16_t* y, const uint16_t* x, const float* post_in,
                                const float* comb_in, const float* pre_in, int T, int n, int C,
                                mhc_weights w, const uint16_t* norm_weight, float eps,
                                int sinkhorn_iters, uint16_t* x_out, float* pre_out, float* post,
                                float* comb, uint16_t* layer_input, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return pre_common(kModeFused, x, pre_in, T, n, C, w, norm_weight, eps, sinkhorn_iters, x_out,
                    pre_out, post, comb, layer_input, workspace, workspace_bytes, stream,
                    PostIn{y, post_in, comb_in});
}

mhc_status mhc_post_pre_delayed_noalloc(const uint16_t* y, const uint16_t* x, const float* post_in,
                                        const float* comb_in, const float* pre_in, int T, int n, int C,
                                        mhc_weights w, const uint16_t* norm_weight, float eps,
                                        int sinkhorn_iters, uint16_t* x_out, float* pre_out, float* post,
                                        float* comb, uint16_t* layer_input, void* stream) {
  return pre_common(kModeFused, x, pre_in, T, n, C, w, norm_weight, eps, sinkhorn_iters, x_out, pre_out,
                    post, comb, layer_input, nullptr, 0, stream, PostIn{y, post_in, comb_in},
                    /*noalloc=*/true);
}

mhc_status mhc_post(const uint16_t* y, const uint16_t* x, const float* post, const float* comb,
                    int T, int n, int C, uint16_t* out, void* stream) {
  mhc_status st = check_common(T, n, C);
  if (st != MHC_OK) return st;
  if (!y || !x || !post || !comb || !out) return MHC_ERR_NULL;
  const void* ptrs[] = {y, x, post, comb, out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MHC_ERR_ALIGN;
  const size_t Tz = (size_t)T;
  const size_t xbytes = Tz * n * C * 2;
  const Range o = {out, xbytes};
  const Range ins_wo_x[] = {{y, Tz * C * 2}, {post, Tz * 16}, {comb, Tz * 64}};
  for (const Range& r : ins_wo_x)
    if (overlap(o, r)) return MHC_ERR_ALIAS;
  if (static_cast<const void*>(out) != static_cast<const void*>(x) && overlap(o, {x, xbytes}))
    return MHC_ERR_ALIAS;
  if (T == 0) return MHC_OK;
  launch_post(reinterpret_cast<const uint4*>(y), reinterpret_cast<const uint4*>(x), post, comb,
              reinterpret_cast<uint4*>(out), T, C / 8, static_cast<hipStream_t>(stream));
  return launched();
}

mhc_status mhc_collapse(const uint16_t* x, const float* p, int T, int n, int C,
                        const uint16_t* norm_weight, float eps, uint16_t* out, void* stream) {
  mhc_status st = check_common(T, n, C);
  if (st != MHC_OK) return st;
  if (norm_weight && (!(eps >= 0.0f) || !std::isfinite(eps))) return MHC_ERR_SHAPE;
  if (!x || !p || !out) return MHC_ERR_NULL;
  const void* ptrs[] = {x, p, norm_weight, out};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return MHC_ERR_ALIGN;
  const size_t Tz = (size_t)T;
  const Range ins[] = {{x, Tz * n * C * 2}, {p, Tz * 16}, {norm_weight, norm_weight ? (size_t)C * 2 : 0}};
  const Range outs[] = {{out, Tz * C * 2}};
  if (any_alias(outs, 1, ins, 3)) return MHC_ERR_ALIAS;
  if (T == 0) return MHC_OK;
  PreParams prm = {};
  prm.x = x;
  prm.pre_in = p;
  prm.nw = norm_weight;
  prm.li = out;
  prm.eps = eps;
  prm.T = T;
  prm.C = C;
  prm.K = n * C;
  // Streaming accesses once the call moves more than the memory-side cache
  // holds (measured, C = 5120, norm on: T = 16384 146.6 -> 131.2 us; at T =
  // 4096, with the rows cache-resident across calls, 32.6 us cached vs 35.4 us).
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (Tz * (size_t)(n + 1) * C * 2 > kStreamBytes)
    hipLaunchKernelGGL(mhc_collapse_kernel<true>, dim3(T), dim3(kThreads), 0, s, prm);
  else
    hipLaunchKernelGGL(mhc_collapse_kernel<false>, dim3(T), dim3(kThreads), 0, s, prm);
  return launched();
}

mhc_status mhc_debug_force_wait_timeouts(int sleeps) {
  if (sleeps < 0 || sleeps > kWaitBudget) return MHC_ERR_SHAPE;
  g_wait_bias = sleeps ? 0x40000000u : 0u;
  g_wait_budget = sleeps ? sleeps : kWaitBudget;
  return MHC_OK;
}

const char* mhc_status_str(mhc_status s) {
  switch (s) {
    case MHC_OK: return "MHC_OK";
    case MHC_ERR_NULL: return "MHC_ERR_NULL: a required pointer is NULL";
    case MHC_ERR_SHAPE: return "MHC_ERR_SHAPE: bad token count, eps or iteration count";
    case MHC_ERR_UNSUPPORTED: return "MHC_ERR_UNSUPPORTED: n must be 4 and C a multiple of 256 in [256, 16384]";
    case MHC_ERR_ALIGN: return "MHC_ERR_ALIGN: pointers must be 16-byte aligned";
    case MHC_ERR_ALIAS: return "MHC_ERR_ALIAS: an output overlaps an input or another output";
    case MHC_ERR_WORKSPACE: return "MHC_ERR_WORKSPACE: workspace missing or too small";
    case MHC_ERR_HIP: return "MHC_ERR_HIP: the HIP runtime rejected the launch";
  }
  return "unknown mhc_status";
}

}  // extern "C"
