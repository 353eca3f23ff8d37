// mhc_kernels.hpp -- the seam kernels of libmhc for gfx950.
//
//   mhc_pack_fn_kernel          one-time weight packing (bf16 hi/lo split, MFMA order)
//   mhc_pre_split_kernel<MODE>  pre stage for any T: projection split over
//                               workgroups (few tokens) or one workgroup per
//                               16-token tile, last-arriver reduction, gates +
//                               Sinkhorn, collapse + folded RMSNorm.
//   mhc_pre_group_kernel        delayed pre stage for many tokens (C = 5120):
//                               one sweep over x; a 64-token tile split over a
//                               group of workgroups on one XCD; projection, both
//                               sums of squares, collapse and norm fused.
//   mhc_post_kernel             post stage: post_i * y + sum_j comb_ij x_j.
#pragma once

#include "mhc_device.hpp"

namespace mhc {

enum Mode { kModePre = 0, kModeDelayed = 1, kModeEntry = 2 };

struct PreParams {
  const uint16_t* x;      // [T][K] bf16: residual [T][4][C] flattened, or h [T][C] (entry)
  const float* pre_in;    // [T][4] carried pre-mix (delayed)
  const uint4* fnp;       // packed projection weight, KB * 3 * 64 vectors of 8 bf16
  const float* bias;      // [24]
  const float* alpha;     // [3]
  const uint16_t* nw;     // [C] bf16 norm weight or nullptr (no norm)
  float* pre;             // [T][4]  pre-mix of this seam (pre / pre_out)
  float* post;            // [T][4]
  float* comb;            // [T][16]
  uint16_t* li;           // [T][C] layer_input (entry: may be nullptr)
  uint16_t* xout;         // [T][4][C] broadcast residual (entry)
  float* part;            // workspace: partial sums [ntile][nsplit][16][25]
  unsigned* cnt;          // workspace: arrival counters [ntile]
  float eps;
  int iters;
  int T, C, K, KB;        // K = row length, KB = K / 32
  int ntile, nsplit, nproj;
};

constexpr int kPS = 28;      // LDS row per token: P[0..23], sum x^2 [24], sum y^2 [25]
constexpr int kJMax = 8;     // k-steps a wave issues together in the split kernel
constexpr int kRedChunk = 16;  // partials loaded together by the last arriver

// ------------------------------------------------------------------ packing
// Packed layout: for 32-row block kb and column tile q (0..2, columns 16q..16q+15
// of [hi 0..23 | lo 0..23]), lane L of a wave holds the 8 values
// fn_part[k = 32 kb + 8 (L >> 4) + e][col = 16 q + (L & 15)], e = 0..7, which is
// the B-operand order of v_mfma_f32_16x16x32_bf16.  Vector index: (kb*3 + q)*64 + L.
__global__ __launch_bounds__(256) void mhc_pack_fn_kernel(const float* __restrict__ fn, int KB,
                                                         uint4* __restrict__ out) {
  const int gid = blockIdx.x * 256 + threadIdx.x;
  if (gid >= KB * kFragPerKB * kWave) return;
  const int lane = gid & (kWave - 1);
  const int q = (gid / kWave) % kFragPerKB;
  const int kb = gid / (kWave * kFragPerKB);
  const int col = 16 * q + (lane & 15);
  const int j = col < kNL ? col : col - kNL;
  const bool lo = col >= kNL;
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int k = kb * kKB + 8 * (lane >> 4) + e;
    const float f = fn[(size_t)k * kNL + j];
    const float hi = (float)(__bf16)f;  // nearest even
    v[e] = lo ? (f - hi) : hi;          // f - hi is exact in float
  }
  out[gid] = pack8(v);
}

// ------------------------------------------------------------------ gates + Sinkhorn
// One full wave handles a 16-token tile: lane L owns token L >> 2 and comb row
// L & 3 (four entries).  Row sums stay in the lane; column sums are a butterfly
// over the four lanes of a quad (DPP), so every lane of a column divides by the
// same bits.  The row maximum is subtracted before exp (removed exactly by the
// first row step); reciprocals are the hardware's (error <= 1 ulp).
__device__ __forceinline__ void tile_gates(const PreParams& p, const float (*s_P)[kPS], int t0,
                                           float (*s_pre)[kNS], bool write = true) {
  const int lane = threadIdx.x & (kWave - 1);
  const int tt = lane >> 2;
  const int row = lane & 3;
  const int tk = t0 + tt;
  const bool ok = tk < p.T;
  const float r = 1.0f / sqrtf(s_P[tt][24] / (float)p.K + p.eps);
  const float ac = p.alpha[2];
  float m[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) m[j] = ac * (r * s_P[tt][8 + 4 * row + j]) + p.bias[8 + 4 * row + j];
  const float mx = fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3]));
#pragma unroll
  for (int j = 0; j < 4; ++j) m[j] = expf(m[j] - mx);
  for (int it = 0; it < p.iters; ++it) {
    const float inv = __builtin_amdgcn_rcpf((m[0] + m[1]) + (m[2] + m[3]));
#pragma unroll
    for (int j = 0; j < 4; ++j) m[j] *= inv;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float c = m[j] + dpp_quad_xor1(m[j]);
      c = c + dpp_quad_xor2(c);
      m[j] *= __builtin_amdgcn_rcpf(c);
    }
  }
  const float lp = p.alpha[0] * (r * s_P[tt][row]) + p.bias[row];
  const float lq = p.alpha[1] * (r * s_P[tt][4 + row]) + p.bias[4 + row];
  const float pr = 1.0f / (1.0f + expf(-lp));
  const float po = 2.0f / (1.0f + expf(-lq));
  s_pre[tt][row] = pr;
  if (ok && write) {
    reinterpret_cast<float4*>(p.comb)[(size_t)tk * 4 + row] = make_float4(m[0], m[1], m[2], m[3]);
    p.pre[(size_t)tk * kNS + row] = pr;
    p.post[(size_t)tk * kNS + row] = po;
  }
}

// ------------------------------------------------------------------ collapse + norm, one token
// The whole 256-thread workgroup handles token `tok`: y (float) stays in
// registers, sum(y^2) is reduced over the workgroup, then layer_input is written.
template <bool kBcast>
__device__ __forceinline__ void collapse_norm_token(const PreParams& p, int tok, float p0, float p1,
                                                    float p2, float p3, float* s_tmp) {
  const int C8 = p.C >> 3;
  const uint4* xs = reinterpret_cast<const uint4*>(p.x) + (size_t)tok * (kBcast ? C8 : kNS * C8);
  uint4* lo = reinterpret_cast<uint4*>(p.li) + (size_t)tok * C8;
  const uint4* w8 = reinterpret_cast<const uint4*>(p.nw);
  const bool norm = p.nw != nullptr;
  float y[8][8];
  float ss = 0.f;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int c8 = threadIdx.x + s * kThreads;
    if (c8 < C8) {
      const uint4 v0 = xs[c8];
      const uint4 v1 = kBcast ? v0 : xs[C8 + c8];
      const uint4 v2 = kBcast ? v0 : xs[2 * C8 + c8];
      const uint4 v3 = kBcast ? v0 : xs[3 * C8 + c8];
      collapse8(v0, v1, v2, v3, p0, p1, p2, p3, y[s]);
      if (norm) {
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(y[s][e], y[s][e], ss);
      } else {
        lo[c8] = pack8(y[s]);
      }
    }
  }
  if (!norm) return;
  const float tot = block_sum(ss, s_tmp);
  const float ry = 1.0f / sqrtf(tot / (float)p.C + p.eps);
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int c8 = threadIdx.x + s * kThreads;
    if (c8 < C8) {
      float w[8], o[8];
      unpack8(w8[c8], w);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (y[s][e] * ry) * w[e];
      lo[c8] = pack8(o);
    }
  }
}

// ------------------------------------------------------------------ pre kernel, split form
// Workgroups [0, nproj): projection of a 16-token tile over one K-split.  With
// nsplit > 1 the last split of a tile to arrive (counter in the workspace)
// sums the partials in split order.  It then runs gates + Sinkhorn and, unless
// delayed, the collapse.  Delayed only: workgroups [nproj, nproj + T) collapse
// one token each with the carried pre-mix; they need nothing from the
// projection, so no workgroup ever waits for another.
template <int MODE>
__global__ __launch_bounds__(256) void mhc_pre_split_kernel(PreParams p) {
  __shared__ float s_red[4][kTileT][52];   // per-wave partial D (48 cols) + sumsq
  __shared__ float s_P[kTileT][kPS];
  __shared__ float s_pre[kTileT][kNS];
  __shared__ float s_tmp[4];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int b = blockIdx.x;

  if (MODE == kModeDelayed && b >= p.nproj) {
    const int tok = b - p.nproj;
    const float4 pin = reinterpret_cast<const float4*>(p.pre_in)[tok];
    collapse_norm_token<false>(p, tok, pin.x, pin.y, pin.z, pin.w, &s_tmp[0]);
    return;
  }

  const int tile = b / p.nsplit;
  const int sp = b - tile * p.nsplit;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int li_ = lane & 15;   // row (token) of the A operand / column of B
  const int g = lane >> 4;     // k-group of 8 within the 32-k step
  const int t0 = tile * kTileT;
  const int tok = t0 + li_;
  const bool valid = tok < p.T;
  const int kb0 = (int)(((long long)sp * p.KB) / p.nsplit);
  const int kb1 = (int)(((long long)(sp + 1) * p.KB) / p.nsplit);

  // ---- projection over this split's k-blocks: wave w takes kb0 + w, +4, ...,
  // issuing up to kJMax steps' loads before the first MFMA.
  const uint16_t* xrow = p.x + (size_t)(valid ? tok : 0) * p.K + g * 8;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0, acc2 = acc0;
  float ssq = 0.f;
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
  for (int base = kb0 + wave; base < kb1; base += 4 * kJMax) {
    uint4 xv[kJMax], b0[kJMax], b1[kJMax], b2[kJMax];
#pragma unroll
    for (int j = 0; j < kJMax; ++j) {
      const int kb = base + 4 * j;
      if (kb < kb1) {
        xv[j] = valid ? *reinterpret_cast<const uint4*>(xrow + (size_t)kb * kKB) : zero;
        const uint4* bp = p.fnp + (size_t)kb * (kFragPerKB * kWave) + lane;
        b0[j] = bp[0];
        b1[j] = bp[kWave];
        b2[j] = bp[2 * kWave];
      }
    }
#pragma unroll
    for (int j = 0; j < kJMax; ++j) {
      const int kb = base + 4 * j;
      if (kb < kb1) {
        ssq += sumsq8(xv[j]);
        acc0 = mfma_bf16(xv[j], b0[j], acc0);
        acc1 = mfma_bf16(xv[j], b1[j], acc1);
        acc2 = mfma_bf16(xv[j], b2[j], acc2);
        if (MODE == kModeEntry && valid) {
          // broadcast h to the four streams while it is in registers
          const size_t c = (size_t)kb * kKB + g * 8;
          uint4* xo = reinterpret_cast<uint4*>(p.xout + (size_t)tok * kNS * p.C + c);
          const size_t C8 = (size_t)(p.C >> 3);
          xo[0] = xv[j];
          xo[C8] = xv[j];
          xo[2 * C8] = xv[j];
          xo[3 * C8] = xv[j];
        }
      }
    }
  }
  // sum of squares: lanes (g, i) for g = 0..3 hold parts of token i's sum
  ssq += __shfl_xor(ssq, 16);
  ssq += __shfl_xor(ssq, 32);
  // D layout: lane L holds rows 4*(L>>4)+r, column L&15 of each 16x16 tile
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    s_red[wave][4 * g + r][li_] = acc0[r];
    s_red[wave][4 * g + r][16 + li_] = acc1[r];
    s_red[wave][4 * g + r][32 + li_] = acc2[r];
  }
  if (g == 0) s_red[wave][li_][48] = ssq;
  __syncthreads();

  // thread (tt, q): token row tt = tid >> 4, logit q (and q + 16 when q < 8)
  const int tt = tid >> 4;
  const int q = tid & 15;
  float v0, v1 = 0.f, vs = 0.f;
  {
    float hi = 0.f, lo = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) { hi += s_red[w][tt][q]; lo += s_red[w][tt][kNL + q]; }
    v0 = hi + lo;
    if (q < 8) {
      hi = 0.f; lo = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) { hi += s_red[w][tt][16 + q]; lo += s_red[w][tt][kNL + 16 + q]; }
      v1 = hi + lo;
    }
    if (q == 15) {
#pragma unroll
      for (int w = 0; w < 4; ++w) vs += s_red[w][tt][48];
    }
  }

  if (p.nsplit > 1) {
    float* dst = p.part + ((size_t)(tile * p.nsplit + sp) * kTileT + tt) * kPartStride;
    dst[q] = v0;
    if (q < 8) dst[16 + q] = v1;
    if (q == 15) dst[24] = vs;
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const unsigned old = atomicAdd(&p.cnt[tile], 1u);
      s_last = (old == (unsigned)(p.nsplit - 1));
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    // sum the partials of every split in split order; each (token, value) pair
    // is one thread, and its loads are issued kRedChunk at a time
    const float* src = p.part + (size_t)tile * p.nsplit * kTileT * kPartStride;
    const size_t sstride = (size_t)kTileT * kPartStride;
#pragma unroll
    for (int rep = 0; rep < 2; ++rep) {
      const int pair = tid + rep * kThreads;
      if (pair < kTileT * kPartStride) {
        const int pt = pair / kPartStride;
        const int pv = pair - pt * kPartStride;
        float acc = 0.f;
        if (t0 + pt < p.T) {
          for (int s0 = 0; s0 < p.nsplit; s0 += kRedChunk) {
            float v[kRedChunk];
#pragma unroll
            for (int u = 0; u < kRedChunk; ++u)
              v[u] = (s0 + u < p.nsplit) ? __builtin_nontemporal_load(src + (s0 + u) * sstride + pair) : 0.f;
#pragma unroll
            for (int u = 0; u < kRedChunk; ++u)
              if (s0 + u < p.nsplit) acc += v[u];
          }
        }
        s_P[pt][pv] = acc;
      }
    }
    if (tid == 0) atomicExch(&p.cnt[tile], 0u);  // leave the workspace as found
  } else {
    s_P[tt][q] = v0;
    if (q < 8) s_P[tt][16 + q] = v1;
    if (q == 15) s_P[tt][24] = vs;
  }
  __syncthreads();

  if (wave == 0) tile_gates(p, s_P, t0, s_pre);

  if (MODE == kModeDelayed || p.li == nullptr) return;
  __syncthreads();
  // ---- collapse with this seam's own pre-mix, token by token
  const int nt = min(kTileT, p.T - t0);
  for (int k = 0; k < nt; ++k)
    collapse_norm_token<MODE == kModeEntry>(p, t0 + k, s_pre[k][0], s_pre[k][1], s_pre[k][2],
                                             s_pre[k][3], &s_tmp[0]);
}

// ------------------------------------------------------------------ pre kernel, grouped delayed form
// Many tokens, hidden size fixed at compile time.  A tile of 64 tokens is
// covered by a group of kGR workgroups; member r owns hidden columns
// [r*C/kGR, (r+1)*C/kGR) of all four streams, and its wave w owns tokens
// 16w..16w+15 of the tile.  The four waves walk the same 32-column blocks in
// step, so each weight fragment is fetched from L2 once per workgroup and
// served to the other waves from L1: the weight costs 1/64 of its size per
// token instead of 1/16.  Per block a lane loads 8 bf16 of each stream for
// one token (the MFMA A operand), so one sweep over x feeds, without
// re-reading:
//   - the partial projection (3 MFMAs per stream against the packed weight),
//   - the partial row sum of squares (MFMA of the fragment with itself: its
//     diagonal is the per-token sum),
//   - the exact-order collapse with the carried pre-mix,
//   - the partial sum of squares of the collapsed row (folded RMSNorm).
// The collapsed rows stay on chip until the norm factor is known: most blocks
// in registers, kYL blocks per wave in LDS; the registers this frees hold a
// rotating prefetch kD blocks deep.  The members then exchange their partial
// sums through the workspace (group barrier, below), every member reduces them
// in member order -- the same bits in every member -- and runs gates +
// Sinkhorn; member 0 writes the gates, every member writes its columns of
// layer_input.
//
// Group barrier.  A group is kGR consecutive blocks.  Blocks are dealt to the
// XCDs round-robin and dispatched in order within each XCD, so a group's members
// are the k-th blocks of kGR different XCDs; every group whose index is at most
// the smallest index any of those XCDs has reached is fully resident and
// completes, which frees slots for the next ones -- no cycle of waits can form.
// (Under a single in-order dispatch queue the members are simply consecutive.)
// The wait is nevertheless bounded (kSpinMax sleeps, well over a second), so it
// always ends.  Arrival and departure counters are reset by the last member to
// leave, so the workspace is left as found.
// All global traffic of the sweep uses buffer instructions on per-tile
// descriptors: rows past the last token of a ragged tile read as zero and
// their stores are dropped by the descriptor's range check.
constexpr int kGroupThreads = 256;   // 4 waves, one per SIMD
constexpr int kGR = 4;               // workgroups per tile
constexpr int kGT = 64;              // tokens per tile (16 per wave)
constexpr int kSpinMax = 1 << 24;
constexpr int kGPart = 26;           // exchanged per token: P[24], sum x^2, sum y^2

// Partial sums cross workgroups (possibly XCDs) through device-coherent
// accesses: agent-scope atomic stores and loads, each coherent on its own, so
// no release fence has to write back the L2 (measured: such a fence cost ~20 us
// per workgroup here, flushing other workgroups' dirty layer_input lines).  A
// writer waits for its own stores to complete before the workgroup barrier
// that precedes the arrival increment.
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned ld_agent(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores() { __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// LDS-only barrier: waits for this wave's LDS traffic, then s_barrier.  Unlike
// __syncthreads it does not wait for outstanding global loads, so the
// prefetched blocks stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int kC, int kYL, int kD>
__global__ __launch_bounds__(kGroupThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mhc_pre_group_kernel(PreParams p) {
  constexpr int kNW = kGroupThreads / kWave;
  constexpr int kKBC = kC / kKB;          // 32-column blocks per stream
  constexpr int kCBW = kKBC / kGR;        // blocks per member (all waves walk the same ones)
  constexpr int kRow = kNS * kC * 2;      // bytes of one token's residual row
  constexpr int kSlots = kD + 1;
  constexpr int kFrag = kFragPerKB * kWave * 16;  // bytes of one k-block of packed weight
  static_assert(kKBC % kGR == 0, "hidden size must split evenly over the group");
  static_assert(kNW * kTileT == kGT, "one 16-token MFMA tile per wave");
  static_assert(kNW == kNS, "wave w fetches the weight fragments of stream w");
  static_assert(kYL <= kCBW, "more LDS blocks than blocks");
  __shared__ float4 s_y[kNW][kYL > 0 ? kYL : 1][2][kWave];  // collapsed rows kept in LDS
  __shared__ float s_pre[kGT][kNS];
  __shared__ float s_ry[kGT];
  __shared__ uint4 s_w[kCBW][4];    // this member's columns of the norm weight (bf16)
  // the weight block ring (2 x 12 KB) is only live during the sweep; afterwards
  // the same bytes hold the per-wave partial sums and the reduced tile sums
  typedef uint4 FnRing[2][kNS][kFragPerKB][kWave];
  typedef float RedBuf[kNW][kTileT][52];
  typedef float TileBuf[kGT][kPS];
  static_assert(sizeof(RedBuf) + sizeof(TileBuf) <= sizeof(FnRing), "reuse of the ring");
  __shared__ FnRing s_fn;
  RedBuf& s_red = *reinterpret_cast<RedBuf*>(&s_fn[0][0][0][0]);
  TileBuf& s_P = *reinterpret_cast<TileBuf*>(reinterpret_cast<char*>(&s_fn[0][0][0][0]) + sizeof(RedBuf));

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int i = lane & 15;
  const int g = lane >> 4;
  // a group is kGR consecutive blocks; with blocks dealt to the XCDs round-robin,
  // member r always lands on the XCDs with index = r (mod kGR), so each XCD's
  // L2 only ever holds one quarter of the packed weight
  const int mem = blockIdx.x % kGR;             // member of the group
  const int tile = blockIdx.x / kGR;
  const int t0 = tile * kGT;
  if (t0 >= p.T) return;                        // the whole group agrees
  const int wt0 = t0 + wave * kTileT;           // this wave's first token
  // descriptors depend on the block only (they must stay in SGPRs); a lane's
  // token row within the tile goes into its offset, which the range check covers
  const int nvalid = min(kGT, p.T - t0);
  const int tw = wave * kTileT + i;             // the lane's token within the tile
  const rsrc_t rx = make_rsrc(p.x + (size_t)t0 * (kNS * kC), nvalid * kRow);
  const rsrc_t rf = make_rsrc(p.fnp, p.KB * kFrag);
  const rsrc_t rp = make_rsrc(p.pre_in + (size_t)t0 * kNS, nvalid * 16);
  const int xlane = tw * kRow + g * 16;
  const int flane = lane * 16;
  const uint4 pv = buf_load16(rp, tw * 16, 0);
  const float p0 = __uint_as_float(pv.x), p1 = __uint_as_float(pv.y);
  const float p2 = __uint_as_float(pv.z), p3 = __uint_as_float(pv.w);
  const int cb0 = mem * kCBW;                   // first column block of this member
  if (p.nw && tid < kCBW * 4)
    s_w[tid >> 2][tid & 3] = reinterpret_cast<const uint4*>(p.nw)[cb0 * 4 + tid];
  // tiles walk their blocks from different starting points, so that at any
  // time the chip's x reads spread over many columns (and L2 channels)
  const int rot = (tile * 7) % kCBW;

  // rotating prefetch: slot k holds block b with b % kSlots == k; per block a
  // wave fetches its tokens' x (4 streams) and one stream's weight fragments
  uint4 xq[kSlots][kNS];
  uint4 fq[kSlots][kFragPerKB];
  auto issue = [&](int cb, int slot) {
    int blk = cb + rot;
    blk = blk >= kCBW ? blk - kCBW : blk;
    const int cbg = cb0 + blk;
#pragma unroll
    for (int s = 0; s < kNS; ++s) xq[slot][s] = buf_load16(rx, xlane, (s * kC + cbg * kKB) * 2);
#pragma unroll
    for (int f = 0; f < kFragPerKB; ++f)
      fq[slot][f] = buf_load16(rf, flane, (wave * kKBC + cbg) * kFrag + f * kWave * 16);
  };
#pragma unroll
  for (int d = 0; d < kD; ++d) issue(d, d);

  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, a2 = a0, as = a0;
  float ssy = 0.f;
  float y[kCBW - kYL][8];
#pragma unroll
  for (int cb = 0; cb < kCBW; ++cb) {
    if (cb + kD < kCBW) issue(cb + kD, (cb + kD) % kSlots);
    const int slot = cb % kSlots;
    // publish this wave's stream of the weight block, then read all four
#pragma unroll
    for (int f = 0; f < kFragPerKB; ++f) s_fn[cb & 1][wave][f][lane] = fq[slot][f];
    lds_barrier();
#pragma unroll
    for (int s = 0; s < kNS; ++s) {
      a0 = mfma_bf16(xq[slot][s], s_fn[cb & 1][s][0][lane], a0);
      a1 = mfma_bf16(xq[slot][s], s_fn[cb & 1][s][1][lane], a1);
      a2 = mfma_bf16(xq[slot][s], s_fn[cb & 1][s][2][lane], a2);
      as = mfma_bf16(xq[slot][s], xq[slot][s], as);
    }
    float yb[8];
    collapse8(xq[slot][0], xq[slot][1], xq[slot][2], xq[slot][3], p0, p1, p2, p3, yb);
#pragma unroll
    for (int e = 0; e < 8; ++e) ssy = __builtin_fmaf(yb[e], yb[e], ssy);
    if (cb < kYL) {
      s_y[wave][cb][0][lane] = make_float4(yb[0], yb[1], yb[2], yb[3]);
      s_y[wave][cb][1][lane] = make_float4(yb[4], yb[5], yb[6], yb[7]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) y[cb - kYL][e] = yb[e];
    }
  }

  // diagonal of x.x^T: row 4g + r of lane (g, i) is token i when i == 4g + r
  float ssx = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (i == 4 * g + r) ssx = as[r];
  ssy += __shfl_xor(ssy, 16);
  ssy += __shfl_xor(ssy, 32);
  __syncthreads();  // every wave is done with the weight ring
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    s_red[wave][4 * g + r][i] = a0[r];
    s_red[wave][4 * g + r][16 + i] = a1[r];
    s_red[wave][4 * g + r][32 + i] = a2[r];
  }
  if ((i >> 2) == g) s_red[wave][i][48] = ssx;
  if (g == 0) s_red[wave][i][49] = ssy;
  __syncthreads();

  // ---- publish this member's partials: token (wave, tt), values 6*part .. 6*part+5
  float* part = p.part + (size_t)tile * kGR * kGT * kGPart;
  {
    const int tt = lane >> 2, pp = lane & 3;
    float* dst = part + ((size_t)mem * kGT + wave * kTileT + tt) * kGPart;
#pragma unroll
    for (int u = 0; u < 6; ++u) {
      const int j = pp * 6 + u;
      st_agent(dst + j, s_red[wave][tt][j] + s_red[wave][tt][kNL + j]);
    }
    if (pp < 2) st_agent(dst + kNL + pp, s_red[wave][tt][48 + pp]);
  }
  wait_stores();
  __syncthreads();
  unsigned* arrive = p.cnt + 2 * tile;
  unsigned* depart = arrive + 1;
  if (tid == 0) {
    __hip_atomic_fetch_add(arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int spins = 0;
    while (ld_agent(arrive) < (unsigned)kGR && spins < kSpinMax) {
      __builtin_amdgcn_s_sleep(2);
      ++spins;
    }
  }
  __syncthreads();
  {
    // sum the members' partials in member order: token tid >> 2, values of part tid & 3
    const int tt = tid >> 2, pp = tid & 3;
    const int nj = pp < 2 ? 7 : 6;  // parts 0/1 also carry sum x^2 / sum y^2
#pragma unroll
    for (int u = 0; u < 7; ++u) {
      if (u < nj) {
        const int j = u < 6 ? pp * 6 + u : kNL + pp;
        float acc = 0.f;
#pragma unroll
        for (int m = 0; m < kGR; ++m)
          acc += ld_agent(part + ((size_t)m * kGT + tt) * kGPart + j);
        s_P[tt][j] = acc;
      }
    }
  }
  __syncthreads();
  if (tid == 0 && atomicAdd(depart, 1u) == (unsigned)(kGR - 1)) {
    atomicExch(arrive, 0u);  // every member has passed the barrier: reset for the next call
    atomicExch(depart, 0u);
  }

  // ---- gates (member 0 writes them) and norm factor, each wave its 16 tokens
  tile_gates(p, &s_P[wave * kTileT], wt0, &s_pre[wave * kTileT], mem == 0);
  if (lane < kTileT) {
    const int tt = wave * kTileT + lane;
    s_ry[tt] = p.nw ? 1.0f / sqrtf(s_P[tt][25] / (float)kC + p.eps) : 1.0f;
  }
  __syncthreads();

  const float ry = s_ry[tw];
  const rsrc_t rl = make_rsrc(p.li + (size_t)t0 * kC, nvalid * kC * 2);
  const int llane = tw * (kC * 2) + g * 16;
  const bool norm = p.nw != nullptr;
#pragma unroll
  for (int cb = 0; cb < kCBW; ++cb) {
    int blk = cb + rot;
    blk = blk >= kCBW ? blk - kCBW : blk;
    const int c = (cb0 + blk) * kKB;
    float yb[8];
    if (cb < kYL) {
      const float4 u = s_y[wave][cb][0][lane], v = s_y[wave][cb][1][lane];
      yb[0] = u.x; yb[1] = u.y; yb[2] = u.z; yb[3] = u.w;
      yb[4] = v.x; yb[5] = v.y; yb[6] = v.z; yb[7] = v.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) yb[e] = y[cb - kYL][e];
    }
    float o[8];
    if (norm) {
      float w[8];
      unpack8(s_w[c / kKB - cb0][g], w);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (yb[e] * ry) * w[e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = yb[e];
    }
    buf_store16(pack8(o), rl, llane, c * 2);
  }
}

// ------------------------------------------------------------------ post kernel
// One thread per (token, 8 hidden elements): reads y (16 B) and the four
// streams (4 x 16 B), writes four streams.  Every byte is touched once, so all
// traffic is non-temporal (streaming): measured ~14% faster than cached
// accesses at T = 16384.  Exact in-place (out == x) is safe: a thread reads
// all of its x before it writes.
__global__ __launch_bounds__(256) void mhc_post_kernel(const uint4* __restrict__ y,
                                                       const uint4* x,
                                                       const float* __restrict__ post,
                                                       const float* __restrict__ comb, uint4* out,
                                                       int T, int C8) {
  const long long idx = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (long long)T * C8) return;
  const int t = (int)(idx / C8);
  const int c8 = (int)(idx - (long long)t * C8);
  const size_t xb = (size_t)t * kNS * C8 + c8;
  const uint4 yq = nt_load16(y + (size_t)t * C8 + c8);
  const uint4 q0 = nt_load16(x + xb);
  const uint4 q1 = nt_load16(x + xb + C8);
  const uint4 q2 = nt_load16(x + xb + 2 * (size_t)C8);
  const uint4 q3 = nt_load16(x + xb + 3 * (size_t)C8);
  const float4 pg = reinterpret_cast<const float4*>(post)[t];
  const float4* cb = reinterpret_cast<const float4*>(comb) + (size_t)t * 4;
  const float4 cr[4] = {cb[0], cb[1], cb[2], cb[3]};
  float yv[8], x0[8], x1[8], x2[8], x3[8];
  unpack8(yq, yv);
  unpack8(q0, x0);
  unpack8(q1, x1);
  unpack8(q2, x2);
  unpack8(q3, x3);
  const float pw[4] = {pg.x, pg.y, pg.z, pg.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float a = pw[i] * yv[e];
      a = __builtin_fmaf(cr[i].x, x0[e], a);
      a = __builtin_fmaf(cr[i].y, x1[e], a);
      a = __builtin_fmaf(cr[i].z, x2[e], a);
      a = __builtin_fmaf(cr[i].w, x3[e], a);
      o[e] = a;
    }
    nt_store16(pack8(o), out + xb + (size_t)i * C8);
  }
}

}  // namespace mhc
