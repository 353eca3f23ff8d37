// mhc_kernels.hpp -- the seam kernels of libmhc for gfx950.
//
//   mhc_pack_fn_kernel          one-time weight packing (bf16 hi/lo split, MFMA order)
//   mhc_pre_split_kernel<MODE>  pre stage for any T: projection split over
//                               workgroups (few tokens) or one workgroup per
//                               16-token tile, last-arriver reduction, gates +
//                               Sinkhorn, collapse + folded RMSNorm.
//   mhc_persist_kernel          (mhc_persist.hpp) pre stage for many tokens at
//                               C = 4096, 5120, 7168: persistent groups of
//                               workgroups, one sweep over x per 64-token tile;
//                               projection (weight slice resident in LDS), both
//                               sums of squares, collapse and norm fused; the
//                               fused seam and the gates-only pass as variants.
//   mhc_collapse_kernel         standalone collapse (+ folded norm), one token per workgroup.
//   mhc_post_kernel             post stage: post_i * y + sum_j comb_ij x_j.
#pragma once

#include "mhc_device.hpp"

namespace mhc {

enum Mode { kModePre = 0, kModeDelayed = 1, kModeEntry = 2, kModeFused = 3 };

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
  uint16_t* xout;         // [T][4][C] broadcast residual (entry) / next residual (fused)
  const uint16_t* ysub;   // [T][C] sublayer output (fused)
  const float* post_in;   // [T][4] post gates of the previous seam (fused)
  const float* comb_in;   // [T][16] comb of the previous seam (fused)
  float* part;            // workspace: partial sums [ntile][nsplit][16][25]
  unsigned* cnt;          // workspace: arrival counters [ntile]
  float eps;
  int iters;
  int T, C, K, KB;        // K = row length, KB = K / 32
  int ntile, nsplit, nproj;
  int own_wgs;            // own pre-mix: workgroups [nproj, nproj + T) collapse one token each
  unsigned wait_bias;     // added to every wait target; non-zero makes every wait run out (tests)
  int wait_budget;        // sleeps a bounded wait may take (per collapse workgroup / per wave)
};

constexpr int kPS = 28;      // LDS row per token: P[0..23], sum x^2 [24], sum y^2 [25]
// Split-form workspace from p.cnt: the tile arrival counters (32-bit words
// [0, kSplitFlagStride)), a word set when a wait ran out (kSplitWaitErr), and
// from byte kSplitRecBytes the own-pre-mix records, 16 bytes per token: the
// four pre-mix values with the sign bit set.  A pre-mix value is >= 0, so a set
// sign bit marks a written word and zero an empty one; the consumer clears its
// record, so the region is back at zero after every call.
constexpr int kSplitFlagStride = 256;          // at least the most tiles a split call has
constexpr int kSplitWaitErr = kSplitFlagStride;
constexpr int kSplitRecBytes = 4096;
constexpr int kOwnMaxTokens = 2048;            // tokens an own-pre-mix call with collapse workgroups may have
constexpr int kSplitBytes = kSplitRecBytes + kOwnMaxTokens * 16;
constexpr int kWaitBudget = 1 << 20;           // sleeps a bounded wait may take (about a second)
constexpr unsigned kRecSet = 0x80000000u;
constexpr int kJMax = 8;     // k-steps a wave issues together in the split kernel
constexpr int kRedChunk = 32;  // partials loaded together by the last arriver

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
// The four waves of the workgroup take a 16-token tile, four tokens each: a
// token's 16 lanes (one DPP row) hold its 4x4 comb matrix, lane 4i + j entry
// (i, j), so an iteration is two butterflies, two reciprocals and two
// multiplies per lane.  Row sums: quad butterflies; column sums: rotations of
// the 16-lane row by 8 (the same as exchanging with lane ^ 8) and then by 4,
// which pairs (0,2) and (1,3) in every lane.  Either way every lane of a row
// or column divides by the same bits.  The row maximum is subtracted before
// exp (removed exactly by the first row step); reciprocals, the exponential and
// the reciprocal square root are the hardware's (about 1 ulp each).  The lanes of
// row 0 also make the token's pre and post gates (gate index j).  `ba` holds
// bias[24] then alpha[3] (LDS).
// `rec` (or nullptr): the own-pre-mix records the tile's collapse workgroups wait on.
__device__ __forceinline__ void tile_gates(const PreParams& p, const float* ba, const float (*s_P)[kPS], int t0,
                                           float (*s_pre)[kNS], unsigned* rec) {
  const int lane = threadIdx.x & (kWave - 1);
  const int tt = (threadIdx.x / kWave) * 4 + (lane >> 4);
  const int i = (lane >> 2) & 3;
  const int j = lane & 3;
  const int tk = t0 + tt;
  const bool ok = tk < p.T;
  const float r = hw_rsqrt(s_P[tt][24] * (1.0f / (float)p.K) + p.eps);
  float m = ba[kNL + 2] * (r * s_P[tt][8 + 4 * i + j]) + ba[8 + 4 * i + j];
  float mx = fmaxf(m, dpp_quad_xor1(m));
  mx = fmaxf(mx, dpp_quad_xor2(mx));
  m = hw_exp(m - mx);
  for (int it = 0; it < p.iters; ++it) {
    float rs = m + dpp_quad_xor1(m);
    rs = rs + dpp_quad_xor2(rs);
    m *= __builtin_amdgcn_rcpf(rs);
    float cs = m + dpp_row_ror8(m);
    cs = cs + dpp_row_ror4(cs);
    m *= __builtin_amdgcn_rcpf(cs);
  }
  if (i == 0) {
    const float lp = ba[kNL] * (r * s_P[tt][j]) + ba[j];
    const float lq = ba[kNL + 1] * (r * s_P[tt][4 + j]) + ba[4 + j];
    const float pr = hw_sigmoid(lp);
    const float po = 2.0f * hw_sigmoid(lq);
    s_pre[tt][j] = pr;
    if (ok) {
      p.pre[(size_t)tk * kNS + j] = pr;
      p.post[(size_t)tk * kNS + j] = po;
      if (rec != nullptr) st_agent(rec + (size_t)tk * kNS + j, __float_as_uint(pr) | kRecSet);
    }
  }
  if (ok) p.comb[(size_t)tk * 16 + 4 * i + j] = m;
}

// ------------------------------------------------------------------ collapse + norm, one token
// The whole 256-thread workgroup handles token `tok`: y (float) stays in
// registers, sum(y^2) is reduced over the workgroup, then layer_input is written.
// kPost: the streams collapsed are the post stage's output, computed here from
// the previous residual, the sublayer output and the previous seam's gates,
// and written out as the next residual on the way.
// kStream: the residual rows are read and layer_input written with streaming
// (non-temporal) accesses, for a call that streams more than the memory-side
// cache holds; the split kernel's collapse workgroups read rows its projection
// workgroups have just read, so they keep them cached.
template <bool kBcast, bool kPost = false, bool kStream = false>
__device__ __forceinline__ void collapse_norm_token(const PreParams& p, int tok, float p0, float p1,
                                                    float p2, float p3, float* s_tmp) {
  const int C8 = p.C >> 3;
  const uint4* xs = reinterpret_cast<const uint4*>(p.x) + (size_t)tok * (kBcast ? C8 : kNS * C8);
  uint4* lo = reinterpret_cast<uint4*>(p.li) + (size_t)tok * C8;
  const uint4* w8 = reinterpret_cast<const uint4*>(p.nw);
  const bool norm = p.nw != nullptr;
  float pw[4] = {0.f, 0.f, 0.f, 0.f};
  float4 cr[4];
  if (kPost) {
    const float4 pg = reinterpret_cast<const float4*>(p.post_in)[tok];
    pw[0] = pg.x;
    pw[1] = pg.y;
    pw[2] = pg.z;
    pw[3] = pg.w;
#pragma unroll
    for (int i = 0; i < 4; ++i) cr[i] = reinterpret_cast<const float4*>(p.comb_in)[(size_t)tok * 4 + i];
  }
  float y[8][8];
  float ss = 0.f;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int c8 = threadIdx.x + s * kThreads;
    if (c8 < C8) {
      uint4 v0 = kStream ? nt_load16(xs + c8) : xs[c8];
      uint4 v1 = kBcast ? v0 : kStream ? nt_load16(xs + C8 + c8) : xs[C8 + c8];
      uint4 v2 = kBcast ? v0 : kStream ? nt_load16(xs + 2 * C8 + c8) : xs[2 * C8 + c8];
      uint4 v3 = kBcast ? v0 : kStream ? nt_load16(xs + 3 * C8 + c8) : xs[3 * C8 + c8];
      if (kBcast) {
        // the entry seam's residual: h broadcast to the four streams, whole rows
        uint4* xo = reinterpret_cast<uint4*>(p.xout) + (size_t)tok * kNS * C8 + c8;
        xo[0] = v0;
        xo[C8] = v0;
        xo[2 * C8] = v0;
        xo[3 * C8] = v0;
        if (p.li == nullptr) continue;
      }
      if (kPost) {
        float yv[8], a0[8], a1[8], a2[8], a3[8];
        unpack8(reinterpret_cast<const uint4*>(p.ysub)[(size_t)tok * C8 + c8], yv);
        unpack8(v0, a0);
        unpack8(v1, a1);
        unpack8(v2, a2);
        unpack8(v3, a3);
        v0 = post_stream8(pw[0], cr[0].x, cr[0].y, cr[0].z, cr[0].w, yv, a0, a1, a2, a3);
        v1 = post_stream8(pw[1], cr[1].x, cr[1].y, cr[1].z, cr[1].w, yv, a0, a1, a2, a3);
        v2 = post_stream8(pw[2], cr[2].x, cr[2].y, cr[2].z, cr[2].w, yv, a0, a1, a2, a3);
        v3 = post_stream8(pw[3], cr[3].x, cr[3].y, cr[3].z, cr[3].w, yv, a0, a1, a2, a3);
        uint4* xo = reinterpret_cast<uint4*>(p.xout) + (size_t)tok * kNS * C8 + c8;
        xo[0] = v0;
        xo[C8] = v1;
        xo[2 * C8] = v2;
        xo[3 * C8] = v3;
      }
      collapse8(v0, v1, v2, v3, p0, p1, p2, p3, y[s]);
      if (norm) {
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(y[s][e], y[s][e], ss);
      } else {
        if (kStream)
          nt_store16(pack8(y[s]), lo + c8);
        else
          lo[c8] = pack8(y[s]);
      }
    }
  }
  if (!norm || (kBcast && p.li == nullptr)) return;
  const float tot = block_sum(ss, s_tmp);
  const float ry = hw_rsqrt(tot * (1.0f / (float)p.C) + p.eps);
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int c8 = threadIdx.x + s * kThreads;
    if (c8 < C8) {
      float w[8], o[8];
      unpack8(w8[c8], w);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (y[s][e] * ry) * w[e];
      if (kStream)
        nt_store16(pack8(o), lo + c8);
      else
        lo[c8] = pack8(o);
    }
  }
}

// ------------------------------------------------------------------ collapse + norm, one token per wave
// For the 16 tokens a projection workgroup has just gated (own pre-mix): with
// hidden sizes up to 5120 a token's collapsed row fits one wave's registers (at
// most 10 chunks of 8 per lane), so the four waves take a token each instead
// of the whole workgroup taking the tokens one after another (measured at
// T = 16384: mhc_pre 392 -> 373 us, entry seam 437 -> 394 us; at T = 128:
// 56 -> 45 and 51 -> 40 us).  The one-workgroup-per-token form above stays for
// the delayed forms' collapse workgroups and the standalone collapse, where it
// is faster (standalone at T = 16384: 146 vs 164 us).  Same exact-order collapse
// and folded norm; the sum of squares is taken per lane over its chunks in
// order, then over the wave, so with the norm the two forms may differ in the
// last bit of the norm factor.  Its stores (layer_input, the entry seam's
// broadcast residual) are written once and never re-read here, so they are
// streaming (entry seam at T = 16384: 289 -> 190 us).
constexpr int kWaveCollapseMaxC = 5120;
template <bool kBcast>
__device__ __forceinline__ void collapse_token_wave(const PreParams& p, int tok, float p0, float p1, float p2,
                                                    float p3) {
  constexpr int kCh = kWaveCollapseMaxC / 8 / kWave;   // chunks per lane at most
  constexpr int kCG = 5;                               // chunks loaded together
  const int lane = threadIdx.x & (kWave - 1);
  const int C8 = p.C >> 3;
  const uint4* xs = reinterpret_cast<const uint4*>(p.x) + (size_t)tok * (kBcast ? C8 : kNS * C8);
  uint4* lo = reinterpret_cast<uint4*>(p.li) + (size_t)tok * C8;
  const uint4* w8 = reinterpret_cast<const uint4*>(p.nw);
  const bool norm = p.nw != nullptr;
  float y[kCh][8];
  float ss = 0.f;
#pragma unroll
  for (int g0 = 0; g0 < kCh; g0 += kCG) {
    uint4 q[kCG][4];
#pragma unroll
    for (int u = 0; u < kCG; ++u) {
      const int c8 = lane + (g0 + u) * kWave;
      if (c8 < C8) {
        q[u][0] = xs[c8];
        q[u][1] = kBcast ? q[u][0] : xs[C8 + c8];
        q[u][2] = kBcast ? q[u][0] : xs[2 * C8 + c8];
        q[u][3] = kBcast ? q[u][0] : xs[3 * C8 + c8];
      }
    }
#pragma unroll
    for (int u = 0; u < kCG; ++u) {
      const int ch = g0 + u;
      const int c8 = lane + ch * kWave;
      if (c8 < C8) {
        if (kBcast) {
          // the entry seam's residual: h broadcast to the four streams, whole rows
          uint4* xo = reinterpret_cast<uint4*>(p.xout) + (size_t)tok * kNS * C8 + c8;
          nt_store16(q[u][0], xo);
          nt_store16(q[u][0], xo + C8);
          nt_store16(q[u][0], xo + 2 * C8);
          nt_store16(q[u][0], xo + 3 * C8);
          if (p.li == nullptr) continue;
        }
        collapse8(q[u][0], q[u][1], q[u][2], q[u][3], p0, p1, p2, p3, y[ch]);
        if (norm) {
#pragma unroll
          for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(y[ch][e], y[ch][e], ss);
        } else {
          nt_store16(pack8(y[ch]), lo + c8);
        }
      }
    }
  }
  if (!norm || (kBcast && p.li == nullptr)) return;
  const float tot = wave_sum(ss);
  const float ry = hw_rsqrt(tot * (1.0f / (float)p.C) + p.eps);
#pragma unroll
  for (int ch = 0; ch < kCh; ++ch) {
    const int c8 = lane + ch * kWave;
    if (c8 < C8) {
      float w[8], o[8];
      unpack8(w8[c8], w);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (y[ch][e] * ry) * w[e];
      nt_store16(pack8(o), lo + c8);
    }
  }
}

// ------------------------------------------------------------------ own pre-mix collapse, waiting workgroup
// One workgroup per token, for the forms that collapse with the seam's own
// pre-mix (mhc_pre, the entry seam) when the projection is split: the token's
// residual row is loaded first, then the workgroup waits until its tile's last
// arriving projection workgroup has published the token's pre-mix record (the
// four values with their sign bits set, polled with device-coherent loads and
// cleared once read), so the collapse overlaps the projection instead of
// following it in one workgroup per tile.  The entry seam writes its broadcast
// residual before waiting, and does not wait at all when no layer_input is
// requested.
// Forward progress: projection workgroups have the lower indices and are
// dispatched first; none of them waits for anything.  The wait is bounded
// nevertheless (p.wait_budget sleeps): if it runs out the workgroup records
// it in p.cnt[kSplitWaitErr] and goes on, so the kernel always ends.  A
// non-zero p.wait_bias counts every record as missing, so each wait runs out.
// Hidden sizes up to kWaveCollapseMaxC (3 chunks of 8 per thread).
template <bool kBcast>
__device__ __forceinline__ void collapse_own_token(const PreParams& p, int tok, float* s_tmp, float* s_pm) {
  constexpr int kCh = 3;
  const int tid = threadIdx.x;
  const int C8 = p.C >> 3;
  const uint4* xs = reinterpret_cast<const uint4*>(p.x) + (size_t)tok * (kBcast ? C8 : kNS * C8);
  uint4 q[kCh][4];
#pragma unroll
  for (int s = 0; s < kCh; ++s) {
    const int c8 = tid + s * kThreads;
    if (c8 < C8) {
      q[s][0] = xs[c8];
      q[s][1] = kBcast ? q[s][0] : xs[C8 + c8];
      q[s][2] = kBcast ? q[s][0] : xs[2 * C8 + c8];
      q[s][3] = kBcast ? q[s][0] : xs[3 * C8 + c8];
    }
  }
  if (kBcast) {
#pragma unroll
    for (int s = 0; s < kCh; ++s) {
      const int c8 = tid + s * kThreads;
      if (c8 < C8) {
        uint4* xo = reinterpret_cast<uint4*>(p.xout) + (size_t)tok * kNS * C8 + c8;
        xo[0] = q[s][0];
        xo[C8] = q[s][0];
        xo[2 * C8] = q[s][0];
        xo[3 * C8] = q[s][0];
      }
    }
    if (p.li == nullptr) return;
  }
  if (tid == 0) {
    // the token's record: four words, each written with its sign bit set
    const rsrc_t rr = make_rsrc(reinterpret_cast<char*>(p.cnt) + kSplitRecBytes, p.T * 16);
    int budget = p.wait_budget;
    const bool never = p.wait_bias != 0u;
    uint4 v = buf_load16_agent(rr, tok * 16, 0);
    while ((never || ((v.x & v.y & v.z & v.w) & kRecSet) == 0u) && budget > 0) {
      --budget;
      __builtin_amdgcn_s_sleep(2);
      v = buf_load16_agent(rr, tok * 16, 0);
    }
    if (never || ((v.x & v.y & v.z & v.w) & kRecSet) == 0u) st_agent(p.cnt + kSplitWaitErr, 1u);
    buf_store16_agent(make_uint4(0u, 0u, 0u, 0u), rr, tok * 16, 0);   // consumed: back to empty
    s_pm[0] = __uint_as_float(v.x & ~kRecSet);
    s_pm[1] = __uint_as_float(v.y & ~kRecSet);
    s_pm[2] = __uint_as_float(v.z & ~kRecSet);
    s_pm[3] = __uint_as_float(v.w & ~kRecSet);
  }
  __syncthreads();
  const float p0 = s_pm[0], p1 = s_pm[1], p2 = s_pm[2], p3 = s_pm[3];
  uint4* lo = reinterpret_cast<uint4*>(p.li) + (size_t)tok * C8;
  const bool norm = p.nw != nullptr;
  float y[kCh][8];
  float ss = 0.f;
#pragma unroll
  for (int s = 0; s < kCh; ++s) {
    const int c8 = tid + s * kThreads;
    if (c8 < C8) {
      collapse8(q[s][0], q[s][1], q[s][2], q[s][3], p0, p1, p2, p3, y[s]);
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
  const float ry = hw_rsqrt(tot * (1.0f / (float)p.C) + p.eps);
  const uint4* w8 = reinterpret_cast<const uint4*>(p.nw);
#pragma unroll
  for (int s = 0; s < kCh; ++s) {
    const int c8 = tid + s * kThreads;
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
// Fused (post of the previous seam, then the delayed pre): the projection
// splits the hidden columns instead of the 4C row, so that each 32-column
// block's five loads (sublayer output, four residual streams) give all four
// next-residual fragments; the collapse workgroups recompute the token's next
// residual with the same arithmetic (same bits) and are the ones that write it.
constexpr int kJFused = 2;   // column blocks a wave loads together in the fused projection
template <int MODE>
__global__ __launch_bounds__(256) void mhc_pre_split_kernel(PreParams p) {
  __shared__ float s_red[4][kTileT][52];   // per-wave partial D (48 cols) + sumsq
  __shared__ float s_P[kTileT][kPS];
  __shared__ float s_pre[kTileT][kNS];
  __shared__ float s_tmp[4];
  __shared__ float s_pm[4];    // own-pre-mix collapse workgroups: the token's pre-mix
  __shared__ float s_ba[32];   // bias[24], alpha[3]
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int b = blockIdx.x;

  if ((MODE == kModeDelayed || MODE == kModeFused) && b >= p.nproj) {
    const int tok = b - p.nproj;
    const float4 pin = reinterpret_cast<const float4*>(p.pre_in)[tok];
    collapse_norm_token<false, MODE == kModeFused>(p, tok, pin.x, pin.y, pin.z, pin.w, &s_tmp[0]);
    return;
  }
  if ((MODE == kModePre || MODE == kModeEntry) && p.own_wgs && b >= p.nproj) {
    collapse_own_token<MODE == kModeEntry>(p, b - p.nproj, &s_tmp[0], &s_pm[0]);
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
  // bias and alpha, loaded now and staged in LDS with the first barrier, so
  // that the gates after the reduction wait on no global load
  const float bav = tid < kNL ? p.bias[tid] : (tid >= 32 && tid < 35) ? p.alpha[tid - 32] : 0.f;
  const int kb0 = (int)(((long long)sp * p.KB) / p.nsplit);
  const int kb1 = (int)(((long long)(sp + 1) * p.KB) / p.nsplit);

  // ---- projection over this split's k-blocks: wave w takes kb0 + w, +4, ...,
  // issuing up to kJMax steps' loads before the first MFMA.  Residual rows
  // through a descriptor covering the tile's tokens: rows past the last token
  // read as zero without a memory access.
  const int ntok = min(kTileT, p.T - t0);
  const rsrc_t xr = make_rsrc(p.x + (size_t)t0 * p.K, ntok * p.K * 2);
  const int xoff = li_ * p.K * 2 + g * 16;   // bytes: the lane's row and 8-column group
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0, acc2 = acc0;
  float ssq = 0.f;
  if constexpr (MODE == kModeFused) {
    // column blocks [cbA, cbB) of all four streams; wave w takes cbA + w, +4, ...
    const int CB = p.C / kKB;
    const int cbA = (int)(((long long)sp * CB) / p.nsplit);
    const int cbB = (int)(((long long)(sp + 1) * CB) / p.nsplit);
    const rsrc_t yr = make_rsrc(p.ysub + (size_t)t0 * p.C, ntok * p.C * 2);
    const int yoff = li_ * p.C * 2 + g * 16;
    float pw[4] = {0.f, 0.f, 0.f, 0.f};
    float4 cr[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) cr[s] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (valid) {
      const float4 pg = reinterpret_cast<const float4*>(p.post_in)[tok];
      pw[0] = pg.x;
      pw[1] = pg.y;
      pw[2] = pg.z;
      pw[3] = pg.w;
#pragma unroll
      for (int s = 0; s < 4; ++s) cr[s] = reinterpret_cast<const float4*>(p.comb_in)[(size_t)tok * 4 + s];
    }
    for (int base = cbA + wave; base < cbB; base += 4 * kJFused) {
      uint4 yv[kJFused], xv[kJFused][kNS], bw[kJFused][kNS][kFragPerKB];
#pragma unroll
      for (int j = 0; j < kJFused; ++j) {
        const int cb = base + 4 * j;
        if (cb < cbB) {
          yv[j] = buf_load16(yr, yoff + cb * kKB * 2, 0);
#pragma unroll
          for (int s = 0; s < kNS; ++s) {
            xv[j][s] = buf_load16(xr, xoff + (s * p.C + cb * kKB) * 2, 0);
            const uint4* bp = p.fnp + (size_t)(s * CB + cb) * (kFragPerKB * kWave) + lane;
#pragma unroll
            for (int f = 0; f < kFragPerKB; ++f) bw[j][s][f] = bp[f * kWave];
          }
        }
      }
#pragma unroll
      for (int j = 0; j < kJFused; ++j) {
        const int cb = base + 4 * j;
        if (cb < cbB) {
          float yf[8], x0[8], x1[8], x2[8], x3[8];
          unpack8(yv[j], yf);
          unpack8(xv[j][0], x0);
          unpack8(xv[j][1], x1);
          unpack8(xv[j][2], x2);
          unpack8(xv[j][3], x3);
#pragma unroll
          for (int s = 0; s < kNS; ++s) {
            const uint4 xn = post_stream8(pw[s], cr[s].x, cr[s].y, cr[s].z, cr[s].w, yf, x0, x1, x2, x3);
            ssq += sumsq8(xn);
            acc0 = mfma_bf16(xn, bw[j][s][0], acc0);
            acc1 = mfma_bf16(xn, bw[j][s][1], acc1);
            acc2 = mfma_bf16(xn, bw[j][s][2], acc2);
          }
        }
      }
    }
  } else
  for (int base = kb0 + wave; base < kb1; base += 4 * kJMax) {
    uint4 xv[kJMax], b0[kJMax], b1[kJMax], b2[kJMax];
#pragma unroll
    for (int j = 0; j < kJMax; ++j) {
      const int kb = base + 4 * j;
      if (kb < kb1) {
        xv[j] = buf_load16(xr, xoff + kb * kKB * 2, 0);
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
  if (tid < kNL) s_ba[tid] = bav;
  if (tid >= 32 && tid < 35) s_ba[kNL + tid - 32] = bav;
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
    // The partials cross workgroups (and XCDs) through device-coherent stores
    // and loads, each coherent on its own: no fence, so no write-back or
    // invalidation of the L2 (which would also drop the cached weight).  A
    // wave's stores are complete once its store counter drains, before the
    // workgroup's arrival is counted; the last arriver's loads are ordered
    // after its counter update by the barrier and its control dependence.
    float* dst = p.part + ((size_t)(tile * p.nsplit + sp) * kTileT + tt) * kPartStride;
    st_agent(dst + q, v0);
    if (q < 8) st_agent(dst + 16 + q, v1);
    if (q == 15) st_agent(dst + 24, vs);
    wait_vmem();
    __syncthreads();
    if (tid == 0) {
      const unsigned old = __hip_atomic_fetch_add(&p.cnt[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = (old == (unsigned)(p.nsplit - 1));
    }
    __syncthreads();
    if (!s_last) return;
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
              v[u] = (s0 + u < p.nsplit) ? ld_agent(src + (s0 + u) * sstride + pair) : 0.f;
#pragma unroll
            for (int u = 0; u < kRedChunk; ++u)
              if (s0 + u < p.nsplit) acc += v[u];
          }
        }
        s_P[pt][pv] = acc;
      }
    }
    if (tid == 0) st_agent(&p.cnt[tile], 0u);  // leave the workspace as found
  } else {
    s_P[tt][q] = v0;
    if (q < 8) s_P[tt][16 + q] = v1;
    if (q == 15) s_P[tt][24] = vs;
  }
  __syncthreads();

  const bool own = (MODE == kModePre || MODE == kModeEntry) && p.own_wgs;
  tile_gates(p, s_ba, s_P, t0, s_pre,
             own && p.li != nullptr ? reinterpret_cast<unsigned*>(reinterpret_cast<char*>(p.cnt) + kSplitRecBytes)
                                    : nullptr);
  // own pre-mix: the tile's collapse workgroups take it from here (records)
  if (own) return;

  // the entry seam always goes on: its collapse pass also writes the broadcast residual
  if (MODE == kModeDelayed || MODE == kModeFused || (MODE != kModeEntry && p.li == nullptr)) return;
  __syncthreads();
  // ---- collapse with this seam's own pre-mix, token by token
  const int nt = min(kTileT, p.T - t0);
  if (p.C <= kWaveCollapseMaxC) {
    for (int k = wave; k < nt; k += kThreads / kWave)
      collapse_token_wave<MODE == kModeEntry>(p, t0 + k, s_pre[k][0], s_pre[k][1], s_pre[k][2],
                                                      s_pre[k][3]);
  } else {
    for (int k = 0; k < nt; ++k)
      collapse_norm_token<MODE == kModeEntry>(p, t0 + k, s_pre[k][0], s_pre[k][1], s_pre[k][2],
                                               s_pre[k][3], &s_tmp[0]);
  }
}

// ------------------------------------------------------------------ pre kernel, persistent form
}  // namespace mhc
#include "mhc_persist.hpp"
namespace mhc {

// ------------------------------------------------------------------ standalone collapse
// One workgroup per token: the exact-order collapse with p[token] and the
// optional folded norm (collapse_norm_token), nothing else.  kStream: streaming
// accesses (a call larger than the memory-side cache).
template <bool kStream>
__global__ __launch_bounds__(kThreads) void mhc_collapse_kernel(PreParams p) {
  __shared__ float s_tmp[4];
  const int tok = blockIdx.x;
  const float4 pv = reinterpret_cast<const float4*>(p.pre_in)[tok];
  collapse_norm_token<false, false, kStream>(p, tok, pv.x, pv.y, pv.z, pv.w, s_tmp);
}

// ------------------------------------------------------------------ post kernel
// One thread per (token, 8 hidden elements): reads y (16 B) and the four
// streams (4 x 16 B), writes four streams.  Every byte is touched once, so all
// traffic is non-temporal (streaming): measured ~14% faster than cached
// accesses at T = 16384.  Exact in-place (out == x) is safe: a thread reads
// all of its x before it writes.  kWaveToken (C / 8 a multiple of 64): a wave's
// 64 threads share one token, whose 20 gate values are then loaded once per
// wave through the scalar unit instead of by every lane.
template <bool kWaveToken>
__global__ __launch_bounds__(256) void mhc_post_kernel(const uint4* __restrict__ y,
                                                       const uint4* x,
                                                       const float* __restrict__ post,
                                                       const float* __restrict__ comb, uint4* out,
                                                       int T, int C8) {
  const long long idx = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (long long)T * C8) return;
  int t;
  if constexpr (kWaveToken) {
    // the wave's first thread is in range (it has the wave's lowest index)
    const long long widx = (long long)blockIdx.x * kThreads + (threadIdx.x & ~(kWave - 1));
    t = __builtin_amdgcn_readfirstlane((int)(widx / C8));
  } else {
    t = (int)(idx / C8);
  }
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
  for (int i = 0; i < 4; ++i)
    nt_store16(post_stream8(pw[i], cr[i].x, cr[i].y, cr[i].z, cr[i].w, yv, x0, x1, x2, x3),
               out + xb + (size_t)i * C8);
}

}  // namespace mhc
