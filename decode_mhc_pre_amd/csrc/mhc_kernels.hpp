// mhc_kernels.hpp -- the seam kernels of libmhc for gfx950.
//
//   mhc_pack_fn_kernel   one-time weight packing (bf16 hi/lo split, MFMA order)
//   mhc_pre_kernel<MODE> pre stage: projection + RMS (bf16 MFMA, split over
//                        workgroups when few tokens), gates, Sinkhorn, collapse,
//                        folded RMSNorm.  MODE = own pre-mix / delayed / entry.
//   mhc_post_kernel      post stage: post_i * y + sum_j comb_ij x_j, streamed.
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

// ------------------------------------------------------------------ pre kernel
// Workgroups [0, nproj): projection tile (16 tokens) x K-split.  The last split
// of a tile to arrive (counter in the workspace) reduces the partials in split
// order, computes gates + Sinkhorn and, unless delayed, the collapse.
// Delayed only: workgroups [nproj, nproj + T) collapse one token each with the
// carried pre-mix -- independent of the projection, so no wait between them.
template <int MODE>
__global__ __launch_bounds__(256) void mhc_pre_kernel(PreParams p) {
  __shared__ float s_red[4][kTileT][52];   // per-wave partial D (48 cols) + sumsq
  __shared__ float s_P[kTileT][kPartStride];
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

  // ---- projection over this split's k-blocks: wave w takes kb0 + w, +4, ...
  const uint16_t* xrow = p.x + (size_t)(valid ? tok : 0) * p.K + g * 8;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0, acc2 = acc0;
  float ssq = 0.f;
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll 2
  for (int kb = kb0 + wave; kb < kb1; kb += 4) {
    const uint4 xv = valid ? *reinterpret_cast<const uint4*>(xrow + (size_t)kb * kKB) : zero;
    const uint4* bp = p.fnp + (size_t)kb * (kFragPerKB * kWave) + lane;
    const uint4 b0 = bp[0], b1 = bp[kWave], b2 = bp[2 * kWave];
    ssq += sumsq8(xv);
    acc0 = mfma_bf16(xv, b0, acc0);
    acc1 = mfma_bf16(xv, b1, acc1);
    acc2 = mfma_bf16(xv, b2, acc2);
    if (MODE == kModeEntry && valid) {
      // broadcast h to the four streams while it is in registers
      const size_t c = (size_t)kb * kKB + g * 8;
      uint4* xo = reinterpret_cast<uint4*>(p.xout + (size_t)tok * kNS * p.C + c);
      const size_t C8 = (size_t)(p.C >> 3);
      xo[0] = xv;
      xo[C8] = xv;
      xo[2 * C8] = xv;
      xo[3 * C8] = xv;
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
    const float* src = p.part + ((size_t)tile * p.nsplit * kTileT + tt) * kPartStride;
    v0 = 0.f; v1 = 0.f; vs = 0.f;
    for (int s = 0; s < p.nsplit; ++s) {
      const float* ps = src + (size_t)s * kTileT * kPartStride;
      v0 += __builtin_nontemporal_load(ps + q);
      if (q < 8) v1 += __builtin_nontemporal_load(ps + 16 + q);
      if (q == 15) vs += __builtin_nontemporal_load(ps + 24);
    }
    if (tid == 0) atomicExch(&p.cnt[tile], 0u);  // leave the workspace as found
  }
  s_P[tt][q] = v0;
  if (q < 8) s_P[tt][16 + q] = v1;
  if (q == 15) s_P[tt][24] = vs;
  __syncthreads();

  // ---- gates and Sinkhorn: thread (tt, e) owns comb entry e = 4i + j of token tt
  {
    const int e = q;
    const int tk = t0 + tt;
    const bool ok = tk < p.T;
    const float r = 1.0f / sqrtf(s_P[tt][24] / (float)p.K + p.eps);
    const float a_pre = p.alpha[0], a_post = p.alpha[1], a_comb = p.alpha[2];
    float m = expf(a_comb * (r * s_P[tt][8 + e]) + p.bias[8 + e]);
    for (int it = 0; it < p.iters; ++it) {
      float rs = m + __shfl_xor(m, 1);     // row i: lanes differ in bits 0..1
      rs += __shfl_xor(rs, 2);
      m = m / rs;
      float cs = m + __shfl_xor(m, 4);     // column j: lanes differ in bits 2..3
      cs += __shfl_xor(cs, 8);
      m = m / cs;
    }
    if (ok) p.comb[(size_t)tk * 16 + e] = m;
    if (e < 4) {
      const float l = a_pre * (r * s_P[tt][e]) + p.bias[e];
      const float pr = 1.0f / (1.0f + expf(-l));
      s_pre[tt][e] = pr;
      if (ok) p.pre[(size_t)tk * kNS + e] = pr;
    } else if (e < 8) {
      const float l = a_post * (r * s_P[tt][e]) + p.bias[e];
      if (ok) p.post[(size_t)tk * kNS + (e - 4)] = 2.0f / (1.0f + expf(-l));
    }
  }

  if (MODE == kModeDelayed || p.li == nullptr) return;
  __syncthreads();
  // ---- collapse with this seam's own pre-mix, token by token
  const int nt = min(kTileT, p.T - t0);
  for (int k = 0; k < nt; ++k)
    collapse_norm_token<MODE == kModeEntry>(p, t0 + k, s_pre[k][0], s_pre[k][1], s_pre[k][2],
                                             s_pre[k][3], &s_tmp[0]);
}

// ------------------------------------------------------------------ post kernel
// One thread per (token, 8 hidden elements): reads y (16 B) and the four
// streams (4 x 16 B), writes four streams.  Exact in-place (out == x) is safe:
// a thread reads all of its x before it writes.
__global__ __launch_bounds__(256) void mhc_post_kernel(const uint4* __restrict__ y,
                                                       const uint4* x,
                                                       const float* __restrict__ post,
                                                       const float* __restrict__ comb, uint4* out,
                                                       int T, int C8) {
  const long long idx = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (long long)T * C8) return;
  const int t = (int)(idx / C8);
  const int c8 = (int)(idx - (long long)t * C8);
  const float4 pg = reinterpret_cast<const float4*>(post)[t];
  const float4* cb = reinterpret_cast<const float4*>(comb) + (size_t)t * 4;
  const float4 c0 = cb[0], c1 = cb[1], c2 = cb[2], c3 = cb[3];
  const size_t xb = (size_t)t * kNS * C8 + c8;
  float yv[8], x0[8], x1[8], x2[8], x3[8];
  unpack8(y[(size_t)t * C8 + c8], yv);
  unpack8(x[xb], x0);
  unpack8(x[xb + C8], x1);
  unpack8(x[xb + 2 * (size_t)C8], x2);
  unpack8(x[xb + 3 * (size_t)C8], x3);
  const float pw[4] = {pg.x, pg.y, pg.z, pg.w};
  const float4 cr[4] = {c0, c1, c2, c3};
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
    out[xb + (size_t)i * C8] = pack8(o);
  }
}

}  // namespace mhc
