// mhc_device.hpp -- device building blocks of libmhc for gfx950 (CDNA4, wave64).
//
// The seam's hot path (vLLM PR "[ROCm][DSV4.1][Perf] Use AITER mHC for the
// delayed pre block", Approach): projection of the flattened 4C row against fn
// plus the row sum of squares, the gates and every Sinkhorn iteration, the
// collapse of the four streams, and the folded RMSNorm of the "Fix TileLang
// mHC pre on 64-wide wavefronts" PR (Measurements).  Every cross-lane
// reduction here spans the full 64-lane wavefront and every role split is
// wave-aligned: that PR's bug was a 32-lane role split inside a 64-lane wave
// that summed only half of the squares (The bug).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mhc {

constexpr int kNS = 4;        // residual streams (hc_mult)
constexpr int kNL = 24;       // logits per token: pre 4 | post 4 | comb 16
constexpr int kTileT = 16;    // tokens per projection tile = rows of one MFMA
constexpr int kThreads = 256; // four waves per workgroup
constexpr int kWave = 64;
constexpr int kKB = 32;       // k elements per MFMA step (16x16x32)
constexpr int kFragPerKB = 3; // 48 packed columns (24 hi | 24 lo) = 3 tiles of 16
constexpr int kPartStride = 25; // 24 partial projections + partial sum of squares

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- bf16 helpers
__device__ __forceinline__ float bf_even(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_odd(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Two floats -> two bf16 (round to nearest even), packed little-endian.
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Component t (compile-time) of a uint4, as a float.
__device__ __forceinline__ float u4_comp(const uint4& v, int t) {
  return __uint_as_float(t == 0 ? v.x : t == 1 ? v.y : t == 2 ? v.z : v.w);
}

__device__ __forceinline__ void unpack8(const uint4& v, float (&f)[8]) {
  f[0] = bf_even(v.x); f[1] = bf_odd(v.x);
  f[2] = bf_even(v.y); f[3] = bf_odd(v.y);
  f[4] = bf_even(v.z); f[5] = bf_odd(v.z);
  f[6] = bf_even(v.w); f[7] = bf_odd(v.w);
}

__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
  return make_uint4(pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7]));
}

__device__ __forceinline__ float sumsq8(const uint4& v) {
  float f[8];
  unpack8(v, f);
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) s = __builtin_fmaf(f[e], f[e], s);
  return s;
}

__device__ __forceinline__ f32x4 mfma_bf16(const uint4& a, const uint4& b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

// Streaming (non-temporal) 16-byte load and store, for data touched exactly once.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 nt_load16(const void* ptr) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ptr)));
}
__device__ __forceinline__ void nt_store16(uint4 v, void* ptr) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4*>(ptr));
}

// ---------------------------------------------------------------- buffer access
// Raw buffer descriptors: base in SGPRs, per-lane 32-bit offset.  A load whose
// offset is at or past `bytes` returns zero and such a store is dropped.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // raw (untyped) 32-bit buffer, gfx9 family
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcWord3);
}
__device__ __forceinline__ uint4 buf_load16(rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
// streaming (non-temporal) variant for data read exactly once
__device__ __forceinline__ uint4 buf_load16_nt(rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2));
}
__device__ __forceinline__ void buf_store16(uint4 v, rsrc_t r, int voff, int soff) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, voff, soff, 0);
}
// streaming (non-temporal) variant for data written once and not read back by this call
__device__ __forceinline__ void buf_store16_nt(uint4 v, rsrc_t r, int voff, int soff) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, voff, soff, 2);
}

// ---------------------------------------------------------------- device-coherent access
// Values passed between workgroups (which may sit on different XCDs, each with
// its own L2) use agent-scope atomic loads and stores: each is coherent on its
// own, so no fence has to write back or invalidate an L2.
template <typename T>
__device__ __forceinline__ T ld_agent(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ void st_agent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The same for 16-byte buffer accesses: cache policy coherent at device scope (sc1).
constexpr int kAuxAgent = 16;
__device__ __forceinline__ uint4 buf_load16_agent(rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kAuxAgent));
}
__device__ __forceinline__ void buf_store16_agent(uint4 v, rsrc_t r, int voff, int soff) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, voff, soff, kAuxAgent);
}
// Wait until every vector memory access of the wave has completed (stores
// included); also a compiler barrier for memory.
__device__ __forceinline__ void wait_vmem() { __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ---------------------------------------------------------------- gate arithmetic
// The hardware's exponential, reciprocal and reciprocal square root (each within
// about 1 ulp; exp(x) as 2^(x log2 e), whose product adds |x| 2^-24 relative).
// The gates' error budget is 1e-4 relative; these keep the gate set-up short.
__device__ __forceinline__ float hw_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504088896341f); }
__device__ __forceinline__ float hw_rsqrt(float x) { return __builtin_amdgcn_rsqf(x); }
__device__ __forceinline__ float hw_sigmoid(float x) { return __builtin_amdgcn_rcpf(1.0f + hw_exp(-x)); }

// ---------------------------------------------------------------- quad shuffles (DPP)
// Lane l reads lane l^1 / l^2 of its quad; all 64 lanes must be active.
__device__ __forceinline__ float dpp_quad_xor1(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1,
                                                               0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_quad_xor2(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E,
                                                               0xF, 0xF, false));
}

// Rotations within a 16-lane DPP row: lane l reads lane (l - 8) mod 16 (the
// same as lane l ^ 8) / (l - 4) mod 16 of its row.
__device__ __forceinline__ float dpp_row_ror8(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128,
                                                               0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_row_ror4(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124,
                                                               0xF, 0xF, false));
}

// ---------------------------------------------------------------- collapse
// y_c = fl(fl(fl(fl(p0 x0) + fl(p1 x1)) + fl(p2 x2)) + fl(p3 x3)): each product
// rounded to float, summed left to right over the streams, never fused --
// the single-precision multiply-and-sum that the delayed-pre PR (Result)
// reports as bit-exact between its paths.
__device__ __forceinline__ float collapse1(float p0, float p1, float p2, float p3, float x0,
                                           float x1, float x2, float x3) {
#pragma clang fp contract(off)
  float a = p0 * x0;
  float b = p1 * x1;
  float c = p2 * x2;
  float d = p3 * x3;
  return ((a + b) + c) + d;
}

__device__ __forceinline__ void collapse8(const uint4& v0, const uint4& v1, const uint4& v2,
                                          const uint4& v3, float p0, float p1, float p2, float p3,
                                          float (&y)[8]) {
  float a[8], b[8], c[8], d[8];
  unpack8(v0, a);
  unpack8(v1, b);
  unpack8(v2, c);
  unpack8(v3, d);
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = collapse1(p0, p1, p2, p3, a[e], b[e], c[e], d[e]);
}

// ---------------------------------------------------------------- post stage
// Residual stream i of the post stage for 8 hidden elements:
//   a = fl(post_i * y);  a = fma(comb[i][j], x_j, a) for j = 0, 1, 2, 3;  bf16(a)
// (single precision, this order, one rounding).  Every kernel that writes or
// consumes the next residual uses this one definition, so the bf16 residual
// the next seam reads is the same bits whichever kernel produced it.
__device__ __forceinline__ uint4 post_stream8(float pw, float c0, float c1, float c2, float c3,
                                              const float (&y)[8], const float (&x0)[8],
                                              const float (&x1)[8], const float (&x2)[8],
                                              const float (&x3)[8]) {
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float a = pw * y[e];
    a = __builtin_fmaf(c0, x0[e], a);
    a = __builtin_fmaf(c1, x1[e], a);
    a = __builtin_fmaf(c2, x2[e], a);
    a = __builtin_fmaf(c3, x3[e], a);
    o[e] = a;
  }
  return pack8(o);
}

// One stream of the post stage from packed inputs (the same operations and
// order as post_stream8): only the five inputs' packed words and this
// stream's gates are live, at the price of unpacking the inputs per stream.
__device__ __forceinline__ uint4 post_packed8(float pw, float c0, float c1, float c2, float c3, const uint4& yv,
                                             const uint4& v0, const uint4& v1, const uint4& v2,
                                             const uint4& v3) {
  uint32_t o[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const uint32_t yw = h == 0 ? yv.x : h == 1 ? yv.y : h == 2 ? yv.z : yv.w;
    const uint32_t w0 = h == 0 ? v0.x : h == 1 ? v0.y : h == 2 ? v0.z : v0.w;
    const uint32_t w1 = h == 0 ? v1.x : h == 1 ? v1.y : h == 2 ? v1.z : v1.w;
    const uint32_t w2 = h == 0 ? v2.x : h == 1 ? v2.y : h == 2 ? v2.z : v2.w;
    const uint32_t w3 = h == 0 ? v3.x : h == 1 ? v3.y : h == 2 ? v3.z : v3.w;
    float r[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      float a = pw * (b ? bf_odd(yw) : bf_even(yw));
      a = __builtin_fmaf(c0, b ? bf_odd(w0) : bf_even(w0), a);
      a = __builtin_fmaf(c1, b ? bf_odd(w1) : bf_even(w1), a);
      a = __builtin_fmaf(c2, b ? bf_odd(w2) : bf_even(w2), a);
      a = __builtin_fmaf(c3, b ? bf_odd(w3) : bf_even(w3), a);
      r[b] = a;
    }
    o[h] = pack2(r[0], r[1]);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// ---------------------------------------------------------------- reductions
// Butterfly over all 64 lanes: every lane ends with the same bits (float
// addition is commutative, so partner lanes form identical sums).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

// Sum over the 256-thread workgroup in a fixed order; every thread gets it.
__device__ __forceinline__ float block_sum(float v, float* s_tmp) {
  v = wave_sum(v);
  if ((threadIdx.x & (kWave - 1)) == 0) s_tmp[threadIdx.x / kWave] = v;
  __syncthreads();
  float t = (s_tmp[0] + s_tmp[1]) + (s_tmp[2] + s_tmp[3]);
  __syncthreads();
  return t;
}

}  // namespace mhc
