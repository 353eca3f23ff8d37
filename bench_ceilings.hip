// bench_ceilings.hip -- reference rates of the memory system, for bench.py.
//
// Not part of the library: the benchmark loads it to set the seam kernels'
// bandwidth beside what this GPU's memory delivers for the same traffic with no
// arithmetic at all.
//
//   ceil_stream: 16-byte non-temporal accesses over a whole buffer: read only,
//     write only, or copy.
//   ceil_pattern_run: the one-sweep pre kernels' traffic at C = 5120 with no
//     arithmetic and no exchange -- the same persistent grid (groups of 16
//     workgroups walking 64-token tiles, 136 KB of LDS so one workgroup per CU),
//     the same loads (each wave: its eight tokens' 128-byte lines of the
//     member's 640-byte column window in each stream, plus the sublayer output
//     for the fused seam; two lines in flight) and the same non-temporal stores
//     (next residual lines for the fused seam, layer_input lines).  The values
//     stored are bitwise mixes of the loaded lines.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kAuxNT = 2;   // non-temporal hint of buffer accesses

__device__ __forceinline__ rsrc_t rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 load_line(rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ void store_nt(u32x4 v, rsrc_t r, int off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kAuxNT);
}

// ---------------------------------------------------------------- streams
// The configurations that measured fastest here (1 GiB and 640 MB buffers): reads
// grid-stride with one load per thread in flight over 2048 workgroups (7.2 TB/s);
// writes and copies with one 16-byte access per thread over as many workgroups as
// that takes (6.9 and 6.6 TB/s: the dispatcher hands out workgroups in address
// order, so the accesses in flight stay within a few MB).
constexpr int kStreamThreads = 256;
constexpr int kReadBlocks = 2048;

__global__ __launch_bounds__(kStreamThreads) void ceil_read_kernel(const u32x4* a, long long n, u32x4* sink) {
  const long long stride = (long long)gridDim.x * kStreamThreads;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (long long i = (long long)blockIdx.x * kStreamThreads + threadIdx.x; i < n; i += stride)
    acc ^= __builtin_nontemporal_load(a + i);
  // kept only if it hits a fixed 64-bit pattern: the loads cannot be dropped
  if (acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u) sink[threadIdx.x] = acc;
}
__global__ __launch_bounds__(kStreamThreads) void ceil_write_kernel(u32x4* b, long long n) {
  const long long i = (long long)blockIdx.x * kStreamThreads + threadIdx.x;
  if (i < n) __builtin_nontemporal_store(u32x4{1u, 2u, 3u, 4u}, b + i);
}
__global__ __launch_bounds__(kStreamThreads) void ceil_copy_kernel(const u32x4* a, u32x4* b, long long n) {
  const long long i = (long long)blockIdx.x * kStreamThreads + threadIdx.x;
  if (i < n) __builtin_nontemporal_store(__builtin_nontemporal_load(a + i), b + i);
}

// ---------------------------------------------------------------- access pattern
constexpr int kNS = 4, kC = 5120, kL = 5, kPG = 16, kPT = 64, kWaves = 8;
constexpr int kRow = kNS * kC * 2;   // bytes of a residual row
constexpr int kYRow = kC * 2;        // bytes of a sublayer-output / layer_input row
constexpr int kLdsWords = 139264 / 16;

template <bool kFused>
__global__ __launch_bounds__(kWaves * 64) void ceil_pattern_kernel(const uint16_t* x, const uint16_t* y,
                                                                   uint16_t* xo, uint16_t* li, int T,
                                                                   int ngroups) {
  __shared__ u32x4 lds[kLdsWords];
  if (T < 0) {   // never taken (the launcher checks T): keeps the LDS allocation
    lds[threadIdx.x] = u32x4{1u, 2u, 3u, 4u};
    __syncthreads();
    store_nt(lds[threadIdx.x ^ 1], rsrc(li, 1 << 16), (int)threadIdx.x * 16);
    return;
  }
  constexpr int kIn = kFused ? 5 : 4;   // loads per line: four streams (+ the sublayer output)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tok = lane & 7;                                  // the lane's token of the wave's eight
  const int chunk = ((lane >> 3) & 1) * 4 + (lane >> 4);     // its 16 bytes of a 128-byte line
  const int mem = blockIdx.x % kPG, grp = blockIdx.x / kPG;
  const int ntiles = (T + kPT - 1) / kPT;
  const int nk = grp < ntiles ? (ntiles - 1 - grp) / ngroups + 1 : 0;
  const int nlines = nk * kL;
  const int col = kL * 128 * mem + chunk * 16;
  const int xl = (wave * 8 + tok) * kRow + col;
  const int yl = (wave * 8 + tok) * kYRow + col;
  // line g of the walk: tile grp + (g / kL) ngroups, line g % kL of the window;
  // past the end a zero-size descriptor (loads read zero, stores are dropped)
  auto tile_of = [&](int g) { return g < nlines ? grp + (g / kL) * ngroups : -1; };
  auto rows = [&](int t) { return t >= 0 ? min(kPT, T - t * kPT) : 0; };
  auto issue = [&](u32x4 (&r)[kIn], int g) {
    const int t = tile_of(g), u = g % kL;
    const rsrc_t rx = rsrc(x + (size_t)(t >= 0 ? t : 0) * kPT * kNS * kC, rows(t) * kRow);
#pragma unroll
    for (int s = 0; s < kNS; ++s) r[s] = load_line(rx, xl + s * kC * 2 + u * 128);
    if constexpr (kFused)
      r[4] = load_line(rsrc(y + (size_t)(t >= 0 ? t : 0) * kPT * kC, rows(t) * kYRow), yl + u * 128);
  };
  auto consume = [&](const u32x4 (&r)[kIn], int g) {
    const int t = tile_of(g), u = g % kL;
    if constexpr (kFused) {
      const rsrc_t ro = rsrc(xo + (size_t)t * kPT * kNS * kC, rows(t) * kRow);
#pragma unroll
      for (int s = 0; s < kNS; ++s) store_nt(r[s] ^ r[4], ro, xl + s * kC * 2 + u * 128);
    }
    store_nt(r[0] ^ r[1] ^ r[2] ^ r[3], rsrc(li + (size_t)t * kPT * kC, rows(t) * kYRow), yl + u * 128);
  };
  u32x4 a[kIn], b[kIn];
  issue(a, 0);
  issue(b, 1);
  for (int g = 0; g < nlines; g += 2) {
    consume(a, g);
    issue(a, g + 2);
    if (g + 1 < nlines) {
      consume(b, g + 1);
      issue(b, g + 3);
    }
  }
}

}  // namespace

// kind: 0 read `bytes` of src, 1 write `bytes` of dst, 2 copy `bytes` of src to
// dst.  bytes: a multiple of 16, at most 16 GiB; sink: 4 KB of device memory.
// Returns 0, -1 for bad arguments, or the launch's HIP error code.
extern "C" int ceil_stream(int kind, const void* src, void* dst, size_t bytes, void* sink, void* stream) {
  if (kind < 0 || kind > 2 || bytes == 0 || bytes % 16 != 0 || bytes > ((size_t)1 << 34) || sink == nullptr) return -1;
  if ((kind != 1 && src == nullptr) || (kind != 0 && dst == nullptr)) return -1;
  const long long n = (long long)(bytes / 16);
  const unsigned blocks = (unsigned)((n + kStreamThreads - 1) / kStreamThreads);
  const hipStream_t s = (hipStream_t)stream;
  const u32x4* a = (const u32x4*)src;
  u32x4* b = (u32x4*)dst;
  switch (kind) {
    case 0: hipLaunchKernelGGL(ceil_read_kernel, dim3(kReadBlocks), dim3(kStreamThreads), 0, s, a, n, (u32x4*)sink); break;
    case 1: hipLaunchKernelGGL(ceil_write_kernel, dim3(blocks), dim3(kStreamThreads), 0, s, b, n); break;
    default: hipLaunchKernelGGL(ceil_copy_kernel, dim3(blocks), dim3(kStreamThreads), 0, s, a, b, n); break;
  }
  return (int)hipGetLastError();
}

// The pre kernels' traffic at hidden size 5120, four streams: x [T][4][5120] bf16
// read; fused: y [T][5120] read and xo [T][4][5120] written; li [T][5120] written.
// ngroups in [1, 16] groups of 16 workgroups.  Returns 0, -1 for bad arguments,
// or the launch's HIP error code.
extern "C" int ceil_pattern_run(int fused, const void* x, const void* y, void* xo, void* li, int T, int ngroups,
                                void* stream) {
  if (T < 1 || T > (1 << 22) || ngroups < 1 || ngroups > 16 || x == nullptr || li == nullptr) return -1;
  if (fused && (y == nullptr || xo == nullptr)) return -1;
  const hipStream_t s = (hipStream_t)stream;
  const dim3 grid(ngroups * kPG), block(kWaves * 64);
  if (fused)
    hipLaunchKernelGGL(ceil_pattern_kernel<true>, grid, block, 0, s, (const uint16_t*)x, (const uint16_t*)y,
                       (uint16_t*)xo, (uint16_t*)li, T, ngroups);
  else
    hipLaunchKernelGGL(ceil_pattern_kernel<false>, grid, block, 0, s, (const uint16_t*)x, (const uint16_t*)y,
                       (uint16_t*)xo, (uint16_t*)li, T, ngroups);
  return (int)hipGetLastError();
}
