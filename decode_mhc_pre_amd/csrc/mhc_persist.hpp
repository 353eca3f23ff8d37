// mhc_persist.hpp -- the one-sweep pre kernel for many tokens (delayed pre, the
// fused seam, and the gates-only pass of the own-pre-mix form) on gfx950.
//
// The seam's pre stage (vLLM PR "[ROCm][DSV4.1][Perf] Use AITER mHC for the
// delayed pre block", Approach): projection of the flattened 4C row against fn
// with the row sum of squares, gates and Sinkhorn; the collapse with the carried
// pre-mix (Purpose) and the folded RMSNorm of the "Fix TileLang mHC pre on
// 64-wide wavefronts" PR (Measurements); in the fused form the post stage of
// the previous seam in front of it (the first PR's Notes / follow-ups).
//
// Decomposition.  Tokens are cut into tiles of 64.  A group of kPG workgroups
// covers one tile at a time; member r owns kLines 64-column "lines" of every
// stream, hidden columns [64 kLines r, 64 kLines (r + 1)), so its slice of the
// packed projection weight fits in LDS and is loaded once per call.  A
// workgroup is 8 waves, two per SIMD; wave w owns tokens 8w .. 8w + 7 of the
// tile.  The grid is persistent: group j walks tiles j, j + ngroups, ...
//
// Loads.  Lane L of a wave reads 16 bytes of token (L & 7) at chunk
// 4 ((L >> 3) & 1) + (L >> 4) of a 128-byte line, so one load covers eight
// whole lines, and the loaded register is already the A operand of
// v_mfma_f32_16x16x32_bf16: rows 0-7 are the eight tokens' first half-lines,
// rows 8-15 their second half-lines.  The weight operand carries the
// matching halves in its output columns 0-7 and 8-15 (8 outputs of each half
// per instruction, so 6 instructions give the 48 packed outputs, hi 0..23 and
// lo 0..23; the hi and lo instructions of the same outputs accumulate into one
// register set, which is f(x . hi) + f(x . lo) with its roundings spread over
// the sum); the two diagonal blocks of the result are the useful ones and are
// added once per tile.  The fragment times itself gives the sums of squares on
// its diagonal.  Each load also feeds one stream's step of the exact-order
// collapse; the collapsed rows of a tile (40 floats per lane at C = 5120) stay
// in registers until the tile's norm factors are known.
//
// Exchange.  Each wave shares its 8 tokens with the waves of the same index in
// the other members.  A record per (group, wave, slot) holds a value block
// [token 8][member][32 floats] (24 projections, sum x^2, sum y^2, padding to a
// 128-byte line) and a sum-y^2 block [member][token 8].  Tile k's record is
// written at the start of tile k + 1 (one whole-line store per wave); a load
// issued right after those stores (a wave's vector memory operations complete
// in issue order) tells when they are complete, and the arrival is counted
// then.  Late in tile k + 1 the wave checks that every member arrived (the
// counter read a few sub-steps before) and issues the loads of the records:
// the sum-y^2 block (norm factors, every member) and its gate token's lines
// (members 0-7 take the wave's tokens 0-7 of even tiles, members 8-15 those
// of odd tiles).  They are summed at the start of tile k + 2, whose sub-steps
// then run the gate token's gates and one Sinkhorn iteration each.  Tile k's
// layer_input is written during tile k + 2, each line just before the sweep
// overwrites its row buffer, so two row buffers give the exchange more than a
// tile of slack.  Record slots alternate (slot k % 2 is rewritten at the start
// of tile k + 2, after its writer saw every member arrive for tile k + 1,
// which each does after its loads of tile k's records are back: they were
// issued before the fence load that the arrival waits for).
//
// Forward progress: a group is kPG consecutive blocks, dispatched in order, so
// groups become resident whole or behind groups that are; those finish all of
// their tiles and free their CUs.  Every wait is bounded all the same: a wave
// sleeps at most p.wait_budget times per call, and when the budget runs out it
// sets workspace word 2 and stops waiting, so the kernel always ends.  The last
// wave of the grid to finish sets every counter back to zero.
#pragma once

#include <type_traits>

#include "mhc_device.hpp"

namespace mhc {

// f(integral_constant<int, I>) for I = 0 .. N-1: loop bodies whose index must be
// a compile-time constant (register arrays, schedules).
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>());
    static_for<N, I + 1>(f);
  }
}
template <bool B, class T>
__device__ __forceinline__ T& pick(T& a, T& b) {
  if constexpr (B)
    return a;
  else
    return b;
}

// Geometry per hidden size: lines per member (kLines, at most 5: the weight
// slice takes 24 KB per line of LDS) and members per group (kPG).  kRefill: the
// sub-step of a line at which the fused form issues the next line's loads (the
// earliest that fits the registers and measured fastest: at C = 4096 one sub-step
// earlier than at 5120 and 7168, T = 16384 281.6 -> 274.0 us).  kLateDelayed: the
// delayed form reads the arrival counter one sub-step later and checks it one
// sub-step earlier than the default schedule (C = 7168, T = 16384: 286.5 -> 281.3
// us; no change for the fused form or at C = 4096).
template <int kC> struct PersistGeom;
template <> struct PersistGeom<4096> {
  static constexpr int kLines = 4, kPG = 16, kRefill = 1;
  static constexpr bool kLateDelayed = false;
};
template <> struct PersistGeom<5120> {
  static constexpr int kLines = 5, kPG = 16, kRefill = 2;
  static constexpr bool kLateDelayed = false;
};
template <> struct PersistGeom<7168> {
  static constexpr int kLines = 4, kPG = 28, kRefill = 2;
  static constexpr bool kLateDelayed = true;
};

constexpr int kPT = 64;                   // tokens per tile
constexpr int kPW = 8;                    // waves per workgroup (two per SIMD)
constexpr int kPTW = 8;                   // tokens per wave
constexpr int kPThreads = kPW * kWave;
constexpr int kPQ = 6;                    // weight fragments per (line, stream): 48 packed outputs / 8
constexpr int kPA = 3;                    // accumulators: fragments q and q + 3 (hi, lo parts of the
                                          // same 8 outputs) add into accumulator q
constexpr int kPMaxGroups = 16;           // the workspace holds records for this many groups
constexpr int kPRing = 2;                 // record slots per (group, wave)
constexpr int kPSlots = kPRing + 1;       // counters per (group, wave): the slots, and one for "tile -1"
constexpr int kPLine = 32;                // floats per (token, member) line of the value block
constexpr int kPMaxPG = 28;               // the largest group of the geometries above
// Workspace: word 0 counts finished waves, word 2 is set by a wait that ran out;
// arrival counters from word kPCntBase, one per (group, wave, slot), each in a
// 128-byte line of its own; records from byte kPPartOffset.
constexpr int kPCntBase = 64;
constexpr int kPCntStride = 32;           // words
constexpr size_t kPPartOffset = 192 * 1024;
static_assert(kPCntBase * 4 + (size_t)kPMaxGroups * kPW * kPSlots * kPCntStride * 4 <= 96 * 1024,
              "arrival counters overlap the split form's counters");
__host__ __device__ constexpr int persist_rec_floats(int pg) { return pg * (kPTW * kPLine + kPTW); }
inline size_t persist_ws_bytes(int pg) {
  return kPPartOffset + (size_t)kPMaxGroups * kPW * kPRing * persist_rec_floats(pg) * sizeof(float);
}

constexpr int kWaitVmem0 = 0x0f70;   // s_waitcnt vmcnt(0), expcnt and lgkmcnt unconstrained (gfx9 encoding)

// An opaque zero that the compiler cannot compute before `v` is in a register:
// whatever uses it waits for the load that produced `v`.
__device__ __forceinline__ unsigned zero_after(unsigned v) {
  unsigned z;
  __asm__ volatile("v_and_b32 %0, 0, %1" : "=v"(z) : "v"(v));
  return z;
}

// Gates and Sinkhorn of one token, in pieces.  The token's 25 summed values
// (P[24], sum x^2) sit in `v`; `ba` holds bias[24] then alpha[3] (both LDS).
// Each 16-lane DPP row of the wave holds the token's 4x4 comb matrix, lane
// 4i + j entry (i, j) (the four rows compute the same): row sums by quad
// butterflies, column sums by rotating the row by 8 and then by 4, so every
// lane of a row or column divides by the same bits.  Lanes 0-15 write comb,
// lanes 0-3 the pre and post gates (gate index j).
struct TokenGates {
  float m;
  float pr, po;
  int tok, it;
  bool write;

  // in three pieces (each a short dependent chain): logits, exponentials, gates
  __device__ __forceinline__ void init_a(const PreParams& p, const float* v, const float* ba, int t,
                                         bool w, int lane) {
    const int e = lane & 15;       // 4 i + j
    const int j = lane & 3;
    const float r = hw_rsqrt(v[24] * (1.0f / (float)p.K) + p.eps);
    m = ba[kNL + 2] * (r * v[8 + e]) + ba[8 + e];
    pr = ba[kNL] * (r * v[j]) + ba[j];          // the pre logit, until init_c
    po = ba[kNL + 1] * (r * v[4 + j]) + ba[4 + j];
    tok = t;
    it = 0;
    write = w;
  }
  __device__ __forceinline__ void init_b() {
    float mx = fmaxf(m, dpp_quad_xor1(m));
    mx = fmaxf(mx, dpp_quad_xor2(mx));
    m = hw_exp(m - mx);
  }
  __device__ __forceinline__ void init_c() {
    pr = hw_sigmoid(pr);
    po = 2.0f * hw_sigmoid(po);
  }
  // one Sinkhorn iteration (row normalisation, then column), if this wave holds a
  // gate token with iterations left
  __device__ __forceinline__ void step(int iters) {
    if (write && it < iters) {
      float rs = m + dpp_quad_xor1(m);
      rs = rs + dpp_quad_xor2(rs);
      m *= __builtin_amdgcn_rcpf(rs);
      float cs = m + dpp_row_ror8(m);
      cs = cs + dpp_row_ror4(cs);
      m *= __builtin_amdgcn_rcpf(cs);
      ++it;
    }
  }
  __device__ __forceinline__ void finish(const PreParams& p, int lane) {
    if (!write) return;
    while (it < p.iters) step(p.iters);
    if (lane < 16 && tok < p.T) {
      p.comb[(size_t)tok * 16 + lane] = m;
      if (lane < 4) {
        p.pre[(size_t)tok * kNS + lane] = pr;
        p.post[(size_t)tok * kNS + lane] = po;
      }
    }
    write = false;
  }
};

// kFused: the post stage of the previous seam in front (x_out written, the
// collapse and projection on it).  kGates: projection, exchange and gates only
// (no pre_in, collapse or layer_input): the first pass of the own-pre-mix form,
// whose collapse needs this seam's gates.
template <int kC, bool kFused, bool kGates = false>
__global__ __launch_bounds__(kPThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mhc_persist_kernel(PreParams p, int ngroups) {
  using G = PersistGeom<kC>;
  constexpr int kL = G::kLines;
  constexpr int kPG = G::kPG;
  constexpr int kRow = kNS * kC * 2;            // bytes of a residual row
  constexpr int kYRow = kC * 2;                 // bytes of a sublayer-output / layer_input row
  constexpr int kFrags = kL * kNS * kPQ;        // weight fragments of the member's slice
  constexpr int kRecF = persist_rec_floats(kPG);
  constexpr int kValF = kPTW * kPG * kPLine;    // floats of the value block
  constexpr int kSS = kNS * kL;                 // sub-steps (stream loads) per tile
  constexpr int kGL = (kPG + 7) / 8;            // 1 KB loads of a gate token's lines
  constexpr int kRaw = kFused ? 5 : kNS;        // raw loads per line: [stream 0..3, sublayer output]
  static_assert(kC == 64 * kL * kPG && kL >= 2 && kL <= 5, "geometry");
  static_assert(kPG <= kPMaxPG && kPG >= kPTW, "every token of a wave needs a gate member");
  static_assert(!(kFused && kGates), "the gates-only form has no post stage");
  static_assert((kFrags * kWave) % kPThreads == 0, "weight fragments split evenly over the threads");
  // exchange sub-steps (counted in stream loads, 4 per line).  In tile k, for
  // tile k - 1: the arrival, the counter read and, late, the check and the
  // record loads (every sub-step between the arrival and the check is slack for
  // members that run behind); the loads are summed at the start of tile k + 1,
  // so that the wait for them has several sub-steps of loads in flight in front
  // of it.  In tile k, for tile k - 2: its records summed (norm factors, gate
  // token's values), then its gate token's gates and Sinkhorn iterations.
  constexpr int kArrive = 2;                    // the fence load issued after the record stores is back
  constexpr bool kLate = G::kLateDelayed && !kFused && !kGates;
  constexpr int kCntRead = kSS - (kLate ? 6 : 7);
  constexpr int kCheck = kSS - (kLate ? 3 : 4);
  constexpr int kStage = 0;                     // tile k - 2's records summed, before its layer_input
  constexpr int kInit = 1;                      // its gate token: logits, exponentials, gates
  constexpr int kGateEnd = kSS - 2;             // its remaining iterations, written
  static_assert(kCntRead > kArrive + 2 && kCheck < kSS && kGateEnd > kInit + 1, "exchange schedule");

  __shared__ uint4 s_w[kFrags * kWave];         // [line][stream][fragment][lane]
  __shared__ uint4 s_nw[kL * 8];                // the member's columns of the norm weight
  __shared__ float s_red[kPW][kPTW][kPLine];    // per wave: a tile's partial sums, token rows
  __shared__ float s_g[kPW][kPTW][24];          // per wave: post[4], comb[16], pre_in[4] of its tokens
  __shared__ float s_gv[kPW][32];               // per wave: the gate token's summed values
  __shared__ float s_ry[kPW][kPTW];             // per wave: the tile's summed y^2 per token
  __shared__ float s_ba[32];                    // bias[24], alpha[3]

  const int tid = threadIdx.x;
  // lane, tok and chunk are made opaque again at every tile's start (see
  // tile_body), so that addresses derived from them are formed where they are
  // used instead of being hoisted out of the tile loop into registers of their own
  int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  int tok = lane & 7;                                // the lane's token of the wave's eight
  int chunk = ((lane >> 3) & 1) * 4 + (lane >> 4);   // its 16-byte chunk of a 128-byte line
  const int mem = blockIdx.x % kPG;
  const int grp = blockIdx.x / kPG;
  const int ntiles = (p.T + kPT - 1) / kPT;
  const int nk = (ntiles - 1 - grp) / ngroups + 1;   // tiles of this group (launch: ngroups <= ntiles)
  const int mcol = kL * 128 * mem;                   // byte offset of the member's first line in a row
  // The member's column offset is part of the lane offsets, and every buffer
  // access passes a literal zero as its scalar offset: the compiler inserts the
  // wait state a 16-byte store needs before its data registers are written again
  // only for stores without a scalar offset register, and on gfx950 a store with
  // one showed the hazard (a move into a store's first data register right after
  // it changed what the store wrote in lanes 12-15 of each 16).
  const int xlane = (wave * kPTW + tok) * kRow + chunk * 16 + mcol;
  int ylane = (wave * kPTW + tok) * kYRow + chunk * 16 + mcol;
  // lane offset of each stream (the line offset, at most 4 x 128 bytes, fits the
  // instructions' immediate field; opaque, so the compiler forms base + constant
  // at each access instead of keeping one register per (stream, line))
  int xls[kNS];
#pragma unroll
  for (int s = 0; s < kNS; ++s) xls[s] = xlane + s * kC * 2;
  __asm__ volatile("" : "+v"(xls[0]), "+v"(xls[1]), "+v"(xls[2]), "+v"(xls[3]), "+v"(ylane));
  const bool norm = p.nw != nullptr;

  auto tile_of = [&](int k) { return (k >= 0 && k < nk) ? grp + k * ngroups : -1; };
  auto tile_rows = [&](int t) { return t >= 0 ? min(kPT, p.T - t * kPT) : 0; };
  auto x_rsrc = [&](int t) { return make_rsrc(p.x + (size_t)max(t, 0) * kPT * (kNS * kC), tile_rows(t) * kRow); };
  auto y_rsrc = [&](int t) { return make_rsrc(p.ysub + (size_t)max(t, 0) * kPT * kC, tile_rows(t) * kYRow); };
  auto xo_rsrc = [&](int t) { return make_rsrc(p.xout + (size_t)max(t, 0) * kPT * (kNS * kC), tile_rows(t) * kRow); };
  auto li_rsrc = [&](int t) { return make_rsrc(p.li + (size_t)max(t, 0) * kPT * kC, tile_rows(t) * kYRow); };
  // the wave's eight tokens of tile t: rows of post_in / comb_in / pre_in
  auto wave_rows = [&](int t) { return t >= 0 ? max(0, min(kPTW, p.T - t * kPT - wave * kPTW)) : 0; };
  auto wtok0 = [&](int t) { return (size_t)max(t, 0) * kPT + wave * kPTW; };

  // ---- prologue: the weight slice's loads first (a wave's loads retire in
  // issue order, so weight loads behind the first residual loads would wait
  // for those), then the first residual loads, then the slice into LDS.  The
  // slice is gathered from the packed layout (32-row blocks, 16-column tiles)
  // into fragment order: fragment (line u, stream s, output group q) lane M
  // holds the 16-byte unit of k-block (s C + 64 (kL mem + u)) / 32 + half,
  // column tile j / 16, lane 16 (M >> 4) + (j & 15), with half = (M & 15) >> 3
  // and j = 8 q + (M & 7).
  constexpr int kPer = kFrags * kWave / kPThreads;
  uint4 fv[kPer];
  {
    const rsrc_t rf = make_rsrc(p.fnp, p.KB * kFragPerKB * kWave * 16);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int idx = tid + i * kPThreads;
      const int M = idx & (kWave - 1);
      const int f = idx / kWave;
      const int q = f % kPQ;
      const int us = f / kPQ;
      const int s = us % kNS, u = us / kNS;
      const int half = (M & 15) >> 3;
      const int j = 8 * q + (M & 7);
      const int kb = (s * kC + 64 * (kL * mem + u)) / kKB + half;
      fv[i] = buf_load16(rf, ((kb * kFragPerKB + (j >> 4)) * kWave + 16 * (M >> 4) + (j & 15)) * 16, 0);
    }
  }
  // raw loads of one line: streams 0..3, then (fused) the sublayer output
  uint4 ra[kRaw], rb[kRaw];
  auto issue_line = [&](uint4 (&r)[kRaw], rsrc_t rx, rsrc_t ryy, int u) {
#pragma unroll
    for (int s = 0; s < kNS; ++s) r[s] = buf_load16(rx, xls[s] + u * 128, 0);
    if constexpr (kFused) r[4] = buf_load16(ryy, ylane + u * 128, 0);
  };
  // the gates a tile needs for the wave's eight tokens, one 16-byte load per
  // lane: pre_in rows to lanes 0-7, (fused) post_in rows to lanes 8-15 and
  // comb_in rows to lanes 16-47.  Every lane loads (lanes without a row of
  // their own read row 0 of pre_in and drop it), so the load is not under a
  // branch and waiting for it does not wait for the loads issued after it.
  uint4 gq = make_uint4(0u, 0u, 0u, 0u);
  bool gq_ok = false;
  auto issue_gates = [&](int t) {
    if constexpr (kGates) return;   // no pre_in (the pointer is null), no post stage
    const int n = wave_rows(t);
    const size_t t0 = wtok0(t);
    const int r = kFused && lane >= 2 * kPTW ? (lane - 2 * kPTW) >> 2 : lane & (kPTW - 1);
    gq_ok = r < n && (lane < kPTW || (kFused && lane < 6 * kPTW));
    const size_t tk = gq_ok ? t0 + r : 0;
    const float* src = lane < kPTW || !kFused ? p.pre_in + tk * kNS
                       : lane < 2 * kPTW      ? p.post_in + tk * kNS
                                              : p.comb_in + tk * 16 + (gq_ok ? 4 * ((lane - 2 * kPTW) & 3) : 0);
    gq = *reinterpret_cast<const uint4*>(src);
  };
  // Non-fused forms: a ring of 8 single loads (two lines): each stream load is
  // refilled with the load two lines ahead as soon as its sub-step has used it.
  // Fused form: whole lines (ra, rb), since every raw input of a line feeds all
  // four output streams of its post stage.
  constexpr int kRing = 2 * kNS;
  uint4 xq[kRing];
  if constexpr (kFused) {
    issue_line(ra, x_rsrc(tile_of(0)), y_rsrc(tile_of(0)), 0);
  } else {
#pragma unroll
    for (int g = 0; g < kRing; ++g) {
      const int u = g / kNS;
      const int t = tile_of(u / kL);
      xq[g] = buf_load16(x_rsrc(t), xls[g % kNS] + (u % kL) * 128, 0);
    }
  }
  issue_gates(tile_of(0));
#pragma unroll
  for (int i = 0; i < kPer; ++i) s_w[tid + i * kPThreads] = fv[i];
  if (norm && tid < kL * 8) s_nw[tid] = reinterpret_cast<const uint4*>(p.nw)[(mcol >> 4) + tid];
  if (tid < kNL) s_ba[tid] = p.bias[tid];
  if (tid >= 32 && tid < 35) s_ba[kNL + tid - 32] = p.alpha[tid - 32];
  if (lane < kPTW) {
#pragma unroll
    for (int c = 26; c < kPLine; ++c) s_red[wave][lane][c] = 0.f;
  }
  __syncthreads();

  // ---- per-wave state
  // Counter, arrival target and record of the group's k-th tile.  "Tile -1"
  // (the exchange before the first tile) has a counter of its own that nobody
  // waits on, target 0 and records of zero bytes (stores dropped, loads zero),
  // so the first tiles run the same code as the others.
  unsigned* cnt_base = p.cnt + kPCntBase + (grp * kPW + wave) * kPSlots * kPCntStride;
  float* rec_base = p.part + (size_t)(grp * kPW + wave) * kPRing * kRecF;
  auto cnt_of = [&](int k) { return cnt_base + (k >= 0 ? k % kPRing : kPRing) * kPCntStride; };
  // (p.wait_bias, zero in a normal call, puts every target out of reach)
  auto target_of = [&](int k) {
    return (k >= 0 ? (unsigned)kPG * (unsigned)(k / kPRing + 1) : 0u) + p.wait_bias;
  };
  auto rec_of = [&](int k) { return rec_base + (size_t)(k >= 0 ? k % kPRing : 0) * kRecF; };
  auto rec_bytes = [&](int k, int bytes) { return k >= 0 ? bytes : 0; };

  f32x4 acc[kPA], as;
#pragma unroll
  for (int q = 0; q < kPA; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  as = f32x4{0.f, 0.f, 0.f, 0.f};
  float ssy = 0.f;
  float gv[24];          // the lane token's post[4], comb[16] and pre_in[4] for the current tile
  float ybA[kL][8], ybB[kL][8];   // collapsed rows: tiles of even / odd index in the group
  float ryA = 1.f, ryB = 1.f;     // their norm factors, once known
  uint4 pssy = make_uint4(0u, 0u, 0u, 0u);   // tile k - 1's sum-y^2 block, in flight
  uint4 pg[4] = {};                          // the gate token's lines, in flight
  unsigned cv = 0;
  TokenGates gt;
  gt.m = 1.0f;
  gt.pr = gt.po = 0.0f;
  gt.tok = -1;
  gt.write = false;
  gt.it = 0;
  int budget = p.wait_budget;
  // weight fragments: two LDS bases, every access within the 16-bit immediate
  // offset of ds_read from one of them (the slice is up to 120 KB)
  constexpr int kHalfF = kFrags / 2;
  int fb0 = lane, fb1 = lane + kHalfF * kWave;
  __asm__ volatile("" : "+v"(fb0), "+v"(fb1));
  auto frag = [&](int fi) -> uint4 {
    return fi < kHalfF ? s_w[fb0 + fi * kWave] : s_w[fb1 + (fi - kHalfF) * kWave];
  };
  // the first two fragments of the coming sub-step, read during the one before
  uint4 fpre[2] = {frag(0), frag(1)};

  // the gates of a tile: loaded registers -> this wave's LDS rows (at the tile's
  // start), then the lane token's row into registers at each line's start
  auto stage_gates = [&]() {
    if constexpr (!kGates) {
      float* row = nullptr;
      if (lane < kPTW)
        row = &s_g[wave][lane][20];
      else if (kFused && lane < 2 * kPTW)
        row = &s_g[wave][lane - kPTW][0];
      else if (kFused && lane < 6 * kPTW)
        row = &s_g[wave][(lane - 2 * kPTW) >> 2][4 + 4 * ((lane - 2 * kPTW) & 3)];
      if (row) *reinterpret_cast<uint4*>(row) = gq_ok ? gq : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  stage_gates();   // tile 0's gates

  auto read_pre = [&]() {
    const float4 v = *reinterpret_cast<const float4*>(&s_g[wave][tok][20]);
    gv[20] = v.x;
    gv[21] = v.y;
    gv[22] = v.z;
    gv[23] = v.w;
  };

  // v of lane (lane ^ m): the lane index is the per-tile opaque one, so the
  // partner addresses are formed at the exchange instead of held across the loop
  auto xshfl = [&](float v, int m) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ m) << 2, __builtin_bit_cast(int, v)));
  };

  auto wait_count = [&](const unsigned* c, unsigned target, unsigned v) {
    while ((int)(v - target) < 0 && budget > 0) {
      --budget;
      __builtin_amdgcn_s_sleep(2);
      v = ld_agent(c);
    }
    if ((int)(v - target) < 0 && lane == 0)
      __hip_atomic_store(p.cnt + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // every load of this wave is complete when the loop ends, so the straight
    // path's wait counts stay valid after it
    __builtin_amdgcn_s_waitcnt(kWaitVmem0);
  };

  // tile kk's partial sums: accumulators -> token rows of this wave's LDS
  // (the two half-lines of lanes L and L ^ 40 added)
  auto publish_a = [&]() {
    float tot[kPA][4];
#pragma unroll
    for (int q = 0; q < kPA; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) tot[q][i] = acc[q][i] + xshfl(acc[q][i], 40);
    float sx = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if ((lane & 15) == 4 * (lane >> 4) + i) sx = as[i];
    sx += xshfl(sx, 40);
    float sy = ssy + xshfl(ssy, 8);
    sy += xshfl(sy, 16);
    sy += xshfl(sy, 32);
    float (*red)[kPLine] = s_red[wave];
    if ((lane & 8) == 0 && lane < 24) {
      const int t0 = 4 * (lane >> 4), c = lane & 7;
#pragma unroll
      for (int q = 0; q < kPA; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[t0 + i][8 * q + c] = tot[q][i];
    }
    if (lane < 4) red[lane][24] = sx;
    if (lane >= 20 && lane < 24) red[lane - 16][24] = sx;
    if (lane < kPTW) red[lane][25] = sy;
  };
  // ... and -> the record of the group's kk-th tile: one whole-line store of the
  // value block (lane L: token L >> 3, floats 4 (L & 7) ..), 32 bytes of sum y^2
  auto publish_b = [&](int kk) {
    const float (*red)[kPLine] = s_red[wave];
    const rsrc_t rr = make_rsrc(rec_of(kk), rec_bytes(kk, kRecF * 4));
    const int t = lane >> 3, c = 4 * (lane & 7);
    const float4 v = *reinterpret_cast<const float4*>(&red[t][c]);
    buf_store16_agent(__builtin_bit_cast(uint4, v), rr, ((t * kPG + mem) * kPLine + c) * 4, 0);
    if (lane < 2)
      buf_store16_agent(make_uint4(__float_as_uint(red[4 * lane][25]), __float_as_uint(red[4 * lane + 1][25]),
                                   __float_as_uint(red[4 * lane + 2][25]), __float_as_uint(red[4 * lane + 3][25])),
                        rr, (kValF + mem * kPTW + 4 * lane) * 4, 0);
  };
  // The gate token of tile kk this member takes: members 0-7 take the wave's
  // tokens 0-7 of even tiles, members 8-15 those of odd tiles (out of [0, 8):
  // none), so that the Sinkhorn work alternates between the two halves.
  auto gate_tok = [&](int kk) { return mem - kPTW * (kk & 1); };
  // the group's records of tile kk: the sum-y^2 block (every member), the gate
  // token's lines (its gate member)
  auto load_records = [&](int kk) {
    const float* rec = rec_of(kk);
    pssy = buf_load16_agent(make_rsrc(rec + kValF, rec_bytes(kk, kPG * kPTW * 4)), lane * 16, 0);
    const int gk = gate_tok(kk);
    const rsrc_t rg = make_rsrc(rec + (size_t)min(max(gk, 0), kPTW - 1) * kPG * kPLine,
                                gk >= 0 && gk < kPTW ? rec_bytes(kk, kPG * kPLine * 4) : 0);
#pragma unroll
    for (int n = 0; n < kGL; ++n) pg[n] = buf_load16_agent(rg, n * 1024 + lane * 16, 0);
  };
  // ... summed: norm factor of the lane's token (-> ry), the gate token's values
  // (-> s_gv); every member adds in the same order, so all hold the same bits
  auto sum_records = [&](float& ry) {
    float a[4] = {__uint_as_float(pssy.x), __uint_as_float(pssy.y), __uint_as_float(pssy.z),
                  __uint_as_float(pssy.w)};
#pragma unroll
    for (int m = 2; m < kWave; m <<= 1)
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] += xshfl(a[e], m);
    if (lane < 2) *reinterpret_cast<float4*>(&s_ry[wave][4 * lane]) = make_float4(a[0], a[1], a[2], a[3]);
    float g[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < kGL; ++n) {
      g[0] += __uint_as_float(pg[n].x);
      g[1] += __uint_as_float(pg[n].y);
      g[2] += __uint_as_float(pg[n].z);
      g[3] += __uint_as_float(pg[n].w);
    }
#pragma unroll
    for (int m = 8; m < kWave; m <<= 1)
#pragma unroll
      for (int e = 0; e < 4; ++e) g[e] += xshfl(g[e], m);
    if (lane < 8) *reinterpret_cast<float4*>(&s_gv[wave][4 * lane]) = make_float4(g[0], g[1], g[2], g[3]);
    const float sy = s_ry[wave][tok];
    ry = norm ? hw_rsqrt(sy * (1.0f / (float)kC) + p.eps) : 1.0f;
  };
  // one line of layer_input from a row buffer (non-temporal, as the next residual:
  // 3% off the delayed pre and 1% off the fused seam at T = 16384, C = 5120; the
  // residual streamed through the same call evicts them from the memory-side cache
  // before anything reads them back)
  auto li_store = [&](const float (&yb)[8], float ry, rsrc_t rl, int u) {
    float o[8];
    if (norm) {
      float w[8];
      unpack8(s_nw[u * 8 + chunk], w);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (yb[e] * ry) * w[e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = yb[e];
    }
    buf_store16_nt(pack8(o), rl, ylane + u * 128, 0);
  };

  // One tile: the sweep of the group's k-th tile into yb (which held tile k - 2:
  // its norm factor into ry at the start, then its layer_input leaves line by
  // line just before the line is overwritten), and the exchange of tile k - 1.
  // P: the tile's parity (which raw-load buffer each line uses).
  auto tile_body = [&](auto par, int k, float (&yb)[kL][8], float& ry) __attribute__((always_inline)) {
#pragma clang fp contract(off)
    constexpr int P = decltype(par)::value;
    // re-define the base offsets and lane indices in every tile (see xls, fb0, fb1, lane)
    __asm__ volatile("" : "+v"(xls[0]), "+v"(xls[1]), "+v"(xls[2]), "+v"(xls[3]), "+v"(ylane), "+v"(fb0),
                     "+v"(fb1));
    __asm__ volatile("" : "+v"(lane), "+v"(tok), "+v"(chunk));
    const int t = tile_of(k);
    const int tn = tile_of(k + 1);
    const rsrc_t rx = x_rsrc(t), ryy = y_rsrc(t);
    const rsrc_t rxn = x_rsrc(tn), ryn = y_rsrc(tn);
    const rsrc_t rxo = xo_rsrc(t);
    const rsrc_t rl2 = li_rsrc(tile_of(k - 2));   // zero bytes for k < 2: stores dropped
    const int tq = tile_of(k - 2);                   // -1 for k < 2
    // fused form: the two waves of a SIMD take turns at the higher issue priority,
    // tile by tile (left alone, the older wave of each SIMD runs ~20% ahead and the
    // other finishes the call alone; 1.5% at T = 16384, C = 5120; the delayed form
    // measured 1% slower with it)
    if constexpr (kFused) {
      if (((k + (wave >> 2)) & 1) != 0)
        __builtin_amdgcn_s_setprio(1);
      else
        __builtin_amdgcn_s_setprio(0);
    }
    // ---- exchange of tile k - 1: partial sums out, before the next line's loads
    publish_a();
#pragma unroll
    for (int q = 0; q < kPA; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    as = f32x4{0.f, 0.f, 0.f, 0.f};
    ssy = 0.f;
    publish_b(k - 1);
    // a load issued after the record stores: once it is back, they are complete
    // (a wave's vector memory operations complete in issue order)
    __asm__ volatile("" ::: "memory");
    const unsigned fence = ld_agent(cnt_of(k - 1));
    static_for<kL>([&](auto uc) __attribute__((always_inline)) {
#pragma clang fp contract(off)
      constexpr int u = decltype(uc)::value;
      constexpr bool cur_a = ((P * kL + u) & 1) == 0;
      uint4 (&rc)[kRaw] = pick<cur_a>(ra, rb);
      uint4 (&rn)[kRaw] = pick<!cur_a>(ra, rb);
      // refill: the next line of this tile, or the next tile's first line; the
      // next tile's gates a line earlier and ahead of that line's loads, so that
      // staging them at the tile's start does not wait for the line queue
      auto refill = [&]() {
        if constexpr (u + 1 < kL)
          issue_line(rn, rx, ryy, u + 1);
        else
          issue_line(rn, rxn, ryn, 0);
      };
      // the next tile's gates, a line and a half ahead of their staging
      if constexpr (u + 2 == kL) issue_gates(tn);
      if constexpr (!kGates) read_pre();
      // the line's four streams as the projection and collapse see them: the raw
      // residual, or (fused) the post stage's next residual, stream by stream
      // with that stream's gates read from LDS
      // (fused: each output stream of the post stage at its own sub-step, from
      // opaque copies of the packed inputs -- sharing their unpacking across the
      // sub-steps would keep forty unpacked values live -- and the next line's
      // loads at sub-step kRefill of the line (the second or third), into the
      // buffer the previous line freed: at C = 5120 the third gives two sub-steps
      // more lead than the last, 1% faster at T = 16384, and any earlier runs out
      // of registers)
      static_for<kNS>([&](auto sc) __attribute__((always_inline)) {
#pragma clang fp contract(off)
        constexpr int s = decltype(sc)::value;
        constexpr int ss = kNS * u + s;
        // keep each sub-step's weight reads, matrix instructions and collapse
        // together (hoisting a whole line's fragment reads would spill)
        __builtin_amdgcn_sched_barrier(0);
        // tile k - 2's records (loaded during tile k - 1): its norm factor, first
        // needed just below, and its gate token's values
        if constexpr (ss == kStage) sum_records(ry);
        // Sinkhorn of tile k - 2's gate token: one iteration per sub-step
        if constexpr (ss > kInit && ss < kGateEnd) gt.step(p.iters);
        if constexpr (ss == kGateEnd) gt.finish(p, lane);
        // tile k - 2's layer_input for this line, before the line's first write
        if constexpr (!kGates && s == 0) li_store(yb[u], ry, rl2, u);
        uint4 xv;
        if constexpr (kFused) {
          uint4 in[5] = {rc[4], rc[0], rc[1], rc[2], rc[3]};
#pragma unroll
          for (int k = 0; k < 5; ++k) __asm__ volatile("" : "+v"(in[k].x), "+v"(in[k].y), "+v"(in[k].z), "+v"(in[k].w));
          const float pw = s_g[wave][tok][s];
          const float4 c = *reinterpret_cast<const float4*>(&s_g[wave][tok][4 + 4 * s]);
          xv = post_packed8(pw, c.x, c.y, c.z, c.w, in[0], in[1], in[2], in[3], in[4]);
          if constexpr (s == G::kRefill) refill();
          buf_store16_nt(xv, rxo, xls[s] + u * 128, 0);
        } else {
          xv = xq[(kNS * (P * kL + u) + s) % kRing];
        }
        // weight fragments two at a time (all six would take 24 registers); the
        // first two of each sub-step were read during the one before
        constexpr int fi = (u * kNS + s) * kPQ;
        constexpr int fn = ((u * kNS + s + 1) % kSS) * kPQ;   // the next sub-step's (this tile's or the next)
        acc[0] = mfma_bf16(xv, fpre[0], acc[0]);
        acc[1] = mfma_bf16(xv, fpre[1], acc[1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 2; q < kPQ; ++q) {
          acc[q % kPA] = mfma_bf16(xv, frag(fi + q), acc[q % kPA]);
          if (q % 2 == 1) __builtin_amdgcn_sched_barrier(0);
        }
        as = mfma_bf16(xv, xv, as);
        fpre[0] = frag(fn);
        fpre[1] = frag(fn + 1);
        if constexpr (!kGates) {
          float f[8];
          unpack8(xv, f);
          const float ps = gv[20 + s];
#pragma unroll
          for (int e = 0; e < 8; ++e) yb[u][e] = s == 0 ? ps * f[e] : yb[u][e] + ps * f[e];
          if constexpr (s == kNS - 1) {
#pragma unroll
            for (int e = 0; e < 8; ++e) ssy = __builtin_fmaf(yb[u][e], yb[u][e], ssy);
          }
        }
        // non-fused: this load is used up; its slot takes the load two lines ahead
        if constexpr (!kFused) {
          constexpr int g = kNS * (P * kL + u) + s;
          constexpr int un = u + 2;   // line of the refill, counted from this tile's first
          const rsrc_t rr = un < kL ? rx : rxn;
          xq[g % kRing] = buf_load16(rr, xls[s] + (un % kL) * 128, 0);
        }
        // ---- exchange of tile k - 1, continued
        if constexpr (ss == kArrive) {
          // the first load issued after the record stores has returned
          const unsigned z = zero_after(fence);
          if (lane == 0) __hip_atomic_fetch_add(cnt_of(k - 1), 1u + z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if constexpr (ss == kCntRead) {
          cv = ld_agent(cnt_of(k - 1));
          __asm__ volatile("" ::: "memory");   // keep the read here, ahead of its use
        }
        if constexpr (ss == kCheck) {
          cv += zero_after(kFused ? rc[1].y : xv.y);   // the check cannot move above this sub-step
          const unsigned tg = target_of(k - 1);
          if ((int)(cv - tg) < 0) wait_count(cnt_of(k - 1), tg, cv);
          load_records(k - 1);
          __asm__ volatile("" ::: "memory");
        }
        if constexpr (ss == kInit) {
          gt.init_a(p, s_gv[wave], s_ba, tq * kPT + wave * kPTW + gate_tok(k - 2),
                    tq >= 0 && gate_tok(k - 2) >= 0 && gate_tok(k - 2) < kPTW, lane);
          gt.init_b();
          gt.init_c();
        }
      });
    });
    // the next tile's gates (loaded a line and a half ago) into LDS, now that
    // this tile's are no longer read; in the same loop iteration as their load,
    // so waiting for them does not wait for the loads issued after them
    stage_gates();
  };

  // After the last tile kl: its partial sums out; tile kl - 1's records (loaded
  // during tile kl): norm factor, gates and layer_input; then tile kl's
  // exchange, gates and layer_input.
  auto drain = [&](int kl, float (&ylast)[kL][8], float (&yprev)[kL][8], float& ry_prev, float& ry_last) {
    publish_a();
    publish_b(kl);
    wait_vmem();   // tile kl's records are stored, tile kl - 1's are loaded
    if (lane == 0) __hip_atomic_fetch_add(cnt_of(kl), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sum_records(ry_prev);
    const int tq = tile_of(kl - 1);
    gt.init_a(p, s_gv[wave], s_ba, tq * kPT + wave * kPTW + gate_tok(kl - 1),
              tq >= 0 && gate_tok(kl - 1) >= 0 && gate_tok(kl - 1) < kPTW, lane);
    gt.init_b();
    gt.init_c();
    gt.finish(p, lane);
    if (!kGates && kl >= 1) {
      const rsrc_t rl = li_rsrc(tq);
#pragma unroll
      for (int u = 0; u < kL; ++u) li_store(yprev[u], ry_prev, rl, u);
    }
    const unsigned v = ld_agent(cnt_of(kl));
    if ((int)(v - target_of(kl)) < 0) wait_count(cnt_of(kl), target_of(kl), v);
    load_records(kl);
    wait_vmem();
    sum_records(ry_last);
    const int tl = tile_of(kl);
    gt.init_a(p, s_gv[wave], s_ba, tl * kPT + wave * kPTW + gate_tok(kl), gate_tok(kl) >= 0 && gate_tok(kl) < kPTW,
              lane);
    gt.init_b();
    gt.init_c();
    gt.finish(p, lane);
    if (!kGates) {
      const rsrc_t rl = li_rsrc(tl);
#pragma unroll
      for (int u = 0; u < kL; ++u) li_store(ylast[u], ry_last, rl, u);
    }
  };

  // two tile bodies (the row buffers alternate; each body's code stays small
  // enough for the instruction cache)
  for (int k = 0; k < nk; k += 2) {
    tile_body(std::integral_constant<int, 0>(), k, ybA, ryA);
    if (k + 1 < nk) tile_body(std::integral_constant<int, 1>(), k + 1, ybB, ryB);
  }
  if ((nk - 1) % 2 == 0)
    drain(nk - 1, ybA, ybB, ryB, ryA);
  else
    drain(nk - 1, ybB, ybA, ryA, ryB);

  // ---- the last wave of the grid to finish resets the counters
  wait_vmem();
  unsigned old = 0;
  if (lane == 0) old = __hip_atomic_fetch_add(p.cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __shfl(old, 0);
  if (old == gridDim.x * kPW - 1) {
    const int ncnt = ngroups * kPW * kPSlots;
    for (int c = lane; c < ncnt; c += kWave)
      __hip_atomic_store(p.cnt + kPCntBase + c * kPCntStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (lane == 0) __hip_atomic_store(p.cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace mhc
