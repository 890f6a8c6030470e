// vmscan: fused bidirectional selective scan (Vision Mamba) and SS2D cross-scan (VMamba) for
// MI355X / gfx950, behind the C ABI declared in include/vmscan.h.
//
// What is computed is stated in that header with the page citations; this file holds the
// kernels and the host-side validation and dispatch.
//
// Design (gfx950: wave64, 4 SIMDs and 160 KB LDS per CU; fp32 VALU with a transcendental rate
// of about a third of the FMA rate, so this path is bound by VALU issue, not by HBM; no dense
// contraction, so no MFMA):
//  * One wave issues at most about one VALU instruction every 8 cycles, so a SIMD needs three
//    or more resident waves to keep its VALU busy.  A workgroup is therefore four wavefronts
//    over the same 64 channels (lane = channel) of one batch row: waves 0 and 2 run the forward
//    direction, waves 1 and 3 the backward direction, and waves 0/1 keep states 0-7 of every
//    channel, waves 2/3 states 8-15, in VGPRs.  At the Vim-Ti shape this is 3072 waves, three
//    per SIMD.  Per state and token the VALU work is exp2(Δ2·A), h·a, h + (Δ2·u)·B' and
//    y + C·h, with Δ carried in base-2 units (Δ2 = Δ·log2 e) and B' = B·ln 2 stored in the B/C
//    copy, so that neither factor costs an instruction in the loop.
//  * B and C are the same for every channel of a batch row, so each wave reads its 8 B and 8 C
//    values per token as wave-uniform scalars (one s_load_dwordx16) from an fp32
//    [batch][direction][part][position][16] copy that a small transpose kernel writes first.
//    No VALU instruction is spent on B/C.
//  * u, Δ_raw (and z) are read per lane in windows of 8 consecutive tokens (16-byte loads;
//    the hardware accepts the 2-byte-aligned rows of odd-length bf16 sequences), one window
//    ahead of use.  Δ2 = log2(1 + 2^t), t = (Δ_raw + bias)·log2 e, is computed as
//    max(t, 0) + log2(1 + e), e = 2^-|t|, with a compensated log1p: log2(1 + e) = log2(s) +
//    (e - (s - 1))·log2 e, s = 1 + e.
//  * All four waves advance in lockstep: at step i the forward waves are at chunk position i,
//    the backward waves at Kc-1-i.  The channel's y at a position is the sum of four partial
//    readouts (two directions x two state halves).  They meet in one fp32 LDS row per channel in
//    a fixed order, so the result is deterministic: per window the lower-half wave of a direction
//    stores (first half of the steps) or adds (second half) its partial y, including the D·u
//    term, and publishes the window in an LDS counter; the upper-half wave waits for that count
//    and adds its own.  A workgroup barrier separates the halves of the chunk, and a cooperative
//    epilogue then applies the gate once, rounds once, and writes 16-byte stores.  No reversed
//    copy of any tensor is made.
//  * Sequences longer than one LDS row are split into chunks.  A first kernel computes each
//    chunk's end state from a zero start and its Σ Δ2; a small prefix kernel walks the chunks in
//    scan order and turns these into the state entering each chunk (exp2(A Σ Δ2) being a
//    chunk's total decay); the main kernel starts each chunk from that state, so the carry
//    crosses workgroups without re-running the recurrence.
//  * SS2D runs as two such bidirectional pairs, both over contiguous rows: the column pair
//    (column-major and its reverse) scans a transposed copy of x and writes an fp32 image in
//    column-major order; that image is transposed, and the row pair (row-major and its reverse)
//    adds it in its epilogue and stores.  Tiled transposes keep every access contiguous.
//  * Workgroup ids are remapped so that the workgroups one XCD receives (the hardware deals
//    them round-robin over 8 XCDs) are consecutive tiles of the same batch row, which then
//    share their B/C reads in that XCD's L2.
//  * d_state 32 keeps 8 states per wave: four state parts per direction, eight waves per
//    workgroup, whose partial readouts meet in the LDS row in part order (each part waits for the
//    one below it).
//  * The backward pass (gradients of every input) recomputes the forward: a checkpoint pass
//    stores each direction's state every 8 steps, then the adjoint walk goes back window by
//    window, rebuilding a window's states from its checkpoint.  Long sequences with few
//    workgroups are split into chunks; the adjoint carry between chunks comes from per-chunk
//    records and the same carry prefix run against the scan order.  Its state parts are
//    independent, so its workgroups stay at four waves; d_state 32 runs two per tile.
//  * The front convolutions that produce the scan input (Vim: causal conv1d + SiLU for both
//    branches; SS2D: 3 x 3 conv2d + SiLU written row-major and transposed) are streaming kernels.

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "vmscan.h"

namespace {

constexpr int kN = 16;                 // the smaller d_state (four-wave forward workgroup); 32 also taken
constexpr int kH = 8;                  // states per wave: d_state / 8 waves (parts) per (channel, direction)
constexpr int kW = 64;                 // channels per workgroup = lanes per wave
constexpr int kThreads = 4 * kW;       // d_state 16 workgroup: (fwd, lo) (bwd, lo) (fwd, hi) (bwd, hi)
constexpr int kWin = 8;                // tokens per register window
constexpr int kBC = 2 * kH;            // floats per (position, state part) in the B/C copy: 8 B, 8 C
constexpr int kKMax = 206;             // longest LDS row: 3 workgroups of 64 x 207 floats per CU
constexpr int kMinChunk = 32;          // shortest chunk the planner picks
constexpr int kTargetBlocks = 768;     // planner: three workgroups on each of 256 CUs
constexpr int kKSplit = 158;           // split sequences: chunks of <= 158 positions (LDS rows of 159), four workgroups per CU
constexpr int kSplitSlots = 1024;      // ... so a round is four workgroups on each of 256 CUs
constexpr int kTransThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

thread_local int g_last_hip_error = 0;

typedef __attribute__((address_space(4))) const float* scalar_fp;  // read-only: uniform loads -> s_load

// ---------------------------------------------------------------------------------------------
// device helpers

__device__ __forceinline__ float ld_act(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld_act(const uint16_t* p, int64_t i) {
  return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}

// Round to bfloat16, nearest-even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const __bf16 v = static_cast<__bf16>(f);
  uint16_t r;
  __builtin_memcpy(&r, &v, sizeof(r));
  return r;
}
__device__ __forceinline__ void st_act(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void st_act(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16_rne(v); }

// Eight consecutive elements (any element alignment), kept as loaded until unpacked so that a
// prefetch is not waited for before its values are used.
template <typename T>
struct Run8;
template <>
struct Run8<uint16_t> {
  uint4 r;
  __device__ __forceinline__ void load(const uint16_t* p) { __builtin_memcpy(&r, p, sizeof(r)); }
  // elements 0 .. n - 1 only (n may be <= 0); the others read as zero
  __device__ __forceinline__ void load_part(const uint16_t* p, int n) {
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = 2 * q < n ? p[2 * q] : 0u, hi = 2 * q + 1 < n ? p[2 * q + 1] : 0u;
      w[q] = lo | (hi << 16);
    }
    r = make_uint4(w[0], w[1], w[2], w[3]);
  }
  template <bool REV>
  __device__ __forceinline__ void unpack(float (&v)[kWin]) const {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[REV ? kWin - 1 - 2 * k : 2 * k] = __uint_as_float(w[k] << 16);
      v[REV ? kWin - 2 - 2 * k : 2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
  }
};
template <>
struct Run8<float> {
  float4 r0, r1;
  __device__ __forceinline__ void load(const float* p) {
    __builtin_memcpy(&r0, p, sizeof(r0));
    __builtin_memcpy(&r1, p + 4, sizeof(r1));
  }
  __device__ __forceinline__ void load_part(const float* p, int n) {
    float t[kWin];
#pragma unroll
    for (int j = 0; j < kWin; ++j) t[j] = j < n ? p[j] : 0.0f;
    r0 = make_float4(t[0], t[1], t[2], t[3]);
    r1 = make_float4(t[4], t[5], t[6], t[7]);
  }
  template <bool REV>
  __device__ __forceinline__ void unpack(float (&v)[kWin]) const {
    const float t[kWin] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
#pragma unroll
    for (int j = 0; j < kWin; ++j) v[j] = t[REV ? kWin - 1 - j : j];
  }
};

// The kernels carry Δ in base-2 units, Δ2 = Δ log2 e: then the decay is exp2(Δ2 A) with the
// natural A = -exp(A_log), Δ u B = Δ2 u (B ln 2) with B pre-scaled in the B/C copy, and the
// softplus argument x log2 e is one FMA of the raw input with the scaled bias.
//
// softplus in base-2 units: given t = x log2 e, returns log2(1 + 2^t) = softplus(x) log2 e,
// evaluated as max(t, 0) + log2(1 + e) with e = 2^-|t| <= 1.  With s = fl(1 + e) in [1, 2],
// c = e - (s - 1) is exactly the rounding error of s, and log2(1 + e) = log2(s) + log2(1 + c/s)
// ~= log2(s) + c log2 e, off by at most |c| (1 - 1/s) log2 e < 2^-24: full fp32 relative
// accuracy both for the e ~ 1e-3 that the Δ bias range produces (where a plain log2(1 + e) loses
// about three digits) and for every large t, with no threshold branch.  (Applying the
// correction to 1 + 2^t itself would be wrong for t > 24: there c is the rounding error of a
// number above 2^24, up to 1, not a small fraction of s.)
__device__ __forceinline__ float softplus2(float t) {
  const float e = __builtin_amdgcn_exp2f(-__builtin_fabsf(t));
  const float s = 1.0f + e;
  const float c = e - (s - 1.0f);
  return __builtin_fmaxf(t, 0.0f) + __builtin_fmaf(c, kLog2e, __builtin_amdgcn_logf(s));
}

// softplus2(t) and, from the same e = 2^-|t|, sigmoid(x) (the derivative of softplus):
// 1 / (1 + e) for x >= 0, e / (1 + e) for x < 0.
__device__ __forceinline__ float softplus2_sig(float t, float& sig) {
  const float e = __builtin_amdgcn_exp2f(-__builtin_fabsf(t));
  const float s = 1.0f + e;
  const float c = e - (s - 1.0f);
  const float q = __builtin_amdgcn_rcpf(s);
  sig = t >= 0.0f ? q : e * q;
  return __builtin_fmaxf(t, 0.0f) + __builtin_fmaf(c, kLog2e, __builtin_amdgcn_logf(s));
}

// Base-2 softplus argument from the raw Δ input and the bias already multiplied by log2 e.
__device__ __forceinline__ float delta2(float raw, float bias2) {
  return softplus2(__builtin_fmaf(raw, kLog2e, bias2));
}

__device__ __forceinline__ float silu_f(float v) {
  return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-v * kLog2e));
}

// Hardware dispatch deals workgroup i to XCD i % 8.  Return the logical tile id so that the
// tiles one XCD runs are contiguous in logical order.
__device__ __forceinline__ int logical_block(int bid, int nblocks) {
  const int xcd = bid & 7, local = bid >> 3;
  const int q = nblocks >> 3, r = nblocks & 7;
  return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

// The SIMD issue arbiter favours the oldest wave, so of the scan workgroups sharing a CU the first
// would finish well before the last, which then runs alone at a fraction of the issue rate (the
// Vim-Ti grid is a single round of three workgroups per CU).  Rotating the waves' priority every
// window across workgroups makes them progress evenly and finish together.  `step` counts
// windows; co-resident workgroups differ in blockIdx / 256.  (The chunk-state pass runs many
// rounds of workgroups and is faster with the default order.)
__device__ __forceinline__ void rotate_priority(int step) {
  const int pr = (static_cast<int>(blockIdx.x >> 8) + step) % 3;
  if (pr == 0) __builtin_amdgcn_s_setprio(0);
  else if (pr == 1) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(2);
}

struct DirArgs {
  const void* u;       // scan input, [batch][dim][L] in position order (batch stride u_bs)
  const void* draw;    // Δ_raw; element (b, d, idx) at b*draw_bs + d*L + idx
  int64_t draw_bs;
  const void* B;       // (b, n, idx) at b*bc_bs + n*L + idx
  const void* C;
  int64_t bc_bs;
  const float* A_log;  // [dim][16]
  const float* Dp;     // [dim]
  const float* bias;   // [dim]
  int rev;             // 1: this direction's Δ_raw/B/C are stored in reversed position order
};

struct ScanArgs {
  int64_t u_bs;    // batch stride of u, z, out, wsy
  const void* z;   // gate, same layout as u, or null
  void* out;
  float* wsy;      // fp32 image of the first SS2D pair
  float* bct;      // [batch][2][parts][L][kBC] fp32 B/C copy in position order
  float* agg;      // [batch][dim][2][nch][ns + 1]
  DirArgs d0, d1;  // forward and backward direction of the pair
  int64_t L;
  int dim, batch, K, nch, ngroups;
  int ns, parts;   // d_state and its parts of 8 states (one wave per direction and part)
  float* ck;       // kModeVimSum of an unsplit sequence, or null: the state entering each window of
  int ck_wpc;      // the two-phase walk, [batch][dir][part][ck_wpc][dim][8] (the backward checkpoints)
  // kModeVimSum: the gate's backward in the epilogue, from the un-gated sum y_f + y_b and
  // dout (same layout as u): gout = dout silu(z) / 2 (float32), dzout = dout (y_f + y_b) silu'(z) / 2.
  const void* dout;
  float* gout;
  void* dzout;
  // The call's wait status word (the first word of the workspace): set to 1 by a wave whose bounded
  // wait for another state part gave up; cleared by the call's first B/C copy (werr_clear).
  int* werr;
  int werr_clear;
  int lane_path;   // kModeVim: run lane_scan_kernel instead of the chunked pair kernels
};

// kModeVimSum: Vim order, but the epilogue turns the un-gated sum y_f + y_b into the gate's
// backward (g and dz, see ScanArgs::dout);
// kModeSecondPairSum: the SS2D row pair, storing the un-gated fp32 sum of all four directions to
// out (as float).  The backward passes need these sums for dL/dz.
enum { kModeVim = 0, kModeFirstPair = 1, kModeSecondPair = 2, kModeVimSum = 3, kModeSecondPairSum = 4 };

// ---------------------------------------------------------------------------------------------
// B/C transpose: for state part q, bct[b][dir][q][s][0..7] = B_dir[b][8q + 0..7, si(s)] ln 2 and
// bct[b][dir][q][s][8..15] = C_dir[b][8q + 0..7, si(s)].

template <typename T, int KH = kH>
__global__ __launch_bounds__(kTransThreads) void bc_transpose_kernel(ScanArgs a) {
  const int64_t ntile = (a.L + kTransThreads - 1) / kTransThreads;
  const int64_t blk = blockIdx.x;
  const int64_t tile = blk % ntile;
  const int dir = static_cast<int>((blk / ntile) & 1);
  const int b = static_cast<int>(blk / (2 * ntile));
  const int64_t s = tile * kTransThreads + threadIdx.x;
  if (a.werr_clear && blk == 0 && threadIdx.x == 0) *a.werr = 0;  // the call's first kernel with the word
  if (s >= a.L) return;
  const DirArgs& da = dir == 0 ? a.d0 : a.d1;
  const int64_t si = da.rev ? a.L - 1 - s : s;
  const T* bb = static_cast<const T*>(da.B) + static_cast<int64_t>(b) * da.bc_bs + si;
  const T* cb = static_cast<const T*>(da.C) + static_cast<int64_t>(b) * da.bc_bs + si;
  constexpr int NB = 2 * KH;
  for (int q = 0; q < a.parts; ++q) {
    float v[NB];
#pragma unroll
    for (int k = 0; k < KH; ++k) {
      v[k] = ld_act(bb, static_cast<int64_t>(KH * q + k) * a.L) * kLn2;  // B ln 2: Δ2 u (B ln 2) = Δ u B
      v[KH + k] = ld_act(cb, static_cast<int64_t>(KH * q + k) * a.L);
    }
    float4* dst = reinterpret_cast<float4*>(a.bct + (((static_cast<int64_t>(b) * 2 + dir) * a.parts + q) * a.L + s) * NB);
#pragma unroll
    for (int k = 0; k < NB / 4; ++k) dst[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
  }
}

// ---------------------------------------------------------------------------------------------
// Batched 2-D transpose through an LDS tile: out[img][c][r] = in[img][r][c] for R x Cc images.
// Reads and writes run along the contiguous dimension of their side.

constexpr int kTile = 64;

template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ in, T* __restrict__ out, int R, int Cc,
                                                        int tiles_r, int tiles_c) {
  __shared__ T tile[kTile][kTile + 1];
  const int64_t blk = blockIdx.x;
  const int tc = static_cast<int>(blk % tiles_c);
  const int tr = static_cast<int>((blk / tiles_c) % tiles_r);
  const int64_t img = blk / (static_cast<int64_t>(tiles_c) * tiles_r);
  const T* src = in + img * R * Cc;
  T* dst = out + img * R * Cc;
  const int r0 = tr * kTile, c0 = tc * kTile;
  if (sizeof(T) == 4 && (R & 3) == 0 && (Cc & 3) == 0) {
    // 4-byte elements, both sides multiples of 4: runs of 4 along each side's contiguous
    // dimension as single 16-byte accesses (the images start 16-byte aligned)
    const int tq = threadIdx.x & 15, tw = threadIdx.x >> 4;  // run of 4, row (column) of the pass
    for (int i = tw; i < kTile; i += 16) {
      const int r = r0 + i, c = c0 + 4 * tq;
      if (r < R && c < Cc) {
        T v[4];
        __builtin_memcpy(v, src + static_cast<int64_t>(r) * Cc + c, sizeof(v));
#pragma unroll
        for (int k = 0; k < 4; ++k) tile[i][4 * tq + k] = v[k];
      }
    }
    __syncthreads();
    for (int i = tw; i < kTile; i += 16) {
      const int c = c0 + i, r = r0 + 4 * tq;
      if (c < Cc && r < R) {
        T v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = tile[4 * tq + k][i];
        __builtin_memcpy(dst + static_cast<int64_t>(c) * R + r, v, sizeof(v));
      }
    }
    return;
  }
  const int tx = threadIdx.x & (kTile - 1), ty = threadIdx.x >> 6;
  for (int i = ty; i < kTile; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    if (r < R && c < Cc) tile[i][tx] = src[static_cast<int64_t>(r) * Cc + c];
  }
  __syncthreads();
  for (int i = ty; i < kTile; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (c < Cc && r < R) dst[static_cast<int64_t>(c) * R + r] = tile[tx][i];
  }
}

// The same for 2-byte elements, moved in pairs: each lane reads two neighbouring columns of a row
// and writes two neighbouring rows of a column as one 32-bit access.
__global__ __launch_bounds__(256) void transpose16_kernel(const uint16_t* __restrict__ in, uint16_t* __restrict__ out,
                                                          int R, int Cc, int tiles_r, int tiles_c) {
  __shared__ uint16_t tile[kTile][kTile + 2];
  const int64_t blk = blockIdx.x;
  const int tc = static_cast<int>(blk % tiles_c);
  const int tr = static_cast<int>((blk / tiles_c) % tiles_r);
  const int64_t img = blk / (static_cast<int64_t>(tiles_c) * tiles_r);
  const int64_t base = img * R * Cc;  // element offset of the image; pairs need an even total offset
  const uint16_t* src = in + base;
  uint16_t* dst = out + base;
  const int r0 = tr * kTile, c0 = tc * kTile;
  if ((R & 7) == 0 && (Cc & 7) == 0) {
    // both sides multiples of 8: runs of 8 elements as single 16-byte accesses (the images start
    // 16-byte aligned)
    const int tq = threadIdx.x & 7, tw = threadIdx.x >> 3;  // run of 8, row (column) of the pass
    for (int i = tw; i < kTile; i += 32) {
      const int r = r0 + i, c = c0 + 8 * tq;
      if (r < R && c < Cc) {
        uint16_t v[8];
        __builtin_memcpy(v, src + static_cast<int64_t>(r) * Cc + c, sizeof(v));
#pragma unroll
        for (int k = 0; k < 8; ++k) tile[i][8 * tq + k] = v[k];
      }
    }
    __syncthreads();
    for (int i = tw; i < kTile; i += 32) {
      const int c = c0 + i, r = r0 + 8 * tq;
      if (c < Cc && r < R) {
        uint16_t v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = tile[8 * tq + k][i];
        __builtin_memcpy(dst + static_cast<int64_t>(c) * R + r, v, sizeof(v));
      }
    }
    return;
  }
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 pairs x 8 rows per pass
  for (int i = ty; i < kTile; i += 8) {
    const int r = r0 + i, c = c0 + 2 * tx;
    if (r < R) {
      if (c + 1 < Cc) {
        const int64_t e = static_cast<int64_t>(r) * Cc + c;
        if (((base + e) & 1) == 0) {
          const uint32_t w = *reinterpret_cast<const uint32_t*>(src + e);
          tile[i][2 * tx] = static_cast<uint16_t>(w & 0xffffu);
          tile[i][2 * tx + 1] = static_cast<uint16_t>(w >> 16);
        } else {
          tile[i][2 * tx] = src[e];
          tile[i][2 * tx + 1] = src[e + 1];
        }
      } else if (c < Cc) {
        tile[i][2 * tx] = src[static_cast<int64_t>(r) * Cc + c];
      }
    }
  }
  __syncthreads();
  for (int i = ty; i < kTile; i += 8) {
    const int c = c0 + i, r = r0 + 2 * tx;
    if (c < Cc) {
      const int64_t e = static_cast<int64_t>(c) * R + r;
      if (r + 1 < R) {
        if (((base + e) & 1) == 0) {
          *reinterpret_cast<uint32_t*>(dst + e) = static_cast<uint32_t>(tile[2 * tx][i]) |
                                                   (static_cast<uint32_t>(tile[2 * tx + 1][i]) << 16);
        } else {
          dst[e] = tile[2 * tx][i];
          dst[e + 1] = tile[2 * tx + 1][i];
        }
      } else if (r < R) {
        dst[e] = tile[2 * tx][i];
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Scan kernels.  What differs between the forward and backward waves, the Vim and SS2D pairs and
// the two scan orders is a template parameter, so the token loop has no data-dependent branches:
//   DIR   0: step i visits chunk position i; 1: position Kc-1-i
//   MODE  kModeVim / kModeVimSum / kModeFirstPair / kModeSecondPair (SS2D backward tensors are
//         stored in reversed position order; the modes differ in the epilogue)
// The state part of a wave is a wave-uniform run-time value (it only selects data).

struct Lane {
  int b, c, lane, d, dd, part;  // dd: channel clamped into range for the loads of inactive lanes
  bool valid;
  int64_t s_lo;
  int Kc;
};

__device__ __forceinline__ Lane lane_at(const ScanArgs& a, int tile) {
  Lane l;
  const int g = tile % a.ngroups;
  const int rest = tile / a.ngroups;
  l.c = rest % a.nch;
  l.b = rest / a.nch;
  l.lane = threadIdx.x & (kW - 1);
  l.part = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 7);  // state part: wave / 2
  l.d = g * kW + l.lane;
  l.valid = l.d < a.dim;
  l.dd = l.valid ? l.d : a.dim - 1;
  l.s_lo = static_cast<int64_t>(l.c) * a.K;
  l.Kc = static_cast<int>(a.L - l.s_lo < a.K ? a.L - l.s_lo : a.K);
  return l;
}

__device__ __forceinline__ Lane lane_ctx(const ScanArgs& a, int bid) {
  return lane_at(a, logical_block(bid, a.batch * a.nch * a.ngroups));
}

__device__ __forceinline__ Lane lane_ctx(const ScanArgs& a) { return lane_ctx(a, static_cast<int>(blockIdx.x)); }

template <int MODE, int DIR>
struct Dir {
  static constexpr bool kRev =
      (MODE == kModeFirstPair || MODE == kModeSecondPair || MODE == kModeSecondPairSum) && DIR == 1;  // stored reversed
  static constexpr int kPosSgn = DIR == 0 ? 1 : -1;
  static constexpr int kSidxSgn = kRev ? -kPosSgn : kPosSgn;
  // global position of step i
  static __device__ __forceinline__ int64_t pos(const Lane& l, int i) {
    return DIR == 0 ? l.s_lo + i : l.s_lo + l.Kc - 1 - i;
  }
  // Δ_raw / B / C storage index of step i
  static __device__ __forceinline__ int64_t sidx(const ScanArgs& a, const Lane& l, int i) {
    return kRev ? a.L - 1 - pos(l, i) : pos(l, i);
  }
};

// Raw u and Δ_raw of a full window of 8 steps of one direction, kept as loaded until unpacked.
template <typename T, int MODE, int DIR>
struct Window {
  using Dr = Dir<MODE, DIR>;
  Run8<T> u, x;
  __device__ __forceinline__ void load(const ScanArgs& a, const Lane& l, const DirArgs& da, int i0) {
    const T* ub = static_cast<const T*>(da.u) + static_cast<int64_t>(l.b) * a.u_bs + static_cast<int64_t>(l.dd) * a.L;
    const T* db = static_cast<const T*>(da.draw) + static_cast<int64_t>(l.b) * da.draw_bs + static_cast<int64_t>(l.dd) * a.L;
    const int64_t p = Dr::pos(l, i0);
    u.load(ub + (Dr::kPosSgn > 0 ? p : p - (kWin - 1)));
    const int64_t si = Dr::sidx(a, l, i0);
    x.load(db + (Dr::kSidxSgn > 0 ? si : si - (kWin - 1)));
  }
  __device__ __forceinline__ void unpack(float (&uu)[kWin], float (&xr)[kWin]) const {
    u.template unpack<(Dr::kPosSgn < 0)>(uu);
    x.template unpack<(Dr::kSidxSgn < 0)>(xr);
  }
};

// A = -exp(A_log) for the wave's KH states (the decay of a step is exp2(Δ2 A)); ns = d_state.
template <int KH>
__device__ __forceinline__ void load_a2(const DirArgs& da, const Lane& l, int ns, float (&A2)[KH]) {
#pragma unroll
  for (int k = 0; k < KH; ++k) A2[k] = -expf(da.A_log[static_cast<int64_t>(l.dd) * ns + KH * l.part + k]);
}

// B/C of one position for the wave's state part: KH + KH wave-uniform floats (one s_load_dwordx16
// for 8 states, s_load_dwordx8 for 4).
template <int NB>
__device__ __forceinline__ void load_bc(scalar_fp p, float (&bc)[NB]) {
#pragma unroll
  for (int q = 0; q < NB; ++q) bc[q] = p[q];
}

// The wave's row of the B/C copy (2 KH floats per position and part of KH states).
template <int DIR, int KH = kH>
__device__ __forceinline__ scalar_fp bc_row(const ScanArgs& a, const Lane& l) {
  return (scalar_fp)(a.bct) + (((static_cast<int64_t>(l.b) * 2 + DIR) * a.parts + l.part) * a.L) * (2 * KH);
}

// One token for the wave's KH states, h = exp2(Δ2 A) h + (Δ2 u)(B ln 2); returns yi + Σ C h.
// Scalar loads may return out of order, so any wait for one covers every scalar load in flight: the
// token first waits for its own B/C (requested a token ago), then requests the next token's (nxt),
// which so has this whole token's work to arrive before the next token waits for it.  4 KH SGPRs
// hold B/C.
template <int KH>
__device__ __forceinline__ float token_update(float dl, float du, float yi, const float (&A2)[KH], float (&h)[KH],
                                             const float* cur) {
  float an[KH];
#pragma unroll
  for (int n = 0; n < KH; ++n) an[n] = __builtin_amdgcn_exp2f(dl * A2[n]);
#pragma unroll
  for (int n = 0; n < KH; ++n) {
    h[n] = h[n] * an[n];
    h[n] = __builtin_fmaf(du, cur[n], h[n]);
  }
  // one accumulator: the readout chain is not on the critical path (the next token's decays do
  // not depend on it), and a second accumulator costs a final add per token (measured 3% slower)
  float y = yi;
#pragma unroll
  for (int n = 0; n < KH; ++n) y = __builtin_fmaf(cur[KH + n], h[n], y);
  return y;
}

template <int KH>
__device__ __forceinline__ float scan_token(float dl, float du, float yi, const float (&A2)[KH], float (&h)[KH],
                                           const float (&cur)[2 * KH], float (&nxt)[2 * KH], scalar_fp nxt_p) {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited for
  __builtin_amdgcn_sched_barrier(0);
  load_bc(nxt_p, nxt);
  __builtin_amdgcn_sched_barrier(0);
  return token_update(dl, du, yi, A2, h, cur);
}

// Steps [i0, i0 + kWin) of one direction.  On entry bcA holds the B/C of step i0; on exit bcA
// holds the B/C of step i0 + kWin.  The buffers alternate between the steps, so no register
// copies are needed.  The one-past-the-end prefetch of a row's last step stays inside the B/C
// copy: forward rows are followed by another row, and backward rows follow another row.
template <int MODE, int DIR, int KH>
__device__ __forceinline__ void run_steps(const Lane& l, int i0, const float (&dl)[kWin], const float (&du)[kWin],
                                          const float (&yi)[kWin], const float (&A2)[KH], float (&h)[KH],
                                          float (&bcA)[2 * KH], float (&bcB)[2 * KH], scalar_fp bct,
                                          float (&y)[kWin]) {
  using Dr = Dir<MODE, DIR>;
  constexpr int NB = 2 * KH;  // B/C floats per position
  // Address of step i0 + k as a window base plus an immediate offset.
  const int64_t p0 = Dr::pos(l, i0);
  scalar_fp base = DIR == 0 ? bct + p0 * NB : bct + (p0 - kWin) * NB;
#pragma unroll
  for (int j = 0; j < kWin; j += 2) {
    y[j] = scan_token(dl[j], du[j], yi[j], A2, h, bcA, bcB, base + (DIR == 0 ? j + 1 : kWin - j - 1) * NB);
    y[j + 1] = scan_token(dl[j + 1], du[j + 1], yi[j + 1], A2, h, bcB, bcA,
                          base + (DIR == 0 ? j + 2 : kWin - j - 2) * NB);
  }
}

// Steps [i0, i0 + kWin) of a wave of 4 states.  Two adjacent steps' B/C (8 floats each) are
// adjacent in the B/C copy, so a pair comes with one 64-byte scalar load and is requested two steps
// before it is used: a wave's token is too short to cover a scalar load's latency on its own.  A
// pair buffer holds its two positions in address order: the first step's values first in the
// forward direction, second in the backward one.  On entry pA holds the pair of steps i0, i0 + 1;
// on exit that of i0 + kWin, i0 + kWin + 1 (the read past a row's end stays inside the copy, as in
// run_steps).
template <int MODE, int DIR>
__device__ __forceinline__ void run_steps2(const Lane& l, int i0, const float (&dl)[kWin], const float (&du)[kWin],
                                           const float (&yi)[kWin], const float (&A2)[4], float (&h)[4],
                                           float (&pA)[16], float (&pB)[16], scalar_fp bct, float (&y)[kWin]) {
  using Dr = Dir<MODE, DIR>;
  constexpr int NB = 8;
  const int64_t p0 = Dr::pos(l, i0);
  // the pair of steps s, s + 1 starts at window base + s (forward) or + kWin - 1 - s (backward)
  scalar_fp base = DIR == 0 ? bct + p0 * NB : bct + (p0 - kWin) * NB;
  constexpr int kF = DIR == 0 ? 0 : NB, kS = DIR == 0 ? NB : 0;  // offsets of the first and second step
#pragma unroll
  for (int j = 0; j < kWin; j += 4) {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): pA, requested two steps ago
    __builtin_amdgcn_sched_barrier(0);
    load_bc(base + (DIR == 0 ? j + 2 : kWin - 3 - j) * NB, pB);
    __builtin_amdgcn_sched_barrier(0);
    y[j] = token_update(dl[j], du[j], yi[j], A2, h, pA + kF);
    y[j + 1] = token_update(dl[j + 1], du[j + 1], yi[j + 1], A2, h, pA + kS);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // pB
    __builtin_amdgcn_sched_barrier(0);
    load_bc(base + (DIR == 0 ? j + 4 : kWin - 5 - j) * NB, pA);
    __builtin_amdgcn_sched_barrier(0);
    y[j + 2] = token_update(dl[j + 2], du[j + 2], yi[j + 2], A2, h, pB + kF);
    y[j + 3] = token_update(dl[j + 3], du[j + 3], yi[j + 3], A2, h, pB + kS);
  }
}

// Steps j, j + 1 (of the window at i0) of a walk that needs the state only (the chunk pass, the
// backward's checkpoint pass), so only B is read.  A step is too short to cover a scalar load's
// latency at the two or three waves per SIMD these passes get, so B comes two steps at a time: the
// pair waits for its own B (requested two steps ago), then requests that of steps j + 2, j + 3 into
// nxt (one wait per pair: scalar loads may return out of order).  Reads past a row's end stay
// inside the B/C copy, as in run_steps.
template <int MODE, int DIR>
__device__ __forceinline__ void ckpt_pair(const Lane& l, int i0, int j, const float (&dl)[kWin], const float (&du)[kWin],
                                          const float (&A2)[kH], float (&h)[kH], const float (&cur)[2 * kH],
                                          float (&nxt)[2 * kH], scalar_fp bct) {
  using Dr = Dir<MODE, DIR>;
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_sched_barrier(0);
  const scalar_fp p0 = bct + Dr::pos(l, i0 + j + 2) * kBC, p1 = bct + Dr::pos(l, i0 + j + 3) * kBC;
#pragma unroll
  for (int q = 0; q < kH; ++q) {
    nxt[q] = p0[q];
    nxt[kH + q] = p1[q];
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    float an[kH];
#pragma unroll
    for (int n = 0; n < kH; ++n) an[n] = __builtin_amdgcn_exp2f(dl[j + k] * A2[n]);
#pragma unroll
    for (int n = 0; n < kH; ++n) {
      h[n] = h[n] * an[n];
      h[n] = __builtin_fmaf(du[j + k], cur[kH * k + n], h[n]);
    }
  }
}

// Steps [i0, i0 + kWin) of a state-only walk.  On entry bA holds B of steps i0, i0 + 1 (kH floats
// each, in step order); on exit that of i0 + kWin, i0 + kWin + 1.
template <int MODE, int DIR>
__device__ __forceinline__ void ckpt_steps(const Lane& l, int i0, const float (&dl)[kWin], const float (&du)[kWin],
                                           const float (&A2)[kH], float (&h)[kH], float (&bA)[2 * kH],
                                           float (&bB)[2 * kH], scalar_fp bct) {
#pragma unroll
  for (int j = 0; j < kWin; j += 4) {
    ckpt_pair<MODE, DIR>(l, i0, j, dl, du, A2, h, bA, bB, bct);
    ckpt_pair<MODE, DIR>(l, i0, j + 2, dl, du, A2, h, bB, bA, bct);
  }
}

// Δ2 and Δ2·u of a window from its raw u and Δ_raw (bias2 = bias log2 e).
__device__ __forceinline__ void prep_window(const float (&uu)[kWin], const float (&xr)[kWin], float bias2,
                                            float (&dl)[kWin], float (&du)[kWin]) {
#pragma unroll
  for (int j = 0; j < kWin; ++j) {
    dl[j] = delta2(xr[j], bias2);
    du[j] = dl[j] * uu[j];
  }
}

// One step i outside the full windows (chunk tails): raw loads, Δ, the token update and the B/C
// prefetch of step i + 1 into bcA.  Returns the wave's partial y (with its D·u share) and sets
// *dl_out = Δ2.
template <typename T, int MODE, int DIR, int KH>
__device__ __forceinline__ float single_step(const ScanArgs& a, const Lane& l, const DirArgs& da, float bias, float Dh,
                                             int i, const float (&A2)[KH], float (&h)[KH], scalar_fp bct,
                                             float (&bcA)[2 * KH], float* dl_out) {
  using Dr = Dir<MODE, DIR>;
  const T* ub = static_cast<const T*>(da.u) + static_cast<int64_t>(l.b) * a.u_bs + static_cast<int64_t>(l.dd) * a.L;
  const T* db = static_cast<const T*>(da.draw) + static_cast<int64_t>(l.b) * da.draw_bs + static_cast<int64_t>(l.dd) * a.L;
  const float uu = ld_act(ub, Dr::pos(l, i));
  const float dl = delta2(ld_act(db, Dr::sidx(a, l, i)), bias);
  float bcB[2 * KH];
  const float y = scan_token(dl, dl * uu, Dh * uu, A2, h, bcA, bcB, bct + Dr::pos(l, i + 1) * (2 * KH));
#pragma unroll
  for (int q = 0; q < 2 * KH; ++q) bcA[q] = bcB[q];
  *dl_out = dl;
  return y;
}

// Ordering of the state parts of one direction, without a workgroup barrier: part 0 publishes the
// number of the last combine unit it has written to the LDS rows, and part p > 0 waits for part
// p - 1's number before adding (and, unless it is the last part, publishes its own).  A wave's
// LDS operations execute in issue order, so the data writes are complete when the flag write is,
// and the compiler barriers keep the instructions in that order.  Part 0 never waits and each
// wait is on a lower part, so every wait ends; the bound only keeps a mistake from turning into
// a hang, and a wait that gives up sets the call's status word (a vector store) so that the
// mistake is reported instead of returning silently wrong results.
__device__ __forceinline__ void unit_signal(int* flag, int unit) {
  asm volatile("" ::: "memory");
  __hip_atomic_store(flag, unit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ void unit_wait(int* flag, int unit, int* werr) {
  for (int n = 0; n < (1 << 22); ++n) {
    if (__builtin_amdgcn_readfirstlane(__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) >= unit) {
      asm volatile("" ::: "memory");
      return;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  // The wait gave up: the results of this call are unspecified.  Say so in the status word.
  if (werr) *werr = 1;
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------------------------
// Pass A: per chunk, direction and state part, the end states of the chunk scanned from a zero
// state, and Σ Δ2 (base-2 units).

// Δ and Δ·u exchange between the NP state parts of a direction: each wave computes them for 8/NP
// of a window's steps and reads the rest from the other parts, so softplus is evaluated once per
// (channel, step) instead of once per wave.  Double-buffered by window parity; a wave overwrites
// a buffer only after every other part has published the next window, which each does only after
// reading that buffer.
template <int NP>
struct ChunkXchg {
  static constexpr int kX = kWin / NP;  // steps per part and window
  float v[2][2][NP][2][kW][kX];         // [dir][window parity][part][Δ, Δ·u][lane][step]
  int prod[2][NP];                      // [dir][part]: windows published
};

template <typename T, int MODE, int DIR, int PART, int NP>
__device__ __forceinline__ void chunk_state_dir(const ScanArgs& a, const Lane& l, ChunkXchg<NP>& xc) {
  // The last chunk in scan order carries into nothing.
  if (DIR == 0 ? l.c == a.nch - 1 : l.c == 0) return;
  const DirArgs& da = DIR == 0 ? a.d0 : a.d1;
  float A2[kH], h[kH];
  load_a2(da, l, a.ns, A2);
#pragma unroll
  for (int n = 0; n < kH; ++n) h[n] = 0.0f;
  const float bias = da.bias[l.dd] * kLog2e;  // base-2 units
  const scalar_fp bct = bc_row<DIR>(a, l);
  float S = 0.0f;
  using Dr = Dir<MODE, DIR>;
  float bcA[kBC], bA[2 * kH], bB[2 * kH];  // bA, bB: B of two steps (ckpt_steps)
  Window<T, MODE, DIR> win;
  const int full_end = (l.Kc / kWin) * kWin;
  constexpr int me = PART, kX = ChunkXchg<NP>::kX;
  if (full_end > 0) {
#pragma unroll
    for (int q = 0; q < kH; ++q) {
      bA[q] = bct[Dr::pos(l, 0) * kBC + q];
      bA[kH + q] = bct[Dr::pos(l, 1) * kBC + q];
    }
    win.load(a, l, da, 0);
  }
  int w = 0;
  for (int i0 = 0; i0 < full_end; i0 += kWin, ++w) {
    float uu[kWin], xr[kWin], dl[kWin], du[kWin];
    win.unpack(uu, xr);
    // The prefetch must not be hoisted above the unpack: the window registers are loop-carried,
    // and a load into other registers would need a copy (and so a wait) at the loop back edge.
    // It is unconditional for the same reason (the last window reloads itself).
    __builtin_amdgcn_sched_barrier(0);
    win.load(a, l, da, i0 + kWin < full_end ? i0 + kWin : i0);
    float (&mine)[2][kW][kX] = xc.v[DIR][w & 1][me];
#pragma unroll
    for (int k = 0; k < kX; ++k) {
      const int j = kX * me + k;
      dl[j] = delta2(xr[j], bias);
      du[j] = dl[j] * uu[j];
      mine[0][l.lane][k] = dl[j];
      mine[1][l.lane][k] = du[j];
    }
    unit_signal(&xc.prod[DIR][me], w + 1);
#pragma unroll
    for (int q = 0; q < NP; ++q)
      if (q != me) unit_wait(&xc.prod[DIR][q], w + 1, a.werr);
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      if (q == me) continue;
#pragma unroll
      for (int k = 0; k < kX; ++k) {
        dl[kX * q + k] = xc.v[DIR][w & 1][q][0][l.lane][k];
        du[kX * q + k] = xc.v[DIR][w & 1][q][1][l.lane][k];
      }
    }
#pragma unroll
    for (int j = 0; j < kWin; ++j) S += dl[j];
    ckpt_steps<MODE, DIR>(l, i0, dl, du, A2, h, bA, bB, bct);
  }
  if (full_end < l.Kc) load_bc(bct + Dr::pos(l, full_end) * kBC, bcA);  // single steps: one B/C at a time
  for (int i = full_end; i < l.Kc; ++i) {
    float dl;
    single_step<T, MODE, DIR>(a, l, da, bias, 0.0f, i, A2, h, bct, bcA, &dl);
    S += dl;
  }
  if (l.valid) {
    constexpr int kStride = kH * NP + 1;
    float* ag = a.agg + ((((static_cast<int64_t>(l.b) * a.dim + l.d) * 2 + DIR) * a.nch) + l.c) * kStride;
#pragma unroll
    for (int n = 0; n < kH; ++n) ag[kH * l.part + n] = h[n];
    if (l.part == 0) ag[kH * NP] = S;
  }
}

template <typename T, int MODE, int DIR, int NP>
__device__ __forceinline__ void chunk_state_part(const ScanArgs& a, const Lane& l, ChunkXchg<NP>& xc) {
  switch (l.part) {
    case 0: chunk_state_dir<T, MODE, DIR, 0, NP>(a, l, xc); break;
    case 1: chunk_state_dir<T, MODE, DIR, 1, NP>(a, l, xc); break;
    case 2: if constexpr (NP > 2) chunk_state_dir<T, MODE, DIR, 2, NP>(a, l, xc); break;
    default: if constexpr (NP > 3) chunk_state_dir<T, MODE, DIR, 3, NP>(a, l, xc); break;
  }
}

template <typename T, int MODE, int NP>
__global__ __launch_bounds__(2 * kW * NP) void chunk_state_kernel(ScanArgs a) {
  __shared__ ChunkXchg<NP> xc;
  const Lane l = lane_ctx(a);
  if (threadIdx.x < 2 * NP) xc.prod[threadIdx.x / NP][threadIdx.x % NP] = 0;
  __syncthreads();
  const int dir = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6) & 1;
  if (dir == 0) chunk_state_part<T, MODE, 0, NP>(a, l, xc);
  else chunk_state_part<T, MODE, 1, NP>(a, l, xc);
}

// Carry prefix: per (batch, channel, direction, state), walk the chunks in scan order and replace
// each chunk's record (end state from a zero start, Σ Δ2) by the state entering that chunk:
//   h_in(first) = 0,  h_in(next) = exp2(A Σ Δ2) h_in + h_end,
// exp(A Σ Δ) being the chunk's total decay.  With `reverse` the walk runs against the scan order
// (the adjoint records of the backward pass, whose carries flow from later chunks to earlier
// ones).  One thread per (batch, channel, direction, state).
__global__ __launch_bounds__(256) void carry_prefix_kernel(ScanArgs a, float* recs, int reverse) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int ns = a.ns, stride = ns + 1;
  const int64_t total = static_cast<int64_t>(a.batch) * a.dim * 2 * ns;
  if (t >= total) return;
  const int n = static_cast<int>(t % ns);
  const int dir = static_cast<int>((t / ns) & 1);
  const int64_t bd = t / (2 * ns);  // b * dim + d
  const int d = static_cast<int>(bd % a.dim);
  const DirArgs& da = dir == 0 ? a.d0 : a.d1;
  const float A2 = -expf(da.A_log[static_cast<int64_t>(d) * ns + n]);  // with Σ Δ2: exp2(A Σ Δ2) = exp(A Σ Δ)
  float* rec = recs + (bd * 2 + dir) * a.nch * stride;
  const bool up = (dir == 0) != (reverse != 0);  // the walk visits chunks in increasing order
  float h = 0.0f;
  // kPB chunks at a time, the next group's records requested before this group's dependent
  // updates run: the walk waits for memory about once per sequence instead of once per group
  constexpr int kPB = 16;
  auto fetch = [&](int k0, float (&hend)[kPB], float (&S)[kPB]) {
#pragma unroll
    for (int j = 0; j < kPB; ++j) {
      const int k = k0 + j < a.nch ? k0 + j : a.nch - 1;
      const float* e = rec + (up ? k : a.nch - 1 - k) * stride;
      hend[j] = e[n];
      S[j] = e[ns];
    }
  };
  auto walk = [&](int k0, const float (&hend)[kPB], const float (&S)[kPB]) {
#pragma unroll
    for (int j = 0; j < kPB; ++j) {
      const int k = k0 + j;
      if (k < a.nch) {
        rec[(up ? k : a.nch - 1 - k) * stride + n] = h;
        if (k + 1 < a.nch) h = __builtin_fmaf(__builtin_amdgcn_exp2f(A2 * S[j]), h, hend[j]);
      }
    }
  };
  float hA[kPB], SA[kPB], hB[kPB], SB[kPB];
  fetch(0, hA, SA);
  for (int k0 = 0; k0 < a.nch; k0 += 2 * kPB) {
    fetch(k0 + kPB < a.nch ? k0 + kPB : k0, hB, SB);
    walk(k0, hA, SA);
    if (k0 + kPB >= a.nch) break;
    fetch(k0 + 2 * kPB < a.nch ? k0 + 2 * kPB : k0, hA, SA);
    walk(k0 + kPB, hB, SB);
  }
}

// ---------------------------------------------------------------------------------------------
// Main pass: fused bidirectional scan of one chunk with meet-in-the-middle combination.
// Phase 0 (steps [0, M)) stores each direction's y, including its D·u term, in the channel's LDS
// row at the chunk positions; phase 1 (steps [M, Kc)) adds it to the other direction's stored
// value.  Within a direction the part-0 wave writes (phase 0) or adds (phase 1) first and, in
// part order, each other part adds once the part below has signalled that unit; one workgroup
// barrier separates the phases and one precedes the epilogue.  For an odd chunk both
// directions reach the middle token at their last phase-0 step; the backward value of that step
// goes to the spare slot Kc, which the backward part-0 wave folds into the middle slot after
// the phase barrier.  After both phases every row holds y_f + y_b.  In kModeVimSum with a
// checkpoint buffer the walk also stores the state entering each of its windows and single-step
// runs, which the backward walk then visits in the same two-phase schedule.

// LDS update of one value by part 0: a write (PHASE 0) or an add (PHASE 1).
template <int PHASE>
__device__ __forceinline__ void lds_first(float* slot, float v) {
  *slot = PHASE == 1 ? *slot + v : v;
}

// Eight consecutive values of one lane, stored as one 16-byte (bf16) or two 16-byte (fp32) writes.
template <typename T>
__device__ __forceinline__ void store8(T* p, const float (&v)[kWin]);
template <>
__device__ __forceinline__ void store8(uint16_t* p, const float (&v)[kWin]) {
  uint32_t w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    w[k] = static_cast<uint32_t>(f32_to_bf16_rne(v[2 * k])) | (static_cast<uint32_t>(f32_to_bf16_rne(v[2 * k + 1])) << 16);
  const uint4 r = make_uint4(w[0], w[1], w[2], w[3]);
  __builtin_memcpy(p, &r, sizeof(r));
}
template <>
__device__ __forceinline__ void store8(float* p, const float (&v)[kWin]) {
  const float4 r0 = make_float4(v[0], v[1], v[2], v[3]), r1 = make_float4(v[4], v[5], v[6], v[7]);
  __builtin_memcpy(p, &r0, sizeof(r0));
  __builtin_memcpy(p + 4, &r1, sizeof(r1));
}

template <typename T, int MODE, int DIR, int PHASE, int NP>
__device__ __forceinline__ void run_phase(const ScanArgs& a, const Lane& l, const DirArgs& da, float bias, float Dh,
                                          int i_begin, int n_win, int i_end, int spare_step, const float (&A2)[kH],
                                          float (&h)[kH], scalar_fp bct, float (&bcA)[kBC], float (&bcB)[kBC],
                                          float* myY, int* flags, int& unit, int slot0) {
  Window<T, MODE, DIR> win;
  const int full_end = i_begin + n_win * kWin;
  // kModeVimSum with a checkpoint buffer: the state entering each window and the single steps
  // (slots slot0, slot0 + 1, ...), for the backward walk.
  float* ckp = nullptr;
  if constexpr (MODE == kModeVimSum) {
    if (a.ck)
      ckp = a.ck + ((static_cast<int64_t>(l.b) * 2 + DIR) * a.parts + l.part) * a.ck_wpc * a.dim * kH +
            (static_cast<int64_t>(slot0) * a.dim + l.dd) * kH;
  }
  const int64_t ck_slot = static_cast<int64_t>(a.dim) * kH;  // floats per slot
  constexpr int kStep = DIR == 0 ? 1 : -1;  // LDS row direction of consecutive steps
  if (full_end > i_begin) win.load(a, l, da, i_begin);
  // Part 0: in the second phase its slots already hold the other direction's values, which are
  // read before the window's arithmetic and added after it.  Other parts: the add of window w
  // waits for the lower part's unit w and is done while window w + 1 is prepared, so its LDS
  // reads overlap the Δ arithmetic instead of stalling the wave.
  const bool lo = l.part == 0;
  int* const wait_flag = flags + (lo ? 0 : l.part - 1);
  int* const own_flag = flags + l.part;
  const bool relay = NP > 2 && !lo && l.part < NP - 1;  // a middle part publishes its own adds
  float yp[kWin];
  int pp = -1;  // parts above 0: chunk position of the pending window's first step, -1 when none
  // The readout's starting value: the lane's D·u share in part 0, zero in the other parts (which so
  // skip the product).
  float yi[kWin];
#pragma unroll
  for (int j = 0; j < kWin; ++j) yi[j] = 0.0f;
  for (int i0 = i_begin; i0 < full_end; i0 += kWin) {
    float uu[kWin], xr[kWin], dl[kWin], du[kWin], y[kWin], r[kWin];
    rotate_priority(i0 / kWin);
    win.unpack(uu, xr);
    __builtin_amdgcn_sched_barrier(0);  // see chunk_state_dir
    win.load(a, l, da, i0 + kWin < full_end ? i0 + kWin : i0);
    const int p0 = DIR == 0 ? i0 : l.Kc - 1 - i0;  // chunk position of step i0
    if (lo) {
      if (PHASE == 1) {
#pragma unroll
        for (int j = 0; j < kWin; ++j) r[j] = myY[p0 + kStep * j];
      }
    } else if (pp >= 0) {
      unit_wait(wait_flag, unit, a.werr);
#pragma unroll
      for (int j = 0; j < kWin; ++j) r[j] = myY[pp + kStep * j];
    }
    prep_window(uu, xr, bias, dl, du);
    if (lo) {
#pragma unroll
      for (int j = 0; j < kWin; ++j) yi[j] = Dh * uu[j];
    }
    if (!lo && pp >= 0) {
#pragma unroll
      for (int j = 0; j < kWin; ++j) myY[pp + kStep * j] = r[j] + yp[j];
      if (relay) unit_signal(own_flag, unit);
    }
    if constexpr (MODE == kModeVimSum) {
      if (ckp && l.valid) store8(ckp + ((i0 - i_begin) / kWin) * ck_slot, h);
    }
    run_steps<MODE, DIR>(l, i0, dl, du, yi, A2, h, bcA, bcB, bct, y);
    ++unit;
    if (lo) {
#pragma unroll
      for (int j = 0; j < kWin; ++j) myY[p0 + kStep * j] = PHASE == 1 ? r[j] + y[j] : y[j];
      unit_signal(own_flag, unit);
    } else {
#pragma unroll
      for (int j = 0; j < kWin; ++j) yp[j] = y[j];
      pp = p0;
    }
  }
  if (!lo && pp >= 0) {
    unit_wait(wait_flag, unit, a.werr);
#pragma unroll
    for (int j = 0; j < kWin; ++j) myY[pp + kStep * j] += yp[j];
    if (relay) unit_signal(own_flag, unit);
  }
  if constexpr (MODE == kModeVimSum) {
    if (ckp && l.valid && full_end < i_end) store8(ckp + n_win * ck_slot, h);
  }
  for (int i = full_end; i < i_end; ++i) {
    float dl;
    const float v = single_step<T, MODE, DIR>(a, l, da, bias, Dh, i, A2, h, bct, bcA, &dl);
    const int pos = i == spare_step ? l.Kc : (DIR == 0 ? i : l.Kc - 1 - i);
    ++unit;
    if (lo) {
      lds_first<PHASE>(myY + pos, v);
      unit_signal(own_flag, unit);
    } else {
      unit_wait(wait_flag, unit, a.werr);
      myY[pos] += v;
      if (relay) unit_signal(own_flag, unit);
    }
  }
}

template <typename T>
struct EpiZ;
template <typename T, int MODE, int NP>
__device__ __forceinline__ void epi_prefetch(const ScanArgs& a, const Lane& l, EpiZ<T>& e);

template <typename T, int MODE, int DIR, int NP>
__device__ __forceinline__ void scan_pair_dir(const ScanArgs& a, const Lane& l, float* ybuf, int ybs, int* flags,
                                              EpiZ<T>& epi) {
  using Dr = Dir<MODE, DIR>;
  const DirArgs& da = DIR == 0 ? a.d0 : a.d1;
  const int Kc = l.Kc;
  const int M = (Kc + 1) >> 1;  // steps of the first phase
  const bool odd = (Kc & 1) != 0;

  float A2[kH], h[kH];
  load_a2(da, l, a.ns, A2);
#pragma unroll
  for (int n = 0; n < kH; ++n) h[n] = 0.0f;
  const float bias = da.bias[l.dd] * kLog2e;  // base-2 units
  const float Dh = l.part == 0 ? da.Dp[l.dd] : 0.0f;  // part 0 adds the D·u term

  // Carry-in: the state entering this chunk, which the carry-prefix kernel left in the chunk's
  // carry record.
  if (a.nch > 1) {
    const float* e = a.agg + ((((static_cast<int64_t>(l.b) * a.dim + l.dd) * 2 + DIR) * a.nch) + l.c) * (kH * NP + 1);
#pragma unroll
    for (int n = 0; n < kH; ++n) h[n] = e[kH * l.part + n];
  }

  const scalar_fp bct = bc_row<DIR>(a, l);
  float* myY = ybuf + l.lane * ybs;
  float bcA[kBC], bcB[kBC];
  load_bc(bct + Dr::pos(l, 0) * kBC, bcA);

  // The same window/step structure for both directions: the windows of phase 0 stop before the
  // middle token of an odd chunk, which is then a single step of both directions.
  const int nw0 = (odd ? M - 1 : M) / kWin;
  const int spare = (DIR == 1 && odd) ? M - 1 : -1;
  int unit = 0;
  run_phase<T, MODE, DIR, 0, NP>(a, l, da, bias, Dh, 0, nw0, M, spare, A2, h, bct, bcA, bcB, myY, flags, unit, 0);
  __syncthreads();
  // Fold the backward value of an odd chunk's middle token (kept in the spare slot) into the
  // middle slot; no wave touches either slot in the second phase.
  if (DIR == 1 && odd && l.part == 0) myY[M - 1] += myY[Kc];
  epi_prefetch<T, MODE, NP>(a, l, epi);
  run_phase<T, MODE, DIR, 1, NP>(a, l, da, bias, Dh, M, (Kc - M) / kWin, Kc, -1, A2, h, bct, bcA, bcB, myY, flags,
                                 unit, nw0 + (nw0 * kWin < M ? 1 : 0));
}

// Combined value of chunk position q of LDS row c.
__device__ __forceinline__ float row_val(const float* ybuf, int ybs, int c, int q) { return ybuf[c * ybs + q]; }

// Outputs of one chunk from the combined LDS rows.  Row-major order: the chunk's part of each
// channel row is cut into groups of 8 positions; the threads take groups in turn (consecutive
// threads on consecutive groups of a row, so the 16-byte loads and stores are contiguous), and
// each thread issues the gate loads of kEpiBatch groups before using any of them.  Column order
// (second SS2D pair): position by position, pixel index advanced incrementally.
constexpr int kEpiBatch = 8;  // threads * kEpiBatch >= 64 * (kKMax / 8): one batch per chunk

// Gate values of the first epilogue batch, requested before the second phase so that they have
// arrived when the epilogue starts.
template <typename T>
struct EpiZ {
  Run8<T> zr[kEpiBatch];
};

// Row c and first position q of epilogue item it (items: groups of 8 positions, row-major).
__device__ __forceinline__ void epi_item(int it, int items, int ngr, int& c, int& q) {
  const int itc = it < items ? it : items - 1;  // clamped: loads stay in range
  c = itc / ngr;
  q = (itc - c * ngr) * kWin;
}

// Finish one batch of groups (first group it0, then every NTH-th) with its gate values.
template <typename T, int MODE, int NTH>
__device__ __forceinline__ void epi_batch(const ScanArgs& a, const float* ybuf, int ybs, int64_t base,
                                          int items, int ngr, int it0, const Run8<T> (&zr)[kEpiBatch]) {
  const T* zb = static_cast<const T*>(a.z);
  T* ob = static_cast<T*>(a.out);
#pragma unroll
  for (int k = 0; k < kEpiBatch; ++k) {
    if (it0 + k * NTH >= items) break;
    int c, q;
    epi_item(it0 + k * NTH, items, ngr, c, q);
    const int64_t gi = base + static_cast<int64_t>(c) * a.L + q;
    float v[kWin], zz[kWin];
#pragma unroll
    for (int j = 0; j < kWin; ++j) v[j] = row_val(ybuf, ybs, c, q + j);
    if (MODE == kModeVim) {
      zr[k].template unpack<false>(zz);
#pragma unroll
      for (int j = 0; j < kWin; ++j) v[j] = 0.5f * v[j] * silu_f(zz[j]);  // (y_f + y_b) / 2 * silu(z)
      store8(ob + gi, v);
    } else if (MODE == kModeVimSum) {
      float go[kWin], gv[kWin], dv[kWin];
      Run8<T> dr;
      dr.load(static_cast<const T*>(a.dout) + gi);
      zr[k].template unpack<false>(zz);
      dr.template unpack<false>(go);
#pragma unroll
      for (int j = 0; j < kWin; ++j) {
        const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-zz[j] * kLog2e));
        gv[j] = 0.5f * go[j] * zz[j] * sg;
        dv[j] = 0.5f * go[j] * v[j] * sg * (1.0f + zz[j] * (1.0f - sg));
      }
      store8(a.gout + gi, gv);
      store8(static_cast<T*>(a.dzout) + gi, dv);
    } else if (MODE == kModeFirstPair) {
      store8(a.wsy + gi, v);
    } else if (MODE == kModeSecondPairSum) {
      float w[kWin];
      Run8<float> wr;
      wr.load(a.wsy + gi);
      wr.template unpack<false>(w);
#pragma unroll
      for (int j = 0; j < kWin; ++j) v[j] += w[j];
      store8(static_cast<float*>(a.out) + gi, v);
    } else {
      float w[kWin];
      Run8<float> wr;
      wr.load(a.wsy + gi);
      wr.template unpack<false>(w);
      if (zb) zr[k].template unpack<false>(zz);
#pragma unroll
      for (int j = 0; j < kWin; ++j) v[j] = zb ? (v[j] + w[j]) * silu_f(zz[j]) : v[j] + w[j];
      store8(ob + gi, v);
    }
  }
}

template <typename T, int MODE, int NTH>
__device__ __forceinline__ void epi_load(const ScanArgs& a, int64_t base, int items, int ngr, int it0,
                                         Run8<T> (&zr)[kEpiBatch]) {
  const T* zb = static_cast<const T*>(a.z);
  if (!(MODE == kModeVim || MODE == kModeVimSum || (MODE == kModeSecondPair && zb))) return;
#pragma unroll
  for (int k = 0; k < kEpiBatch; ++k) {
    int c, q;
    epi_item(it0 + k * NTH, items, ngr, c, q);
    zr[k].load(zb + base + static_cast<int64_t>(c) * a.L + q);
  }
}

template <typename T, int MODE, int NP>
__device__ __forceinline__ void epi_prefetch(const ScanArgs& a, const Lane& l, EpiZ<T>& e) {
  if (MODE != kModeVim) return;
  const int g_d0 = l.d - l.lane;
  const int nch_here = a.dim - g_d0 < kW ? a.dim - g_d0 : kW;
  const int ngr = l.Kc / kWin;
  const int items = nch_here * ngr;
  if (static_cast<int>(threadIdx.x) >= items) return;
  const int64_t base = static_cast<int64_t>(l.b) * a.u_bs + static_cast<int64_t>(g_d0) * a.L + l.s_lo;
  epi_load<T, MODE, 2 * kW * NP>(a, base, items, ngr, static_cast<int>(threadIdx.x), e.zr);
}

template <typename T, int MODE, int NP>
__device__ __forceinline__ void pair_epilogue(const ScanArgs& a, const Lane& l, const float* ybuf, int ybs,
                                              const EpiZ<T>& pre) {
  constexpr int NTH = 2 * kW * NP;  // threads of the workgroup
  const int g_d0 = l.d - l.lane;  // first channel of the group
  const int Kc = l.Kc;
  const int tid = threadIdx.x;
  const int nch_here = a.dim - g_d0 < kW ? a.dim - g_d0 : kW;
  const T* zb = static_cast<const T*>(a.z);
  T* ob = static_cast<T*>(a.out);
  const int64_t base = static_cast<int64_t>(l.b) * a.u_bs + static_cast<int64_t>(g_d0) * a.L + l.s_lo;
  {
    const int ngr = Kc / kWin;            // full groups per row
    const int items = nch_here * ngr;
    if (tid < items) {
      if (MODE == kModeVim) {
        epi_batch<T, MODE, NTH>(a, ybuf, ybs, base, items, ngr, tid, pre.zr);
      } else {
        Run8<T> zr[kEpiBatch];
        epi_load<T, MODE, NTH>(a, base, items, ngr, tid, zr);
        epi_batch<T, MODE, NTH>(a, ybuf, ybs, base, items, ngr, tid, zr);
      }
    }
    for (int it0 = tid + NTH * kEpiBatch; it0 < items; it0 += NTH * kEpiBatch) {
      Run8<T> zr[kEpiBatch];
      epi_load<T, MODE, NTH>(a, base, items, ngr, it0, zr);
      epi_batch<T, MODE, NTH>(a, ybuf, ybs, base, items, ngr, it0, zr);
    }
    // positions past the last full group of each row
    const int rem = Kc - ngr * kWin;
    for (int it = tid; it < nch_here * rem; it += NTH) {
      const int c = it / rem, q = ngr * kWin + (it - (it / rem) * rem);
      const int64_t gi = base + static_cast<int64_t>(c) * a.L + q;
      const float v = row_val(ybuf, ybs, c, q);
      if (MODE == kModeVim) {
        st_act(ob, gi, 0.5f * v * silu_f(ld_act(zb, gi)));
      } else if (MODE == kModeVimSum) {
        const float zz = ld_act(zb, gi), go = ld_act(static_cast<const T*>(a.dout), gi);
        const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-zz * kLog2e));
        a.gout[gi] = 0.5f * go * zz * sg;
        st_act(static_cast<T*>(a.dzout), gi, 0.5f * go * v * sg * (1.0f + zz * (1.0f - sg)));
      } else if (MODE == kModeFirstPair) {
        a.wsy[gi] = v;
      } else if (MODE == kModeSecondPairSum) {
        static_cast<float*>(a.out)[gi] = v + a.wsy[gi];
      } else {
        float w = v + a.wsy[gi];
        if (zb) w *= silu_f(ld_act(zb, gi));
        st_act(ob, gi, w);
      }
    }
  }
}

// Workgroup: 2 NP waves, wave w on direction w & 1 and state part w >> 1 (states 8p .. 8p + 7).
template <typename T, int MODE, int NP>
__global__ __launch_bounds__(2 * kW * NP) void scan_pair_kernel(ScanArgs a) {
  extern __shared__ float ybuf[];    // [kW][ybs]: combined y of the chunk
  __shared__ int unit_flag[2][NP];   // per direction and part: last combine unit the part has written
  const int ybs = (a.K + 1) | 1;     // odd row stride spreads the 64 lanes over the banks
  const Lane l = lane_ctx(a);
  if (threadIdx.x < 2 * NP) unit_flag[threadIdx.x / NP][threadIdx.x % NP] = 0;
  __syncthreads();
  EpiZ<T> epi;
  if ((__builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6) & 1) == 0)
    scan_pair_dir<T, MODE, 0, NP>(a, l, ybuf, ybs, unit_flag[0], epi);
  else
    scan_pair_dir<T, MODE, 1, NP>(a, l, ybuf, ybs, unit_flag[1], epi);
  __syncthreads();
  pair_epilogue<T, MODE, NP>(a, l, ybuf, ybs, epi);
}

// ---------------------------------------------------------------------------------------------
// Whole-sequence walk of one bidirectional pair (SS2D sequences too long for an LDS row).
//
// A sequence longer than an LDS row would otherwise be cut into chunks, and every chunk but the
// last needs its end state from a second pass over it (the chunk pass), about 0.8 of a scan's
// work.  When the (batch, channel-group) tiles alone fill the GPU, each pair instead walks its
// sequence whole: the same meet-in-the-middle schedule as scan_pair_kernel, but the channel's y
// row lives in global memory, position-major ([position][64 lanes] per tile), so every store of
// one step is one 256-byte line whatever the order of the positions.  Within a direction the
// state parts add their partial readouts in part order through a small LDS ring of windows (the
// last part adds its own and does the global store or, in the second half, the read-add of the
// other direction's value); the first part reuses a ring slot only after the last part has
// consumed it.  The fp32 sums of both directions are what the merge kernel then reads.
//
// Δ2 = softplus(Δ_raw + bias) log2 e and Δ2 u are the same for every state part of a direction,
// so each part computes them for kWin / NP steps of a window and publishes them in a second LDS
// ring, from which all parts read the whole window.  A part publishes its share of window w + 1
// (from raw inputs loaded two windows ahead) before it waits for the shares of window w, so the
// parts exchange without waiting as long as none is a window behind.

constexpr int kRing = 2;   // windows in flight between the first and the last state part
constexpr int kXRing = 4;  // windows of shared Δ2, Δ2 u: at most three in use (w - 1 .. w + 1)

template <int NP>
struct WalkShared {
  static constexpr int kX = kWin / NP;  // steps per part and window
  float ring[2][kRing][kWin][kW];       // [dir][slot][step][lane]: partial y of a window, parts so far
  int prod[2][NP];                      // [dir][part]: units the part has added to its ring slot
  int cons[2];                          // [dir]: units the last part has consumed
  float xv[2][kXRing][NP][2][kW][kX];   // [dir][window % kXRing][part][Δ2, Δ2 u][lane][step]
  int xprod[2][NP];                     // [dir][part]: windows whose share the part has published
};

// One window (len steps at positions p0 + kStep j) of partial readouts y: combined over the state
// parts in part order through the ring; the last part then stores the direction's value (PHASE
// 0) or adds it to the other direction's value r (PHASE 1) in the global row G.  keep >= 0: the
// step at that index is the odd sequence's middle token in the backward direction, whose value
// is returned in *vkeep instead of being stored (it is added after the phase barrier).
template <int DIR, int PHASE, int NP, int LEN>
__device__ __forceinline__ void walk_combine(WalkShared<NP>& sh, const Lane& l, int unit, const float (&y)[LEN],
                                             const float (&r)[LEN], float* G, int64_t p0, int kStep, int keep,
                                             float* vkeep, int* werr) {
  float* slot = &sh.ring[DIR][unit % kRing][0][0];
  if (l.part == 0) {
    unit_wait(&sh.cons[DIR], unit - kRing + 1, werr);  // the last part is done with this slot's previous use
#pragma unroll
    for (int j = 0; j < LEN; ++j) slot[j * kW + l.lane] = y[j];
    unit_signal(&sh.prod[DIR][0], unit + 1);
    return;
  }
  unit_wait(&sh.prod[DIR][l.part - 1], unit + 1, werr);
  float v[LEN];
#pragma unroll
  for (int j = 0; j < LEN; ++j) v[j] = slot[j * kW + l.lane] + y[j];
  if (l.part < NP - 1) {
#pragma unroll
    for (int j = 0; j < LEN; ++j) slot[j * kW + l.lane] = v[j];
    unit_signal(&sh.prod[DIR][l.part], unit + 1);
    return;
  }
  asm volatile("" ::: "memory");  // the slot is read before it is released
  unit_signal(&sh.cons[DIR], unit + 1);
#pragma unroll
  for (int j = 0; j < LEN; ++j) {
    float* g = G + (p0 + kStep * j) * kW + l.lane;
    if (PHASE == 1) *g = r[j] + v[j];
    else if (j == keep) *vkeep = v[j];
    else *g = v[j];
  }
}

template <typename T, int DIR, int PHASE, int NP, int KH, int PART>
__device__ __forceinline__ void walk_phase(const ScanArgs& a, const Lane& l, const DirArgs& da, float bias, float Dh,
                                           int i_begin, int n_win, int i_end, int keep_step, const float (&A2)[KH],
                                           float (&h)[KH], scalar_fp bct, float (&bcA)[2 * KH], float (&bcB)[2 * KH],
                                           float* G, WalkShared<NP>& sh, int& unit, int& xw, float* vkeep) {
  constexpr int MODE = kModeFirstPair;  // pair semantics: the backward direction's inputs are stored reversed
  constexpr int kX = WalkShared<NP>::kX;
  static_assert(kWin % NP == 0, "a window's steps split evenly over the state parts");
  Window<T, MODE, DIR> win;
  constexpr int kStep = DIR == 0 ? 1 : -1;
  constexpr bool last = PART == NP - 1;
  float yn[kWin];  // part 0: D u of the window whose share was published last
  // Parts above 0 add a window's readout to the ring at the start of the next window, after the
  // lower part has had that window's work to publish its own: the wait then rarely stalls.
  float yd[kWin], rd[kWin];  // the pending window's readout (and, last part, second half: the other direction's)
  int64_t pd = -1;           // its first position, -1 when none
  int ud = 0;                // its unit
  // This part's share of window wi (raw inputs uu, xr): Δ2 and Δ2 u of steps kX PART .. + kX - 1.
  auto publish = [&](const float (&uu)[kWin], const float (&xr)[kWin], int wi) {
    float (&mine)[2][kW][kX] = sh.xv[DIR][wi % kXRing][PART];
#pragma unroll
    for (int k = 0; k < kX; ++k) {
      const int j = kX * PART + k;
      const float d = delta2(xr[j], bias);
      mine[0][l.lane][k] = d;
      mine[1][l.lane][k] = d * uu[j];
    }
    if (PART == 0) {
#pragma unroll
      for (int j = 0; j < kWin; ++j) yn[j] = Dh * uu[j];
    }
    unit_signal(&sh.xprod[DIR][PART], wi + 1);
  };
  using Dr = Dir<MODE, DIR>;
  constexpr bool kPairs = KH == 4;  // B/C two steps at a time (run_steps2)
  float pA[16], pB[16];
  if (kPairs && n_win > 0) load_bc(bct + (DIR == 0 ? Dr::pos(l, i_begin) : Dr::pos(l, i_begin) - 1) * 8, pA);
  if (n_win > 0) {
    float uu[kWin], xr[kWin];
    win.load(a, l, da, i_begin);
    win.unpack(uu, xr);
    __builtin_amdgcn_sched_barrier(0);
    win.load(a, l, da, n_win > 1 ? i_begin + kWin : i_begin);
    publish(uu, xr, xw);
  }
  for (int k = 0; k < n_win; ++k, ++xw) {
    const int i0 = i_begin + k * kWin;
    float dl[kWin], du[kWin], yi[kWin], y[kWin], r[kWin];
    rotate_priority(i0 / kWin);
#pragma unroll
    for (int j = 0; j < kWin; ++j) yi[j] = PART == 0 ? yn[j] : 0.0f;
    {
      // raw inputs of window k + 1 (window k again at the last, unused): the window registers
      // are loop-carried, so the next load is unconditional and stays after the unpack
      float uu[kWin], xr[kWin];
      win.unpack(uu, xr);
      __builtin_amdgcn_sched_barrier(0);
      win.load(a, l, da, k + 2 < n_win ? i0 + 2 * kWin : i0);
      if (k + 1 < n_win) publish(uu, xr, xw + 1);
    }
#pragma unroll
    for (int q = 0; q < NP; ++q)
      if (q != PART) unit_wait(&sh.xprod[DIR][q], xw + 1, a.werr);
    const float (&xs)[NP][2][kW][kX] = sh.xv[DIR][xw % kXRing];
#pragma unroll
    for (int q = 0; q < NP; ++q) {
#pragma unroll
      for (int kk = 0; kk < kX; ++kk) {
        dl[kX * q + kk] = xs[q][0][l.lane][kk];
        du[kX * q + kk] = xs[q][1][l.lane][kk];
      }
    }
    const int64_t p0 = DIR == 0 ? i0 : l.Kc - 1 - i0;
    if (PART > 0 && pd >= 0) {
      walk_combine<DIR, PHASE, NP, kWin>(sh, l, ud, yd, rd, G, pd, kStep, -1, vkeep, a.werr);
      pd = -1;
    }
    if (PHASE == 1 && last) {
      // the other direction's values, requested a window's work before they are added
#pragma unroll
      for (int j = 0; j < kWin; ++j) r[j] = G[(p0 + kStep * j) * kW + l.lane];
    }
    if constexpr (kPairs) run_steps2<MODE, DIR>(l, i0, dl, du, yi, A2, h, pA, pB, bct, y);
    else run_steps<MODE, DIR>(l, i0, dl, du, yi, A2, h, bcA, bcB, bct, y);
    if (PART == 0) {
      walk_combine<DIR, PHASE, NP, kWin>(sh, l, unit, y, r, G, p0, kStep, -1, vkeep, a.werr);
    } else {
#pragma unroll
      for (int j = 0; j < kWin; ++j) {
        yd[j] = y[j];
        rd[j] = r[j];
      }
      pd = p0;
      ud = unit;
    }
    ++unit;
  }
  if (PART > 0 && pd >= 0) walk_combine<DIR, PHASE, NP, kWin>(sh, l, ud, yd, rd, G, pd, kStep, -1, vkeep, a.werr);
  // single steps take their B/C one at a time in bcA
  if (kPairs && i_begin + n_win * kWin < i_end) load_bc(bct + Dr::pos(l, i_begin + n_win * kWin) * 8, bcA);
  for (int i = i_begin + n_win * kWin; i < i_end; ++i) {
    float dl, y[1], r[1];
    const int64_t pos = DIR == 0 ? i : l.Kc - 1 - i;
    if (PHASE == 1 && last) r[0] = G[pos * kW + l.lane];
    y[0] = single_step<T, MODE, DIR>(a, l, da, bias, Dh, i, A2, h, bct, bcA, &dl);
    walk_combine<DIR, PHASE, NP, 1>(sh, l, unit, y, r, G, pos, kStep, i == keep_step ? 0 : -1, vkeep, a.werr);
    ++unit;
  }
}

template <typename T, int DIR, int NP, int KH, int PART>
__device__ __forceinline__ void walk_dir(const ScanArgs& a, const Lane& l, WalkShared<NP>& sh) {
  using Dr = Dir<kModeFirstPair, DIR>;
  const DirArgs& da = DIR == 0 ? a.d0 : a.d1;
  const int L = l.Kc;
  const int M = (L + 1) >> 1;  // steps of the first half
  const bool odd = (L & 1) != 0;
  float A2[KH], h[KH];
  load_a2(da, l, a.ns, A2);
#pragma unroll
  for (int n = 0; n < KH; ++n) h[n] = 0.0f;
  const float bias = da.bias[l.dd] * kLog2e;
  const float Dh = l.part == 0 ? da.Dp[l.dd] : 0.0f;
  const scalar_fp bct = bc_row<DIR, KH>(a, l);
  float* G = a.wsy + ((static_cast<int64_t>(l.b) * a.ngroups + l.d / kW) * a.L) * kW;
  float bcA[2 * KH], bcB[2 * KH];
  load_bc(bct + Dr::pos(l, 0) * (2 * KH), bcA);
  const int nw0 = (odd ? M - 1 : M) / kWin;
  // In an odd sequence both directions reach the middle token at step M - 1: the forward one
  // stores it, the backward one adds its value after the phase barrier.
  const int keep = (DIR == 1 && odd) ? M - 1 : -1;
  float vmid = 0.0f;
  int unit = 0, xw = 0;
  walk_phase<T, DIR, 0, NP, KH, PART>(a, l, da, bias, Dh, 0, nw0, M, keep, A2, h, bct, bcA, bcB, G, sh, unit, xw,
                                      &vmid);
  __syncthreads();  // first halves of both directions stored (global memory, workgroup scope)
  if (keep >= 0 && l.part == NP - 1) G[static_cast<int64_t>(M - 1) * kW + l.lane] += vmid;
  walk_phase<T, DIR, 1, NP, KH, PART>(a, l, da, bias, Dh, M, (L - M) / kWin, L, -1, A2, h, bct, bcA, bcB, G, sh,
                                      unit, xw, &vmid);
}

// Workgroup: 2 NP waves on one (batch, channel group) tile of one pair, wave w on direction w & 1
// and state part w >> 1 (KH states each; d_state = NP KH).  Two pairs (argument sets) per launch,
// the first set's tiles first.  A whole-sequence walk has no chunks to add parallelism, so the
// state is cut into four parts whatever d_state is: at d_state 16 four parts of 4 states give the
// 56 x 56 workload four waves per SIMD, which outweighs the per-token work shared by fewer states.
template <typename T, int NP, int KH>
__global__ __launch_bounds__(2 * kW * NP) void walk_pair_kernel(ScanArgs a0, ScanArgs a1) {
  __shared__ WalkShared<NP> sh;
  const int nb = a0.batch * a0.ngroups, bid = static_cast<int>(blockIdx.x);
  const bool first = bid < nb;
  const ScanArgs* ap = first ? &a0 : &a1;
  const ScanArgs& a = *ap;
  const Lane l = lane_at(a, logical_block(first ? bid : bid - nb, nb));
  if (threadIdx.x < 2 * NP) {
    sh.prod[threadIdx.x / NP][threadIdx.x % NP] = 0;
    sh.xprod[threadIdx.x / NP][threadIdx.x % NP] = 0;
  }
  if (threadIdx.x < 2) sh.cons[threadIdx.x] = 0;
  __syncthreads();
  static_assert(NP == 4, "one instantiation per state part");
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);  // direction w & 1, part w >> 1
  switch (w) {
    case 0: walk_dir<T, 0, NP, KH, 0>(a, l, sh); break;
    case 1: walk_dir<T, 1, NP, KH, 0>(a, l, sh); break;
    case 2: walk_dir<T, 0, NP, KH, 1>(a, l, sh); break;
    case 3: walk_dir<T, 1, NP, KH, 1>(a, l, sh); break;
    case 4: walk_dir<T, 0, NP, KH, 2>(a, l, sh); break;
    case 5: walk_dir<T, 1, NP, KH, 2>(a, l, sh); break;
    case 6: walk_dir<T, 0, NP, KH, 3>(a, l, sh); break;
    default: walk_dir<T, 1, NP, KH, 3>(a, l, sh); break;
  }
}

// Cross-merge of the two pairs' sums: out[b][d][h][w] = (R[h W + w] + C[w H + h]) (times
// silu(z)), with R (row pair, row-major positions) and C (column pair, column-major positions)
// the walk's [batch][group][position][64] float32 rows.  A workgroup takes 64 pixels of one
// (batch, channel group): it reads the 64 x 64 sums pixel by pixel (256-byte lines), turns them
// channel-major through LDS and stores each channel's 64 pixels contiguously.
template <typename T>
__global__ __launch_bounds__(256) void walk_merge_kernel(const float* __restrict__ R, const float* __restrict__ Cs,
                                                         const T* __restrict__ z, T* __restrict__ out, int dim, int H,
                                                         int W, int ngroups) {
  __shared__ float tile[64][kW + 1];
  const int L = H * W;
  const int nblk = (L + 63) / 64;
  const int64_t blk = blockIdx.x;
  const int pb = static_cast<int>(blk % nblk);
  const int64_t bg = blk / nblk;  // b * ngroups + g
  const int g = static_cast<int>(bg % ngroups);
  const int64_t b = bg / ngroups;
  const int p0 = pb * 64;
  const float* Rt = R + bg * L * kW;
  const float* Ct = Cs + bg * L * kW;
  {
    const int k = threadIdx.x >> 2, cq = (threadIdx.x & 3) * 16;  // pixel, 16 channels
    const int p = p0 + k;
    if (p < L) {
      const int hh = p / W, ww = p - hh * W;
      const float4* rr = reinterpret_cast<const float4*>(Rt + static_cast<int64_t>(p) * kW + cq);
      const float4* cc = reinterpret_cast<const float4*>(Ct + (static_cast<int64_t>(ww) * H + hh) * kW + cq);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 a = rr[q], c = cc[q];
        tile[k][cq + 4 * q] = a.x + c.x;
        tile[k][cq + 4 * q + 1] = a.y + c.y;
        tile[k][cq + 4 * q + 2] = a.z + c.z;
        tile[k][cq + 4 * q + 3] = a.w + c.w;
      }
    }
  }
  __syncthreads();
  const int c = threadIdx.x >> 3, k0 = (threadIdx.x & 7) * kWin;  // channel (pass 1: 0-31), 8 pixels
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int cc = c + 32 * pass;
    const int d = g * kW + cc;
    if (d >= dim) break;
    const int64_t e0 = (b * dim + d) * L + p0 + k0;  // first element of the run
    float v[kWin];
#pragma unroll
    for (int j = 0; j < kWin; ++j) v[j] = tile[k0 + j][cc];
    if (p0 + k0 + kWin <= L && (e0 & 7) == 0) {
      // a whole run of 8 starting at a multiple of 8 elements: 16-byte (bf16) / 32-byte accesses
      if (z) {
        Run8<T> zr;
        float zz[kWin];
        zr.load(z + e0);
        zr.template unpack<false>(zz);
#pragma unroll
        for (int j = 0; j < kWin; ++j) v[j] *= silu_f(zz[j]);
      }
      store8(out + e0, v);
    } else {
      for (int j = 0; j < kWin && p0 + k0 + j < L; ++j) {
        float w = v[j];
        if (z) w *= silu_f(ld_act(z, e0 + j));
        st_act(out, e0 + j, w);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Long Vim sequences: lanes over positions, with an associative scan of (decay, state) pairs.
//
// A sequence longer than an LDS row is otherwise split into chunks whose end states a chunk pass
// recomputes from a zero start: a second exp2 per (position, state, direction) for almost the
// whole sequence.  Here one workgroup of two waves takes one (batch, channel): wave 0 the forward
// direction, wave 1 the backward one.  A lane owns a run of kRun consecutive positions, so a wave
// covers a segment of kSeg positions, and the segments are walked in scan order with the state
// carried between them.  Per state n and segment each lane
//  * computes its run's decays a_t = exp2(Δ2_t A_n) and inputs b_t = Δ_t u_t B_t,n once and
//    keeps them in registers, folding them into the run's transform h -> P h + H from a zero
//    state (P = exp2(A_n Σ Δ2) is the run's total decay);
//  * combines the transforms of the earlier lanes with an inclusive DPP scan across the wave
//    (row_shr 1, 2, 4, 8 within rows of 16 lanes, then row_bcast 15 and 31 across rows), the
//    pair (P1, H1) followed by (P2, H2) composing to (P1 P2, P2 H1 + H2);
//  * shifts that scan by one lane (wave_shr 1) for the state entering its run, applies it to the
//    state entering the segment, and walks the run again from there with the kept a_t, b_t,
//    accumulating y_t += C_t,n h_t.
// So the carry between lanes costs the scan's few operations per run and state, not a second
// exp2.  The backward wave takes the runs of a segment in reverse lane order (lane k the run
// 63 - k, walked backwards), so its scan also runs up the lanes.  Positions past the sequence end
// have Δ = 0 and input 0, the identity transform.
//
// The two directions meet in the middle through an LDS row of the whole sequence: in the first
// phase the forward wave takes the first half of the segments and the backward wave the second
// half, each storing its y (with D u) in the row; after a barrier each takes the other half, adds
// the stored value, applies the gate 0.5 (y_f + y_b) silu(z) and stores the outputs.  A lane's
// run is contiguous in memory, so a wave's loads and stores are whole contiguous segments.
// B and C are read directly from the inputs ([batch][state][position]): every lane of a segment
// reads a different run, so no copy would be shared.

constexpr int kRun = 16;              // positions per lane
constexpr int kSeg = kW * kRun;       // positions per wave segment
constexpr int kLaneMaxL = 8192;       // longest sequence taken (its LDS row is 32 KB)
constexpr int kNMax = 32;             // largest d_state

// N consecutive elements of a row, any alignment; past n (n <= 0: all) they read as zero and are
// not accessed.
template <typename T, int N>
struct RunN {
  Run8<T> r[N / kWin];
  __device__ __forceinline__ void load(const T* p, int n) {
    if (n >= N) {
#pragma unroll
      for (int k = 0; k < N / kWin; ++k) r[k].load(p + kWin * k);
    } else {
#pragma unroll
      for (int k = 0; k < N / kWin; ++k) r[k].load_part(p + kWin * k, n - kWin * k);
    }
  }
  // v[i] = element i (REV: element N - 1 - i)
  template <bool REV>
  __device__ __forceinline__ void unpack(float (&v)[N]) const {
#pragma unroll
    for (int k = 0; k < N / kWin; ++k) {
      float t[kWin];
      r[k].template unpack<REV>(t);
#pragma unroll
      for (int j = 0; j < kWin; ++j) v[REV ? N - kWin * (k + 1) + j : kWin * k + j] = t[j];
    }
  }
};

// One DPP step of the inclusive scan: each lane composes the transform of the lane the control
// selects (earlier in the wave) before its own, H += P H_src, P *= P_src.  Both are single VOP2
// instructions with the shifted operand read through DPP; a lane without a source (row_shr past its
// row's start) or outside the row mask is not written, which is the identity (1, 0) for free.  A
// DPP operand must not be read within two wait states of the VALU write that produced it, so each
// DPP instruction is preceded by s_nop 1.
#define VMSCAN_SCAN_STEP(CTRL)                                                                    \
  asm volatile("s_nop 1\n\tv_fmac_f32_dpp %0, %0, %1 " CTRL " bank_mask:0xf\n\t"                 \
               "s_nop 1\n\tv_mul_f32_dpp %1, %1, %1 " CTRL " bank_mask:0xf"                        \
               : "+v"(H), "+v"(P))

// Inclusive scan of the lanes' transforms over the wave (lane 0 first), then shifted by one lane:
// on return (P, H) is the composition of the transforms of lanes 0 .. lane - 1 (lane 0: identity).
__device__ __forceinline__ void wave_exclusive_scan(float& P, float& H) {
  VMSCAN_SCAN_STEP("row_shr:1 row_mask:0xf");
  VMSCAN_SCAN_STEP("row_shr:2 row_mask:0xf");
  VMSCAN_SCAN_STEP("row_shr:4 row_mask:0xf");
  VMSCAN_SCAN_STEP("row_shr:8 row_mask:0xf");
  VMSCAN_SCAN_STEP("row_bcast:15 row_mask:0xa");  // lane 15 of rows 0 and 2 into rows 1 and 3
  VMSCAN_SCAN_STEP("row_bcast:31 row_mask:0xc");  // lane 31 into rows 2 and 3
  asm volatile("s_nop 1" ::: "memory");            // the shift below reads P and H through DPP too
  P = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.0f), __float_as_int(P), 0x138, 0xf, 0xf, false));
  H = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(H), 0x138, 0xf, 0xf, false));  // wave_shr:1
}
#undef VMSCAN_SCAN_STEP

// One segment of one direction: the lane's run, every state, and its half of the combination.
// FULL: the whole segment lies inside the sequence (every segment but possibly the last), so no
// lane needs bound checks.
template <typename T, int DIR, int PHASE, bool FULL>
__device__ __forceinline__ void lane_segment(const ScanArgs& a, const DirArgs& da, int b, int d, int s, int lane,
                                             float* row, float* carry) {
  const int L = static_cast<int>(a.L);
  const int ns = a.ns;
  const int p0 = s * kSeg + kRun * (DIR == 0 ? lane : kW - 1 - lane);  // the run's first position
  const int nv = FULL ? kRun : L - p0;                                   // positions of it in the sequence
  constexpr bool kRev = DIR == 1;  // index i of the run in scan order: position p0 + i, or p0 + kRun - 1 - i
  const int64_t rbase = static_cast<int64_t>(b) * a.u_bs + static_cast<int64_t>(d) * L + p0;
  float dl[kRun], du[kRun], y[kRun];
  float S = 0.0f;
  {
    RunN<T, kRun> ur, xr;
    ur.load(static_cast<const T*>(da.u) + rbase, nv);
    xr.load(static_cast<const T*>(da.draw) + static_cast<int64_t>(b) * da.draw_bs + static_cast<int64_t>(d) * L + p0, nv);
    float uu[kRun], xx[kRun];
    ur.template unpack<kRev>(uu);
    xr.template unpack<kRev>(xx);
    const float bias2 = da.bias[d] * kLog2e;
    const float Dd = da.Dp[d];
#pragma unroll
    for (int i = 0; i < kRun; ++i) {
      const bool in = (kRev ? kRun - 1 - i : i) < nv;
      dl[i] = in ? delta2(xx[i], bias2) : 0.0f;
      du[i] = dl[i] * uu[i] * kLn2;  // Δ u = Δ2 u ln 2
      y[i] = Dd * uu[i];
      S += dl[i];
    }
  }
  const T* Bp = static_cast<const T*>(da.B) + static_cast<int64_t>(b) * da.bc_bs + p0;
  const T* Cp = static_cast<const T*>(da.C) + static_cast<int64_t>(b) * da.bc_bs + p0;
  const float* Al = da.A_log + static_cast<int64_t>(d) * ns;
  RunN<T, kRun> br, cr;
  br.load(Bp, nv);
  cr.load(Cp, nv);
  for (int n = 0; n < ns; ++n) {
    const float A = -expf(Al[n]);
    const int64_t nxt = static_cast<int64_t>(n + 1 < ns ? n + 1 : n) * L;  // the next state's rows (the last: again)
    float bv[kRun], av[kRun];
    br.template unpack<kRev>(bv);
    br.load(Bp + nxt, nv);
    float h = 0.0f;
#pragma unroll
    for (int i = 0; i < kRun; ++i) {
      av[i] = __builtin_amdgcn_exp2f(dl[i] * A);
      bv[i] *= du[i];
      h = __builtin_fmaf(av[i], h, bv[i]);
    }
    float P = __builtin_amdgcn_exp2f(A * S), H = h;
    wave_exclusive_scan(P, H);
    h = __builtin_fmaf(P, carry[n], H);  // the state entering the run
    float cv[kRun];
    cr.template unpack<kRev>(cv);
    cr.load(Cp + nxt, nv);
#pragma unroll
    for (int i = 0; i < kRun; ++i) {
      h = __builtin_fmaf(av[i], h, bv[i]);
      y[i] = __builtin_fmaf(cv[i], h, y[i]);
    }
    // the state leaving the segment: the last lane's (positions past the end leave it unchanged)
    const float hl = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(h), kW - 1));
    if (lane == 0) carry[n] = hl;  // read by this wave only, in order
  }
  if (PHASE == 0) {
#pragma unroll
    for (int i = 0; i < kRun; ++i) {
      const int q = kRev ? kRun - 1 - i : i;
      if (q < nv) row[p0 + q] = y[i];
    }
    return;
  }
  RunN<T, kRun> zr;
  zr.load(static_cast<const T*>(a.z) + rbase, nv);
  float zz[kRun], o[kRun];
  zr.template unpack<false>(zz);
#pragma unroll
  for (int i = 0; i < kRun; ++i) {
    const int q = kRev ? kRun - 1 - i : i;  // o and zz in position order
    o[q] = 0.5f * (y[i] + (q < nv ? row[p0 + q] : 0.0f)) * silu_f(zz[q]);
  }
  T* op = static_cast<T*>(a.out) + rbase;
  if (nv >= kRun) {
#pragma unroll
    for (int k = 0; k < kRun / kWin; ++k) {
      float w[kWin];
#pragma unroll
      for (int j = 0; j < kWin; ++j) w[j] = o[kWin * k + j];
      store8(op + kWin * k, w);
    }
  } else {
#pragma unroll
    for (int q = 0; q < kRun; ++q)
      if (q < nv) st_act(op, q, o[q]);
  }
}

template <typename T, int DIR>
__device__ __forceinline__ void lane_dir(const ScanArgs& a, int b, int d, int lane, float* row, float* carry) {
  const DirArgs& da = DIR == 0 ? a.d0 : a.d1;
  const int nseg = static_cast<int>((a.L + kSeg - 1) / kSeg);
  const int mid = nseg / 2;  // forward: segments [0, mid) first; backward: [mid, nseg) first
  if (lane < a.ns) carry[lane] = 0.0f;
  const int L = static_cast<int>(a.L);
  // segment s with or without bound checks (only the last one can reach past the sequence)
  auto seg = [&](int s, auto phase) {
    constexpr int PH = decltype(phase)::value;
    if ((s + 1) * kSeg <= L) lane_segment<T, DIR, PH, true>(a, da, b, d, s, lane, row, carry);
    else lane_segment<T, DIR, PH, false>(a, da, b, d, s, lane, row, carry);
  };
  using Ph0 = std::integral_constant<int, 0>;
  using Ph1 = std::integral_constant<int, 1>;
  if (DIR == 0) {
    for (int s = 0; s < mid; ++s) seg(s, Ph0{});
  } else {
    for (int s = nseg - 1; s >= mid; --s) seg(s, Ph0{});
  }
  __syncthreads();  // the first phase's values are in the row
  if (DIR == 0) {
    for (int s = mid; s < nseg; ++s) seg(s, Ph1{});
  } else {
    for (int s = mid - 1; s >= 0; --s) seg(s, Ph1{});
  }
}

// Workgroup: two waves on one (batch, channel), wave 0 forward, wave 1 backward.
template <typename T>
__global__ __launch_bounds__(2 * kW) void lane_scan_kernel(ScanArgs a) {
  extern __shared__ float lrow[];           // [L]: the first phase's y
  __shared__ float carry[2][kNMax];         // per direction: the state entering the next segment
  const int nblk = a.batch * a.dim;
  const int lb = logical_block(static_cast<int>(blockIdx.x), nblk);  // one XCD: consecutive channels of a batch row
  const int b = lb / a.dim, d = lb - b * a.dim;
  const int lane = threadIdx.x & (kW - 1);
  if (a.werr_clear && blockIdx.x == 0 && threadIdx.x == 0) *a.werr = 0;  // no bounded waits here
  if (__builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6) == 0)
    lane_dir<T, 0>(a, b, d, lane, lrow, carry[0]);
  else
    lane_dir<T, 1>(a, b, d, lane, lrow, carry[1]);
}

// ---------------------------------------------------------------------------------------------
// Front convolutions: the local mixing that produces the scan input.  Both are streaming kernels
// bound by HBM: the scans are bound by the vector ALU, so recomputing the convolution and SiLU
// in every wave of a scan would cost more issue slots than one pass over the activations, and the
// projections that make Δ, B and C need the convolved activations anyway.

constexpr int kConvMax = 4;  // widest conv1d

// Taps of one channel's width-K filter placed in a width-4 window: causal, tap k multiplies
// x[t - 3 + k] (the filter sits at the right end); reversed, tap i multiplies x[t + i]
// (w[K - 1 - i]).  Width 4 is one 16-byte load (the weights start 16-byte aligned).
__device__ __forceinline__ void conv_taps(const float* w, int64_t d, int K, bool rev, float (&t)[kConvMax]) {
  if (K == kConvMax) {
    const float4 q = *reinterpret_cast<const float4*>(w + d * kConvMax);
    const float v[kConvMax] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int k = 0; k < kConvMax; ++k) t[k] = v[rev ? kConvMax - 1 - k : k];
    return;
  }
#pragma unroll
  for (int k = 0; k < kConvMax; ++k) {
    if (rev) t[k] = k < K ? w[d * K + K - 1 - k] : 0.0f;
    else t[k] = k >= kConvMax - K ? w[d * K + k - (kConvMax - K)] : 0.0f;
  }
}

// Vim: u = silu(b + Σ_k w[k] x[t - (K-1) + k]) (causal, the forward branch) and
// u_b = silu(b_b + Σ_k w_b[k] x[t + (K-1) - k]) (the flipped branch's causal convolution, in
// original token order), depthwise, from one read of x.
//
// Vim front, flat form: thread k computes the E outputs at flat positions f = E k .. E k + E - 1 of
// the [rows][L] tensors (both branches) from the aligned 16-byte blocks x[f - 8, f + E + 8): no
// staging and no barrier, so every wave goes from its loads to its stores on its own, and the
// neighbours' reads of the same blocks hit in L1.  (A form that stages each span of rows in LDS
// and a grid-stride form that keeps the next run's loads in flight take the same time on the
// Vim-Ti front, 21-22 us: the write-heavy stream, one read for two outputs, sets it.)  With E = 16
// the halo blocks are a third of the loads instead of two thirds, and the fronts take 1.5-4% less
// time than with 8 (32 costs registers and is slower).  A run can cross one row boundary (rows of
// at least E positions): positions of the window are masked per row (the previous row, the run's
// first row r0, the next row r0 + 1), and each output takes the convolution of its own row, with
// its row's taps.  Rows shorter than E positions go element by element.
constexpr int kConvRun = 16;  // outputs per thread of the Vim front (E)

template <typename T, int E>
__global__ __launch_bounds__(256) void conv1d_flat_kernel(const T* __restrict__ x, const float* __restrict__ w,
                                                          const float* __restrict__ bias,
                                                          const float* __restrict__ w_b,
                                                          const float* __restrict__ bias_b, T* __restrict__ u,
                                                          T* __restrict__ u_b, int64_t total, int dim, int L, int K) {
  static_assert(E % kWin == 0, "whole 8-element runs per thread");
  constexpr int kHalo = kConvMax - 1;
  constexpr int kR = E / kWin;  // runs of 8 per thread
  const int64_t f = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * E;
  if (f >= total) return;
  const int nbr = u_b ? 2 : 1;
  if (L < E) {
    for (int j = 0; j < E && f + j < total; ++j) {
      const int64_t p = f + j, r = p / L;
      const int t = static_cast<int>(p - r * L);
      const int d = static_cast<int>(r % dim);
      for (int br = 0; br < nbr; ++br) {
        float tap[kConvMax];
        conv_taps(br == 0 ? w : w_b, d, K, br == 1, tap);
        float acc = (br == 0 ? bias : bias_b)[d];
        for (int k = 0; k < kConvMax; ++k) {
          const int tt = br == 0 ? t - kHalo + k : t + k;
          if (tt >= 0 && tt < L) acc = __builtin_fmaf(tap[k], ld_act(x, r * L + tt), acc);
        }
        st_act(br == 0 ? u : u_b, p, silu_f(acc));
      }
    }
    return;
  }
  // xs[i] = x at flat position f - 3 + i, i = 0 .. E + 5 (past either end of the tensor: 0)
  float xs[E + 2 * kHalo];
  {
    float pv[kWin], cv[kR][kWin], nv[kWin];
    Run8<T> rp, rc[kR], rn;
    if (f >= kWin) rp.load(x + f - kWin);
    else rp.load_part(x, 0);
#pragma unroll
    for (int c = 0; c < kR; ++c) {
      const int64_t o = f + kWin * c;
      if (o + kWin <= total) rc[c].load(x + o);
      else rc[c].load_part(x + o, static_cast<int>(total - o > 0 ? total - o : 0));
    }
    if (f + E + kWin <= total) rn.load(x + f + E);
    else rn.load_part(x + f + E, static_cast<int>(total - f - E > 0 ? total - f - E : 0));
    rp.template unpack<false>(pv);
#pragma unroll
    for (int c = 0; c < kR; ++c) rc[c].template unpack<false>(cv[c]);
    rn.template unpack<false>(nv);
#pragma unroll
    for (int i = 0; i < kHalo; ++i) xs[i] = pv[kWin - kHalo + i];
#pragma unroll
    for (int c = 0; c < kR; ++c)
#pragma unroll
      for (int i = 0; i < kWin; ++i) xs[kHalo + kWin * c + i] = cv[c][i];
#pragma unroll
    for (int i = 0; i < kHalo; ++i) xs[kHalo + E + i] = nv[i];
  }
  const int64_t r0 = f / L;
  const int t0 = static_cast<int>(f - r0 * L);
  const int q = L - t0;  // outputs j < q are in row r0, the others in row r0 + 1 (q >= 1, E <= L)
  // the window masked to row r0 (x0) and to row r0 + 1 (x1): window position i is at row
  // position t0 - 3 + i
  float x0[E + 2 * kHalo], x1[E + 2 * kHalo];
#pragma unroll
  for (int i = 0; i < E + 2 * kHalo; ++i) {
    const int tt = t0 - kHalo + i;
    x0[i] = tt >= 0 && tt < L ? xs[i] : 0.0f;
    x1[i] = tt >= L && tt < 2 * L ? xs[i] : 0.0f;
  }
  const int d0 = static_cast<int>(r0 % dim), d1 = d0 + 1 < dim ? d0 + 1 : 0;
  float o[2][E];
#pragma unroll
  for (int br = 0; br < 2; ++br) {
    if (br == 1 && !u_b) break;
    const float* wp = br == 0 ? w : w_b;
    const float* bp = br == 0 ? bias : bias_b;
    float ta[kConvMax], tb[kConvMax];
    conv_taps(wp, d0, K, br == 1, ta);
    conv_taps(wp, d1, K, br == 1, tb);
    const float ba = bp[d0], bb = bp[d1];
#pragma unroll
    for (int j = 0; j < E; ++j) {
      float aa = ba, ab = bb;
#pragma unroll
      for (int k = 0; k < kConvMax; ++k) {
        const int i = br == 0 ? j + k : kHalo + j + k;  // causal: x[t - 3 + k]; reversed: x[t + k]
        aa = __builtin_fmaf(ta[k], x0[i], aa);
        ab = __builtin_fmaf(tb[k], x1[i], ab);
      }
      o[br][j] = silu_f(j < q ? aa : ab);
    }
  }
#pragma unroll
  for (int br = 0; br < 2; ++br) {
    if (br == 1 && !u_b) break;
    T* out = br == 0 ? u : u_b;
#pragma unroll
    for (int c = 0; c < kR; ++c) {
      const int64_t oo = f + kWin * c;
      float v[kWin];
#pragma unroll
      for (int j = 0; j < kWin; ++j) v[j] = o[br][kWin * c + j];
      if (oo + kWin <= total) {
        store8(out + oo, v);
      } else {
        for (int j = 0; j < kWin; ++j)
          if (oo + j < total) st_act(out, oo + j, v[j]);
      }
    }
  }
}

// SS2D: x' = act(b + Σ_{a,c} w[a][c] x[i - 1 + a][j - 1 + c]) (3 x 3, depthwise, zero padding),
// written both row-major (the row scans) and transposed (the column scans), from one read of x.
// One workgroup per 64 x 64 tile of one image.  The tile and its one-pixel border are staged in
// LDS as float (all of a thread's loads issued before any is used; an image that is a single
// aligned tile, like 56 x 56, is read as one flat run of 16-byte blocks); each thread computes a strip
// of 16 rows of one column, sliding the 3 x 3 window down in registers (3 LDS reads per pixel);
// the results then replace the input tile in LDS, and both copies are stored from there in pairs
// of neighbouring elements (one 4-byte store per pair when aligned), rows of the tile for the
// row-major copy and columns for the transposed one.  One LDS tile per workgroup keeps eight
// workgroups resident per CU.
template <typename T>
__device__ __forceinline__ void store_pair(T* p, int64_t e, float v0, float v1, bool two) {
  if (!two) {
    st_act(p, e, v0);
    return;
  }
  if constexpr (sizeof(T) == 2) {
    if ((e & 1) == 0) {
      *reinterpret_cast<uint32_t*>(p + e) =
          static_cast<uint32_t>(f32_to_bf16_rne(v0)) | (static_cast<uint32_t>(f32_to_bf16_rne(v1)) << 16);
      return;
    }
  } else {
    if ((e & 1) == 0) {
      *reinterpret_cast<float2*>(p + e) = make_float2(v0, v1);
      return;
    }
  }
  st_act(p, e, v0);
  st_act(p, e + 1, v1);
}

template <typename T>
__global__ __launch_bounds__(256) void conv2d_front_kernel(const T* __restrict__ x, const float* __restrict__ w,
                                                           const float* __restrict__ bias, int act,
                                                           T* __restrict__ xo, T* __restrict__ xto, int dim, int H,
                                                           int W, int tiles_r, int tiles_c) {
  constexpr int kIn = kTile + 2;
  constexpr int kInS = kIn + 1;        // input tile row stride
  constexpr int kOutS = kTile + 1;     // output tile row stride (same storage)
  constexpr int kLoads = (kIn * kIn + 255) / 256;
  constexpr int kStrip = kTile / 4;    // rows per thread
  __shared__ float tile[kIn * kInS];
  const int64_t blk = blockIdx.x;
  const int tc = static_cast<int>(blk % tiles_c);
  const int tr = static_cast<int>((blk / tiles_c) % tiles_r);
  const int64_t img = blk / (static_cast<int64_t>(tiles_c) * tiles_r);
  const int d = static_cast<int>(img % dim);
  const int64_t base = img * H * W;
  const int r0 = tr * kTile, c0 = tc * kTile;
  float wk[9];
#pragma unroll
  for (int k = 0; k < 9; ++k) wk[k] = w[static_cast<int64_t>(d) * 9 + k];
  const float b = bias[d];
  if (tiles_r == 1 && tiles_c == 1 && (base & (kWin - 1)) == 0) {
    // The image is one tile and starts 8-element aligned: read it as one flat run of aligned
    // 8-element blocks (its tail element by element) and zero the tile cells outside it.
    const int hw = H * W, nblk = hw / kWin;
    for (int c = threadIdx.x; c < nblk; c += 256) {
      Run8<T> r;
      r.load(x + base + c * kWin);
      float v[kWin];
      r.template unpack<false>(v);
#pragma unroll
      for (int j = 0; j < kWin; ++j) {
        const int e = c * kWin + j, rr = e / W;
        tile[(rr + 1) * kInS + e - rr * W + 1] = v[j];
      }
    }
    for (int e = nblk * kWin + threadIdx.x; e < hw; e += 256) {
      const int rr = e / W;
      tile[(rr + 1) * kInS + e - rr * W + 1] = ld_act(x, base + e);
    }
    for (int idx = threadIdx.x; idx < kIn * kIn; idx += 256) {
      const int r = idx / kIn, c = idx - (idx / kIn) * kIn;
      if (r == 0 || c == 0 || r > H || c > W) tile[r * kInS + c] = 0.0f;
    }
  } else {
    float ld[kLoads];
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
      const int idx = static_cast<int>(threadIdx.x) + 256 * k;
      const int r = idx / kIn, c = idx - (idx / kIn) * kIn;
      const int gr = r0 - 1 + r, gc = c0 - 1 + c;
      const bool in = idx < kIn * kIn && gr >= 0 && gr < H && gc >= 0 && gc < W;
      ld[k] = in ? ld_act(x, base + static_cast<int64_t>(gr) * W + gc) : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
      const int idx = static_cast<int>(threadIdx.x) + 256 * k;
      if (idx < kIn * kIn) tile[(idx / kIn) * kInS + idx - (idx / kIn) * kIn] = ld[k];
    }
  }
  __syncthreads();
  const int tx = threadIdx.x & (kTile - 1), ty = threadIdx.x >> 6;
  const int i0 = ty * kStrip;
  float a0[3], a1[3], a2[3], v[kStrip];
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    a0[c] = tile[i0 * kInS + tx + c];
    a1[c] = tile[(i0 + 1) * kInS + tx + c];
  }
#pragma unroll
  for (int k = 0; k < kStrip; ++k) {
#pragma unroll
    for (int c = 0; c < 3; ++c) a2[c] = tile[(i0 + k + 2) * kInS + tx + c];
    float acc = b;
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      acc = __builtin_fmaf(wk[c], a0[c], acc);
      acc = __builtin_fmaf(wk[3 + c], a1[c], acc);
      acc = __builtin_fmaf(wk[6 + c], a2[c], acc);
    }
    v[k] = act ? silu_f(acc) : acc;
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      a0[c] = a1[c];
      a1[c] = a2[c];
    }
  }
  __syncthreads();  // every read of the input tile is done
#pragma unroll
  for (int k = 0; k < kStrip; ++k) tile[(i0 + k) * kOutS + tx] = v[k];
  __syncthreads();
  // row-major copy: pair p = (row i, columns 2q, 2q + 1); 64 x 32 pairs, 8 per thread
  const int q = threadIdx.x & 31, i1 = threadIdx.x >> 5;
#pragma unroll
  for (int k = 0; k < kTile / 8; ++k) {
    const int i = i1 + 8 * k, gr = r0 + i, gc = c0 + 2 * q;
    if (gr < H && gc < W)
      store_pair(xo, base + static_cast<int64_t>(gr) * W + gc, tile[i * kOutS + 2 * q], tile[i * kOutS + 2 * q + 1],
                 gc + 1 < W);
  }
  if (!xto) return;
  // transposed copy [W][H]: pair = (column c, rows 2q, 2q + 1)
#pragma unroll
  for (int k = 0; k < kTile / 8; ++k) {
    const int c = i1 + 8 * k, gc = c0 + c, gr = r0 + 2 * q;
    if (gc < W && gr < H)
      store_pair(xto, base + static_cast<int64_t>(gc) * H + gr, tile[2 * q * kOutS + c], tile[(2 * q + 1) * kOutS + c],
                 gr + 1 < H);
  }
}

// ---------------------------------------------------------------------------------------------
// host side

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Chunk length for a pair scan over L tokens with `base` = batch * channel-groups workgroups per
// chunk: one chunk when it fits an LDS row and there are enough workgroups, else enough chunks
// of at most kKMax tokens to reach kTargetBlocks workgroups.  "Enough" is a quarter of a round: a
// wave of the unsplit scan runs at its own latency-bound pace, so below a round the unsplit call
// takes about the same time whatever the batch (Vim, d_inner 384, L 197, bf16: 69-73 us from 48 to
// 288 workgroups), while the split call grows with it (37, 61, 78, 94 us at 48, 144, 192, 288).
constexpr int64_t kWholeFrom = kTargetBlocks / 4;
int64_t plan_chunk(int64_t base, int64_t L, int64_t forced) {
  if (forced > 0) return forced < kKMax ? (forced < L ? forced : L) : (kKMax < L ? kKMax : L);
  if (L <= kKMax && (base >= kWholeFrom || L <= kMinChunk)) return L;
  // Split: chunks of at most kKSplit positions (four workgroups per CU), at least one full round of
  // kSplitSlots workgroups, and the chunk count raised to fill the last round.
  int64_t nch = ceil_div(L, kKSplit);
  const int64_t want = ceil_div(kSplitSlots, base);
  if (want > nch) nch = want;
  const int64_t fill = ceil_div(base * nch, kSplitSlots) * kSplitSlots / base;
  if (fill > nch && ceil_div(L, fill) >= kMinChunk) nch = fill;
  int64_t K = ceil_div(L, nch);
  if (K < kMinChunk) K = kMinChunk;
  // Whole windows of 8 steps, so that no chunk but the last has a ragged window.  Rounded down: the
  // extra chunk that leaves is a short tail, whereas rounding up drops the chunk count below the
  // one chosen to fill the last round (measured 1-7% slower on split shapes, 5% on the 1248-pixel
  // Vim-Ti workload).
  K = (K / kWin) * kWin;
  if (K > kKSplit) K = (kKSplit / kWin) * kWin;
  return K < L ? K : L;
}

// Backward chunks.  A split adds two passes over the sequence (the forward carries and the adjoint
// records), which only pays when the unsplit walk would leave CUs idle: from kBwdSplitBelow
// workgroups in the walk's launch (`launch_base`: SS2D runs both pairs in one launch) the sequence
// stays whole.  Measured (Vim, d_inner 384, bf16, split against whole): 258 tiles, L 232: 345
// against 367 us; 288 tiles, L 1000 / 3000: 1.42 / 4.16 against 1.57 / 4.75 ms; 384 tiles, L 400 /
// 1000: 742 / 1875 against 695 / 1773 us; SS2D 56x56 (2 x 256 workgroups): 6.61 against 4.99 ms.
// Otherwise the chunks are whole
// multiples m of the forward's chunks Kf, so that the forward carries give the state entering
// each, and as few as still give kBwdTargetBlocks workgroups: three rounds of two per CU.  On the
// 1248-pixel Vim workload (forward chunks of 144) that is m = 1 at d_state 16 and m = 2 at d_state
// 32, the best of m = 1, 2, 3, 4, 6, 8 at both (a target of 1024 gave m = 3 at d_state 32: 2.86
// against 2.70 ms).
constexpr int64_t kBwdSplitBelow = 320;
constexpr int64_t kBwdTargetBlocks = 1536;
int64_t bwd_chunk(int64_t base, int64_t L, int64_t Kf, int64_t launch_base = -1) {
  const int64_t nch_f = ceil_div(L, Kf);
  if (nch_f <= 1 || (launch_base < 0 ? base : launch_base) >= kBwdSplitBelow) return L;
  int64_t m = nch_f / ceil_div(kBwdTargetBlocks, base);
  if (m < 1) m = 1;
  return m * Kf;
}

int64_t groups(int64_t dim) { return ceil_div(dim, kW); }

size_t round256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Every workspace starts with the call's wait status word (int32, 0 = every wait ended), padded
// to 256 bytes; the scratch regions follow.
constexpr size_t kStatusBytes = 256;

// d_state values the forward kernels take: whole parts of 8 states, one wave per direction and part.
bool d_state_ok(int d_state) { return d_state == 16 || d_state == 32; }

// Channel groups weighted by the waves of one workgroup (2 per part), in units of the 4-wave
// workgroup of d_state 16: what the chunk planner counts.
int64_t plan_base(int64_t batch, int64_t dim, int ns) { return batch * groups(dim) * (ns / kN); }

size_t bct_bytes(int64_t batch, int64_t L, int ns = kN) {
  return round256(static_cast<size_t>(batch) * 2 * (ns / kH) * L * kBC * sizeof(float));
}

size_t agg_bytes(int64_t batch, int64_t dim, int64_t L, int64_t K, int ns = kN) {
  const int64_t nch = ceil_div(L, K);
  if (nch <= 1) return 0;
  return round256(static_cast<size_t>(batch) * dim * 2 * nch * (ns + 1) * sizeof(float));
}

bool shape_ok(int64_t batch, int64_t dim, int64_t L) {
  if (batch < 1 || dim < 1 || L < 1) return false;
  if (L >= (int64_t{1} << 31) || dim >= (int64_t{1} << 31) || batch >= (int64_t{1} << 31)) return false;
  if (batch > (int64_t{1} << 62) / dim / L) return false;
  return true;
}

vmscan_status launch_failed(hipError_t e) {
  g_last_hip_error = static_cast<int>(e);
  return VMSCAN_ERR_HIP;
}

// The end of an entry point.  In a build with VMSCAN_CHECK_WAITS the call waits for its kernels and
// reads the workspace's status word, so that a wait between state parts that gave up is reported
// as VMSCAN_ERR_WAIT; otherwise the word is left for the caller to read.
vmscan_status finish_call(vmscan_status st, const void* workspace, hipStream_t stream) {
#ifdef VMSCAN_CHECK_WAITS
  if (st != VMSCAN_OK || !workspace) return st;
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return launch_failed(e);
  int word = 0;
  e = hipMemcpy(&word, workspace, sizeof(word), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return launch_failed(e);
  return word ? VMSCAN_ERR_WAIT : VMSCAN_OK;
#else
  (void)workspace;
  (void)stream;
  return st;
#endif
}

enum { kStagePrepare = 1, kStageScan = 2, kStageAll = 3 };

// Stage kStagePrepare writes the fp32 B/C copy and, for a split sequence, runs the chunk-state
// kernel; stage kStageScan runs the main kernel.
template <typename T, int MODE, int NP>
vmscan_status run_pair_np(const ScanArgs& a, hipStream_t stream, int stages) {
  const int64_t nblocks = static_cast<int64_t>(a.batch) * a.nch * a.ngroups;
  const int64_t tblocks = static_cast<int64_t>(a.batch) * 2 * ceil_div(a.L, kTransThreads);
  if (nblocks >= (int64_t{1} << 31) || tblocks >= (int64_t{1} << 31)) return VMSCAN_ERR_SHAPE;
  hipError_t e;
  if (stages & kStagePrepare) {
    hipLaunchKernelGGL(bc_transpose_kernel<T>, dim3(static_cast<unsigned>(tblocks)), dim3(kTransThreads), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return launch_failed(e);
    if (a.nch > 1) {
      hipLaunchKernelGGL((chunk_state_kernel<T, MODE, NP>), dim3(static_cast<unsigned>(nblocks)), dim3(2 * kW * NP),
                         0, stream, a);
      e = hipGetLastError();
      if (e != hipSuccess) return launch_failed(e);
      const int64_t pblocks = ceil_div(static_cast<int64_t>(a.batch) * a.dim * 2 * a.ns, 256);
      hipLaunchKernelGGL(carry_prefix_kernel, dim3(static_cast<unsigned>(pblocks)), dim3(256), 0, stream, a, a.agg, 0);
      e = hipGetLastError();
      if (e != hipSuccess) return launch_failed(e);
    }
  }
  if (!(stages & kStageScan)) return VMSCAN_OK;
  const size_t smem = sizeof(float) * kW * static_cast<size_t>((a.K + 1) | 1);
  hipLaunchKernelGGL((scan_pair_kernel<T, MODE, NP>), dim3(static_cast<unsigned>(nblocks)), dim3(2 * kW * NP), smem,
                     stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return launch_failed(e);
  return VMSCAN_OK;
}

template <typename T, int MODE>
vmscan_status run_pair(const ScanArgs& a, hipStream_t stream, int stages) {
  if (a.parts == 2) return run_pair_np<T, MODE, 2>(a, stream, stages);
  if (a.parts == 4) return run_pair_np<T, MODE, 4>(a, stream, stages);
  return VMSCAN_ERR_UNSUPPORTED;
}

template <int MODE>
vmscan_status run_pair_dtype(const ScanArgs& a, vmscan_dtype dtype, hipStream_t stream, int stages = kStageAll) {
  return dtype == VMSCAN_F32 ? run_pair<float, MODE>(a, stream, stages)
                             : run_pair<uint16_t, MODE>(a, stream, stages);
}

// The long-sequence Vim forward: one launch, nothing to prepare (stage kStagePrepare is empty).
template <typename T>
vmscan_status run_lane(const ScanArgs& a, hipStream_t stream, int stages) {
  if (!(stages & kStageScan)) return VMSCAN_OK;
  const int64_t nblocks = static_cast<int64_t>(a.batch) * a.dim;
  if (nblocks >= (int64_t{1} << 31) || a.L > kLaneMaxL || a.ns > kNMax) return VMSCAN_ERR_SHAPE;
  hipLaunchKernelGGL(lane_scan_kernel<T>, dim3(static_cast<unsigned>(nblocks)), dim3(2 * kW),
                     sizeof(float) * static_cast<size_t>(a.L), stream, a);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? VMSCAN_OK : launch_failed(e);
}

vmscan_status run_vim(const ScanArgs& a, vmscan_dtype dtype, hipStream_t stream, int stages) {
  if (a.lane_path) return dtype == VMSCAN_F32 ? run_lane<float>(a, stream, stages) : run_lane<uint16_t>(a, stream, stages);
  return run_pair_dtype<kModeVim>(a, dtype, stream, stages);
}

// SS2D workspace: the column pair's fp32 image, its transpose, the transposed x, then the B/C copy
// and the chunk carries shared by both pairs.
struct Ss2dLayout {
  size_t col_img, row_img, xt, bct, agg, total;
};

Ss2dLayout ss2d_layout(int64_t batch, int64_t dim, int64_t L, int64_t K, size_t esz, int ns = kN) {
  Ss2dLayout w{};
  const size_t img = round256(static_cast<size_t>(batch) * dim * L * sizeof(float));
  w.col_img = kStatusBytes;
  w.row_img = w.col_img + img;
  w.xt = w.row_img + img;
  w.bct = w.xt + round256(static_cast<size_t>(batch) * dim * L * esz);
  w.agg = w.bct + bct_bytes(batch, L, ns);
  w.total = w.agg + agg_bytes(batch, dim, L, K, ns);
  return w;
}

// SS2D whole-sequence walk (walk_pair_kernel) or chunked pairs, for sequences longer than an LDS row
// (a chunk length of at least the sequence forces the walk, a shorter one the chunks).  The walk
// runs one wave per state part along the whole sequence, so with fewer (batch, channel-group) tiles
// it fills fewer SIMDs and its time grows with L; the chunked path fills the GPU at any tile count but
// pays the chunk pass.  Measured at d_state 16 (bf16, d_inner 512, walk against the chunked default):
// the walk wins at every L from 160 tiles up (192 tiles, 56x56: 1075 against 1287 us); at 128 tiles
// up to L = 1936 (44x44: 568 against 586 us) but not at 2304 or 3136 (671 against 619 us at 48x48);
// at 96 tiles up to L = 900 (30x30: 243 against 279 us); at 64 tiles nowhere.  d_state 32 keeps the
// threshold its walk was measured at (256 tiles).
constexpr int64_t kWalkTiles = 256;        // d_state 32
constexpr int64_t kWalkTilesAnyL = 160;    // d_state 16: the walk at any L
constexpr int64_t kWalkTilesMid = 128;     // ... for L <= kWalkMidL
constexpr int64_t kWalkMidL = 2048;
constexpr int64_t kWalkTilesShort = 96;    // ... for L <= kWalkShortL
constexpr int64_t kWalkShortL = 1024;
constexpr int kWalkParts = 4;  // state parts per direction in the walk: 4 states each at d_state 16, 8 at 32
bool ss2d_walk(int64_t batch, int64_t dim, int64_t L, int ns, int64_t chunk_len) {
  if (chunk_len > 0) return chunk_len >= L;
  if (L <= kKMax) return false;
  const int64_t tiles = batch * groups(dim);
  if (ns != kN) return tiles >= kWalkTiles;
  return tiles >= kWalkTilesAnyL || (tiles >= kWalkTilesMid && L <= kWalkMidL) ||
         (tiles >= kWalkTilesShort && L <= kWalkShortL);
}

// Walk workspace: the two pairs' float32 rows [batch][group][L][64], the transposed x, and each
// pair's B/C copy.
struct Ss2dWalkLayout {
  size_t rows_r, rows_c, xt, bct_r, bct_c, total;
};

Ss2dWalkLayout ss2d_walk_layout(int64_t batch, int64_t dim, int64_t L, size_t esz, int ns) {
  Ss2dWalkLayout w{};
  const size_t rows = round256(static_cast<size_t>(batch) * groups(dim) * kW * L * sizeof(float));
  w.rows_r = kStatusBytes;
  w.rows_c = w.rows_r + rows;
  w.xt = w.rows_c + rows;
  w.bct_r = w.xt + round256(static_cast<size_t>(batch) * dim * L * esz);
  w.bct_c = w.bct_r + bct_bytes(batch, L, ns);
  w.total = w.bct_c + bct_bytes(batch, L, ns);
  return w;
}

// Launch the batched transpose of nimg R x Cc images of element size esz.
vmscan_status launch_transpose(const void* in, void* out, int64_t nimg, int R, int Cc, size_t esz,
                               hipStream_t stream) {
  const int tr = static_cast<int>(ceil_div(R, kTile)), tc = static_cast<int>(ceil_div(Cc, kTile));
  const int64_t blocks = nimg * tr * tc;
  if (blocks >= (int64_t{1} << 31)) return VMSCAN_ERR_SHAPE;
  if (esz == 4)
    hipLaunchKernelGGL(transpose_kernel<float>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                       static_cast<const float*>(in), static_cast<float*>(out), R, Cc, tr, tc);
  else
    hipLaunchKernelGGL(transpose16_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(in), static_cast<uint16_t*>(out), R, Cc, tr, tc);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? VMSCAN_OK : launch_failed(e);
}

// The workspace: may be absent when nothing is needed, else at least `need` bytes; 16-byte
// aligned when given.
vmscan_status check_workspace(const void* workspace, size_t workspace_bytes, size_t need) {
  if (need > 0 && (!workspace || workspace_bytes < need)) return VMSCAN_ERR_WORKSPACE;
  return workspace && !aligned16(workspace) ? VMSCAN_ERR_ALIGN : VMSCAN_OK;
}

// Validation and kernel arguments of the bidirectional scan (shared by its entry points).
vmscan_status vim_args(ScanArgs& a, const void* u, const void* delta_raw, const float* delta_bias, const void* u_b,
                       const void* delta_raw_b, const float* delta_bias_b, const void* z, const float* A_log,
                       const float* A_b_log, const void* B, const void* C, const void* B_b, const void* C_b,
                       const float* D, const float* D_b, void* out, int64_t batch, int64_t dim, int64_t seqlen,
                       int d_state, vmscan_dtype dtype, void* workspace, size_t workspace_bytes, int64_t chunk_len) {
  const void* ptrs[] = {u, delta_raw, delta_bias, u_b, delta_raw_b, delta_bias_b, z, A_log, A_b_log, B, C, B_b, C_b,
                        D, D_b, out};
  for (const void* p : ptrs)
    if (!p) return VMSCAN_ERR_NULL;
  if (!shape_ok(batch, dim, seqlen) || (chunk_len < 0 && chunk_len != VMSCAN_CHUNK_LANE_SCAN)) return VMSCAN_ERR_SHAPE;
  if (!d_state_ok(d_state) || (dtype != VMSCAN_F32 && dtype != VMSCAN_BF16)) return VMSCAN_ERR_UNSUPPORTED;
  if (chunk_len == VMSCAN_CHUNK_LANE_SCAN && seqlen > kLaneMaxL) return VMSCAN_ERR_UNSUPPORTED;
  for (const void* p : ptrs)
    if (!aligned16(p)) return VMSCAN_ERR_ALIGN;
  const int ns = d_state;
  const int64_t K = plan_chunk(plan_base(batch, dim, ns), seqlen, chunk_len > 0 ? chunk_len : 0);
  const bool lane = chunk_len == VMSCAN_CHUNK_LANE_SCAN;  // the status word is all that path uses
  const vmscan_status ws = check_workspace(
      workspace, workspace_bytes,
      kStatusBytes + (lane ? 0 : bct_bytes(batch, seqlen, ns) + agg_bytes(batch, dim, seqlen, K, ns)));
  if (ws != VMSCAN_OK) return ws;
  a.u_bs = dim * seqlen;
  a.z = z;
  a.out = out;
  a.wsy = nullptr;
  a.werr = static_cast<int*>(workspace);
  a.werr_clear = 1;
  a.bct = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + kStatusBytes);
  a.agg = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + kStatusBytes + bct_bytes(batch, seqlen, ns));
  a.d0 = DirArgs{u, delta_raw, dim * seqlen, B, C, ns * seqlen, A_log, D, delta_bias, 0};
  a.d1 = DirArgs{u_b, delta_raw_b, dim * seqlen, B_b, C_b, ns * seqlen, A_b_log, D_b, delta_bias_b, 0};
  a.ns = ns;
  a.parts = ns / kH;
  a.L = seqlen;
  a.dim = static_cast<int>(dim);
  a.batch = static_cast<int>(batch);
  a.K = static_cast<int>(K);
  a.nch = static_cast<int>(ceil_div(seqlen, K));
  a.ngroups = static_cast<int>(groups(dim));
  a.lane_path = lane;
  return VMSCAN_OK;
}

// ---------------------------------------------------------------------------------------------
// Backward pass of the bidirectional scan (gradients of vmscan_fwd_bidir_v2).
//
// Per direction, with g_t = dL/ds_t = dout_t silu(z_t) / 2 (the same for both directions) and
// a_t = exp(Δ_t A), the adjoint λ_t = dL/dh_t runs against the scan order:
//   λ_t = g_t C_t + a_{t+1} λ_{t+1},   λ after the last step = 0
// and gives dC_t = g_t h_t, dB_t = λ_t Δ_t u_t, du_t = g_t D + Δ_t Σ λ_t B_t,
// dΔ_t = Σ λ_t (A a_t h_{t-1} + B_t u_t), dΔ_raw_t = dΔ_t sigmoid(Δ_raw_t + bias),
// dA = Σ λ_t Δ_t a_t h_{t-1} (dA_log = dA A), dD = Σ g_t u_t, dbias = Σ dΔ_raw_t.
//
// Stages (one stream): the B/C copy and chunk carries of the forward; the forward scan with the
// un-gated sum y_f + y_b saved (kModeVimSum); gate_bwd_kernel (g and dz); the backward kernels,
// whose four waves per workgroup (direction x state part of 8, lane = channel; d_state 32: two
// workgroups per tile) each run their direction over the chunk twice: forward, storing the state
// at every 8-step window (bwd_ckpt_kernel), then window by window backwards, recomputing the
// window's states from its checkpoint and walking the adjoint (bwd_scan_kernel); and three small
// kernels that sum the partial results (state parts, directions when
// the branches share inputs, channel groups, batch) and round.  In base-2 units (Δ2 = Δ log2 e,
// B' = B ln 2 from the B/C copy): Σ λ B = log2e Σ λ B', du = Δ2 Σ λ B', dB = ln2 λ Δ2 u and
// dA = ln2 Σ λ Δ2 a h_{t-1}; the ln 2 factors are applied when the partial sums are reduced.

constexpr int kRedCols = 32;              // per lane and reduction round: 2 steps x (8 dB + 8 dC)
constexpr int kRedStride = kRedCols + 4;  // floats per LDS row (16-byte aligned rows)
constexpr int kParStride = 16;            // per (batch, direction, part, channel): dA[8], dD, dbias

struct BwdArgs {
  ScanArgs s;       // forward arguments: B/C copy (bct), per-direction u, Δ_raw, A_log, D, bias; the
                    // chunking (K, nch) and, for split sequences, the forward carries (agg: the state
                    // entering each chunk)
  const float* g;   // [batch][dim][L]: dout silu(z) / 2
  const void* gt;   // ungated SS2D with bf16 activations and unsplit walks, or null: g in the activation
                    // dtype (dout itself, or its transpose for the column pair), read instead of g
  float* ck;        // [batch][dir][part][nch * wpc][dim][8]: state entering each window of each chunk
  float* adj;       // split sequences: [batch][dim][dir][nch][ns + 1] adjoint records, then carries
  float* gu;        // [dir][part / 2][batch][dim][L]: the share of du of a pair of state parts
  float* gx;        // [dir][part / 2][batch][dim][L]: the share of dΔ_raw of a pair of state parts
  float* dbc;       // [dir][group][batch][2][ns][L]: sums over the group's channels of λ Δ2 u (dB / ln2), g h (dC)
  float* dpar;      // [dir][part][dim][kParStride][batch * nch]
  // SS2D with one share per direction (d_state 16), or null: the walk stores dΔ_raw itself, rounded
  // once to the activation dtype; element (b, d, idx) of direction DIR at
  // gx_out + DIR * gx_out_dir + b * gx_out_bs + d * L + idx (else the gx planes and a sum pass).
  void* gx_out;
  int64_t gx_out_dir, gx_out_bs;
  // Vim with separate branches at d_state 16 (one share per direction), or null: the walk rounds and
  // stores direction DIR's du and dΔ_raw itself, [batch][dim][L] each (else the planes and a combine pass).
  void* du_out[2];
  void* dx_out[2];
  int wpc;          // checkpoint slots per chunk (at least the windows of the schedule)
  int msched;       // 1: windows of the forward's two-phase walk, whose checkpoints it stored
  int fnch, fm;     // the forward's chunk count, and forward chunks per backward chunk
};

// SS2D gate backward: g = scale dout silu(z) (float32) and dz = scale dout ysum silu'(z), with
// silu'(z) = σ (1 + z (1 - σ)) and scale 1 for the summed directions; without a gate (z NULL)
// g = dout and there is no dz.  Eight elements per thread (16-byte accesses; the flat arrays start
// 16-byte aligned).
template <typename T>
__global__ __launch_bounds__(256) void gate_bwd_kernel(const T* __restrict__ dout, const T* __restrict__ z,
                                                       const float* __restrict__ ysum, float* __restrict__ g,
                                                       T* __restrict__ dz, int64_t n, float scale) {
  const int64_t i0 = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * kWin;
  if (i0 >= n) return;
  if (i0 + kWin <= n) {
    Run8<T> dr, zr;
    Run8<float> yr;
    float go[kWin], zz[kWin], ys[kWin], gv[kWin], dv[kWin];
    dr.load(dout + i0);
    dr.template unpack<false>(go);
    if (!z) {
#pragma unroll
      for (int j = 0; j < kWin; ++j) gv[j] = scale * go[j];
      store8(g + i0, gv);
      return;
    }
    zr.load(z + i0);
    yr.load(ysum + i0);
    zr.template unpack<false>(zz);
    yr.template unpack<false>(ys);
#pragma unroll
    for (int j = 0; j < kWin; ++j) {
      const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-zz[j] * kLog2e));
      gv[j] = scale * go[j] * zz[j] * sg;
      dv[j] = scale * go[j] * ys[j] * sg * (1.0f + zz[j] * (1.0f - sg));
    }
    store8(g + i0, gv);
    store8(dz + i0, dv);
    return;
  }
  for (int64_t i = i0; i < n; ++i) {
    const float go = ld_act(dout, i);
    if (!z) {
      g[i] = scale * go;
      continue;
    }
    const float zz = ld_act(z, i);
    const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-zz * kLog2e));
    g[i] = scale * go * zz * sg;
    st_act(dz, i, scale * go * ysum[i] * sg * (1.0f + zz * (1.0f - sg)));
  }
}

// Weighted column sums over the wave's 64 lanes of the 32 values each lane stored in its LDS row:
// lane c (c < 32) returns the sum over rows r of rows[r][c] * wts[c / 8][r], lanes 32-63 the same
// sums.  Each weight row holds one weight per lane (channel), kWtStride floats apart, so that the
// four rows a 16-byte read touches start in different banks.
constexpr int kWtStride = kW + 4;
constexpr int kWtFloats = 4 * kWtStride;
__device__ __forceinline__ float wave_column_dot(const float* rows, const float* wts, int lane) {
  const int c = lane & 31, r0 = (lane >> 5) * 32;
  const float* wr = wts + (c >> 3) * kWtStride + r0;
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // four chains, so the FMAs overlap the LDS reads
#pragma unroll
  for (int r = 0; r < 32; r += 4) {
    const float4 wv = *reinterpret_cast<const float4*>(wr + r);
    acc[0] = __builtin_fmaf(rows[(r0 + r) * kRedStride + c], wv.x, acc[0]);
    acc[1] = __builtin_fmaf(rows[(r0 + r + 1) * kRedStride + c], wv.y, acc[1]);
    acc[2] = __builtin_fmaf(rows[(r0 + r + 2) * kRedStride + c], wv.z, acc[2]);
    acc[3] = __builtin_fmaf(rows[(r0 + r + 3) * kRedStride + c], wv.w, acc[3]);
  }
  const float s = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  return s + __shfl_xor(s, 32);
}

// Raw inputs of one full 8-step window of the backward walk, loaded one window ahead: u and
// Δ_raw (activation dtype), g (GT: float32, or the activation dtype when it is dout itself) and the
// checkpoint state entering the window.
template <typename T, int MODE, int DIR, typename GT = float>
struct RevWin {
  using Dr = Dir<MODE, DIR>;
  Run8<T> u, x;
  Run8<GT> g;
  Run8<float> ck;
  __device__ __forceinline__ void load(const ScanArgs& a, const T* ub, const T* xb, const GT* gb, const float* ckp,
                                       const Lane& l, int i0) {
    const int64_t p = Dr::pos(l, i0);
    const int64_t lo = Dr::kPosSgn > 0 ? p : p - (kWin - 1);  // lowest position of the window
    const int64_t si = Dr::sidx(a, l, i0);
    u.load(ub + lo);
    x.load(xb + (Dr::kSidxSgn > 0 ? si : si - (kWin - 1)));
    g.load(gb + lo);
    ck.load(ckp);
  }
};

// Steps [i0, i0 + kWin) of the checkpoint walk: the state only, so only B is read.  A step is too
// short to cover a scalar load's latency at the two waves per SIMD this pass gets, so B comes two
// steps at a time, requested two steps before use (one wait per pair: scalar loads may return out
// of order).  On entry bA holds B of steps i0, i0 + 1; on exit that of i0 + kWin, i0 + kWin + 1
// (reads past a row's end stay inside the B/C copy, as in run_steps).
// Forward over the sequence, storing the state entering each 8-step window (the steps of a last,
// partial window are not needed: nothing follows them).  Its own kernel: it needs few registers
// and so runs at full occupancy.
template <typename T, int MODE, int DIR>
__device__ __forceinline__ void bwd_ckpt_dir(const BwdArgs& ba, const Lane& l) {
  const ScanArgs& a = ba.s;
  using Dr = Dir<MODE, DIR>;
  const DirArgs& da = DIR == 0 ? a.d0 : a.d1;
  const int L = l.Kc;  // steps of this chunk
  float A[kH];
  load_a2(da, l, a.ns, A);
  const float bias2 = da.bias[l.dd] * kLog2e;
  const scalar_fp bct = bc_row<DIR>(a, l);
  float* ckw = ba.ck + ((static_cast<int64_t>(l.b) * 2 + DIR) * a.parts + l.part) * a.nch * ba.wpc * a.dim * kH;
  auto ck_at = [&](int w) {
    return ckw + ((static_cast<int64_t>(l.c) * ba.wpc + w) * a.dim + l.dd) * kH;
  };
  const int full_end = (L / kWin) * kWin;
  float h[kH];
  if (ba.fnch > 1) {
    // the state entering the chunk, left by the forward's carry prefix for its forward chunk
    // where this direction enters: the first, or (backward direction) the last of the chunk's
    const int last = (l.c + 1) * ba.fm < ba.fnch ? (l.c + 1) * ba.fm - 1 : ba.fnch - 1;
    const int cf = DIR == 0 ? l.c * ba.fm : last;
    const float* e = a.agg + ((((static_cast<int64_t>(l.b) * a.dim + l.dd) * 2 + DIR) * ba.fnch) + cf) * (a.ns + 1);
#pragma unroll
    for (int n = 0; n < kH; ++n) h[n] = e[kH * l.part + n];
  } else {
#pragma unroll
    for (int n = 0; n < kH; ++n) h[n] = 0.0f;
  }
  Window<T, MODE, DIR> win;
  float bA[2 * kH], bB[2 * kH];
  if (full_end > 0) {
#pragma unroll
    for (int q = 0; q < kH; ++q) {
      bA[q] = bct[Dr::pos(l, 0) * kBC + q];
      bA[kH + q] = bct[Dr::pos(l, 1) * kBC + q];
    }
    win.load(a, l, da, 0);
  }
  for (int i0 = 0; i0 < full_end; i0 += kWin) {
    if (l.valid) store8(ck_at(i0 / kWin), h);
    float uu[kWin], xr[kWin], dl[kWin], du[kWin];
    win.unpack(uu, xr);
    __builtin_amdgcn_sched_barrier(0);  // see chunk_state_dir
    win.load(a, l, da, i0 + kWin < full_end ? i0 + kWin : i0);
    prep_window(uu, xr, bias2, dl, du);
    ckpt_steps<MODE, DIR>(l, i0, dl, du, A, h, bA, bB, bct);
  }
  if (full_end < L && l.valid) store8(ck_at(full_end / kWin), h);
}

// The backward kernels run one argument set, or two (SETS = 2: the two SS2D pairs in one launch,
// the first set's workgroups first); both sets have the same workgroup count and d_state.
// The backward walks of different state parts are independent, so its workgroups always hold four
// waves (two directions x two parts): d_state 32 runs two workgroups per (batch, chunk, channel
// group), adjacent in the XCD-local order (they read the same inputs), the second on parts 2, 3.
__device__ __forceinline__ int bwd_blocks(const ScanArgs& a) { return a.batch * a.nch * a.ngroups * (a.parts >> 1); }

__device__ __forceinline__ Lane bwd_lane(const ScanArgs& a, int bid) {
  const int pq = a.parts >> 1;
  const int t = logical_block(bid, bwd_blocks(a));
  Lane l = lane_at(a, t / pq);
  l.part += 2 * (t % pq);
  return l;
}

template <typename T, int MODE>
__device__ __forceinline__ void bwd_ckpt_block(const BwdArgs& ba, int bid) {
  const Lane l = bwd_lane(ba.s, bid);
  if ((__builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6) & 1) == 0) bwd_ckpt_dir<T, MODE, 0>(ba, l);
  else bwd_ckpt_dir<T, MODE, 1>(ba, l);
}

template <typename T, int MODE, int SETS>
__global__ __launch_bounds__(kThreads) void bwd_ckpt_kernel(BwdArgs b0, BwdArgs b1) {
  const int nb = bwd_blocks(b0.s), bid = static_cast<int>(blockIdx.x);
  if (SETS == 1 || bid < nb) bwd_ckpt_block<T, MODE>(b0, bid);
  else bwd_ckpt_block<T, MODE>(b1, bid - nb);
}

// Adjoint chunk records (split sequences).  Within a chunk the adjoint obeys
//   λ_i = g_i C_i + a_{i+1} λ_{i+1}
// and, written from its last step's successor, λ_i = λ_i^0 + (a_{i+1} ... a_{Kc-1}) μ, where λ^0 is
// the walk started from zero and μ = a λ is what the next chunk in scan order passes back.  So each
// chunk passes X = a_0 λ_0^0 + (a_0 ... a_{Kc-1}) μ to the previous one: a reverse carry prefix over
// the records (X, Σ Δ2) gives every chunk its μ.  This pass computes the records: per direction and
// state part, the walk from zero over the chunk's steps, last first (windows of 8 with the previous
// window's loads in flight).  It needs no forward state.
// Steps j, j - 1 (of the window at i0) of the adjoint-record walk, which runs against the scan
// order: λ = g C + a λ' with a the later step's decay.  Only C is read, two steps at a time as in
// ckpt_pair: the pair waits for its own C (cur, requested two steps ago) and requests that of steps
// j - 2, j - 3 into nxt.  This walk runs towards a row's other end, so the request is clamped to
// the chunk's first step (the last pair re-reads it) instead of reading past the row.
template <int MODE, int DIR>
__device__ __forceinline__ void adj_pair(const Lane& l, int i0, int j, const float (&xr)[kWin], const float (&gg)[kWin],
                                         float bias2, const float (&A)[kH], float (&lam)[kH], float (&anext)[kH],
                                         float& S, const float (&cur)[2 * kH], float (&nxt)[2 * kH], scalar_fp bct) {
  using Dr = Dir<MODE, DIR>;
  const int i2 = i0 + j - 2 > 0 ? i0 + j - 2 : 0, i3 = i0 + j - 3 > 0 ? i0 + j - 3 : 0;
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_sched_barrier(0);
  const scalar_fp p2 = bct + Dr::pos(l, i2) * kBC + kH, p3 = bct + Dr::pos(l, i3) * kBC + kH;
#pragma unroll
  for (int q = 0; q < kH; ++q) {
    nxt[q] = p2[q];
    nxt[kH + q] = p3[q];
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const float d2 = delta2(xr[j - k], bias2);
#pragma unroll
    for (int n = 0; n < kH; ++n) {
      lam[n] = __builtin_fmaf(gg[j - k], cur[kH * k + n], anext[n] * lam[n]);
      anext[n] = __builtin_amdgcn_exp2f(d2 * A[n]);
    }
    S += d2;
  }
}

template <typename T, int MODE, int DIR>
__device__ __forceinline__ void adj_state_dir(const BwdArgs& ba, const Lane& l) {
  const ScanArgs& a = ba.s;
  // The first chunk in scan order passes nothing back.
  if (DIR == 0 ? l.c == 0 : l.c == a.nch - 1) return;
  using Dr = Dir<MODE, DIR>;
  constexpr bool kRevOrder = Dr::kPosSgn < 0;
  const DirArgs& da = DIR == 0 ? a.d0 : a.d1;
  const T* xb = static_cast<const T*>(da.draw) + static_cast<int64_t>(l.b) * da.draw_bs + static_cast<int64_t>(l.dd) * a.L;
  const float* gb = ba.g + static_cast<int64_t>(l.b) * a.u_bs + static_cast<int64_t>(l.dd) * a.L;
  float A[kH];
  load_a2(da, l, a.ns, A);
  const float bias2 = da.bias[l.dd] * kLog2e;
  const scalar_fp bct = bc_row<DIR>(a, l);
  float lam[kH], anext[kH];
#pragma unroll
  for (int n = 0; n < kH; ++n) {
    lam[n] = 0.0f;
    anext[n] = 0.0f;
  }
  float S = 0.0f;
  auto step = [&](float d2, float gv, scalar_fp c) {
#pragma unroll
    for (int n = 0; n < kH; ++n) {
      lam[n] = __builtin_fmaf(gv, c[kH + n], anext[n] * lam[n]);
      anext[n] = __builtin_amdgcn_exp2f(d2 * A[n]);
    }
    S += d2;
  };
  const int Kc = l.Kc, full_end = (Kc / kWin) * kWin;
  for (int i = Kc - 1; i >= full_end; --i)
    step(delta2(ld_act(xb, Dr::sidx(a, l, i)), bias2), gb[Dr::pos(l, i)], bct + Dr::pos(l, i) * kBC);
  Run8<T> xw;
  Run8<float> gw;
  auto wload = [&](int i0) {
    const int64_t p = Dr::pos(l, i0);
    const int64_t si = Dr::sidx(a, l, i0);
    xw.load(xb + (Dr::kSidxSgn > 0 ? si : si - (kWin - 1)));
    gw.load(gb + (Dr::kPosSgn > 0 ? p : p - (kWin - 1)));
  };
  float cA[2 * kH], cB[2 * kH];  // C of two steps, the later one first
  if (full_end > 0) {
    wload(full_end - kWin);
#pragma unroll
    for (int q = 0; q < kH; ++q) {
      cA[q] = bct[Dr::pos(l, full_end - 1) * kBC + kH + q];
      cA[kH + q] = bct[Dr::pos(l, full_end - 2) * kBC + kH + q];
    }
  }
  for (int i0 = full_end - kWin; i0 >= 0; i0 -= kWin) {
    float xr[kWin], gg[kWin];
    xw.template unpack<(Dr::kSidxSgn < 0)>(xr);
    gw.template unpack<kRevOrder>(gg);
    __builtin_amdgcn_sched_barrier(0);
    wload(i0 > 0 ? i0 - kWin : i0);
#pragma unroll
    for (int j = kWin - 1; j >= 0; j -= 4) {
      adj_pair<MODE, DIR>(l, i0, j, xr, gg, bias2, A, lam, anext, S, cA, cB, bct);
      adj_pair<MODE, DIR>(l, i0, j - 2, xr, gg, bias2, A, lam, anext, S, cB, cA, bct);
    }
  }
  if (l.valid) {
    float* rec = ba.adj + ((((static_cast<int64_t>(l.b) * a.dim + l.d) * 2 + DIR) * a.nch) + l.c) * (a.ns + 1);
#pragma unroll
    for (int n = 0; n < kH; ++n) rec[kH * l.part + n] = anext[n] * lam[n];  // X = a_0 λ_0
    if (l.part == 0) rec[a.ns] = S;
  }
}

template <typename T, int MODE>
__device__ __forceinline__ void adj_state_block(const BwdArgs& ba, int bid) {
  const Lane l = bwd_lane(ba.s, bid);
  if ((__builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6) & 1) == 0) adj_state_dir<T, MODE, 0>(ba, l);
  else adj_state_dir<T, MODE, 1>(ba, l);
}

template <typename T, int MODE, int SETS>
__global__ __launch_bounds__(kThreads) void adj_state_kernel(BwdArgs b0, BwdArgs b1) {
  const int nb = bwd_blocks(b0.s), bid = static_cast<int>(blockIdx.x);
  if (SETS == 1 || bid < nb) adj_state_block<T, MODE>(b0, bid);
  else adj_state_block<T, MODE>(b1, bid - nb);
}

// Per-wave LDS staging of one window's outputs, so that each is stored as runs of 8 positions
// (32 bytes per lane) rather than one scattered 4-byte store per step: du and dΔ_raw shares
// [2][step][lane] (conflict-free: lanes on consecutive words) and the dB/dC column sums
// [16 (B/C, state)][step].
constexpr int kStageFloats = 2 * kWin * kW + 2 * kH * kWin;

// Store a window's 8 values v[j] (step j) at the 8 consecutive indices lo..lo+7 that the steps
// occupy in ascending (ASC) or descending order; only the first ns steps when ns < 8.
template <bool ASC, typename O>
__device__ __forceinline__ void store_window(O* base, int64_t lo, const float (&v)[kWin], int ns) {
  if (ns == kWin) {
    float o[kWin];
#pragma unroll
    for (int j = 0; j < kWin; ++j) o[j] = v[ASC ? j : kWin - 1 - j];
    store8(base + lo, o);
    return;
  }
  for (int j = 0; j < ns; ++j) st_act(base, ASC ? lo + j : lo + kWin - 1 - j, v[j]);
}

// Windows of a chunk of Kc steps in the walk's step order: uniform windows of kWin steps from step 0
// (the last one ragged), or, for checkpoints left by the forward scan, its two-phase schedule:
// whole windows up to the middle step M = ceil(Kc / 2) (stopping before the middle token of an
// odd chunk), the steps left before M, whole windows from M, and the steps left at the end.
struct WinSched {
  int Kc, M, nw0, s1, n;
  bool two;
};

__device__ __forceinline__ WinSched win_sched(int msched, int Kc) {
  WinSched w{};
  w.Kc = Kc;
  w.two = msched != 0;
  if (!w.two) {
    w.n = (Kc + kWin - 1) / kWin;
    return w;
  }
  w.M = (Kc + 1) >> 1;
  w.nw0 = ((Kc & 1) ? w.M - 1 : w.M) / kWin;
  w.s1 = w.nw0 + (w.nw0 * kWin < w.M ? 1 : 0);
  w.n = w.s1 + (Kc - w.M + kWin - 1) / kWin;
  return w;
}

// First step i0 and length of window s.
__device__ __forceinline__ void win_at(const WinSched& w, int s, int& i0, int& len) {
  if (!w.two || s < w.nw0) {
    i0 = s * kWin;
  } else if (s < w.s1) {
    i0 = w.nw0 * kWin;
    len = w.M - i0;
    return;
  } else {
    i0 = w.M + (s - w.s1) * kWin;
  }
  len = w.Kc - i0 < kWin ? w.Kc - i0 : kWin;
}

// The adjoint walk of one direction and state part over one chunk, window by window from the last.
template <typename T, int MODE, int DIR, bool GACT = false, bool VDIRECT = false>
__device__ __forceinline__ void bwd_dir(const BwdArgs& ba, const Lane& l, float* rows, float* stage, int* pf) {
  const ScanArgs& a = ba.s;
  using Dr = Dir<MODE, DIR>;
  using GT = typename std::conditional<GACT, T, float>::type;  // g as stored
  constexpr bool kRevOrder = Dr::kPosSgn < 0;  // window positions descend with the step
  const DirArgs& da = DIR == 0 ? a.d0 : a.d1;
  const int L = l.Kc;  // steps of this chunk
  const T* ub = static_cast<const T*>(da.u) + static_cast<int64_t>(l.b) * a.u_bs + static_cast<int64_t>(l.dd) * a.L;
  const T* xb = static_cast<const T*>(da.draw) + static_cast<int64_t>(l.b) * da.draw_bs + static_cast<int64_t>(l.dd) * a.L;
  const GT* gb = (GACT ? static_cast<const GT*>(ba.gt) : reinterpret_cast<const GT*>(ba.g)) +
                 static_cast<int64_t>(l.b) * a.u_bs + static_cast<int64_t>(l.dd) * a.L;
  float A[kH];
  load_a2(da, l, a.ns, A);
  const float bias2 = da.bias[l.dd] * kLog2e;
  const float Dh = l.part == 0 ? da.Dp[l.dd] : 0.0f;
  const scalar_fp bct = bc_row<DIR>(a, l);
  const float vmask = l.valid ? 1.0f : 0.0f;  // lanes past the last channel add nothing to dB/dC
  float* ckw = ba.ck + ((static_cast<int64_t>(l.b) * 2 + DIR) * a.parts + l.part) * a.nch * ba.wpc * a.dim * kH;
  auto ck_at = [&](int w) {
    return ckw + ((static_cast<int64_t>(l.c) * ba.wpc + w) * a.dim + l.dd) * kH;
  };

  // Backward, window by window from the last.
  const int64_t plane = static_cast<int64_t>(a.batch) * a.dim * a.L;
  const int64_t row = static_cast<int64_t>(l.b) * a.u_bs + static_cast<int64_t>(l.dd) * a.L;
  // one plane per direction and pair of parts: [dir][part / 2][batch][dim][L]
  float* guw = ba.gu + (DIR * (a.parts / 2) + l.part / 2) * plane + row;
  float* gxw = ba.gx + (DIR * (a.parts / 2) + l.part / 2) * plane + row;
  const int group = l.d / kW;
  float* dbcw = ba.dbc + ((static_cast<int64_t>(DIR) * a.ngroups + group) * a.batch + l.b) * 2 * a.ns * a.L;
  // The walk starts after the chunk's last step with a λ = μ, passed back by the chunks after it
  // (zero for the last chunk in scan order and for an unsplit sequence).
  // mu = a_{t+1} λ_{t+1}, the part of λ_t that comes from the later steps
  float mu[kH], dA[kH];
  const float* mu0 = ba.adj ? ba.adj + ((((static_cast<int64_t>(l.b) * a.dim + l.dd) * 2 + DIR) * a.nch) + l.c) * (a.ns + 1) +
                                  kH * l.part
                            : nullptr;
#pragma unroll
  for (int n = 0; n < kH; ++n) {
    mu[n] = mu0 ? mu0[n] : 0.0f;
    dA[n] = 0.0f;
  }
  float dD = 0.0f, dbias = 0.0f;
  int nstaged = 0;  // windows staged so far
  float* myrow = rows + l.lane * kRedStride;
  float* wts = rows + kW * kRedStride;  // the column sums' weight rows: [step & 1][B, C][lane]
  RevWin<T, MODE, DIR, GT> rw;
  const WinSched sched = win_sched(ba.msched, L);
  const int nwin = sched.n;
  {
    int i0l, nl;
    win_at(sched, nwin - 1, i0l, nl);
    if (nl == kWin) rw.load(a, ub, xb, gb, ck_at(nwin - 1), l, i0l);
  }
  for (int w = nwin - 1; w >= 0; --w) {
    // Steps j >= ns (only in a partial window) are padding: Δ = 0 and g = 0 make them leave the
    // state and the adjoint unchanged and contribute nothing; their loads use step ns - 1.  A
    // whole window's raw inputs were loaded during the previous window (rw).
    int i0, ns, i0n = 0, nsn = 0;
    win_at(sched, w, i0, ns);
    if (w > 0) win_at(sched, w - 1, i0n, nsn);
    float hs[kH], d2[kWin], uu[kWin], gg[kWin], xr[kWin], sg[kWin];
    if (ns == kWin) {
      rw.u.template unpack<kRevOrder>(uu);
      rw.x.template unpack<(Dr::kSidxSgn < 0)>(xr);
      rw.g.template unpack<kRevOrder>(gg);
      rw.ck.template unpack<false>(hs);
      __builtin_amdgcn_sched_barrier(0);
      if (nsn == kWin) rw.load(a, ub, xb, gb, ck_at(w - 1), l, i0n);  // the next window down
    } else {
      const float* c = ck_at(w);
#pragma unroll
      for (int n = 0; n < kH; ++n) hs[n] = c[n];
#pragma unroll
      for (int j = 0; j < kWin; ++j) {
        const int ij = i0 + (j < ns ? j : ns - 1);
        const int64_t p = Dr::pos(l, ij);
        xr[j] = ld_act(xb, Dr::sidx(a, l, ij));
        uu[j] = ld_act(ub, p);
        gg[j] = j < ns ? ld_act(gb, p) : 0.0f;
      }
      if (nsn == kWin) rw.load(a, ub, xb, gb, ck_at(w - 1), l, i0n);
    }
#pragma unroll
    for (int j = 0; j < kWin; ++j) {
      const float dv = softplus2_sig(__builtin_fmaf(xr[j], kLog2e, bias2), sg[j]);
      d2[j] = j < ns ? dv : 0.0f;
    }
    auto bc_at = [&](int j) { return bct + Dr::pos(l, i0 + (j < ns ? j : ns - 1)) * kBC; };
    // The window is walked in two halves (steps 7..4, then 3..0).  Each half first rebuilds its
    // four states and decays from the checkpoint (the upper half runs through steps 0..3 without
    // keeping them), so only five states and four decays per lane are held at a time.
#pragma unroll
    for (int hf = 1; hf >= 0; --hf) {
      const int j0 = 4 * hf;
      // hiding Δ2 of the lower half's steps from the compiler stops it from keeping the upper
      // half's rebuild decays of those steps through the upper walk (more registers)
      if (hf == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(d2[j]));
      }
      float hq[5][kH];  // hq[0] = state before step j0, hq[1 + k] = state after step j0 + k
      float aq[4][kH];  // aq[k] = decay of step j0 + k
      {
        float hcur[kH], bc0[kBC], bc1[kBC];
#pragma unroll
        for (int n = 0; n < kH; ++n) hcur[n] = hs[n];
        load_bc(bc_at(0), bc0);
#pragma unroll
        for (int j = 0; j < j0 + 4; ++j) {
          float (&cur)[kBC] = (j & 1) ? bc1 : bc0;
          float (&nxt)[kBC] = (j & 1) ? bc0 : bc1;
          __builtin_amdgcn_sched_barrier(0);
          if (j + 1 < j0 + 4) load_bc(bc_at(j + 1), nxt);
          __builtin_amdgcn_sched_barrier(0);
          if (j == j0) {
#pragma unroll
            for (int n = 0; n < kH; ++n) hq[0][n] = hcur[n];
          }
          const float du2 = d2[j] * uu[j];
#pragma unroll
          for (int n = 0; n < kH; ++n) {
            const float an = __builtin_amdgcn_exp2f(d2[j] * A[n]);
            if (j >= j0) aq[j - j0][n] = an;
            hcur[n] = __builtin_fmaf(du2, cur[n], an * hcur[n]);
          }
          if (j >= j0) {
#pragma unroll
            for (int n = 0; n < kH; ++n) hq[1 + j - j0][n] = hcur[n];
          }
        }
      }
      // the upper part's staging area is free once the lower part has read the previous window
      if (hf == 1 && (l.part & 1)) unit_wait(&pf[1], nstaged, a.werr);
      float bc0[kBC], bc1[kBC];
      load_bc(bc_at(j0 + 3), bc1);
#pragma unroll
      for (int r = 1; r >= 0; --r) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int jj = 1; jj >= 0; --jj) {
          const int k = 2 * r + jj, j = j0 + k;
          float (&cur)[kBC] = (j & 1) ? bc1 : bc0;
          float (&nxt)[kBC] = (j & 1) ? bc0 : bc1;
          float lam[kH];
          float P[2] = {0.0f, 0.0f}, Q[2] = {0.0f, 0.0f};  // two chains each
#pragma unroll
          for (int n = 0; n < kH; ++n) {
            lam[n] = __builtin_fmaf(gg[j], cur[kH + n], mu[n]);  // λ_t = g_t C_t + a_{t+1} λ_{t+1}
            mu[n] = aq[k][n] * lam[n];
            const float wv = mu[n] * hq[k][n];  // λ_t a_t h_{t-1}
            Q[n & 1] = __builtin_fmaf(A[n], wv, Q[n & 1]);
            dA[n] = __builtin_fmaf(d2[j], wv, dA[n]);
            P[n & 1] = __builtin_fmaf(lam[n], cur[n], P[n & 1]);
          }
          __builtin_amdgcn_sched_barrier(0);
          if (j > j0) load_bc(bc_at(j - 1), nxt);
          __builtin_amdgcn_sched_barrier(0);
          const float Ps = P[0] + P[1];
          const float dd = __builtin_fmaf(uu[j] * kLog2e, Ps, Q[0] + Q[1]);
          const float gx = sg[j] * dd;
          dbias += j < ns ? gx : 0.0f;
          dD = __builtin_fmaf(gg[j], uu[j], dD);
          stage[j * kW + l.lane] = __builtin_fmaf(d2[j], Ps, Dh * gg[j]);  // du share
          stage[(kWin + j) * kW + l.lane] = gx;                           // dΔ_raw share
          // dB_t and dC_t are channel sums of λ_t Δ2_t u_t and g_t h_t: the lane's λ_t and h_t go to
          // its row, its Δ2_t u_t and g_t to the weight rows (zero past the last channel)
          float4* dst = reinterpret_cast<float4*>(myrow + jj * 2 * kH);
          dst[0] = make_float4(lam[0], lam[1], lam[2], lam[3]);
          dst[1] = make_float4(lam[4], lam[5], lam[6], lam[7]);
          dst[2] = make_float4(hq[k + 1][0], hq[k + 1][1], hq[k + 1][2], hq[k + 1][3]);
          dst[3] = make_float4(hq[k + 1][4], hq[k + 1][5], hq[k + 1][6], hq[k + 1][7]);
          wts[(2 * jj) * kWtStride + l.lane] = vmask * d2[j] * uu[j];
          wts[(2 * jj + 1) * kWtStride + l.lane] = vmask * gg[j];
        }
        // A wave's LDS accesses execute in order, so every lane's row is written before it is
        // read and read before the next round overwrites it; the compiler barriers keep that order.
        asm volatile("" ::: "memory");
        const float sum = wave_column_dot(rows, wts, l.lane);
        asm volatile("" ::: "memory");
        if (l.lane < kRedCols) {
          const int jj = l.lane >> 4, tk = l.lane & 15;  // tk = (B or C) * 8 + state
          stage[2 * kWin * kW + tk * kWin + j0 + 2 * r + jj] = sum;
        }
      }
    }
    // The window's outputs, from the staging areas.  The workgroup's two waves of this direction
    // (parts p and p + 1: waves w and w + 2) walk the same steps: the upper part publishes its du
    // and dΔ_raw shares (pf[0] = windows staged), the lower part adds them to its own, stores the
    // sums and releases the upper part's staging area (pf[1] = windows consumed).  A wave's LDS
    // accesses execute in order, so data written before a flag is seen by whoever sees the flag,
    // and its own dB/dC sums are written before it reads them.
    ++nstaged;
    if (l.part & 1) unit_signal(&pf[0], nstaged);
    else unit_wait(&pf[0], nstaged, a.werr);
    if ((l.part & 1) == 0 && l.valid) {
      const float* up = stage + 2 * kStageFloats;  // wave w + 2
      float v[kWin];
#pragma unroll
      for (int j = 0; j < kWin; ++j) v[j] = stage[j * kW + l.lane] + up[j * kW + l.lane];
      const int64_t plo = Dr::kPosSgn > 0 ? Dr::pos(l, i0) : Dr::pos(l, i0) - (kWin - 1);
      if constexpr (VDIRECT) store_window<(Dr::kPosSgn > 0)>(static_cast<T*>(ba.du_out[DIR]) + row, plo, v, ns);
      else store_window<(Dr::kPosSgn > 0)>(guw, plo, v, ns);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < kWin; ++j) v[j] = stage[(kWin + j) * kW + l.lane] + up[(kWin + j) * kW + l.lane];
      const int64_t slo = Dr::kSidxSgn > 0 ? Dr::sidx(a, l, i0) : Dr::sidx(a, l, i0) - (kWin - 1);
      bool direct = false;  // SS2D only: the Vim walk would carry the branch's registers too
      if constexpr (MODE == kModeSecondPair) direct = ba.gx_out != nullptr;
      if constexpr (VDIRECT) {
        store_window<(Dr::kSidxSgn > 0)>(static_cast<T*>(ba.dx_out[DIR]) + row, slo, v, ns);
      } else if (direct) {
        T* gxo = static_cast<T*>(ba.gx_out) + DIR * ba.gx_out_dir + static_cast<int64_t>(l.b) * ba.gx_out_bs +
                 static_cast<int64_t>(l.dd) * a.L;
        store_window<(Dr::kSidxSgn > 0)>(gxo, slo, v, ns);
      } else {
        store_window<(Dr::kSidxSgn > 0)>(gxw, slo, v, ns);  // Δ_raw's own storage order
      }
    }
    if (l.lane < 2 * kH) {
      const int ty = l.lane >> 3, kk = l.lane & 7;
      float v[kWin];
#pragma unroll
      for (int j = 0; j < kWin; ++j) v[j] = stage[2 * kWin * kW + l.lane * kWin + j];
      const int64_t slo = Dr::kSidxSgn > 0 ? Dr::sidx(a, l, i0) : Dr::sidx(a, l, i0) - (kWin - 1);
      store_window<(Dr::kSidxSgn > 0)>(dbcw + (static_cast<int64_t>(ty) * a.ns + kH * l.part + kk) * a.L, slo, v, ns);
    }
    if ((l.part & 1) == 0) unit_signal(&pf[1], nstaged);
    asm volatile("" ::: "memory");
  }
  if (l.valid) {
    // [dir][part][dim][kParStride][batch * nch]: the sums over batch and chunks read contiguous runs
    const int64_t nbc = static_cast<int64_t>(a.batch) * a.nch;
    float* pp = ba.dpar + ((static_cast<int64_t>(DIR) * a.parts + l.part) * a.dim + l.d) * kParStride * nbc +
                static_cast<int64_t>(l.b) * a.nch + l.c;
#pragma unroll
    for (int n = 0; n < kH; ++n) pp[n * nbc] = dA[n];
    pp[kH * nbc] = l.part == 0 ? dD : 0.0f;
    pp[(kH + 1) * nbc] = dbias;
  }
}

template <typename T, int MODE, bool GACT, bool VDIRECT>
__device__ __forceinline__ void bwd_scan_block(const BwdArgs& ba, int bid, float* rows, float* stage, int (*pflag)[2]) {
  const Lane l = bwd_lane(ba.s, bid);
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  if ((w & 1) == 0) bwd_dir<T, MODE, 0, GACT, VDIRECT>(ba, l, rows, stage, pflag[0]);
  else bwd_dir<T, MODE, 1, GACT, VDIRECT>(ba, l, rows, stage, pflag[1]);
}

// Float32 inputs make the window prefetch 8 registers larger, which takes the walk past 256 registers
// and so to one wave per SIMD; asking for two costs a few bytes of spills and is faster (the SS2D
// walk by about 9%).  The bf16 walk fits two waves without the request and is slower with it.
template <typename T, int MODE, int SETS, bool GACT = false, bool VDIRECT = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(std::is_same<T, float>::value ? 2 : 1)))
void bwd_scan_kernel(BwdArgs b0, BwdArgs b1) {
  __shared__ __attribute__((aligned(16))) float rows[4][kW * kRedStride + kWtFloats];
  __shared__ __attribute__((aligned(16))) float stage[4][kStageFloats];
  __shared__ int pflag[2][2];  // per direction: windows staged by the upper part, consumed by the lower
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  if (threadIdx.x < 4) pflag[threadIdx.x >> 1][threadIdx.x & 1] = 0;
  __syncthreads();
  const int nb = bwd_blocks(b0.s), bid = static_cast<int>(blockIdx.x);
  // one copy of the body: the argument set is picked by address (both live in the kernel
  // argument segment)
  const bool first = SETS == 1 || bid < nb;
  const BwdArgs* ba = first ? &b0 : &b1;
  bwd_scan_block<T, MODE, GACT, VDIRECT>(*ba, first ? bid : bid - nb, rows[w], stage[w], pflag);
}

// du, dΔ_raw (and the backward branch's, or their sums when the branches share inputs):
// elementwise over [batch][dim][L], the np shares per direction (one per pair of state parts)
// added in float32 and rounded once to the activation dtype.
template <typename T>
__global__ __launch_bounds__(256) void bwd_combine_kernel(const float* __restrict__ gu, const float* __restrict__ gx,
                                                          T* du, T* dx, T* du_b, T* dx_b, int64_t n, int np) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  float uf = 0.0f, ubk = 0.0f, xf = 0.0f, xbk = 0.0f;
  for (int k = 0; k < np; ++k) {
    uf += gu[k * n + i];
    ubk += gu[(np + k) * n + i];
    xf += gx[k * n + i];
    xbk += gx[(np + k) * n + i];
  }
  if (du_b) {
    st_act(du, i, uf);
    st_act(du_b, i, ubk);
  } else {
    st_act(du, i, uf + ubk);
  }
  if (dx_b) {
    st_act(dx, i, xf);
    st_act(dx_b, i, xbk);
  } else {
    st_act(dx, i, xf + xbk);
  }
}

// dB, dC, dB_b, dC_b: the channel-group partial sums added up (dB scaled by ln 2), rounded once.
// A thread takes 8 consecutive (state, index) elements of one (batch, direction, B or C) row
// (grid: x over the ns * L elements, a multiple of 16; y over batch x 4), as whole 32-byte loads
// and 16/32-byte stores.
template <typename T>
__global__ __launch_bounds__(256) void bwd_bc_kernel(const float* __restrict__ dbc, T* dB, T* dC, T* dB_b, T* dC_b,
                                                     int batch, int ngroups, int64_t L, int64_t out_bstride, int ns) {
  const int64_t NL = static_cast<int64_t>(ns) * L;
  const int64_t q0 = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * kWin;
  if (q0 >= NL) return;
  for (int y = static_cast<int>(blockIdx.y); y < 4 * batch; y += static_cast<int>(gridDim.y)) {
    const int b = y >> 2, dir = (y >> 1) & 1, ty = y & 1;
    float s[kWin] = {};
    for (int gi = 0; gi < ngroups; ++gi) {
      float v[kWin];
      Run8<float> r;
      r.load(dbc + (((static_cast<int64_t>(dir) * ngroups + gi) * batch + b) * 2 + ty) * NL + q0);
      r.template unpack<false>(v);
#pragma unroll
      for (int j = 0; j < kWin; ++j) s[j] += v[j];
    }
    if (ty == 0) {
#pragma unroll
      for (int j = 0; j < kWin; ++j) s[j] *= kLn2;
    }
    T* dst = ty == 0 ? (dir == 0 ? dB : dB_b) : (dir == 0 ? dC : dC_b);
    store8(dst + static_cast<int64_t>(b) * out_bstride + q0, s);
  }
}

template <typename T>
void launch_bwd_bc(const float* dbc, T* dB, T* dC, T* dB_b, T* dC_b, int batch, int ngroups, int64_t L,
                   int64_t out_bstride, int ns, hipStream_t stream) {
  const int64_t NL = static_cast<int64_t>(ns) * L;
  const dim3 grid(static_cast<unsigned>(ceil_div(NL, 256 * kWin)),
                  static_cast<unsigned>(4 * static_cast<int64_t>(batch) < 65535 ? 4 * batch : 65535));
  hipLaunchKernelGGL(bwd_bc_kernel<T>, grid, dim3(256), 0, stream, dbc, dB, dC, dB_b, dC_b, batch, ngroups, L,
                     out_bstride, ns);
}

// dA_log, dD, dbias per direction: sums over batch (and state parts); for shared inputs
// (dbias_b NULL) the backward branch's dbias is added to the forward one.  One wave per output
// value: the lanes take batch entries (contiguous in the partial-sum layout) and a butterfly
// adds them up.
__device__ __forceinline__ float wave_batch_sum(const float* p, int batch, int lane) {
  float s = 0.0f;
  for (int b = lane; b < batch; b += kW) s += p[b];
#pragma unroll
  for (int m = kW / 2; m >= 1; m >>= 1) s += __shfl_xor(s, m);
  return s;
}

__global__ __launch_bounds__(256) void bwd_param_kernel(const float* __restrict__ dpar, const float* A_log,
                                                        const float* A_b_log, float* dA_log, float* dA_b_log,
                                                        float* dD, float* dD_b, float* dbias, float* dbias_b,
                                                        int batch, int dim, int ns) {
  // items: (dir, d, n) for dA_log, then (dir, d, {dD, dbias})
  const int item = blockIdx.x * 4 + static_cast<int>(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int nA = 2 * dim * ns, parts = ns / kH;
  if (item >= nA + 4 * dim) return;
  auto at = [&](int dr, int pt, int k) {
    return dpar + ((static_cast<int64_t>(dr) * parts + pt) * dim) * kParStride * batch + static_cast<int64_t>(k) * batch;
  };
  if (item < nA) {
    const int dir = item / (dim * ns), d = (item / ns) % dim, n = item % ns;
    const float s = wave_batch_sum(at(dir, n / kH, n % kH) + static_cast<int64_t>(d) * kParStride * batch, batch, lane);
    if (lane == 0) {
      const float An = -expf((dir == 0 ? A_log : A_b_log)[static_cast<int64_t>(d) * ns + n]);
      (dir == 0 ? dA_log : dA_b_log)[static_cast<int64_t>(d) * ns + n] = s * kLn2 * An;
    }
    return;
  }
  const int r = item - nA, dir = r / (2 * dim), d = (r / 2) % dim, which = r & 1;
  const int64_t off = static_cast<int64_t>(d) * kParStride * batch;
  if (which == 0) {
    const float s = wave_batch_sum(at(dir, 0, kH) + off, batch, lane);
    if (lane == 0) (dir == 0 ? dD : dD_b)[d] = s;
    return;
  }
  if (dir == 1 && !dbias_b) return;  // added into dbias by the forward item
  float s = 0.0f;
  for (int pt = 0; pt < parts; ++pt) s += wave_batch_sum(at(dir, pt, kH + 1) + off, batch, lane);
  if (dir == 0 && !dbias_b)
    for (int pt = 0; pt < parts; ++pt) s += wave_batch_sum(at(1, pt, kH + 1) + off, batch, lane);
  if (lane == 0) (dir == 0 ? dbias : dbias_b)[d] = s;
}

// out[b][r] (batch stride out_bstride) = the sum of np float32 planes [batch][n_b] (plane k at
// base + k * pstride) and, if given, one more plane `extra`, at (b, r), in float32, rounded once
// to O.  Used for the SS2D gradients: dx from the row pair's partial planes (two directions x
// pairs of state parts) plus the transposed column-pair plane, dΔ_raw per direction from its
// planes.  A thread takes 8 consecutive elements of one batch entry (grid: x over n_b, y over the
// batch); when n_b is a multiple of 8 they move as whole 32-byte loads and 16/32-byte stores.
template <typename O>
__global__ __launch_bounds__(256) void sum_planes_kernel(const float* base, int np, int64_t pstride,
                                                         const float* extra, O* out, int64_t n_b, int batch,
                                                         int64_t out_bstride) {
  const int64_t r0 = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * kWin;
  if (r0 >= n_b) return;
  for (int b = static_cast<int>(blockIdx.y); b < batch; b += static_cast<int>(gridDim.y)) {
    const int64_t i0 = static_cast<int64_t>(b) * n_b + r0;
    O* o = out + static_cast<int64_t>(b) * out_bstride + r0;
    if (n_b % kWin == 0) {
      float s[kWin] = {};
      for (int k = 0; k < np; ++k) {
        float v[kWin];
        Run8<float> r;
        r.load(base + k * pstride + i0);
        r.template unpack<false>(v);
#pragma unroll
        for (int j = 0; j < kWin; ++j) s[j] += v[j];
      }
      if (extra) {
        float v[kWin];
        Run8<float> r;
        r.load(extra + i0);
        r.template unpack<false>(v);
#pragma unroll
        for (int j = 0; j < kWin; ++j) s[j] += v[j];
      }
      store8(o, s);
    } else {
      for (int j = 0; j < kWin && r0 + j < n_b; ++j) {
        float s = 0.0f;
        for (int k = 0; k < np; ++k) s += base[k * pstride + i0 + j];
        if (extra) s += extra[i0 + j];
        st_act(o, j, s);
      }
    }
  }
}

template <typename O>
void launch_sum_planes(const float* base, int np, int64_t pstride, const float* extra, O* out, int64_t n_b, int batch,
                       int64_t out_bstride, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(ceil_div(n_b, 256 * kWin)), static_cast<unsigned>(batch < 65535 ? batch : 65535));
  hipLaunchKernelGGL(sum_planes_kernel<O>, grid, dim3(256), 0, stream, base, np, pstride, extra, out, n_b, batch,
                     out_bstride);
}

// dx of the SS2D backward in one pass.  The column pair's du shares (np float32 planes in the
// transposed images' order, [img][R = W][Cc = H]) are summed and transposed through an LDS tile, the
// row pair's shares (np planes, [img][H][W]) are summed and added, and the result is rounded once:
// dx = (0 + row_0 + row_1 ...) + (0 + col_0 + col_1 ...)^T, the same sums in the same order as
// summing, transposing and summing again in three passes.
template <typename O>
__device__ __forceinline__ void store4(O* p, const float (&v)[4]);
template <>
__device__ __forceinline__ void store4(float* p, const float (&v)[4]) {
  const float4 r = make_float4(v[0], v[1], v[2], v[3]);
  __builtin_memcpy(p, &r, sizeof(r));
}
template <>
__device__ __forceinline__ void store4(uint16_t* p, const float (&v)[4]) {
  const uint2 r = make_uint2(static_cast<uint32_t>(f32_to_bf16_rne(v[0])) | (static_cast<uint32_t>(f32_to_bf16_rne(v[1])) << 16),
                             static_cast<uint32_t>(f32_to_bf16_rne(v[2])) | (static_cast<uint32_t>(f32_to_bf16_rne(v[3])) << 16));
  __builtin_memcpy(p, &r, sizeof(r));
}

template <typename O>
__global__ __launch_bounds__(256) void dx_merge_kernel(const float* __restrict__ colp, const float* __restrict__ rowp,
                                                       int np, int64_t pstride, O* __restrict__ out, int R, int Cc,
                                                       int tiles_r, int tiles_c) {
  __shared__ float tile[kTile][kTile + 1];
  const int64_t blk = blockIdx.x;
  const int tc = static_cast<int>(blk % tiles_c);
  const int tr = static_cast<int>((blk / tiles_c) % tiles_r);
  const int64_t img = blk / (static_cast<int64_t>(tiles_c) * tiles_r);
  const int64_t ioff = img * R * Cc;
  const int r0 = tr * kTile, c0 = tc * kTile;
  if ((R & 3) == 0 && (Cc & 3) == 0) {
    // both sides multiples of 4: runs of 4 as single 16-byte accesses on both sides
    const int tq = threadIdx.x & 15, tw = threadIdx.x >> 4;
    for (int i = tw; i < kTile; i += 16) {
      const int r = r0 + i, c = c0 + 4 * tq;
      if (r < R && c < Cc) {
        float sum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int k = 0; k < np; ++k) {
          float v[4];
          __builtin_memcpy(v, colp + k * pstride + ioff + static_cast<int64_t>(r) * Cc + c, sizeof(v));
#pragma unroll
          for (int q = 0; q < 4; ++q) sum[q] += v[q];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) tile[i][4 * tq + q] = sum[q];
      }
    }
    __syncthreads();
    for (int i = tw; i < kTile; i += 16) {
      const int c = c0 + i, r = r0 + 4 * tq;
      if (c < Cc && r < R) {
        const int64_t o = ioff + static_cast<int64_t>(c) * R + r;
        float sum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int k = 0; k < np; ++k) {
          float v[4];
          __builtin_memcpy(v, rowp + k * pstride + o, sizeof(v));
#pragma unroll
          for (int q = 0; q < 4; ++q) sum[q] += v[q];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) sum[q] += tile[4 * tq + q][i];
        store4(out + o, sum);
      }
    }
    return;
  }
  const int tx = threadIdx.x & (kTile - 1), ty = threadIdx.x >> 6;
  for (int i = ty; i < kTile; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    if (r < R && c < Cc) {
      float sum = 0.0f;
      for (int k = 0; k < np; ++k) sum += colp[k * pstride + ioff + static_cast<int64_t>(r) * Cc + c];
      tile[i][tx] = sum;
    }
  }
  __syncthreads();
  for (int i = ty; i < kTile; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (c < Cc && r < R) {
      const int64_t o = ioff + static_cast<int64_t>(c) * R + r;
      float sum = 0.0f;
      for (int k = 0; k < np; ++k) sum += rowp[k * pstride + o];
      st_act(out, o, sum + tile[tx][i]);
    }
  }
}

// Backward buffers that depend on the chunking (the forward's: chunks of Kf): checkpoints of every
// window of every chunk, the adjoint records (split sequences only) and the per-chunk parameter sums.
// Checkpoint slots per chunk: its windows, one more for the forward's two-phase schedule.
int64_t ck_slots(int64_t K) { return ceil_div(K, kWin) + 1; }
size_t ck_bytes(int64_t batch, int64_t dim, int64_t L, int64_t Kf, int ns) {
  return round256(static_cast<size_t>(batch) * 2 * (ns / kH) * ceil_div(L, Kf) * ck_slots(Kf) * dim * kH *
                  sizeof(float));
}
size_t dpar_bytes(int64_t batch, int64_t dim, int64_t L, int64_t Kf, int ns) {
  return round256(static_cast<size_t>(batch) * ceil_div(L, Kf) * 2 * (ns / kH) * dim * kParStride * sizeof(float));
}
// the dB / dC partial sums: [dir][group][batch][2][ns][L]
size_t dbc_bytes(int64_t batch, int64_t dim, int64_t L, int ns) {
  return round256(static_cast<size_t>(2) * groups(dim) * batch * 2 * ns * L * sizeof(float));
}

struct BwdLayout {
  size_t bct, agg, g, ck, adj, gu, gx, dbc, dpar, total;
};

// The planes of du / dΔ_raw shares are [dir][part / 2][batch][dim][L], rounded up to 256 bytes only
// as a whole block: the kernels index plane k at k * batch * dim * L elements.
BwdLayout bwd_layout(int64_t batch, int64_t dim, int64_t L, int64_t Kf, int ns) {
  BwdLayout w{};
  const size_t planes = round256(static_cast<size_t>(2) * (ns / kH / 2) * batch * dim * L * sizeof(float));
  const size_t plane = round256(static_cast<size_t>(batch) * dim * L * sizeof(float));
  const int64_t Kb = bwd_chunk(plan_base(batch, dim, ns), L, Kf);
  w.bct = kStatusBytes;  // after the status word, as in the forward's workspace
  w.agg = w.bct + bct_bytes(batch, L, ns);
  w.g = w.agg + agg_bytes(batch, dim, L, Kf, ns);
  w.ck = w.g + plane;
  w.adj = w.ck + ck_bytes(batch, dim, L, Kb, ns);
  w.gu = w.adj + agg_bytes(batch, dim, L, Kb, ns);
  w.gx = w.gu + planes;
  w.dbc = w.gx + planes;
  w.dpar = w.dbc + dbc_bytes(batch, dim, L, ns);
  w.total = w.dpar + dpar_bytes(batch, dim, L, Kb, ns);
  return w;
}

// Checkpoints, then (split sequences) the adjoint records and their reverse carry prefix, then the
// adjoint walk; every kernel runs one workgroup per (set, batch, chunk, channel group, pair of
// state parts).  SETS = 2 runs b0 and b1 (same shapes, d_state and chunking) in the same launches.
template <typename T, int MODE, int SETS>
vmscan_status launch_bwd_scans(const BwdArgs& b0, const BwdArgs& b1, hipStream_t stream) {
  const ScanArgs& a = b0.s;
  const int64_t nblocks = static_cast<int64_t>(a.batch) * a.nch * a.ngroups * (a.parts / 2) * SETS;
  if (nblocks >= (int64_t{1} << 31)) return VMSCAN_ERR_SHAPE;
  const dim3 grid(static_cast<unsigned>(nblocks));
  hipError_t e;
  if (!b0.msched) {  // else the forward scan stored the checkpoints
    hipLaunchKernelGGL((bwd_ckpt_kernel<T, MODE, SETS>), grid, dim3(kThreads), 0, stream, b0, b1);
    e = hipGetLastError();
    if (e != hipSuccess) return launch_failed(e);
  }
  if (a.nch > 1) {
    hipLaunchKernelGGL((adj_state_kernel<T, MODE, SETS>), grid, dim3(kThreads), 0, stream, b0, b1);
    e = hipGetLastError();
    if (e != hipSuccess) return launch_failed(e);
    const int64_t pblocks = ceil_div(static_cast<int64_t>(a.batch) * a.dim * 2 * a.ns, 256);
    for (int k = 0; k < SETS; ++k) {
      const BwdArgs& b = k == 0 ? b0 : b1;
      hipLaunchKernelGGL(carry_prefix_kernel, dim3(static_cast<unsigned>(pblocks)), dim3(256), 0, stream, b.s, b.adj, 1);
      e = hipGetLastError();
      if (e != hipSuccess) return launch_failed(e);
    }
  }
  if constexpr (MODE == kModeVim) {
    if (b0.du_out[0]) {  // separate branches: the walk stores du and dΔ_raw
      hipLaunchKernelGGL((bwd_scan_kernel<T, MODE, SETS, false, true>), grid, dim3(kThreads), 0, stream, b0, b1);
      e = hipGetLastError();
      return e == hipSuccess ? VMSCAN_OK : launch_failed(e);
    }
  }
  if constexpr (MODE == kModeSecondPair && std::is_same<T, uint16_t>::value) {
    if (b0.gt) {  // g in the activation dtype (both sets)
      hipLaunchKernelGGL((bwd_scan_kernel<T, MODE, SETS, true>), grid, dim3(kThreads), 0, stream, b0, b1);
      e = hipGetLastError();
      return e == hipSuccess ? VMSCAN_OK : launch_failed(e);
    }
  }
  hipLaunchKernelGGL((bwd_scan_kernel<T, MODE, SETS>), grid, dim3(kThreads), 0, stream, b0, b1);
  e = hipGetLastError();
  return e == hipSuccess ? VMSCAN_OK : launch_failed(e);
}


template <typename T>
vmscan_status run_bwd(const ScanArgs& fwd, const BwdLayout& lay, unsigned char* wsp, const void* dout, const void* z,
                      void* du, void* dx, float* dbias, void* du_b, void* dx_b, float* dbias_b, void* dz,
                      const float* A_log, const float* A_b_log, float* dA_log, float* dA_b_log, void* dB, void* dC,
                      void* dB_b, void* dC_b, float* dD, float* dD_b, hipStream_t stream) {
  const int ns = fwd.ns;
  const int64_t n = static_cast<int64_t>(fwd.batch) * fwd.dim * fwd.L;
  const int64_t nbc = static_cast<int64_t>(2) * fwd.batch * 2 * ns * fwd.L;
  if (ceil_div(n, 256) >= (int64_t{1} << 31) || ceil_div(nbc, 256) >= (int64_t{1} << 31)) return VMSCAN_ERR_SHAPE;
  float* g = reinterpret_cast<float*>(wsp + lay.g);
  BwdArgs ba{};
  ba.s = fwd;  // the forward's carries (the state entering each forward chunk) are in agg
  const int64_t Kb = bwd_chunk(plan_base(fwd.batch, fwd.dim, ns), fwd.L, fwd.K);
  ba.s.K = static_cast<int>(Kb);
  ba.s.nch = static_cast<int>(ceil_div(fwd.L, Kb));
  ba.fnch = ba.s.nch > 1 ? fwd.nch : 1;  // an unsplit walk starts from zero and reads no carries
  ba.fm = ba.s.nch > 1 ? static_cast<int>(Kb / fwd.K) : 1;
  ba.g = g;
  ba.ck = reinterpret_cast<float*>(wsp + lay.ck);
  ba.adj = ba.s.nch > 1 ? reinterpret_cast<float*>(wsp + lay.adj) : nullptr;
  ba.gu = reinterpret_cast<float*>(wsp + lay.gu);
  ba.gx = reinterpret_cast<float*>(wsp + lay.gx);
  ba.dbc = reinterpret_cast<float*>(wsp + lay.dbc);
  ba.dpar = reinterpret_cast<float*>(wsp + lay.dpar);
  ba.wpc = static_cast<int>(ck_slots(Kb));
  // When neither pass splits the sequence, the forward scan below stores the checkpoints itself
  // (the state entering each window of its two-phase walk) and the adjoint walk follows that
  // schedule; otherwise the checkpoint kernel walks each backward chunk again.
  ba.msched = fwd.nch == 1 && ba.s.nch == 1 ? 1 : 0;
  // forward with the un-gated sum y_f + y_b
  ScanArgs a = fwd;
  a.wsy = nullptr;
  a.dout = dout;  // the epilogue computes g and dz (the gate's backward)
  a.gout = g;
  a.dzout = dz;
  if (ba.msched) {
    a.ck = ba.ck;
    a.ck_wpc = ba.wpc;
  }
  vmscan_status st = run_pair<T, kModeVimSum>(a, stream, kStageAll);
  if (st != VMSCAN_OK) return st;
  ba.s.werr_clear = 0;
  hipError_t e;
  // Separate branches at d_state 16: one share per direction, which the walk rounds and stores itself.
  const bool vdirect = du_b && dx_b && fwd.parts == 2;
  if (vdirect) {
    ba.du_out[0] = du;
    ba.du_out[1] = du_b;
    ba.dx_out[0] = dx;
    ba.dx_out[1] = dx_b;
  }
  st = launch_bwd_scans<T, kModeVim, 1>(ba, ba, stream);
  if (st != VMSCAN_OK) return st;
  if (!vdirect)
    hipLaunchKernelGGL(bwd_combine_kernel<T>, dim3(static_cast<unsigned>(ceil_div(n, 256))), dim3(256), 0, stream,
                       ba.gu, ba.gx, static_cast<T*>(du), static_cast<T*>(dx), static_cast<T*>(du_b),
                       static_cast<T*>(dx_b), n, fwd.parts / 2);
  launch_bwd_bc<T>(ba.dbc, static_cast<T*>(dB), static_cast<T*>(dC), static_cast<T*>(dB_b), static_cast<T*>(dC_b),
                   fwd.batch, fwd.ngroups, fwd.L, static_cast<int64_t>(ns) * fwd.L, ns, stream);
  hipLaunchKernelGGL(bwd_param_kernel, dim3(static_cast<unsigned>(ceil_div(2 * fwd.dim * ns + 4 * fwd.dim, 4))),
                     dim3(256), 0, stream, ba.dpar, A_log, A_b_log, dA_log, dA_b_log, dD, dD_b, dbias, dbias_b,
                     fwd.batch * ba.s.nch, fwd.dim, ns);
  e = hipGetLastError();
  return e == hipSuccess ? VMSCAN_OK : launch_failed(e);
}


// SS2D backward workspace: the forward's (images, transposed x, B/C copy, carries), then the
// un-gated sum, the row- and column-order g, the checkpoints and the partial gradients.
// Per-pair backward buffers (the two pairs share launches): the B/C copy and forward carries, the
// checkpoints and adjoint records, the du and dΔ_raw shares, the dB/dC and parameter partials.
// Pair 0 uses the forward layout's B/C copy and carries.
struct PairBufs {
  size_t bct, agg, ck, adj, gu, gx, dbc, dpar;
};

struct Ss2dBwdLayout {
  Ss2dLayout f;
  size_t ysum, g, gcol;
  PairBufs p[2];
  size_t total;
};

Ss2dBwdLayout ss2d_bwd_layout(int64_t batch, int64_t dim, int64_t L, int64_t Kf, size_t esz, int ns) {
  Ss2dBwdLayout w{};
  w.f = ss2d_layout(batch, dim, L, Kf, esz, ns);
  const size_t plane = round256(static_cast<size_t>(batch) * dim * L * sizeof(float));
  const size_t planes = round256(static_cast<size_t>(2) * (ns / kH / 2) * batch * dim * L * sizeof(float));
  const int64_t Kb = bwd_chunk(plan_base(batch, dim, ns), L, Kf, 2 * plan_base(batch, dim, ns));
  w.ysum = round256(w.f.total);
  w.g = w.ysum + plane;
  w.gcol = w.g + plane;
  size_t o = w.gcol + plane;
  for (int k = 0; k < 2; ++k) {
    PairBufs& q = w.p[k];
    if (k == 0) {
      q.bct = w.f.bct;
      q.agg = w.f.agg;
    } else {
      q.bct = o;
      o += bct_bytes(batch, L, ns);
      q.agg = o;
      o += agg_bytes(batch, dim, L, Kf, ns);
    }
    q.ck = o;
    o += ck_bytes(batch, dim, L, Kb, ns);
    q.adj = o;
    o += agg_bytes(batch, dim, L, Kb, ns);
    q.gu = o;
    o += planes;
    q.gx = o;
    o += planes;
    q.dbc = o;
    o += dbc_bytes(batch, dim, L, ns);
    q.dpar = o;
    o += dpar_bytes(batch, dim, L, Kb, ns);
  }
  w.total = o;
  return w;
}

// One SS2D pair (directions k0 and k1 = its reverse) before its adjoint walk: its B/C copy and,
// for a split sequence, its forward carries (in the forward's chunks).
template <typename T>
vmscan_status ss2d_pair_prepare(const BwdArgs& ba, hipStream_t stream) {
  ScanArgs af = ba.s;
  af.K = ba.fnch > 1 ? static_cast<int>(ba.s.K / ba.fm) : static_cast<int>(ba.s.L);
  af.nch = ba.fnch;
  return run_pair<T, kModeSecondPair>(af, stream, kStagePrepare);
}

// ... and after it: dΔ_raw, dB, dC and the parameter sums written for both directions.  The pair's
// du (parts float32 planes in position order: two directions x parts / 2) stays in ba.gu.
template <typename T>
vmscan_status ss2d_pair_post(const BwdArgs& ba, int k0, int k1, void* ddelta_raw, void* dB, void* dC, float* dA_log,
                             const float* A_log, float* dD, float* ddelta_bias, hipStream_t stream) {
  const ScanArgs& a = ba.s;
  const int64_t DL = static_cast<int64_t>(a.dim) * a.L;
  const int64_t n = static_cast<int64_t>(a.batch) * DL;
  const int64_t plane = n;
  T* ddr = static_cast<T*>(ddelta_raw);
  const int np = a.parts / 2;  // planes per direction
  if (!ba.gx_out) {  // else the walk stored dΔ_raw
    launch_sum_planes<T>(ba.gx, np, plane, nullptr, ddr + k0 * DL, DL, a.batch, 4 * DL, stream);
    launch_sum_planes<T>(ba.gx + np * plane, np, plane, nullptr, ddr + k1 * DL, DL, a.batch, 4 * DL, stream);
  }
  const int ns = a.ns;
  const int64_t NL = static_cast<int64_t>(ns) * a.L;
  launch_bwd_bc<T>(ba.dbc, static_cast<T*>(dB) + k0 * NL, static_cast<T*>(dC) + k0 * NL, static_cast<T*>(dB) + k1 * NL,
                   static_cast<T*>(dC) + k1 * NL, a.batch, a.ngroups, a.L, 4 * NL, ns, stream);
  const int64_t dN = static_cast<int64_t>(a.dim) * ns;
  hipLaunchKernelGGL(bwd_param_kernel, dim3(static_cast<unsigned>(ceil_div(2 * a.dim * ns + 4 * a.dim, 4))), dim3(256),
                     0, stream, ba.dpar, A_log + k0 * dN, A_log + k1 * dN, dA_log + k0 * dN, dA_log + k1 * dN,
                     dD + k0 * a.dim, dD + k1 * a.dim, ddelta_bias + k0 * a.dim, ddelta_bias + k1 * a.dim,
                     a.batch * a.nch, a.dim, ns);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? VMSCAN_OK : launch_failed(e);
}

template <typename T>
vmscan_status run_ss2d_bwd(const void* x, const void* delta_raw, const float* A_log, const void* B, const void* C,
                           const float* D, const float* delta_bias, const void* z, const void* dout, void* dx,
                           void* ddelta_raw, float* dA_log, void* dB, void* dC, float* dD, float* ddelta_bias,
                           void* dz, int64_t batch, int64_t dim, int64_t H, int64_t W, int ns, unsigned char* wsp,
                           const Ss2dBwdLayout& lay, int64_t Kf, hipStream_t stream) {
  const int64_t L = H * W;
  const size_t esz = sizeof(T);
  const int64_t nimg = batch * dim, n = nimg * L;
  if (ceil_div(n, 256) >= (int64_t{1} << 31)) return VMSCAN_ERR_SHAPE;
  auto off = [&](const void* p, int64_t elems) {
    return static_cast<const void*>(static_cast<const unsigned char*>(p) + elems * static_cast<int64_t>(esz));
  };
  auto dir_args = [&](const void* u, int k, int rev) {
    return DirArgs{u, off(delta_raw, k * dim * L), 4 * dim * L, off(B, k * ns * L), off(C, k * ns * L), 4 * ns * L,
                   A_log + k * dim * ns, D + k * dim, delta_bias + k * dim, rev};
  };
  float* ysum = reinterpret_cast<float*>(wsp + lay.ysum);
  float* g = reinterpret_cast<float*>(wsp + lay.g);
  float* gcol = reinterpret_cast<float*>(wsp + lay.gcol);
  ScanArgs a{};
  a.ns = ns;
  a.parts = ns / kH;
  a.u_bs = dim * L;
  a.z = nullptr;
  a.werr = reinterpret_cast<int*>(wsp);
  a.werr_clear = 1;  // the first B/C copy of the call clears the status word
  a.bct = reinterpret_cast<float*>(wsp + lay.f.bct);
  a.agg = reinterpret_cast<float*>(wsp + lay.f.agg);
  a.L = L;
  a.dim = static_cast<int>(dim);
  a.batch = static_cast<int>(batch);
  a.K = static_cast<int>(Kf);
  a.nch = static_cast<int>(ceil_div(L, Kf));
  a.ngroups = static_cast<int>(groups(dim));
  const void* xt = wsp + lay.f.xt;
  vmscan_status st = launch_transpose(x, wsp + lay.f.xt, nimg, static_cast<int>(H), static_cast<int>(W), esz, stream);
  if (st != VMSCAN_OK) return st;
  if (z) {
    // the forward's un-gated four-direction sum, as float32 (same pairs as ss2d_cross_scan_fwd)
    a.wsy = reinterpret_cast<float*>(wsp + lay.f.col_img);
    a.d0 = dir_args(xt, 1, 0);
    a.d1 = dir_args(xt, 3, 1);
    st = run_pair<T, kModeFirstPair>(a, stream, kStageAll);
    if (st != VMSCAN_OK) return st;
    a.werr_clear = 0;
    st = launch_transpose(wsp + lay.f.col_img, wsp + lay.f.row_img, nimg, static_cast<int>(W), static_cast<int>(H), 4,
                          stream);
    if (st != VMSCAN_OK) return st;
    a.wsy = reinterpret_cast<float*>(wsp + lay.f.row_img);
    a.out = ysum;
    a.d0 = dir_args(x, 0, 0);
    a.d1 = dir_args(x, 2, 1);
    st = run_pair<T, kModeSecondPairSum>(a, stream, kStageAll);
    if (st != VMSCAN_OK) return st;
  }
  const int64_t Kb = bwd_chunk(plan_base(batch, dim, ns), L, Kf, 2 * plan_base(batch, dim, ns));
  // Without a gate g is dout itself.  With bf16 activations and unsplit walks, the walks read it (and
  // its transpose, for the column pair) as it is instead of a float32 copy; the values are the same.
  const bool gact = !z && sizeof(T) == 2 && ceil_div(L, Kb) == 1;
  hipError_t e;
  if (gact) {
    st = launch_transpose(dout, gcol, nimg, static_cast<int>(H), static_cast<int>(W), esz, stream);
    if (st != VMSCAN_OK) return st;
  } else {
    hipLaunchKernelGGL(gate_bwd_kernel<T>, dim3(static_cast<unsigned>(ceil_div(n, 256 * kWin))), dim3(256), 0, stream,
                       static_cast<const T*>(dout), static_cast<const T*>(z), ysum, g, static_cast<T*>(dz), n, 1.0f);
    e = hipGetLastError();
    if (e != hipSuccess) return launch_failed(e);
    // g in column-major order for the column pair
    st = launch_transpose(g, gcol, nimg, static_cast<int>(H), static_cast<int>(W), 4, stream);
    if (st != VMSCAN_OK) return st;
  }
  // Both pairs' adjoint walks in the same launches (twice the workgroups of one pair), each with its
  // own buffers: the column pair (directions 1 and 3 over x^T, g in column order) and the row
  // pair (directions 0 and 2 over x, g in row order).
  BwdArgs bp[2];
  for (int k = 0; k < 2; ++k) {
    BwdArgs& ba = bp[k];
    const PairBufs& q = lay.p[k];
    ba = BwdArgs{};
    ba.s = a;
    ba.s.bct = reinterpret_cast<float*>(wsp + q.bct);
    ba.s.agg = reinterpret_cast<float*>(wsp + q.agg);
    ba.s.K = static_cast<int>(Kb);
    ba.s.nch = static_cast<int>(ceil_div(L, Kb));
    ba.fnch = ba.s.nch > 1 ? a.nch : 1;  // an unsplit walk needs no forward carries
    ba.fm = ba.s.nch > 1 ? static_cast<int>(Kb / Kf) : 1;
    ba.ck = reinterpret_cast<float*>(wsp + q.ck);
    ba.adj = ba.s.nch > 1 ? reinterpret_cast<float*>(wsp + q.adj) : nullptr;
    ba.gu = reinterpret_cast<float*>(wsp + q.gu);
    ba.gx = reinterpret_cast<float*>(wsp + q.gx);
    ba.dbc = reinterpret_cast<float*>(wsp + q.dbc);
    ba.dpar = reinterpret_cast<float*>(wsp + q.dpar);
    ba.wpc = static_cast<int>(ck_slots(Kb));
    ba.g = k == 0 ? gcol : g;
    ba.gt = gact ? (k == 0 ? static_cast<const void*>(gcol) : dout) : nullptr;
    ba.s.d0 = k == 0 ? dir_args(xt, 1, 0) : dir_args(x, 0, 0);
    ba.s.d1 = k == 0 ? dir_args(xt, 3, 1) : dir_args(x, 2, 1);
    if (a.parts == 2) {  // one dΔ_raw share per direction: the walk rounds and stores it
      ba.gx_out = static_cast<unsigned char*>(ddelta_raw) + (k == 0 ? 1 : 0) * dim * L * static_cast<int64_t>(esz);
      ba.gx_out_dir = 2 * dim * L;  // directions (1, 3) and (0, 2): two planes apart
      ba.gx_out_bs = 4 * dim * L;
    }
    st = ss2d_pair_prepare<T>(ba, stream);
    if (st != VMSCAN_OK) return st;
    a.werr_clear = 0;
  }
  st = launch_bwd_scans<T, kModeSecondPair, 2>(bp[0], bp[1], stream);
  if (st != VMSCAN_OK) return st;
  const BwdArgs& ba = bp[0];
  st = ss2d_pair_post<T>(bp[0], 1, 3, ddelta_raw, dB, dC, dA_log, A_log, dD, ddelta_bias, stream);
  if (st != VMSCAN_OK) return st;
  // the row pair's gradients, and dx = its du plus the column pair's, transposed (one pass)
  const BwdArgs& br = bp[1];
  st = ss2d_pair_post<T>(br, 0, 2, ddelta_raw, dB, dC, dA_log, A_log, dD, ddelta_bias, stream);
  if (st != VMSCAN_OK) return st;
  {
    const int R = static_cast<int>(W), Cc = static_cast<int>(H);
    const int tr = static_cast<int>(ceil_div(R, kTile)), tc = static_cast<int>(ceil_div(Cc, kTile));
    const int64_t blocks = nimg * tr * tc;
    if (blocks >= (int64_t{1} << 31)) return VMSCAN_ERR_SHAPE;
    hipLaunchKernelGGL(dx_merge_kernel<T>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, ba.gu, br.gu,
                       a.parts, n, static_cast<T*>(dx), R, Cc, tr, tc);
  }
  e = hipGetLastError();
  return e == hipSuccess ? VMSCAN_OK : launch_failed(e);
}

// Fixed scratch for vmscan_fwd_bidir_noalloc: device memory the code object brings with it, so
// that entry point never allocates.  Each GPU the library is loaded on holds its own copy until
// the process ends.  In host code `scratch` names a host-side stand-in, not device memory: the
// device address of each GPU's copy comes from hipGetSymbolAddress (scratch_ptr) and only that
// address is ever passed to a kernel.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

}  // namespace

static __device__ __align__(256) unsigned char scratch[VMSCAN_SCRATCH_BYTES];

namespace {

// The current device's copy of `scratch`, looked up once per device (with that device current).
vmscan_status scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return launch_failed(e);
  if (dev < 0 || dev >= kMaxDevices) return VMSCAN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return launch_failed(e);
    if (!p) return launch_failed(hipErrorInvalidSymbol);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return VMSCAN_OK;
}

}  // namespace

// ---------------------------------------------------------------------------------------------
// C ABI

extern "C" {

const char* vmscan_status_string(vmscan_status s) {
  switch (s) {
    case VMSCAN_OK: return "VMSCAN_OK";
    case VMSCAN_ERR_NULL: return "VMSCAN_ERR_NULL: a required pointer is NULL";
    case VMSCAN_ERR_SHAPE: return "VMSCAN_ERR_SHAPE: a size is < 1 or too large";
    case VMSCAN_ERR_UNSUPPORTED:
      return "VMSCAN_ERR_UNSUPPORTED: d_state must be 16 or 32 and dtype F32 or BF16";
    case VMSCAN_ERR_ALIGN: return "VMSCAN_ERR_ALIGN: a pointer is not 16-byte aligned";
    case VMSCAN_ERR_WORKSPACE: return "VMSCAN_ERR_WORKSPACE: workspace missing or too small";
    case VMSCAN_ERR_HIP: return "VMSCAN_ERR_HIP: a HIP call failed (see vmscan_last_hip_error)";
    case VMSCAN_ERR_SCRATCH:
      return "VMSCAN_ERR_SCRATCH: the call needs more workspace than the fixed scratch buffer (VMSCAN_SCRATCH_BYTES)";
    case VMSCAN_ERR_WAIT:
      return "VMSCAN_ERR_WAIT: a wait between the waves of a workgroup gave up; the results are unspecified";
  }
  return "VMSCAN_ERR_UNKNOWN";
}

int vmscan_last_hip_error(void) { return g_last_hip_error; }

int64_t vmscan_fwd_bidir_chunk_len(int64_t batch, int64_t dim, int64_t seqlen, int d_state) {
  if (!shape_ok(batch, dim, seqlen) || !d_state_ok(d_state)) return 0;
  return plan_chunk(plan_base(batch, dim, d_state), seqlen, 0);
}

size_t vmscan_fwd_bidir_workspace_bytes_ex(int64_t batch, int64_t dim, int64_t seqlen, int d_state,
                                           vmscan_dtype dtype, int64_t chunk_len) {
  if (!shape_ok(batch, dim, seqlen) || !d_state_ok(d_state) || (dtype != VMSCAN_F32 && dtype != VMSCAN_BF16) ||
      (chunk_len < 0 && chunk_len != VMSCAN_CHUNK_LANE_SCAN))
    return 0;
  if (chunk_len == VMSCAN_CHUNK_LANE_SCAN) return seqlen <= kLaneMaxL ? kStatusBytes : 0;  // the status word only
  const int64_t K = plan_chunk(plan_base(batch, dim, d_state), seqlen, chunk_len);
  return kStatusBytes + bct_bytes(batch, seqlen, d_state) + agg_bytes(batch, dim, seqlen, K, d_state);
}

size_t vmscan_fwd_bidir_workspace_bytes(int64_t batch, int64_t dim, int64_t seqlen, int d_state,
                                        vmscan_dtype dtype) {
  return vmscan_fwd_bidir_workspace_bytes_ex(batch, dim, seqlen, d_state, dtype, 0);
}

vmscan_status vmscan_fwd_bidir_ex(const void* u, const void* delta_raw, const void* z, const float* A_log,
                                  const float* A_b_log, const void* B, const void* C, const void* B_b,
                                  const void* C_b, const float* D, const float* D_b, const float* delta_bias,
                                  void* out, int64_t batch, int64_t dim, int64_t seqlen, int d_state,
                                  vmscan_dtype dtype, void* workspace, size_t workspace_bytes,
                                  int64_t chunk_len, hipStream_t stream) {
  return vmscan_fwd_bidir_stage(u, delta_raw, z, A_log, A_b_log, B, C, B_b, C_b, D, D_b, delta_bias, out, batch, dim,
                                seqlen, d_state, dtype, workspace, workspace_bytes, chunk_len, 3, stream);
}

size_t vmscan_bwd_bidir_v2_workspace_bytes(int64_t batch, int64_t dim, int64_t seqlen, int d_state,
                                           vmscan_dtype dtype) {
  if (!shape_ok(batch, dim, seqlen) || !d_state_ok(d_state) || (dtype != VMSCAN_F32 && dtype != VMSCAN_BF16)) return 0;
  return bwd_layout(batch, dim, seqlen, plan_chunk(plan_base(batch, dim, d_state), seqlen, 0), d_state).total;
}

vmscan_status vmscan_bwd_bidir_v2(const void* u, const void* delta_raw, const float* delta_bias, const void* u_b,
                                  const void* delta_raw_b, const float* delta_bias_b, const void* z,
                                  const float* A_log, const float* A_b_log, const void* B, const void* C,
                                  const void* B_b, const void* C_b, const float* D, const float* D_b,
                                  const void* dout, void* du, void* ddelta_raw, float* ddelta_bias, void* du_b,
                                  void* ddelta_raw_b, float* ddelta_bias_b, void* dz, float* dA_log, float* dA_b_log,
                                  void* dB, void* dC, void* dB_b, void* dC_b, float* dD, float* dD_b, int64_t batch,
                                  int64_t dim, int64_t seqlen, int d_state, vmscan_dtype dtype, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  const void* need[] = {dout, du, ddelta_raw, ddelta_bias, dz, dA_log, dA_b_log, dB, dC, dB_b, dC_b, dD, dD_b};
  for (const void* p : need)
    if (!p) return VMSCAN_ERR_NULL;
  if (!shape_ok(batch, dim, seqlen)) return VMSCAN_ERR_SHAPE;
  if (!d_state_ok(d_state) || (dtype != VMSCAN_F32 && dtype != VMSCAN_BF16)) return VMSCAN_ERR_UNSUPPORTED;
  const void* opt[] = {du_b, ddelta_raw_b, ddelta_bias_b};
  for (const void* p : need)
    if (!aligned16(p)) return VMSCAN_ERR_ALIGN;
  for (const void* p : opt)
    if (p && !aligned16(p)) return VMSCAN_ERR_ALIGN;
  const int64_t Kf = plan_chunk(plan_base(batch, dim, d_state), seqlen, 0);
  const BwdLayout lay = bwd_layout(batch, dim, seqlen, Kf, d_state);
  ScanArgs a{};
  // The forward arguments; its output pointer is unused in the sum-saving mode.
  vmscan_status st = vim_args(a, u, delta_raw, delta_bias, u_b, delta_raw_b, delta_bias_b, z, A_log, A_b_log, B, C,
                              B_b, C_b, D, D_b, workspace, batch, dim, seqlen, d_state, dtype, workspace,
                              workspace_bytes, 0);
  if (st != VMSCAN_OK) return st;
  st = check_workspace(workspace, workspace_bytes, lay.total);
  if (st != VMSCAN_OK) return st;
  unsigned char* wsp = static_cast<unsigned char*>(workspace);
  st = dtype == VMSCAN_F32
           ? run_bwd<float>(a, lay, wsp, dout, z, du, ddelta_raw, ddelta_bias, du_b, ddelta_raw_b, ddelta_bias_b, dz,
                            A_log, A_b_log, dA_log, dA_b_log, dB, dC, dB_b, dC_b, dD, dD_b, stream)
           : run_bwd<uint16_t>(a, lay, wsp, dout, z, du, ddelta_raw, ddelta_bias, du_b, ddelta_raw_b, ddelta_bias_b,
                               dz, A_log, A_b_log, dA_log, dA_b_log, dB, dC, dB_b, dC_b, dD, dD_b, stream);
  return finish_call(st, workspace, stream);
}

vmscan_status vmscan_fwd_bidir_v2_stage(const void* u, const void* delta_raw, const float* delta_bias, const void* u_b,
                                        const void* delta_raw_b, const float* delta_bias_b, const void* z,
                                        const float* A_log, const float* A_b_log, const void* B, const void* C,
                                        const void* B_b, const void* C_b, const float* D, const float* D_b, void* out,
                                        int64_t batch, int64_t dim, int64_t seqlen, int d_state, vmscan_dtype dtype,
                                        void* workspace, size_t workspace_bytes, int64_t chunk_len, int stage,
                                        hipStream_t stream) {
  if (stage < 1 || stage > 3) return VMSCAN_ERR_UNSUPPORTED;
  ScanArgs a{};
  const vmscan_status st =
      vim_args(a, u, delta_raw, delta_bias, u_b, delta_raw_b, delta_bias_b, z, A_log, A_b_log, B, C, B_b, C_b, D, D_b,
               out, batch, dim, seqlen, d_state, dtype, workspace, workspace_bytes, chunk_len);
  if (st != VMSCAN_OK) return st;
  return finish_call(run_vim(a, dtype, stream, stage), workspace, stream);
}

vmscan_status vmscan_fwd_bidir_v2(const void* u, const void* delta_raw, const float* delta_bias, const void* u_b,
                                  const void* delta_raw_b, const float* delta_bias_b, const void* z,
                                  const float* A_log, const float* A_b_log, const void* B, const void* C,
                                  const void* B_b, const void* C_b, const float* D, const float* D_b, void* out,
                                  int64_t batch, int64_t dim, int64_t seqlen, int d_state, vmscan_dtype dtype,
                                  void* workspace, size_t workspace_bytes, int64_t chunk_len, hipStream_t stream) {
  return vmscan_fwd_bidir_v2_stage(u, delta_raw, delta_bias, u_b, delta_raw_b, delta_bias_b, z, A_log, A_b_log, B, C,
                                   B_b, C_b, D, D_b, out, batch, dim, seqlen, d_state, dtype, workspace,
                                   workspace_bytes, chunk_len, 3, stream);
}

vmscan_status vmscan_fwd_bidir_stage(const void* u, const void* delta_raw, const void* z, const float* A_log,
                                     const float* A_b_log, const void* B, const void* C, const void* B_b,
                                     const void* C_b, const float* D, const float* D_b, const float* delta_bias,
                                     void* out, int64_t batch, int64_t dim, int64_t seqlen, int d_state,
                                     vmscan_dtype dtype, void* workspace, size_t workspace_bytes, int64_t chunk_len,
                                     int stage, hipStream_t stream) {
  return vmscan_fwd_bidir_v2_stage(u, delta_raw, delta_bias, u, delta_raw, delta_bias, z, A_log, A_b_log, B, C, B_b,
                                   C_b, D, D_b, out, batch, dim, seqlen, d_state, dtype, workspace, workspace_bytes,
                                   chunk_len, stage, stream);
}

vmscan_status vmscan_fwd_bidir(const void* u, const void* delta_raw, const void* z, const float* A_log,
                               const float* A_b_log, const void* B, const void* C, const void* B_b,
                               const void* C_b, const float* D, const float* D_b, const float* delta_bias,
                               void* out, int64_t batch, int64_t dim, int64_t seqlen, int d_state,
                               vmscan_dtype dtype, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  return vmscan_fwd_bidir_ex(u, delta_raw, z, A_log, A_b_log, B, C, B_b, C_b, D, D_b, delta_bias, out, batch, dim,
                             seqlen, d_state, dtype, workspace, workspace_bytes, 0, stream);
}

vmscan_status vmscan_fwd_bidir_noalloc(const void* u, const void* delta_raw, const void* z, const float* A_log,
                                       const float* A_b_log, const void* B, const void* C, const void* B_b,
                                       const void* C_b, const float* D, const float* D_b, const float* delta_bias,
                                       void* out, int64_t batch, int64_t dim, int64_t seqlen, int d_state,
                                       vmscan_dtype dtype, hipStream_t stream) {
  // Validate every argument first (a stand-in workspace that passes the workspace checks), so
  // that bad arguments are reported as by vmscan_fwd_bidir, before any HIP call.
  ScanArgs a{};
  vmscan_status st = vim_args(a, u, delta_raw, delta_bias, u, delta_raw, delta_bias, z, A_log, A_b_log, B, C, B_b,
                              C_b, D, D_b, out, batch, dim, seqlen, d_state, dtype,
                              reinterpret_cast<void*>(static_cast<uintptr_t>(256)), SIZE_MAX, 0);
  if (st != VMSCAN_OK) return st;
  if (vmscan_fwd_bidir_workspace_bytes(batch, dim, seqlen, d_state, dtype) > VMSCAN_SCRATCH_BYTES)
    return VMSCAN_ERR_SCRATCH;
  void* ws = nullptr;
  st = scratch_ptr(&ws);
  if (st != VMSCAN_OK) return st;
  return vmscan_fwd_bidir_v2_stage(u, delta_raw, delta_bias, u, delta_raw, delta_bias, z, A_log, A_b_log, B, C, B_b,
                                   C_b, D, D_b, out, batch, dim, seqlen, d_state, dtype, ws, VMSCAN_SCRATCH_BYTES, 0,
                                   kStageAll, stream);
}

size_t ss2d_cross_scan_workspace_bytes_ex(int64_t batch, int64_t dim, int64_t H, int64_t W, int d_state,
                                          vmscan_dtype dtype, int64_t chunk_len) {
  if (H < 1 || W < 1 || H >= (int64_t{1} << 31) || W >= (int64_t{1} << 31)) return 0;
  const int64_t L = H * W;
  if (!shape_ok(batch, dim, L) || !d_state_ok(d_state) || (dtype != VMSCAN_F32 && dtype != VMSCAN_BF16) ||
      chunk_len < 0)
    return 0;
  if (ss2d_walk(batch, dim, L, d_state, chunk_len))
    return ss2d_walk_layout(batch, dim, L, dtype == VMSCAN_F32 ? 4 : 2, d_state).total;
  const int64_t K = plan_chunk(plan_base(batch, dim, d_state), L, chunk_len);
  return ss2d_layout(batch, dim, L, K, dtype == VMSCAN_F32 ? 4 : 2, d_state).total;
}

size_t ss2d_cross_scan_workspace_bytes(int64_t batch, int64_t dim, int64_t H, int64_t W, int d_state,
                                       vmscan_dtype dtype) {
  return ss2d_cross_scan_workspace_bytes_ex(batch, dim, H, W, d_state, dtype, 0);
}

namespace {

// The SS2D forward as two whole-sequence pair walks (column pair over x^T, row pair over x) in one
// launch, then the cross-merge; arguments already validated.
vmscan_status ss2d_walk_fwd(const void* x, const void* xT, const void* delta_raw, const float* A_log, const void* B,
                            const void* C, const float* D, const float* delta_bias, const void* z, void* out,
                            int64_t batch, int64_t dim, int64_t H, int64_t W, int ns, vmscan_dtype dtype,
                            void* workspace, hipStream_t stream) {
  const int64_t L = H * W;
  const size_t esz = dtype == VMSCAN_F32 ? 4 : 2;
  const Ss2dWalkLayout lay = ss2d_walk_layout(batch, dim, L, esz, ns);
  unsigned char* wsp = static_cast<unsigned char*>(workspace);
  const int64_t ngr = groups(dim);
  const int64_t nb = batch * ngr;
  const int64_t tblocks = batch * 2 * ceil_div(L, kTransThreads);
  const int64_t mblocks = nb * ceil_div(L, 64);
  if (2 * nb >= (int64_t{1} << 31) || tblocks >= (int64_t{1} << 31) || mblocks >= (int64_t{1} << 31))
    return VMSCAN_ERR_SHAPE;
  vmscan_status st = VMSCAN_OK;
  if (!xT) {
    st = launch_transpose(x, wsp + lay.xt, batch * dim, static_cast<int>(H), static_cast<int>(W), esz, stream);
    if (st != VMSCAN_OK) return st;
    xT = wsp + lay.xt;
  }
  auto off = [&](const void* p, int64_t elems) {
    return static_cast<const void*>(static_cast<const unsigned char*>(p) + elems * static_cast<int64_t>(esz));
  };
  auto dir_args = [&](const void* u, int k, int rev) {
    return DirArgs{u, off(delta_raw, k * dim * L), 4 * dim * L, off(B, k * ns * L), off(C, k * ns * L), 4 * ns * L,
                   A_log + k * dim * ns, D + k * dim, delta_bias + k * dim, rev};
  };
  ScanArgs a[2] = {};
  for (int k = 0; k < 2; ++k) {  // 0: column pair (directions 1, 3) over x^T; 1: row pair (0, 2) over x
    ScanArgs& s = a[k];
    s.ns = ns;
    s.parts = kWalkParts;  // of ns / kWalkParts states each
    s.u_bs = dim * L;
    s.L = L;
    s.dim = static_cast<int>(dim);
    s.batch = static_cast<int>(batch);
    s.K = static_cast<int>(L);
    s.nch = 1;
    s.ngroups = static_cast<int>(ngr);
    s.wsy = reinterpret_cast<float*>(wsp + (k == 0 ? lay.rows_c : lay.rows_r));
    s.werr = reinterpret_cast<int*>(wsp);
    s.werr_clear = k == 0 ? 1 : 0;
    s.bct = reinterpret_cast<float*>(wsp + (k == 0 ? lay.bct_c : lay.bct_r));
    s.d0 = k == 0 ? dir_args(xT, 1, 0) : dir_args(x, 0, 0);
    s.d1 = k == 0 ? dir_args(xT, 3, 1) : dir_args(x, 2, 1);
    if (dtype == VMSCAN_F32) {
      if (ns == 16)
        hipLaunchKernelGGL((bc_transpose_kernel<float, 4>), dim3(static_cast<unsigned>(tblocks)), dim3(kTransThreads),
                           0, stream, s);
      else
        hipLaunchKernelGGL((bc_transpose_kernel<float, 8>), dim3(static_cast<unsigned>(tblocks)), dim3(kTransThreads),
                           0, stream, s);
    } else {
      if (ns == 16)
        hipLaunchKernelGGL((bc_transpose_kernel<uint16_t, 4>), dim3(static_cast<unsigned>(tblocks)),
                           dim3(kTransThreads), 0, stream, s);
      else
        hipLaunchKernelGGL((bc_transpose_kernel<uint16_t, 8>), dim3(static_cast<unsigned>(tblocks)),
                           dim3(kTransThreads), 0, stream, s);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return launch_failed(e);
  }
  const dim3 grid(static_cast<unsigned>(2 * nb)), block(2 * kW * kWalkParts);
  if (dtype == VMSCAN_F32) {
    if (ns == 16) hipLaunchKernelGGL((walk_pair_kernel<float, kWalkParts, 4>), grid, block, 0, stream, a[0], a[1]);
    else hipLaunchKernelGGL((walk_pair_kernel<float, kWalkParts, 8>), grid, block, 0, stream, a[0], a[1]);
    hipLaunchKernelGGL(walk_merge_kernel<float>, dim3(static_cast<unsigned>(mblocks)), dim3(256), 0, stream,
                       a[1].wsy, a[0].wsy, static_cast<const float*>(z), static_cast<float*>(out),
                       static_cast<int>(dim), static_cast<int>(H), static_cast<int>(W), static_cast<int>(ngr));
  } else {
    if (ns == 16) hipLaunchKernelGGL((walk_pair_kernel<uint16_t, kWalkParts, 4>), grid, block, 0, stream, a[0], a[1]);
    else hipLaunchKernelGGL((walk_pair_kernel<uint16_t, kWalkParts, 8>), grid, block, 0, stream, a[0], a[1]);
    hipLaunchKernelGGL(walk_merge_kernel<uint16_t>, dim3(static_cast<unsigned>(mblocks)), dim3(256), 0, stream,
                       a[1].wsy, a[0].wsy, static_cast<const uint16_t*>(z), static_cast<uint16_t*>(out),
                       static_cast<int>(dim), static_cast<int>(H), static_cast<int>(W), static_cast<int>(ngr));
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? VMSCAN_OK : launch_failed(e);
}

// The SS2D forward with x's transposed copy either made here (xT NULL) or given by the caller.
vmscan_status ss2d_fwd_impl(const void* x, const void* xT, const void* delta_raw, const float* A_log, const void* B,
                            const void* C, const float* D, const float* delta_bias, const void* z, void* out,
                            int64_t batch, int64_t dim, int64_t H, int64_t W, int d_state, vmscan_dtype dtype,
                            void* workspace, size_t workspace_bytes, int64_t chunk_len, hipStream_t stream) {
  const void* ptrs[] = {x, delta_raw, A_log, B, C, D, delta_bias, out};
  for (const void* p : ptrs)
    if (!p) return VMSCAN_ERR_NULL;
  if (H < 1 || W < 1 || H >= (int64_t{1} << 31) || W >= (int64_t{1} << 31) || chunk_len < 0) return VMSCAN_ERR_SHAPE;
  const int64_t L = H * W;
  if (!shape_ok(batch, dim, L)) return VMSCAN_ERR_SHAPE;
  if (!d_state_ok(d_state) || (dtype != VMSCAN_F32 && dtype != VMSCAN_BF16)) return VMSCAN_ERR_UNSUPPORTED;
  for (const void* p : ptrs)
    if (!aligned16(p)) return VMSCAN_ERR_ALIGN;
  if ((z && !aligned16(z)) || (xT && !aligned16(xT))) return VMSCAN_ERR_ALIGN;
  const size_t need = ss2d_cross_scan_workspace_bytes_ex(batch, dim, H, W, d_state, dtype, chunk_len);
  const vmscan_status ws = check_workspace(workspace, workspace_bytes, need);
  if (ws != VMSCAN_OK) return ws;

  const int ns = d_state;
  const size_t esz = dtype == VMSCAN_F32 ? 4 : 2;
  if (ss2d_walk(batch, dim, L, ns, chunk_len))
    return ss2d_walk_fwd(x, xT, delta_raw, A_log, B, C, D, delta_bias, z, out, batch, dim, H, W, ns, dtype, workspace,
                         stream);
  const int64_t K = plan_chunk(plan_base(batch, dim, ns), L, chunk_len);
  const Ss2dLayout lay = ss2d_layout(batch, dim, L, K, esz, ns);
  unsigned char* wsp = static_cast<unsigned char*>(workspace);

  auto off = [&](const void* p, int64_t elems) {
    return static_cast<const void*>(static_cast<const unsigned char*>(p) + elems * static_cast<int64_t>(esz));
  };
  // Direction k of delta_raw [batch, 4, dim, L] and B/C [batch, 4, ns, L]; params [4, dim(, ns)].
  auto dir_args = [&](const void* u, int k, int rev) {
    return DirArgs{u, off(delta_raw, k * dim * L), 4 * dim * L, off(B, k * ns * L), off(C, k * ns * L), 4 * ns * L,
                   A_log + k * dim * ns, D + k * dim, delta_bias + k * dim, rev};
  };

  ScanArgs a{};
  a.ns = ns;
  a.parts = ns / kH;
  a.u_bs = dim * L;
  a.z = z;
  a.out = out;
  a.werr = reinterpret_cast<int*>(wsp);
  a.werr_clear = 1;  // the column pair's B/C copy runs first
  a.bct = reinterpret_cast<float*>(wsp + lay.bct);
  a.agg = reinterpret_cast<float*>(wsp + lay.agg);
  a.L = L;
  a.dim = static_cast<int>(dim);
  a.batch = static_cast<int>(batch);
  a.K = static_cast<int>(K);
  a.nch = static_cast<int>(ceil_div(L, K));
  a.ngroups = static_cast<int>(groups(dim));
  const int64_t nimg = batch * dim;

  // Column pair (direction 1 = column-major order, direction 3 = its reverse) over the transposed
  // image x^T [W][H], whose rows are x's columns: position p = w*H + h is x^T's element p.  It
  // writes its combined values as an fp32 image in the same column-major order.
  vmscan_status st = VMSCAN_OK;
  if (!xT) {
    st = launch_transpose(x, wsp + lay.xt, nimg, static_cast<int>(H), static_cast<int>(W), esz, stream);
    if (st != VMSCAN_OK) return st;
    xT = wsp + lay.xt;
  }
  a.wsy = reinterpret_cast<float*>(wsp + lay.col_img);
  a.d0 = dir_args(xT, 1, 0);
  a.d1 = dir_args(xT, 3, 1);
  st = run_pair_dtype<kModeFirstPair>(a, dtype, stream);
  if (st != VMSCAN_OK) return st;
  // Back to row-major pixels, then the row pair (direction 0 and its reverse, direction 2) adds
  // that image to its own sum, applies the optional gate and stores.  Its transpose and
  // chunk-state kernels reuse the B/C and carry regions after the column pair (same stream).
  st = launch_transpose(wsp + lay.col_img, wsp + lay.row_img, nimg, static_cast<int>(W), static_cast<int>(H), 4,
                        stream);
  if (st != VMSCAN_OK) return st;
  a.wsy = reinterpret_cast<float*>(wsp + lay.row_img);
  a.d0 = dir_args(x, 0, 0);
  a.d1 = dir_args(x, 2, 1);
  a.werr_clear = 0;
  return run_pair_dtype<kModeSecondPair>(a, dtype, stream);
}

}  // namespace

vmscan_status ss2d_cross_scan_fwd_ex(const void* x, const void* delta_raw, const float* A_log, const void* B,
                                     const void* C, const float* D, const float* delta_bias, const void* z,
                                     void* out, int64_t batch, int64_t dim, int64_t H, int64_t W, int d_state,
                                     vmscan_dtype dtype, void* workspace, size_t workspace_bytes,
                                     int64_t chunk_len, hipStream_t stream) {
  return finish_call(ss2d_fwd_impl(x, nullptr, delta_raw, A_log, B, C, D, delta_bias, z, out, batch, dim, H, W,
                                   d_state, dtype, workspace, workspace_bytes, chunk_len, stream),
                     workspace, stream);
}

vmscan_status ss2d_cross_scan_fwd_xt(const void* x, const void* xT, const void* delta_raw, const float* A_log,
                                     const void* B, const void* C, const float* D, const float* delta_bias,
                                     const void* z, void* out, int64_t batch, int64_t dim, int64_t H, int64_t W,
                                     int d_state, vmscan_dtype dtype, void* workspace, size_t workspace_bytes,
                                     int64_t chunk_len, hipStream_t stream) {
  if (!xT) return VMSCAN_ERR_NULL;
  return finish_call(ss2d_fwd_impl(x, xT, delta_raw, A_log, B, C, D, delta_bias, z, out, batch, dim, H, W, d_state,
                                   dtype, workspace, workspace_bytes, chunk_len, stream),
                     workspace, stream);
}

vmscan_status vmscan_conv1d_silu_fwd(const void* x, const float* conv_w, const float* conv_b, const float* conv_w_b,
                                     const float* conv_b_b, void* u, void* u_b, int64_t batch, int64_t dim,
                                     int64_t seqlen, int d_conv, vmscan_dtype dtype, hipStream_t stream) {
  if (!x || !conv_w || !conv_b || !u) return VMSCAN_ERR_NULL;
  // the backward branch's weights, bias and output come together
  const int nb_set = (conv_w_b != nullptr) + (conv_b_b != nullptr) + (u_b != nullptr);
  if (nb_set != 0 && nb_set != 3) return VMSCAN_ERR_NULL;
  if (!shape_ok(batch, dim, seqlen)) return VMSCAN_ERR_SHAPE;
  if (d_conv < 1 || d_conv > kConvMax || (dtype != VMSCAN_F32 && dtype != VMSCAN_BF16)) return VMSCAN_ERR_UNSUPPORTED;
  const void* ptrs[] = {x, conv_w, conv_b, conv_w_b, conv_b_b, u, u_b};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return VMSCAN_ERR_ALIGN;
  const int64_t total = batch * dim * seqlen;
  const int64_t blocks = ceil_div(ceil_div(total, kConvRun), 256);  // a thread per kConvRun outputs
  if (dim >= (int64_t{1} << 31) || seqlen >= (int64_t{1} << 30) || blocks >= (int64_t{1} << 31))
    return VMSCAN_ERR_SHAPE;
  const dim3 grid(static_cast<unsigned>(blocks));
  const int di = static_cast<int>(dim), Li = static_cast<int>(seqlen);
  if (dtype == VMSCAN_F32)
    hipLaunchKernelGGL((conv1d_flat_kernel<float, kConvRun>), grid, dim3(256), 0, stream, static_cast<const float*>(x), conv_w,
                       conv_b, conv_w_b, conv_b_b, static_cast<float*>(u), static_cast<float*>(u_b), total, di, Li,
                       d_conv);
  else
    hipLaunchKernelGGL((conv1d_flat_kernel<uint16_t, kConvRun>), grid, dim3(256), 0, stream, static_cast<const uint16_t*>(x),
                       conv_w, conv_b, conv_w_b, conv_b_b, static_cast<uint16_t*>(u), static_cast<uint16_t*>(u_b),
                       total, di, Li, d_conv);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? VMSCAN_OK : launch_failed(e);
}

vmscan_status ss2d_conv2d_silu_fwd(const void* x, const float* conv_w, const float* conv_b, int act, void* x_out,
                                   void* xT_out, int64_t batch, int64_t dim, int64_t H, int64_t W, int d_conv,
                                   vmscan_dtype dtype, hipStream_t stream) {
  if (!x || !conv_w || !conv_b || !x_out) return VMSCAN_ERR_NULL;
  if (H < 1 || W < 1 || H >= (int64_t{1} << 31) || W >= (int64_t{1} << 31)) return VMSCAN_ERR_SHAPE;
  if (!shape_ok(batch, dim, H * W)) return VMSCAN_ERR_SHAPE;
  if (d_conv != 3 || (act != 0 && act != 1) || (dtype != VMSCAN_F32 && dtype != VMSCAN_BF16))
    return VMSCAN_ERR_UNSUPPORTED;
  const void* ptrs[] = {x, conv_w, conv_b, x_out, xT_out};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return VMSCAN_ERR_ALIGN;
  const int tr = static_cast<int>(ceil_div(H, kTile)), tc = static_cast<int>(ceil_div(W, kTile));
  const int64_t blocks = batch * dim * tr * tc;
  if (blocks >= (int64_t{1} << 31)) return VMSCAN_ERR_SHAPE;
  if (dtype == VMSCAN_F32)
    hipLaunchKernelGGL(conv2d_front_kernel<float>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                       static_cast<const float*>(x), conv_w, conv_b, act, static_cast<float*>(x_out),
                       static_cast<float*>(xT_out), static_cast<int>(dim), static_cast<int>(H), static_cast<int>(W),
                       tr, tc);
  else
    hipLaunchKernelGGL(conv2d_front_kernel<uint16_t>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(x), conv_w, conv_b, act, static_cast<uint16_t*>(x_out),
                       static_cast<uint16_t*>(xT_out), static_cast<int>(dim), static_cast<int>(H),
                       static_cast<int>(W), tr, tc);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? VMSCAN_OK : launch_failed(e);
}

size_t ss2d_cross_scan_bwd_workspace_bytes(int64_t batch, int64_t dim, int64_t H, int64_t W, int d_state,
                                           vmscan_dtype dtype) {
  if (H < 1 || W < 1 || H >= (int64_t{1} << 31) || W >= (int64_t{1} << 31)) return 0;
  const int64_t L = H * W;
  if (!shape_ok(batch, dim, L) || !d_state_ok(d_state) || (dtype != VMSCAN_F32 && dtype != VMSCAN_BF16)) return 0;
  return ss2d_bwd_layout(batch, dim, L, plan_chunk(plan_base(batch, dim, d_state), L, 0), dtype == VMSCAN_F32 ? 4 : 2,
                         d_state)
      .total;
}

vmscan_status ss2d_cross_scan_bwd(const void* x, const void* delta_raw, const float* A_log, const void* B,
                                  const void* C, const float* D, const float* delta_bias, const void* z,
                                  const void* dout, void* dx, void* ddelta_raw, float* dA_log, void* dB, void* dC,
                                  float* dD, float* ddelta_bias, void* dz, int64_t batch, int64_t dim, int64_t H,
                                  int64_t W, int d_state, vmscan_dtype dtype, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  const void* ptrs[] = {x, delta_raw, A_log, B, C, D, delta_bias, dout, dx, ddelta_raw, dA_log, dB, dC, dD,
                        ddelta_bias};
  for (const void* p : ptrs)
    if (!p) return VMSCAN_ERR_NULL;
  if ((z == nullptr) != (dz == nullptr)) return VMSCAN_ERR_NULL;  // the gate and its gradient come together
  if (H < 1 || W < 1 || H >= (int64_t{1} << 31) || W >= (int64_t{1} << 31)) return VMSCAN_ERR_SHAPE;
  const int64_t L = H * W;
  if (!shape_ok(batch, dim, L)) return VMSCAN_ERR_SHAPE;
  if (!d_state_ok(d_state) || (dtype != VMSCAN_F32 && dtype != VMSCAN_BF16)) return VMSCAN_ERR_UNSUPPORTED;
  for (const void* p : ptrs)
    if (!aligned16(p)) return VMSCAN_ERR_ALIGN;
  if (z && (!aligned16(z) || !aligned16(dz))) return VMSCAN_ERR_ALIGN;
  const int64_t Kf = plan_chunk(plan_base(batch, dim, d_state), L, 0);
  const size_t esz = dtype == VMSCAN_F32 ? 4 : 2;
  const Ss2dBwdLayout lay = ss2d_bwd_layout(batch, dim, L, Kf, esz, d_state);
  const vmscan_status ws = check_workspace(workspace, workspace_bytes, lay.total);
  if (ws != VMSCAN_OK) return ws;
  unsigned char* wsp = static_cast<unsigned char*>(workspace);
  const vmscan_status st =
      dtype == VMSCAN_F32
          ? run_ss2d_bwd<float>(x, delta_raw, A_log, B, C, D, delta_bias, z, dout, dx, ddelta_raw, dA_log, dB, dC, dD,
                                ddelta_bias, dz, batch, dim, H, W, d_state, wsp, lay, Kf, stream)
          : run_ss2d_bwd<uint16_t>(x, delta_raw, A_log, B, C, D, delta_bias, z, dout, dx, ddelta_raw, dA_log, dB, dC,
                                   dD, ddelta_bias, dz, batch, dim, H, W, d_state, wsp, lay, Kf, stream);
  return finish_call(st, workspace, stream);
}

vmscan_status ss2d_cross_scan_fwd(const void* x, const void* delta_raw, const float* A_log, const void* B,
                                  const void* C, const float* D, const float* delta_bias, const void* z, void* out,
                                  int64_t batch, int64_t dim, int64_t H, int64_t W, int d_state, vmscan_dtype dtype,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return ss2d_cross_scan_fwd_ex(x, delta_raw, A_log, B, C, D, delta_bias, z, out, batch, dim, H, W, d_state, dtype,
                                workspace, workspace_bytes, 0, stream);
}

}  // extern "C"
