// Decode QMV kernels for gfx950 (wave64): y[m][n] = sum_k x[m][k] * (s*q + b)
// over group-wise affine low-bit weights, M = 1..5 activation rows sharing
// one read of W.
//
// Method: "oMLX Bonsai 自定义内核" article, section 二 -- path 1 (qmv_fast:
// 1-bit codes in uint32, shift-unpacked in registers, never materialized as
// float weights), path 2 (qmv_wide: one read of W serves M = 2..5 rows; the
// symmetric variant implies bias = -scale*ratio and skips the bias read) and
// path 3 (t5 ternary bytes, 13/26 bytes per 64/128-weight group).
//
// gfx950 design
// -------------
// * One workgroup of W = 8 or 12 waves per CU (12 on the long shapes: with
//   4-row units for t5 at M >= 3, 2-row units otherwise).  A wave holds four slots of 16 lanes; the 16 lanes of a slot
//   cover one 1024-code K tile of R = 1, 2 or 4 rows, each lane one chunk:
//   64 codes of 1/2-bit words (8 or 16 bytes) or one 13-byte t5 run (a
//   whole 64-group, or half of a 128-group: 65 + 63 codes).
// * Work unit = (row-group of R rows, K tile).  A workgroup's units, in the
//   order of their bytes, are dealt to its slots cyclically (slot k: units
//   k, k + 4W, ...), so at every step its slots read one contiguous stretch
//   of its rows; a slot keeps a ring of P units in flight, so HBM reads
//   overlap the arithmetic without any barrier.  Each unit's partial sums
//   are reduced over the slot's lanes into LDS, keyed by (row-group, tile),
//   and at the end every row adds its tiles in order.  Nothing in a row's
//   sums depends on M, R, P or the slot that took a unit, so row m of a
//   wide call is bit-identical to a call with that row alone.
// * x is staged per segment of K tiles in LDS, permuted into the order in
//   which the unpack below produces code pairs and pre-scaled per code
//   position.  Its loads are issued before the ring loads so that waiting
//   for x never waits for W.
// * Scaled codes: a code masked in place inside a 16-bit half reads as the
//   fp16 subnormal q * 2^e * 2^-24, e its bit offset in the half;
//   v_dot2_f32_f16 multiplies it by the staged x*2^(c-e), so every product
//   is q*x*2^(c-24) exactly, with no per-code conversion.  c is a power-of-
//   two exponent chosen per staged chunk from its largest |x| (E = that
//   value's fp16 exponent field, c = min(29 - E, 15)): the largest value
//   lands in [2^14, 2^15), or a chunk below 1/2 is scaled by 2^15, so the
//   staged fp16 values stay exact for every input magnitude fp16 can hold
//   (elements below 2^-19 of their chunk's largest excepted), and the
//   result scales with x.  2^-c multiplies the chunk's product sum.
// * t5 bytes go through a 256-entry LDS table that holds a byte's five
//   base-3 digits as 2-bit fields (and a second copy with the fields in the
//   upper half, for the second byte of a pair, so that no shift is needed);
//   two bytes fill one dword and five masks
//   give five half2 code pairs.  The run's single last byte is paired with
//   itself (digits 0/1 and 2/3 in the two halves), so it costs two or three
//   products instead of five.  13-byte runs are loaded as one dword-aligned
//   16-byte window and realigned with v_alignbyte_b32.
// * Epilogue per chunk: b*X + s*(P*2^-c) in fp32 (units of 2^-24), with X
//   the chunk's (or, for 128-groups, the group's) sum of x.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace bq {

typedef _Float16 half_t;
typedef half_t half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// dword-aligned (not 16-byte aligned) view for t5 rows
typedef uint32_t u32x4a __attribute__((ext_vector_type(4), aligned(4)));

enum { FMT_U1 = 1, FMT_U2 = 2, FMT_T5 = 5 };
constexpr int kTile = 1024;        // codes per K tile
constexpr int kKL = 16;            // lanes per slot (chunks per tile)
constexpr int kWaves = 8;          // waves per workgroup at M <= 2 (one workgroup per CU)
constexpr int kThreads = 64 * kWaves;
constexpr int kSlots = kThreads / kKL;
// Instances with kWaves3 = 12 waves (three per SIMD) exist too: a unit's
// loop is a chain of staged-x LDS reads and dot products that two waves per
// SIMD do not hide.  Their registers must fit three waves' share (168).
constexpr int kWaves3 = 12;
constexpr int kR = 2;              // rows per row-group of the scale-staging limit (the kernels take R = 1, 2 or 4)
constexpr int kXD = 36;            // LDS dwords per staged chunk (32-35 used)

struct QmvParams {
  const half_t* x;       // [M][K]
  const uint8_t* w;      // [N][row_bytes]
  const half_t* s;       // [N][G]
  const half_t* b;       // [N][G] (unused when the bias is implied)
  half_t* y;             // [M][N]
  int N, K, G;           // G = K / group_size
  int row_bytes;
  int rows_per_wg;       // rows of one workgroup
  int ntiles;            // ceil(K / kTile)
  int seg_tiles;         // tiles per x segment staged in LDS
  int nseg;              // ceil(ntiles / seg_tiles)
  int x_bytes;           // M * K * 2 (buffer descriptor size)
  int w_bytes;           // N * row_bytes (buffer descriptor size)
  int sb_bytes;          // N * G * 2
  int sb_dwords;         // LDS dwords of the staged scale/bias block
  float ratio;           // implied bias = -scale * ratio
};

// --------------------------------------------------------------------------
// Format traits.  place(pos) maps code `pos` of a K tile (0..1023) to its
// chunk, staged dword, half and exponent; CB = packed bytes per chunk.
// --------------------------------------------------------------------------
template <int FMT, int GS> struct Fmt;

// 2-bit: word i of a chunk holds codes 16i..16i+15; pair p = (code p, code
// p+8); pairs 0..4 are masked in place (offset 2p), pairs 5..7 after >> 10.
template <int GS> struct Fmt<FMT_U2, GS> {
  static constexpr int CB = 16;
  __device__ static inline void place(int pos, int& c, int& d, int& h, int& e) {
    c = pos >> 6;
    const int q = pos & 63, i = q >> 4, j = q & 15, pp = j & 7;
    h = j >> 3;
    d = 8 * i + pp;
    e = 2 * (pp < 5 ? pp : pp - 5);
  }
};

// 1-bit: word i of a chunk holds codes 32i..32i+31; pair p = (code p,
// code p+16); pairs 0..9 masked in place (offset p), 10..15 after >> 10.
template <int GS> struct Fmt<FMT_U1, GS> {
  static constexpr int CB = 8;
  __device__ static inline void place(int pos, int& c, int& d, int& h, int& e) {
    c = pos >> 6;
    const int q = pos & 63, i = q >> 5, j = q & 31, pp = j & 15;
    h = j >> 4;
    d = 16 * i + pp;
    e = pp < 10 ? pp : pp - 10;
  }
};

// t5: a chunk is 13 bytes; bytes (2p, 2p+1), p < 6, form pair p whose digit
// i < 4 is staged at dword 4p+i and digit 4 at 28+p; byte 12 is single and
// pairs its own digits: (0, 1) at dword 24, (2, 3) at 25, digit 4 at 26.
__device__ inline void t5_slot(int t, int i, int& d, int& h) {
  if (t < 12) {
    const int p = t >> 1;
    h = t & 1;
    d = (i < 4) ? 4 * p + i : 28 + p;
  } else {
    h = i < 4 ? (i & 1) : 0;
    d = 24 + (i >> 1);
  }
}

template <> struct Fmt<FMT_T5, 64> {
  static constexpr int CB = 13;
  __device__ static inline void place(int pos, int& c, int& d, int& h, int& e) {
    c = pos >> 6;
    const int q = pos & 63, t = q / 5, i = q - 5 * t;
    e = 2 * i;
    t5_slot(t, i, d, h);
  }
};

// 128-groups are split into bytes 0..12 (codes 0..64) and bytes 13..25
// (codes 65..127 and two zero pad digits): chunks 2g and 2g+1.
template <> struct Fmt<FMT_T5, 128> {
  static constexpr int CB = 13;
  __device__ static inline void place(int pos, int& c, int& d, int& h, int& e) {
    const int g = pos >> 7, r = pos & 127, hi = r >= 65 ? 1 : 0;
    c = 2 * g + hi;
    const int byte = r / 5, i = r - 5 * byte;
    e = 2 * i;
    t5_slot(byte - 13 * hi, i, d, h);
  }
};

// --------------------------------------------------------------------------
// helpers
// --------------------------------------------------------------------------
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c,
                                false);
}

__device__ __forceinline__ float h2f(half_t v) { return (float)v; }
__device__ __forceinline__ float lo_half(uint32_t v) {
  return h2f(__builtin_bit_cast(half_t, (uint16_t)(v & 0xFFFFu)));
}
__device__ __forceinline__ float hi_half(uint32_t v) {
  return h2f(__builtin_bit_cast(half_t, (uint16_t)(v >> 16)));
}

// Sum over the 16 lanes of a DPP row (row_shr 1, 2, 4, 8 with zero fill):
// the last lane of the row gets the total.
__device__ __forceinline__ float row_sum16(float v) {
  int x = __builtin_bit_cast(int, v);
  x = __builtin_bit_cast(int, __builtin_bit_cast(float, x) +
                                  __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false)));
  x = __builtin_bit_cast(int, __builtin_bit_cast(float, x) +
                                  __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false)));
  x = __builtin_bit_cast(int, __builtin_bit_cast(float, x) +
                                  __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false)));
  x = __builtin_bit_cast(int, __builtin_bit_cast(float, x) +
                                  __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false)));
  return __builtin_bit_cast(float, x);
}

// row_sum16 of several values, step by step across all of them, so that no
// step waits for the one just before it.  Same additions, same order.
template <int CTL, int N>
__device__ __forceinline__ void dpp_add_step(float (&v)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i)
    v[i] += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v[i]), CTL, 0xF, 0xF, false));
}
template <int N>
__device__ __forceinline__ void rows_sum16(float (&v)[N]) {
  dpp_add_step<0x111>(v);
  dpp_add_step<0x112>(v);
  dpp_add_step<0x114>(v);
  dpp_add_step<0x118>(v);
}

// Workgroup barrier for LDS hand-offs only.  __syncthreads() also fences
// global memory, which on this GPU waits for every load in flight (loads and
// stores share one counter) and would drain the prefetched weights; here only
// the LDS traffic is waited for.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Forces the partial sums to be computed here: keeps the compiler from
// sinking the dot products of several quads below later loads, which would
// keep a whole chunk of x live in registers.
template <int R, int M>
__device__ __forceinline__ void pin_partials(float (&Pd)[R][M]) {
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) asm volatile("" : "+v"(Pd[r][m]));
}

// Half `h` of dword a next to half `g` of dword b: (a.h, b.g) as one dword.
__device__ __forceinline__ uint32_t pair_halves(uint32_t a, int h, uint32_t b, int g) {
  const uint32_t lo = h ? (a >> 16) : (a & 0xFFFFu);
  const uint32_t hi = g ? (b & 0xFFFF0000u) : (b << 16);
  return lo | hi;
}

// (lo, hi) fp16 pair times 2^k, -14 <= k <= 15 (one fp16 rounding, to
// nearest even, of the exact product).
__device__ __forceinline__ uint32_t scale_pair(uint32_t v, int k) {
  const half2_t f = __builtin_bit_cast(half2_t, v);
  const half_t sc = __builtin_bit_cast(half_t, (uint16_t)((k + 15) << 10));
  const half2_t r = f * half2_t{sc, sc};
  return __builtin_bit_cast(uint32_t, r);
}

// (lo, hi) fp16 pair times (2^klo, 2^khi), each -14 <= k <= 15.
__device__ __forceinline__ uint32_t scale_pair2(uint32_t v, int klo, int khi) {
  const half2_t f = __builtin_bit_cast(half2_t, v);
  const half_t slo = __builtin_bit_cast(half_t, (uint16_t)((klo + 15) << 10));
  const half_t shi = __builtin_bit_cast(half_t, (uint16_t)((khi + 15) << 10));
  const half2_t r = f * half2_t{slo, shi};
  return __builtin_bit_cast(uint32_t, r);
}

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// Staging exponent of a chunk whose largest |x| has the fp16 magnitude bits
// amax: c = min(29 - E, 15), E = amax's exponent field.  Then the largest
// value times 2^c lies in [2^14, 2^15) (for E >= 14), and x * 2^(c-e) for
// a code offset e <= 9 is exact in fp16 unless |x| is below 2^-19 of the
// chunk's largest; chunks below 1/2 get c = 15, where x * 2^(15-e) is
// exact for every fp16 x (subnormal inputs are multiples of 2^-24).
__device__ __forceinline__ int stage_exponent(uint32_t amax) {
  const int E = (int)(amax >> 10);
  return 29 - E < 15 ? 29 - E : 15;
}

// t5 digit table entry: digit i of byte v at bits 2i..2i+1.
__device__ __forceinline__ uint32_t t5_fields(uint32_t v) {
  uint32_t f = 0;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    f |= (v % 3u) << (2 * i);
    v /= 3u;
  }
  return f;
}

// LDS dwords per staged chunk for all M rows: M*kXD, padded so that the 16
// chunks of a tile start on distinct 4-dword bank groups.
template <int M> constexpr int chunk_stride() { return M * kXD + ((M % 2 == 0) ? 4 : 0); }

typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, int bytes) {
  // dword 3 of a raw buffer descriptor on gfx9-class GPUs; reads outside
  // [0, bytes) return zero
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}

// Packed chunk of one row held by one lane.
template <int FMT> struct Chunk;
template <> struct Chunk<FMT_U2> { u32x4 v; };
template <> struct Chunk<FMT_U1> { u32x2 v; };
template <> struct Chunk<FMT_T5> { u32x4 v; };

// The chunk at byte `off` of the packed rows.  The whole offset goes in the
// per-lane operand: only that operand is range-checked against the
// descriptor, so an offset past the end reads zeros and touches no memory.
template <int FMT>
__device__ __forceinline__ void load_chunk(Chunk<FMT>& c, rsrc_t w, uint32_t off) {
  if constexpr (FMT == FMT_U2) {
    c.v = __builtin_amdgcn_raw_buffer_load_b128(w, (int)off, 0, 0);
  } else if constexpr (FMT == FMT_U1) {
    c.v = __builtin_amdgcn_raw_buffer_load_b64(w, (int)off, 0, 0);
  } else {
    // 13 bytes at off, in the dword-aligned 16-byte window that holds them
    // (past the end of W it reads zeros).
    c.v = __builtin_amdgcn_raw_buffer_load_b128(w, (int)(off & ~3u), 0, 0);
  }
}

// --------------------------------------------------------------------------
// x staging of one segment (Ts tiles from tile s0).  Task = (m, tile,
// chunk): one thread loads the chunk's 64 x values (65/63 for the halves of
// a t5 128-group), writes its staged dwords (permuted into the order the
// unpack produces code pairs, pre-scaled by 2^-e) with 16-byte LDS stores
// and its sum of x.  xstage_plan does the index arithmetic (before any load
// is in flight), xstage_load loads into registers and xstage_commit writes
// LDS, so that other loads can be issued in between.
// --------------------------------------------------------------------------
template <int FMT, int GS> struct XSpan {
  // the halves of a t5 128-group need one x dword past the chunk's 64 codes
  static constexpr bool TAIL = FMT == FMT_T5 && GS == 128;
};

// 64 x values from the chunk's nominal start (8 16-byte vectors) and, for
// t5 128-groups, the dword after them; where they go
template <int FMT, int GS> struct XStage {
  u32x4 v[8];
  uint32_t tail;
  uint32_t off;  // byte offset in x
  int c;         // chunk within its tile
  int dst;       // staged dwords: xs + dst
  int xi;        // sum of x: xsum[xi]
  bool live;     // the thread has a task
  bool wave;     // some thread of the wave has a task
};
constexpr int kStageRounds = 2;  // staging tasks per thread

template <int FMT, int GS, int M>
__device__ __forceinline__ void xstage_plan(const QmvParams& p, int s0, int Ts, int task, XStage<FMT, GS>& st) {
  const int ntask = M * Ts * kKL;
  const int c = task % kKL, tt = (task / kKL) % Ts, m = min(task / (kKL * Ts), M);
  st.c = c;
  st.dst = (tt * kKL + c) * chunk_stride<M>() + m * kXD;
  st.xi = (tt * kKL + c) * M + m;
  st.live = task < ntask;
  st.wave = ((int)threadIdx.x & ~63) + (task - (int)threadIdx.x) < ntask;
  // the chunk's nominal first code; t5 128-groups: chunk 2g loads from code
  // 128g, chunk 2g+1 from 128g+64 (both 16-byte aligned).  A chunk past K
  // loads from an offset with bit 31 set (x is below 2^30 bytes): out of the
  // descriptor's range, it reads zeros, so the chunk stages zeros.
  const int k0 = (s0 + tt) * kTile + 64 * c;
  st.off = (2u * ((uint32_t)m * (uint32_t)p.K + (uint32_t)k0)) | (k0 < p.K ? 0u : 0x80000000u);
}

template <int FMT, int GS>
__device__ __forceinline__ void xstage_load(rsrc_t rx, XStage<FMT, GS>& st) {
  if (!st.wave) {  // whole waves without a task issue nothing
    // (and hold zeros: otherwise a skipped round would keep the previous
    // segment's registers live through the whole unit loop)
#pragma unroll
    for (int j = 0; j < 8; ++j) st.v[j] = u32x4{0u, 0u, 0u, 0u};
    return;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) st.v[j] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(st.off + 16u * j), 0, 0);
  if constexpr (XSpan<FMT, GS>::TAIL) st.tail = __builtin_amdgcn_raw_buffer_load_b32(rx, (int)(st.off + 128u), 0, 0);
}

template <int FMT, int GS, int M>
__device__ __forceinline__ void xstage_commit(const XStage<FMT, GS>& st, uint32_t* xs, float2* xsum) {
  if (!st.live) return;
  const int c = st.c;
  // X[j] = (x[2j], x[2j+1]) of the loaded span
  auto X = [&](int j) -> uint32_t { return j < 32 ? st.v[j >> 2][j & 3] : st.tail; };
  auto H = [&](int k) -> uint32_t { return (X(k >> 1) >> (16 * (k & 1))) & 0xFFFFu; };  // x[k] bits
  // the chunk's staging exponent, from the largest |x| of the loaded span
  // (for a t5 128-group half a value or two of the neighbouring half may
  // take part: any exponent is exact as long as staging and epilogue agree)
  // largest |x| = max(largest x, -smallest x), with three-input packed
  // maximum/minimum (IEEE maximum: the same magnitude bits as an integer
  // max of |x|, a NaN giving the NaN exponent as before)
  constexpr int NJ = XSpan<FMT, GS>::TAIL ? 33 : 32;
  half2_t mx = __builtin_bit_cast(half2_t, X(0)), mn = mx;
#pragma unroll
  for (int j = 1; j + 1 < NJ; j += 2) {
    const half2_t a = __builtin_bit_cast(half2_t, X(j)), b2 = __builtin_bit_cast(half2_t, X(j + 1));
    mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx, a), b2);
    mn = __builtin_elementwise_minimum(__builtin_elementwise_minimum(mn, a), b2);
  }
  if constexpr (NJ % 2 == 0) {
    const half2_t a = __builtin_bit_cast(half2_t, X(NJ - 1));
    mx = __builtin_elementwise_maximum(mx, a);
    mn = __builtin_elementwise_minimum(mn, a);
  }
  const half2_t am2 = __builtin_elementwise_maximum(mx, -mn);
  const half_t amh = __builtin_elementwise_maximum(am2.x, am2.y);
  const int ce = stage_exponent(__builtin_bit_cast(uint16_t, amh) & 0x7FFFu);
  // (x[k0], x[k1]) as one dword: one v_perm_b32 of the two loaded dwords
  auto PX = [&](int k0_, int k1_) -> uint32_t {
    const uint32_t sel = ((k0_ & 1) ? 0x0302u : 0x0100u) | ((k1_ & 1) ? 0x07060000u : 0x05040000u);
    return __builtin_amdgcn_perm(X(k1_ >> 1), X(k0_ >> 1), sel);
  };
  auto P2 = [&](int k0_, int k1_, int e) -> uint32_t {  // (x[k0], x[k1]) * 2^(ce-e); k < 0 means 0
    if (k0_ >= 0 && k1_ >= 0) return scale_pair(PX(k0_, k1_), ce - e);
    const uint32_t lo = k0_ >= 0 ? H(k0_) : 0u;
    const uint32_t hi = k1_ >= 0 ? H(k1_) : 0u;
    return scale_pair(lo | (hi << 16), ce - e);
  };
  // (x[k0] * 2^(ce-e0), x[k1] * 2^(ce-e1)); k < 0 means 0
  auto P2x = [&](int k0_, int k1_, int e0, int e1) -> uint32_t {
    if (k0_ >= 0 && k1_ >= 0) return scale_pair2(PX(k0_, k1_), ce - e0, ce - e1);
    const uint32_t lo = k0_ >= 0 ? H(k0_) : 0u;
    const uint32_t hi = k1_ >= 0 ? H(k1_) : 0u;
    return scale_pair2(lo | (hi << 16), ce - e0, ce - e1);
  };
  uint32_t out[36];
#pragma unroll
  for (int d = 0; d < 36; ++d) out[d] = 0u;
  float sum = 0.f;
  const uint32_t ones = 0x3C003C00u;  // (1.0, 1.0)
  if constexpr (FMT == FMT_U2) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int pp = 0; pp < 8; ++pp) {
        const int e = 2 * (pp < 5 ? pp : pp - 5);
        out[8 * i + pp] = P2(16 * i + pp, 16 * i + pp + 8, e);
      }
#pragma unroll
    for (int j = 0; j < 32; ++j) sum = dot2(X(j), ones, sum);
  } else if constexpr (FMT == FMT_U1) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int pp = 0; pp < 16; ++pp) {
        const int e = pp < 10 ? pp : pp - 10;
        out[16 * i + pp] = P2(32 * i + pp, 32 * i + pp + 16, e);
      }
#pragma unroll
    for (int j = 0; j < 32; ++j) sum = dot2(X(j), ones, sum);
  } else if constexpr (GS == 64) {
    // codes 0..63: pairs p < 6 hold codes 10p+i / 10p+5+i; byte 12 (codes
    // 60..63, its digit 4 a pad) pairs its own digits: (0, 1), (2, 3)
#pragma unroll
    for (int pr = 0; pr < 6; ++pr) {
#pragma unroll
      for (int i = 0; i < 4; ++i) out[4 * pr + i] = P2(10 * pr + i, 10 * pr + 5 + i, 2 * i);
      out[28 + pr] = P2(10 * pr + 4, 10 * pr + 9, 8);
    }
    out[24] = P2x(60, 61, 0, 2);
    out[25] = P2x(62, 63, 4, 6);
#pragma unroll
    for (int j = 0; j < 32; ++j) sum = dot2(X(j), ones, sum);
  } else {
    // 128-group halves.  Even chunk: codes 0..64 of the group, loaded from
    // the group start.  Odd chunk: codes 65..127, loaded from code 64 of the
    // group (the chunk's nominal start), so local code q sits at span q+1.
    auto half_group = [&](auto HI) {
      constexpr int off = decltype(HI)::value;  // span index of local code 0
#pragma unroll
      for (int pr = 0; pr < 6; ++pr) {
#pragma unroll
        for (int i = 0; i < 4; ++i) out[4 * pr + i] = P2(off + 10 * pr + i, off + 10 * pr + 5 + i, 2 * i);
        out[28 + pr] = P2(off + 10 * pr + 4, off + 10 * pr + 9, 8);
      }
      // single byte, its own digits paired: (0, 1), (2, 3), (4, -).  Even
      // chunk byte 12 = codes 60..64 (5 digits); odd chunk byte 25 = codes
      // 125..127 (3 digits) = local 60..62
      out[24] = P2x(off + 60, off + 61, 0, 2);
      out[25] = P2x(off + 62, off == 1 ? -1 : off + 63, 4, 6);
      out[26] = P2x(off == 1 ? -1 : 64, -1, 8, 0);
      // sum of this half's codes: even 0..64 (span 0..64), odd 65..127 (span 1..63)
      if constexpr (off == 0) {
#pragma unroll
        for (int j = 0; j < 32; ++j) sum = dot2(X(j), ones, sum);
        sum += h2f(__builtin_bit_cast(half_t, (uint16_t)H(64)));
      } else {
        sum = h2f(__builtin_bit_cast(half_t, (uint16_t)(X(0) >> 16)));
#pragma unroll
        for (int j = 1; j < 32; ++j) sum = dot2(X(j), ones, sum);
      }
    };
    if (c & 1) half_group(std::integral_constant<int, 1>{});
    else half_group(std::integral_constant<int, 0>{});
  }
  if constexpr (FMT == FMT_T5 && GS == 128) {
    // the group's sum goes to its even chunk; odd chunks carry 0
    const float other = __shfl_xor(sum, 1, 64);
    sum = (c & 1) ? 0.f : sum + other;
  }
  // every staged chunk of the segment is written (chunks past K with zeros),
  // so LDS needs no clearing
  uint32_t* dst = xs + st.dst;
#pragma unroll
  for (int q = 0; q < 9; ++q)
    *reinterpret_cast<u32x4*>(dst + 4 * q) = u32x4{out[4 * q], out[4 * q + 1], out[4 * q + 2], out[4 * q + 3]};
  // the sum * 2^-24 (the units of the products) and the factor 2^-ce that
  // brings the chunk's products to those units
  xsum[st.xi] = float2{sum * 5.9604644775390625e-08f, __builtin_bit_cast(float, (uint32_t)(127 - ce) << 23)};
}

// --------------------------------------------------------------------------
// Scale/bias staging.  A workgroup's rows are contiguous in the [N][G] scale
// and bias arrays, so its block is one byte range; it is read with 16-byte
// loads from the aligned address at or below its start and stored in LDS,
// one entry per (row, group), entry 8v+i holding element i of vector v.
// Element (row, group) of the block then sits at entry delta + row*G +
// group, delta = (start mod 16) / 2.  An entry is a (scale, bias) fp16 pair
// in one dword, or, for one or two activation rows (where converting per
// chunk would cost more than the LDS it saves), an fp32 pair whose bias is
// already -scale * ratio when the bias is implied.
// --------------------------------------------------------------------------
constexpr int kSbRounds = 2;  // 16-byte vectors per thread and array
template <int M> constexpr bool sb_f32() { return M <= 2; }
constexpr int sb_entry_dwords(int M) { return M <= 2 ? 2 : 1; }

struct SbStage {
  u32x4 s[kSbRounds], b[kSbRounds];
  int nvec;
};

template <bool IMPLIED, int TH>
__device__ __forceinline__ void sbstage_load(rsrc_t rs, rsrc_t rb, uint32_t lo_al, int nvec, SbStage& st) {
  st.nvec = nvec;
#pragma unroll
  for (int k = 0; k < kSbRounds; ++k) {
    const int v = (int)threadIdx.x + k * TH;
    const int off = (int)((lo_al + 16u * (uint32_t)v) | (v < nvec ? 0u : 0x80000000u));
    st.s[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
    if constexpr (!IMPLIED) st.b[k] = __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0);
  }
}

template <bool IMPLIED, bool F32, int TH>
__device__ __forceinline__ void sbstage_commit(const SbStage& st, uint32_t* sbl, float ratio) {
#pragma unroll
  for (int k = 0; k < kSbRounds; ++k) {
    const int v = (int)threadIdx.x + k * TH;
    if (F32 && v < st.nvec) {
      float o[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t sv = st.s[k][j], bv = IMPLIED ? 0u : st.b[k][j];
        o[4 * j] = lo_half(sv);
        o[4 * j + 2] = hi_half(sv);
        o[4 * j + 1] = IMPLIED ? -o[4 * j] * ratio : lo_half(bv);
        o[4 * j + 3] = IMPLIED ? -o[4 * j + 2] * ratio : hi_half(bv);
      }
      float* dst = reinterpret_cast<float*>(sbl) + 16 * v;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(dst + 4 * q) = float4{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]};
    } else if (!F32 && v < st.nvec) {
      uint32_t o[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t sv = st.s[k][j], bv = IMPLIED ? 0u : st.b[k][j];
        o[2 * j] = __builtin_amdgcn_perm(bv, sv, 0x05040100u);      // (s lo, b lo)
        o[2 * j + 1] = __builtin_amdgcn_perm(bv, sv, 0x07060302u);  // (s hi, b hi)
      }
      *reinterpret_cast<u32x4*>(sbl + 8 * v) = u32x4{o[0], o[1], o[2], o[3]};
      *reinterpret_cast<u32x4*>(sbl + 8 * v + 4) = u32x4{o[4], o[5], o[6], o[7]};
    }
  }
}

// --------------------------------------------------------------------------
// Per-chunk multiply: Pd[r][m] = codes(row r) . xstaged(m).
// xc points at the lane's staged chunk; row m of x is kXD dwords further.
// --------------------------------------------------------------------------
template <int FMT, int GS, int M, int R>
__device__ __forceinline__ void chunk_dot(const Chunk<FMT> (&wc)[R], const uint32_t* xc,
                                          const uint32_t* lut, const uint32_t (&sh)[R], float (&Pd)[R][M]) {
  if constexpr (FMT == FMT_U2 || FMT == FMT_U1) {
    // quad q = 4 staged dwords 4q..4q+3 (2-bit: word q/2, pairs 4(q%2)..;
    // 1-bit: word q/4, pairs 4(q%4)..); the next quad's x is read while
    // this one is multiplied
    u32x4 xb[2][M];
#pragma unroll
    for (int m = 0; m < M; ++m) xb[0][m] = *reinterpret_cast<const u32x4*>(xc + m * kXD);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (q + 1 < 8) {
#pragma unroll
        for (int m = 0; m < M; ++m) xb[(q + 1) & 1][m] = *reinterpret_cast<const u32x4*>(xc + m * kXD + 4 * (q + 1));
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        uint32_t c4[4];
        if constexpr (FMT == FMT_U2) {
          const uint32_t wv = wc[r].v[q >> 1];
          if ((q & 1) == 0) {
#pragma unroll
            for (int u = 0; u < 4; ++u) c4[u] = wv & (0x00030003u << (2 * u));
          } else {
            const uint32_t ws = wv >> 10;
            c4[0] = wv & 0x03000300u;
            c4[1] = ws & 0x00030003u;
            c4[2] = ws & 0x000C000Cu;
            c4[3] = ws & 0x00300030u;
          }
        } else {
          const uint32_t wv = wc[r].v[q >> 2];
          const uint32_t ws = wv >> 10;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int pp = 4 * (q & 3) + u;
            c4[u] = pp < 10 ? (wv & (0x00010001u << pp)) : (ws & (0x00010001u << (pp - 10)));
          }
        }
#pragma unroll
        for (int m = 0; m < M; ++m) {
          // the first product starts from the constant 0 (no register to clear)
          float acc = q == 0 ? 0.f : Pd[r][m];
          acc = dot2(c4[0], xb[q & 1][m][0], acc);
          acc = dot2(c4[1], xb[q & 1][m][1], acc);
          acc = dot2(c4[2], xb[q & 1][m][2], acc);
          acc = dot2(c4[3], xb[q & 1][m][3], acc);
          Pd[r][m] = acc;
        }
      }
      pin_partials<R, M>(Pd);
    }
  } else {
    // t5: realign each row's 13 bytes (they start sh[r] bytes into the first
    // dword), then six byte pairs and the single byte 12 via the table
    uint32_t rb[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        rb[r][j] = __builtin_amdgcn_alignbyte(j < 3 ? wc[r].v[j + 1] : 0u, wc[r].v[j], sh[r]);
    }
    u32x4 xq[2][M];
    uint32_t x4[2][M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      xq[0][m] = *reinterpret_cast<const u32x4*>(xc + m * kXD);
      x4[0][m] = xc[m * kXD + 28];
    }
#pragma unroll
    for (int pr = 0; pr < 7; ++pr) {
      const bool paired = pr < 6;
      if (pr + 1 < 7) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
          xq[(pr + 1) & 1][m] = *reinterpret_cast<const u32x4*>(xc + m * kXD + 4 * (pr + 1));
          if (pr + 1 < 6) x4[(pr + 1) & 1][m] = xc[m * kXD + 28 + pr + 1];
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int t0 = 2 * pr, t1 = 2 * pr + 1;
        const uint32_t b0 = (rb[r][t0 >> 2] >> (8 * (t0 & 3))) & 0xFFu;
        uint32_t v = lut[b0];
        if (paired) {
          const uint32_t b1 = (rb[r][t1 >> 2] >> (8 * (t1 & 3))) & 0xFFu;
          v |= lut[256 + b1];  // the same fields, upper half
          const uint32_t q0 = v & 0x00030003u, q1 = v & 0x000C000Cu, q2 = v & 0x00300030u,
                         q3 = v & 0x00C000C0u, q4 = v & 0x03000300u;
#pragma unroll
          for (int m = 0; m < M; ++m) {
            float acc = pr == 0 ? 0.f : Pd[r][m];
            acc = dot2(q0, xq[pr & 1][m][0], acc);
            acc = dot2(q1, xq[pr & 1][m][1], acc);
            acc = dot2(q2, xq[pr & 1][m][2], acc);
            acc = dot2(q3, xq[pr & 1][m][3], acc);
            acc = dot2(q4, x4[pr & 1][m], acc);
            Pd[r][m] = acc;
          }
        } else {
          // the single byte pairs its own digits: (0, 1), (2, 3), and for
          // 128-groups (4, -); 64-groups have no digit 4 in it
          v |= v << 16;
          const uint32_t q0 = v & 0x000C0003u, q1 = v & 0x00C00030u, q2 = v & 0x00000300u;
#pragma unroll
          for (int m = 0; m < M; ++m) {
            float acc = pr == 0 ? 0.f : Pd[r][m];
            acc = dot2(q0, xq[pr & 1][m][0], acc);
            acc = dot2(q1, xq[pr & 1][m][1], acc);
            if constexpr (GS == 128) acc = dot2(q2, xq[pr & 1][m][2], acc);
            Pd[r][m] = acc;
          }
        }
      }
      pin_partials<R, M>(Pd);
    }
  }
}

// --------------------------------------------------------------------------
// The kernel.
// --------------------------------------------------------------------------
template <int FMT, int GS, int M, bool IMPLIED, int P, int R, int W>
__global__ __launch_bounds__(64 * W) void qmv_kernel(QmvParams p) {
  constexpr int TH = 64 * W;     // threads of the workgroup (W waves)
  constexpr int NSL = TH / kKL;  // its slots
  using F = Fmt<FMT, GS>;
  constexpr int CS = chunk_stride<M>();
  extern __shared__ uint32_t smem[];
  __shared__ uint32_t lut[512];  // t5 digit fields: [b] in the low half, [256 + b] in the high

  const int ST = p.seg_tiles;
  const int T = p.ntiles;
  uint32_t* xs = smem;                                              // [ST*16][CS]
  float2* xsum = reinterpret_cast<float2*>(smem + ST * kKL * CS);   // [ST*16][M]
  uint32_t* sbl = reinterpret_cast<uint32_t*>(xsum + ST * kKL * M);  // [sb_dwords]
  constexpr bool SBF = sb_f32<M>();
  float* part = reinterpret_cast<float*>(sbl + p.sb_dwords);        // [NG*T][R*M]

  const int tid = threadIdx.x;
  const int slot = tid / kKL;
  const int kl = tid % kKL;
  const int base = blockIdx.x * p.rows_per_wg;
  const int nrow_wg = min(p.rows_per_wg, p.N - base);
  const int NG = (nrow_wg + R - 1) / R;  // row-groups of this workgroup
  // Descriptor sizes are rounded up to whole dwords: the range check zeroes
  // every dword that reaches past the size, and the dword holding the last
  // byte never leaves the page of a 4-byte aligned buffer.
  const rsrc_t rw = make_rsrc(p.w, (p.w_bytes + 3) & ~3);
  const rsrc_t rx = make_rsrc(p.x, p.x_bytes);
  // the workgroup's scale/bias block: bytes [sb_lo, sb_lo + nrow_wg*G*2)
  const uint32_t sb_lo = (uint32_t)base * (uint32_t)p.G * 2u;
  const uint32_t sb_lo_al = sb_lo & ~15u;
  const int sb_delta = (int)(sb_lo - sb_lo_al) / 2;
  const int sb_nvec = (int)((sb_lo + (uint32_t)nrow_wg * (uint32_t)p.G * 2u - sb_lo_al + 15u) >> 4);

  // x of segment 0 first, so that waiting for it never waits for W
  XStage<FMT, GS> xst[kStageRounds];
#pragma unroll
  for (int k = 0; k < kStageRounds; ++k) xstage_plan<FMT, GS, M>(p, 0, min(ST, T), tid + k * TH, xst[k]);
#pragma unroll
  for (int k = 0; k < kStageRounds; ++k) xstage_load<FMT, GS>(rx, xst[k]);
  SbStage sbst;
  const int sb_size = (p.sb_bytes + 3) & ~3;
  sbstage_load<IMPLIED, TH>(make_rsrc(p.s, sb_size), make_rsrc(IMPLIED ? p.s : p.b, sb_size), sb_lo_al, sb_nvec, sbst);

  auto seg_tiles = [&](int s) { return min(ST, T - s * ST); };

  // ---- Units of segment s: u = g * Ts + t (row-group g, tile t), in the
  // order of their bytes.  Slot k takes units k, k + NSL, k + 2 NSL,
  // ..., so at every step the workgroup's slots read one contiguous stretch
  // of its rows.  Cursor step: NSL units = dg row-groups + dt tiles.
  // Every fetch issues the same loads (rows past N and chunks past K read
  // zeros or data that is never used), so the compiler can wait for exactly
  // the ring entry it needs.  Fetches past the last unit use an offset
  // outside every buffer: no memory is touched and zeros come back.
  Chunk<FMT> ring[P][R];
  int fTs = 1, fdg = 0, fdt = 0, ft = 0, fleft = 0;
  uint32_t fwrow = 0, fc0 = 0;
  auto fetch_start = [&](int s) {
    fTs = seg_tiles(s);
    fdg = NSL / fTs;
    fdt = NSL - fdg * fTs;
    const int g = slot / fTs;
    ft = slot - g * fTs;
    const int U = NG * fTs;
    fleft = slot < U ? (U - 1 - slot) / NSL + 1 : 0;
    fwrow = (uint32_t)(base + g * R) * (uint32_t)p.row_bytes;
    fc0 = (uint32_t)(s * ST * kKL + kl);
  };
  auto fetch = [&](Chunk<FMT>(&dst)[R]) {
    const uint32_t fc = fc0 + (uint32_t)(ft * kKL);
    const bool live = fleft > 0;
    // buffers are below 2^30 bytes: bit 31 puts a dead fetch out of range
    const uint32_t dead = live ? 0u : 0x80000000u;
    // 24-bit multiply (fc < 2^20): a 64-bit multiply-add here would read a
    // don't-care register that may still be the target of a load in flight
    const uint32_t wo = fwrow + __umul24(fc, (uint32_t)F::CB);
#pragma unroll
    for (int r = 0; r < R; ++r) load_chunk<FMT>(dst[r], rw, (wo + (uint32_t)(r * p.row_bytes)) | dead);
    if (live) {
      --fleft;
      ft += fdt;
      int dg = fdg;
      if (ft >= fTs) {
        ft -= fTs;
        ++dg;
      }
      fwrow += (uint32_t)(dg * R) * (uint32_t)p.row_bytes;
    }
  };

  // Each unit's partial products, summed over the slot's 16 lanes, go to
  // part[(row-group * T + tile) * R*M + r*M + m]; rows then add their tiles
  // in order.  No sum depends on M, on the segment length or on which slot
  // took the unit, so a row's result is the same in every such launch.
  int cg = 0, ct = 0, cdg = 0, cdt = 0, cTs = 1;  // compute cursor, same steps
  auto process = [&](int s, const Chunk<FMT>(&wc)[R]) {
    const int cs = ct * kKL + kl;  // chunk within the staged segment
    const int tile = s * ST + ct;
    const int chunk = tile * kKL + kl;
    // (scale, bias) of the unit's rows.  A chunk past K reads its row's last
    // group; its staged x and x sum are zero, so it adds exactly 0.
    const int grp = min((chunk * 64) / GS, p.G - 1);
    float sc[R], bb[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int e = sb_delta + (cg * R + r) * p.G + grp;
      if constexpr (SBF) {
        const float2 v = *reinterpret_cast<const float2*>(sbl + 2 * e);
        sc[r] = v.x;
        bb[r] = v.y;
      } else {
        const uint32_t v = sbl[e];
        sc[r] = lo_half(v);
        bb[r] = IMPLIED ? -sc[r] * p.ratio : hi_half(v);
      }
    }
    float Pd[R][M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m) Pd[r][m] = 0.f;
    // t5 runs start 13 bytes apart: where each row's run sits in its dword
    uint32_t sh[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
      sh[r] = ((uint32_t)(base + cg * R + r) * (uint32_t)p.row_bytes + 13u * (uint32_t)chunk) & 3u;
    chunk_dot<FMT, GS, M, R>(wc, xs + cs * CS, lut, sh, Pd);
    float X[M], F[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float2 xf = xsum[cs * M + m];
      X[m] = xf.x;
      F[m] = xf.y;
    }
    float v[R * M];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int m = 0; m < M; ++m) v[r * M + m] = __builtin_fmaf(bb[r], X[m], sc[r] * (Pd[r][m] * F[m]));
    rows_sum16<R * M>(v);
    if (kl == kKL - 1) {
      float* dst = part + (cg * T + tile) * (R * M);
#pragma unroll
      for (int i = 0; i < R * M; ++i) dst[i] = v[i];
    }
    ct += cdt;
    cg += cdg;
    if (ct >= cTs) {
      ct -= cTs;
      ++cg;
    }
  };

  // Ring fill for segment 0.  Only kEarly units per slot go out before the
  // staging barrier: the x and scale loads share the memory queues with the
  // weight loads, and every weight byte requested ahead of them delays the
  // start of the arithmetic.  A slot without units fetches nothing.
  constexpr int kEarly = P < 1 ? P : 1;
  fetch_start(0);
#pragma unroll
  for (int j = 0; j < kEarly; ++j) fetch(ring[j]);
  if constexpr (FMT == FMT_T5) {
    if (tid < 256) {
      const uint32_t f = tid < 243 ? t5_fields((uint32_t)tid) : 0u;
      lut[tid] = f;
      lut[256 + tid] = f << 16;
    }
  }
#pragma unroll
  for (int k = 0; k < kStageRounds; ++k) xstage_commit<FMT, GS, M>(xst[k], xs, xsum);
  sbstage_commit<IMPLIED, SBF, TH>(sbst, sbl, p.ratio);
  lds_barrier();  // x of segment 0, scales and biases staged; table built
#pragma unroll
  for (int j = kEarly; j < P; ++j) fetch(ring[j]);

  for (int s = 0; s < p.nseg; ++s) {
    cTs = seg_tiles(s);
    cdg = NSL / cTs;
    cdt = NSL - cdg * cTs;
    cg = slot / cTs;
    ct = slot - cg * cTs;
    const int U = NG * cTs;
    const int n = slot < U ? (U - 1 - slot) / NSL + 1 : 0;  // units of this slot
    for (int i = 0; i < n; i += P) {
#pragma unroll
      for (int j = 0; j < P; ++j) {
        if (i + j < n) process(s, ring[j]);
        fetch(ring[j]);
      }
    }
    if (s + 1 < p.nseg) {
#pragma unroll
      for (int k = 0; k < kStageRounds; ++k)
        xstage_plan<FMT, GS, M>(p, (s + 1) * ST, seg_tiles(s + 1), tid + k * TH, xst[k]);
#pragma unroll
      for (int k = 0; k < kStageRounds; ++k) xstage_load<FMT, GS>(rx, xst[k]);
      fetch_start(s + 1);
#pragma unroll
      for (int j = 0; j < P; ++j) fetch(ring[j]);
      lds_barrier();  // every slot is done with segment s
#pragma unroll
      for (int k = 0; k < kStageRounds; ++k) xstage_commit<FMT, GS, M>(xst[k], xs, xsum);
    }
    lds_barrier();
  }

  // y = sum over the row's tiles, in tile order, * 2^24
  for (int idx = tid; idx < NG * R * M; idx += TH) {
    const int g = idx / (R * M);
    const int rm = idx - g * (R * M);
    const int r = rm / M, m = rm - r * M;
    if (g * R + r >= nrow_wg) continue;
    const float* src = part + g * T * (R * M) + rm;
    float v = 0.f;
    // eight tiles' loads in flight before their adds (same order of adds)
    for (int t = 0; t < T; t += 8) {
      float b[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] = src[min(t + j, T - 1) * (R * M)];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (t + j < T) v += b[j];
    }
    p.y[(size_t)m * p.N + base + g * R + r] = (half_t)(v * 16777216.0f);
  }
}

}  // namespace bq
