// Prefill products on the matrix cores: y[M][N] = x[M][K] . W^T with W
// unpacked tile by tile, from t5 bytes or from 1/2-bit uint32 codes.
//
// Method: "oMLX Bonsai 自定义内核" article, section 二 path 3 -- for prefill
// with more than 16 rows the t5 weights are unpacked and multiplied in one
// fused kernel that reads each t5 byte once per weight tile.  The same
// pipeline with a decoder for uint32 codes replaces section 二 path 1's
// 1-bit prefill (dequantize to float16, then a matrix multiply).
//
// gfx950 design
// -------------
// * A 512-thread workgroup computes a BM x BN tile of y (BM 32 to 256, BN
//   64 or 128, chosen per call by rules from measured sweeps); the K loop
//   steps 64 codes at a time.  Four waves multiply: each owns a
//   (BM/2) x (BN/2) block and runs v_mfma_f32_16x16x32_f16 on it with fp32
//   accumulators.  Four more waves load the next step's x and decode its
//   weights meanwhile; each SIMD holds one wave of each kind, so the matrix
//   cores and the vector ALUs run at the same time.
// * x tiles go straight from HBM/L2 to LDS with buffer loads that write LDS
//   (no registers, no ALU), into a double buffer.  Rows are 128 bytes of
//   eight 16-byte units, stored at unit (q XOR row%8) so that the MFMA
//   operand reads of 16 rows hit distinct banks.
// * Weights: each decoding thread takes BN/4 codes of one weight row per
//   step.  Their t5 bytes (at most 14) are loaded ahead as a 16-byte window
//   from the dword at or below the first byte and realigned with
//   v_alignbyte.  An LDS table gives, for each byte value and each pair of
//   its five digits, a v_perm_b32 selector that picks the pair's two fp16
//   weights out of the row's three possible weights (held in two dwords:
//   {-s, 0, s} when the bias is -scale, exact, otherwise the correctly
//   rounded s*q + b for q = 0, 1, 2), so two codes cost one v_perm.  The
//   uint32 decoder does the same with a table of selectors per byte of
//   four 2-bit or eight 1-bit codes.
// * Per step: the multiplying waves work on one buffer while the others fill
//   the second one (x loads, weight decode, and the byte and scale loads of
//   the step after); then one barrier.
// * Where an iteration is far shorter than a memory round trip (small M;
//   and the larger tiles, whose x loads one iteration ahead leave the
//   matrix cores waiting): a variant requests x and the raw bytes several
//   iterations ahead into register sets (see qmm_deep_kernel).
// * In both, the two kinds of waves run loops of their own.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dequant_kernels.hpp"
#include "qmv_kernels.hpp"

namespace bq {

typedef half_t half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

struct QmmParams {
  const half_t* x;     // [M][K]
  const uint8_t* w;    // [N][row_bytes]
  const half_t* s;     // [N][G]
  const half_t* b;     // [N][G] or null (implied -scale)
  half_t* y;           // [M][N]
  int M, N, K, G, row_bytes;
  int x_bytes, w_bytes, sb_bytes;  // buffer descriptor sizes
  // K split (qmm_deep_kernel only): ksplit workgroups per tile, each over
  // its share of the K iterations, storing fp32 partial tiles to part
  // (ksplit slices of qmm_part_stride(M, N) floats, [M][N] each) instead
  // of y (part == null: ksplit is 1, y direct)
  float* part;
  int ksplit;
  size_t part_cap;  // host side: bytes the caller's workspace holds
};

// floats per partial-sum slice: M*N rounded up to a multiple of 4 (each
// slice starts 16-byte aligned)
__host__ __device__ inline size_t qmm_part_stride(int M, int N) { return ((size_t)M * N + 3) & ~(size_t)3; }

constexpr int kQmmBK = 64;        // codes per K step
constexpr int kQmmThreads = 512;  // 4 MFMA waves (2 x 2 over the tile) + 4 loading/decoding waves

constexpr size_t qmm_lds_bytes(int BM, int BN, int lut_words, int SUB = 1) {
  return (size_t)2 * SUB * BM * kQmmBK * 2 + (size_t)2 * SUB * BN * kQmmBK * 2 + (size_t)lut_words * 4;
}

// 16-byte unit (row, q) of a 128-byte LDS row
__device__ __forceinline__ int qmm_swz(int row, int q) { return row * 8 + (q ^ (row & 7)); }

// v_perm_b32 selector of a code pair (a, b): bytes 2a, 2a+1 and 2b, 2b+1 of
// the row's weight table {w0, w1 | w2} (two fp16 weights per dword), which
// places the fp16 weights of codes a and b in the low and high half.
__device__ __forceinline__ uint32_t t5_pair_sel(uint32_t a, uint32_t b) {
  return (2u * a) | ((2u * a + 1u) << 8) | ((2u * b) << 16) | ((2u * b + 1u) << 24);
}

// Pair table entry k (0..3) of byte v: the selectors of its digit pairs
// (d0, d1), (d2, d3), (d1, d2), (d3, d4); a pair that starts on digit 4
// takes the high half of entry 3 and the low half of the next byte's
// entry 0.  Bytes above 242 are invalid and get 0.
__device__ __forceinline__ uint32_t t5_pair_entry(uint32_t v, int k) {
  if (v >= 243u) return 0u;
  uint32_t d[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    d[i] = v % 3u;
    v /= 3u;
  }
  const int a = k == 0 ? 0 : k == 1 ? 2 : k == 2 ? 1 : 3;
  return t5_pair_sel(d[a], d[a + 1]);
}

// Where code c (0..GS-1) of a group sits in the group's bytes: 64-groups
// hold code 5j+i at digit i of byte j; 128-groups are two 13-byte halves,
// codes 0..64 in bytes 0..12 and codes 65..127 in bytes 13..25.
template <int GS> constexpr int t5_byte_of(int c) { return (GS == 128 && c >= 65) ? 13 + (c - 65) / 5 : c / 5; }
template <int GS> constexpr int t5_digit_of(int c) { return (GS == 128 && c >= 65) ? (c - 65) % 5 : c % 5; }

// A thread's NC codes in a step: codes 64*PAR + NC*H + u of the group
// (PAR: which half of a 128-group the step covers; always 0 for 64-groups).
template <int GS, int PAR, int H, int NC> struct T5Span {
  static constexpr int c0 = 64 * PAR + NC * H;
  static constexpr int start = t5_byte_of<GS>(c0);  // first byte, within the group
};

// Decodes the thread's NC codes: wv = the 16 bytes from the span's first
// byte, wt_lo/wt_hi = the row's three fp16 weights (wt_lo: q = 0 low half,
// q = 1 high half; wt_hi: q = 2 low half), lut = pair table.  Out: NC/2
// dwords, code pairs (2t, 2t+1) in dword t.  Each pair costs one v_perm_b32
// (plus one v_alignbit_b32 where the pair spans two bytes).
template <int GS, int PAR, int H, int NC>
__device__ __forceinline__ void t5_decode(const uint32_t (&wv)[4], uint32_t wt_lo, uint32_t wt_hi,
                                          const uint32_t* lut, uint32_t (&out)[NC / 2]) {
  using S = T5Span<GS, PAR, H, NC>;
  constexpr int nb = t5_byte_of<GS>(S::c0 + NC - 1) - S::start + 1;  // bytes used
  static_assert(nb <= 14, "span of at most 14 bytes");
  u32x4 e[14];
#pragma unroll
  for (int j = 0; j < nb; ++j)
    e[j] = *reinterpret_cast<const u32x4*>(lut + 4 * ((wv[j >> 2] >> (8 * (j & 3))) & 0xFFu));
#pragma unroll
  for (int t = 0; t < NC / 2; ++t) {
    const int ca = S::c0 + 2 * t, cb = ca + 1;
    const int ja = t5_byte_of<GS>(ca) - S::start, jb = t5_byte_of<GS>(cb) - S::start;
    const int ia = t5_digit_of<GS>(ca);
    uint32_t sel;
    if (ja == jb) {
      // digits (ia, ia + 1) of one byte: entry 0, 2, 1 or 3 for ia = 0..3
      sel = e[ja][ia == 0 ? 0 : ia == 1 ? 2 : ia == 2 ? 1 : 3];
    } else {
      // digit 4 of byte ja (high half of its entry 3), digit 0 of byte jb
      // (low half of its entry 0)
      sel = __builtin_amdgcn_alignbit(e[jb][0], e[ja][3], 16);
    }
    out[t] = __builtin_amdgcn_perm(wt_hi, wt_lo, sel);
  }
}

// The span start and the decode for a runtime span index h < 64/NC (the
// same for a whole wave), dispatched to the compile-time instances.
template <int GS, int PAR, int NC>
__device__ __forceinline__ int t5_span_start(int h) {
  int st = T5Span<GS, PAR, 0, NC>::start;
  if constexpr (64 / NC > 1) {
    if (h == 1) st = T5Span<GS, PAR, 1, NC>::start;
  }
  if constexpr (64 / NC > 2) {
    if (h == 2) st = T5Span<GS, PAR, 2, NC>::start;
    if (h == 3) st = T5Span<GS, PAR, 3, NC>::start;
  }
  return st;
}

template <int GS, int PAR, int NC>
__device__ __forceinline__ void t5_decode_h(int h, const uint32_t (&wv)[4], uint32_t wt_lo, uint32_t wt_hi,
                                            const uint32_t* lut, uint32_t (&out)[NC / 2]) {
  if (h == 0) t5_decode<GS, PAR, 0, NC>(wv, wt_lo, wt_hi, lut, out);
  if constexpr (64 / NC > 1) {
    if (h == 1) t5_decode<GS, PAR, 1, NC>(wv, wt_lo, wt_hi, lut, out);
  }
  if constexpr (64 / NC > 2) {
    if (h == 2) t5_decode<GS, PAR, 2, NC>(wv, wt_lo, wt_hi, lut, out);
    if (h == 3) t5_decode<GS, PAR, 3, NC>(wv, wt_lo, wt_hi, lut, out);
  }
}

// Reads every dword of a loaded register set at the point of use.  A
// decoder uses only some of the dwords it loads; without this the compiler
// may give the unused ones of a load still in flight to other values, and
// must then wait for that load before writing them.
__device__ __forceinline__ void keep_loaded(const u32x4& d) { asm volatile("" ::"v"(d)); }
template <int N>
__device__ __forceinline__ void keep_loaded(const uint32_t (&d)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" ::"v"(d[i]));
}

// ---------------------------------------------------------------------------
// Decoders.  A producer thread owns NC = BN/4 codes of one weight row per K
// step (codes 64*step + NC*h .. +NC-1; h is the same for a whole wave).  A
// decoder loads their packed bytes and the group's scale (and bias) one step
// ahead (issue), and turns them into NC/2 dwords of fp16 pairs, codes
// (2t, 2t+1) in dword t (decode).  kRawLoads is the number of loads issue
// makes, for the pipeline's vmcnt bookkeeping; kLutWords the size of the
// decoder's LDS table.
// ---------------------------------------------------------------------------
template <int BN, int GS, bool IMPLIED>
struct T5Decoder {
  static constexpr int NC = BN / 4;
  static constexpr int kRawLoads = IMPLIED ? 2 : 3;
  static constexpr int kLutWords = 1024;  // 4 pair selectors per byte value
  static constexpr int P1 = GS == 128 ? 1 : 0;
  struct Raw {
    u32x4 d;
    uint16_t s, b;
  };
  rsrc_t rw, rs, rb;
  uint32_t row_off, sb_row;
  int h;

  __device__ __forceinline__ static void init_lut(uint32_t* lut, int tid) {
    for (int e = tid; e < kLutWords; e += kQmmThreads) lut[e] = t5_pair_entry((uint32_t)(e >> 2), e & 3);
  }
  __device__ __forceinline__ T5Decoder(const QmmParams& p, int n, int h_) : h(h_) {
    // whole dwords: the dword holding W's last byte is read in full
    rw = make_rsrc(p.w, (p.w_bytes + 3) & ~3);
    rs = make_rsrc(p.s, p.sb_bytes);
    rb = make_rsrc(IMPLIED ? p.s : p.b, p.sb_bytes);
    row_off = (uint32_t)n * (uint32_t)p.row_bytes;
    sb_row = (uint32_t)n * (uint32_t)p.G;
  }
  __device__ __forceinline__ int group_base(int step) const { return GS == 64 ? 13 * step : 26 * (step >> 1); }
  __device__ __forceinline__ int span_start(int step) const {
    const int par = GS == 128 ? (step & 1) : 0;
    return par == 0 ? t5_span_start<GS, 0, NC>(h) : t5_span_start<GS, P1, NC>(h);
  }
  __device__ __forceinline__ void issue(int step, Raw& rw_) const {
    const uint32_t a = row_off + (uint32_t)(group_base(step) + span_start(step));
    // 16 bytes from the dword at or below the span's first byte: a span has
    // at most 13 bytes (14 for the second half of a 128-group, which starts
    // 0 or 2 bytes into its dword), so the window always holds it; dwords
    // past the end of W read as zeros
    rw_.d = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(a & ~3u), 0, 0);
    const uint32_t so = 2u * (sb_row + (uint32_t)((step * kQmmBK) / GS));
    rw_.s = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)so, 0, 0);
    if constexpr (!IMPLIED) rw_.b = __builtin_amdgcn_raw_buffer_load_b16(rb, (int)so, 0, 0);
    else rw_.b = 0;
  }
  __device__ __forceinline__ void decode(int step, const Raw& rw_, const uint32_t* lut,
                                         uint32_t (&out)[NC / 2]) const {
    const uint32_t a = row_off + (uint32_t)(group_base(step) + span_start(step));
    const uint32_t sh = a & 3u;
    uint32_t wv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) wv[k] = __builtin_amdgcn_alignbyte(k < 3 ? rw_.d[k + 1] : 0u, rw_.d[k], sh);
    // the row's weights for q = 0, 1, 2: {-s, 0, +s} exactly when the bias
    // is -scale, else the correctly rounded s*q + b
    uint32_t wt_lo, wt_hi;
    if constexpr (IMPLIED) {
      wt_lo = (uint32_t)(rw_.s ^ 0x8000u) & 0xFFFFu;  // -s, then +0
      wt_hi = rw_.s;                                 // +s
    } else {
      const float s = h2f(__builtin_bit_cast(half_t, rw_.s)), b = h2f(__builtin_bit_cast(half_t, rw_.b));
      const uint32_t v0 = __builtin_bit_cast(uint16_t, affine_to_half(s, 0u, b));
      const uint32_t v1 = __builtin_bit_cast(uint16_t, affine_to_half(s, 1u, b));
      const uint32_t v2 = __builtin_bit_cast(uint16_t, affine_to_half(s, 2u, b));
      wt_lo = v0 | (v1 << 16);
      wt_hi = v2;
    }
    const int par = GS == 128 ? (step & 1) : 0;
    if (par == 0) t5_decode_h<GS, 0, NC>(h, wv, wt_lo, wt_hi, lut, out);
    else t5_decode_h<GS, P1, NC>(h, wv, wt_lo, wt_hi, lut, out);
  }
};

// Selector table of the uint32 decoder: for the byte value v (four 2-bit or
// eight 1-bit codes, LSB first), the v_perm_b32 selectors that place the
// fp16 weight of each code -- bytes 2q and 2q+1 of the row's weight table --
// two codes per dword.
template <int BITS>
__device__ __forceinline__ uint32_t uq_selector(uint32_t v, int pair) {
  const uint32_t qa = (v >> (2 * pair * BITS)) & ((1u << BITS) - 1u);
  const uint32_t qb = (v >> ((2 * pair + 1) * BITS)) & ((1u << BITS) - 1u);
  return (2u * qa) | ((2u * qa + 1u) << 8) | ((2u * qb) << 16) | ((2u * qb + 1u) << 24);
}

template <int BN, int BITS, int GS, bool IMPLIED>
struct UqDecoder {
  static constexpr int NC = BN / 4;
  static constexpr int CPB = 8 / BITS;                          // codes per byte
  static constexpr int SPB = CPB / 2;                           // selectors per byte
  static constexpr int ND = NC * BITS >= 32 ? NC * BITS / 32 : 1;  // dwords loaded
  static constexpr int kRawLoads = IMPLIED ? 2 : 3;
  static constexpr int kLutWords = 256 * SPB;
  struct Raw {
    uint32_t d[ND];
    uint16_t s, b;
  };
  rsrc_t rw, rs, rb;
  uint32_t row_off, sb_row;
  int h;

  __device__ __forceinline__ static void init_lut(uint32_t* lut, int tid) {
    for (int e = tid; e < kLutWords; e += kQmmThreads) lut[e] = uq_selector<BITS>((uint32_t)(e / SPB), e % SPB);
  }
  __device__ __forceinline__ UqDecoder(const QmmParams& p, int n, int h_) : h(h_) {
    rw = make_rsrc(p.w, p.w_bytes);
    rs = make_rsrc(p.s, p.sb_bytes);
    rb = make_rsrc(IMPLIED ? p.s : p.b, p.sb_bytes);
    row_off = (uint32_t)n * (uint32_t)p.row_bytes;
    sb_row = (uint32_t)n * (uint32_t)p.G;
  }
  // first code of the thread's span, within the row
  __device__ __forceinline__ uint32_t k0(int step) const { return (uint32_t)(step * kQmmBK + NC * h); }
  __device__ __forceinline__ void issue(int step, Raw& rw_) const {
    // the dword holding the span's first code; rows are whole dwords
    const uint32_t a = row_off + ((k0(step) * BITS) >> 5) * 4u;
    if constexpr (ND == 1) {
      rw_.d[0] = __builtin_amdgcn_raw_buffer_load_b32(rw, (int)a, 0, 0);
    } else if constexpr (ND == 2) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(rw, (int)a, 0, 0);
      rw_.d[0] = v[0];
      rw_.d[1] = v[1];
    } else {
      static_assert(ND == 4, "spans of 16, 32 or 64 codes");
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)a, 0, 0);
#pragma unroll
      for (int k = 0; k < 4; ++k) rw_.d[k] = v[k];
    }
    const uint32_t so = 2u * (sb_row + (uint32_t)((step * kQmmBK) / GS));
    rw_.s = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)so, 0, 0);
    if constexpr (!IMPLIED) rw_.b = __builtin_amdgcn_raw_buffer_load_b16(rb, (int)so, 0, 0);
    else rw_.b = 0;
  }
  __device__ __forceinline__ void decode(int step, const Raw& rw_, const uint32_t* lut,
                                         uint32_t (&out)[NC / 2]) const {
    // the row's weights for q = 0 .. 2^BITS-1: bytes 2q, 2q+1 of {wt_hi, wt_lo}
    const float s = h2f(__builtin_bit_cast(half_t, rw_.s));
    const float b = IMPLIED ? -s * (BITS == 1 ? 0.5f : 1.5f) : h2f(__builtin_bit_cast(half_t, rw_.b));
    uint32_t wt_lo, wt_hi = 0;
    wt_lo = (uint32_t)__builtin_bit_cast(uint16_t, affine_to_half(s, 0u, b)) |
            ((uint32_t)__builtin_bit_cast(uint16_t, affine_to_half(s, 1u, b)) << 16);
    if constexpr (BITS == 2)
      wt_hi = (uint32_t)__builtin_bit_cast(uint16_t, affine_to_half(s, 2u, b)) |
              ((uint32_t)__builtin_bit_cast(uint16_t, affine_to_half(s, 3u, b)) << 16);
    // 1-bit spans of 16 codes sit in the upper half of their dword for odd h
    uint32_t d[ND];
#pragma unroll
    for (int k = 0; k < ND; ++k) d[k] = rw_.d[k];
    if constexpr (NC * BITS < 32) d[0] >>= (k0(step) * BITS) & 31u;
    constexpr int NBYTES = NC * BITS / 8;
#pragma unroll
    for (int j = 0; j < NBYTES; ++j) {
      const uint32_t v = (d[j >> 2] >> (8 * (j & 3))) & 0xFFu;
#pragma unroll
      for (int e = 0; e < SPB; ++e) out[j * SPB + e] = __builtin_amdgcn_perm(wt_hi, wt_lo, lut[v * SPB + e]);
    }
  }
};

// SUB: K steps per pipeline iteration.  Each iteration's x and weight bytes
// are requested one iteration ahead and waited for at its end, so one
// iteration costs at least a memory round trip (about a microsecond); with
// small tiles a single 64-code step is much shorter than that, and SUB
// steps per iteration divide that floor by SUB.  The products and their
// order are the same for every SUB.
template <int BM, int BN, class Dec, int SUB>
__global__ __launch_bounds__(kQmmThreads) void qmm_kernel(QmmParams p) {
  constexpr int MB = BM / 32;   // 16-row MFMA blocks per wave (wave rows: BM/2)
  constexpr int NB = BN / 32;   // 16-column MFMA blocks per wave (wave columns: BN/2)
  constexpr int NC = Dec::NC;   // codes a thread decodes per step
  constexpr int RPW = 64 / NC;  // spans per weight row (threads per row)
  static_assert(NC == BN / 4, "one span of BN/4 codes per producer thread");
  extern __shared__ __attribute__((aligned(16))) uint32_t qsmem[];
  half_t* xs = reinterpret_cast<half_t*>(qsmem);                        // [2][SUB][BM*64]
  half_t* ws = xs + 2 * SUB * BM * kQmmBK;                              // [2][SUB][BN*64]
  uint32_t* lut = reinterpret_cast<uint32_t*>(ws + 2 * SUB * BN * kQmmBK);  // [Dec::kLutWords]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // waves 0-3 multiply, waves 4-7 load x and decode weights; each SIMD runs
  // one of each, so the matrix cores and the vector ALUs work side by side
  const bool producer = wave >= 4;
  const int pw = wave & 3;             // producer wave index
  const int wm = (wave >> 1) & 1, wn = wave & 1;
  const int tiles_n = (p.N + BN - 1) / BN;
  const int t = (int)blockIdx.x;
  const int m0 = (t / tiles_n) * BM;
  const int n0 = (t % tiles_n) * BN;
  const int S = p.K / kQmmBK;  // K steps, a multiple of SUB
  const int IT = S / SUB;      // pipeline iterations

  const rsrc_t rx = make_rsrc(p.x, p.x_bytes);

  Dec::init_lut(lut, tid);

  // ---- x loads (producers): chunk c = i*4 + pw covers LDS units
  // [64c, 64c+64) of a buffer, rows 8c..8c+7; lane l loads unit 64c+l
  auto issue_x = [&](int step, int buf) {  // buf: buffer slot (iteration buffer * SUB + sub-step)
    const int k0 = step * kQmmBK;
#pragma unroll
    for (int i = 0; i < BM / 32; ++i) {
      const int c = i * 4 + pw;
      const int u = c * 64 + lane;
      const int row = u >> 3, q = (u & 7) ^ (row & 7);
      const uint32_t off = 2u * ((uint32_t)(m0 + row) * (uint32_t)p.K + (uint32_t)(k0 + q * 8));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rx, (__attribute__((address_space(3))) void*)(xs + buf * BM * kQmmBK + c * 512), 16, (int)off, 0, 0, 0);
    }
  };

  // ---- weight rows (producers): thread -> row r, codes NC*h .. NC*h+NC-1
  // of each step (h is the same for a whole wave)
  const int pt = tid & 255;
  const int r = pt % BN, h = pt / BN;
  static_assert(RPW * BN == 256, "one span per producer thread");
  const Dec dec(p, n0 + r, h);
  typename Dec::Raw raw[SUB];
  auto decode = [&](int step, int buf, int u) {  // raw bytes of sub-step u into buffer slot buf
    keep_loaded(raw[u].d);
    uint32_t out[NC / 2];
    dec.decode(step, raw[u], lut, out);
    half_t* wb = ws + buf * BN * kQmmBK;
#pragma unroll
    for (int t = 0; t < NC / 8; ++t)
      *reinterpret_cast<u32x4*>(wb + qmm_swz(r, (NC / 8) * h + t) * 8) =
          u32x4{out[4 * t], out[4 * t + 1], out[4 * t + 2], out[4 * t + 3]};
  };

  float4_t acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};

  // An LDS read may not target a register that an issued MFMA has yet to
  // read.  When two multiplying waves share a SIMD (two workgroups on one
  // CU) the matrix core reads the last lanes of its A/B operands late enough
  // for the data of an LDS read issued after the MFMA to land first.  So the
  // operands of a group of MFMAs (the whole step where they fit in
  // registers, else each 32-code half) are all read into registers of their
  // own before the group's first MFMA, and the group ends by reading every
  // accumulator in a VALU op, which waits until its MFMAs are done, before
  // the next LDS read is issued.
  constexpr int KS = kQmmBK / 32;
  constexpr int KG = (MB + NB) <= 6 ? KS : 1;  // 32-code halves per group
  auto multiply = [&](int buf) {
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
    const half_t* xb = xs + (buf * SUB + u) * BM * kQmmBK;
    const half_t* wb = ws + (buf * SUB + u) * BN * kQmmBK;
#pragma unroll
    for (int g = 0; g < KS; g += KG) {
      half8_t af[KG][MB], bf[KG][NB];
#pragma unroll
      for (int kk = 0; kk < KG; ++kk) {
        const int q = (g + kk) * 4 + (lane >> 4);
#pragma unroll
        for (int j = 0; j < NB; ++j)
          bf[kk][j] = *reinterpret_cast<const half8_t*>(wb + qmm_swz(wn * (BN / 2) + 16 * j + (lane & 15), q) * 8);
#pragma unroll
        for (int i = 0; i < MB; ++i)
          af[kk][i] = *reinterpret_cast<const half8_t*>(xb + qmm_swz(wm * (BM / 2) + 16 * i + (lane & 15), q) * 8);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < KG; ++kk)
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[kk][i], bf[kk][j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      uint32_t done = 0;
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          done |= __builtin_amdgcn_readfirstlane(__builtin_bit_cast(uint32_t, acc[i][j][0]));
      asm volatile("" ::"s"(done) : "memory");
      __builtin_amdgcn_sched_barrier(0);
    }
    }
  };

  // ---- prologue: iteration 0 (steps 0 .. SUB-1) in buffer 0, raw bytes of
  // iteration 1 in registers
  if (producer) {
#pragma unroll
    for (int u = 0; u < SUB; ++u) issue_x(u, u);
#pragma unroll
    for (int u = 0; u < SUB; ++u) dec.issue(u, raw[u]);
  }
  __syncthreads();  // table built (the loads above are waited for by decode)
  if (producer) {
#pragma unroll
    for (int u = 0; u < SUB; ++u) decode(u, u, u);
    if (IT > 1) {
#pragma unroll
      for (int u = 0; u < SUB; ++u) dec.issue(SUB + u, raw[u]);
    }
  }
  __syncthreads();  // x of iteration 0 (the fence waits for the loads) and its weights

  // loads a producer issues after an iteration's x loads: bytes + scale
  // (+ bias) of each of the SUB steps of the iteration after
  constexpr int kRawLoads = Dec::kRawLoads * SUB;
  static_assert(kRawLoads <= 15, "vmcnt field");
  // The two kinds of waves run loops of their own with the same barriers,
  // so that the waits the compiler places for the loading waves' registers
  // follow the loads those waves issued, not a state merged with the
  // multiplying waves' path.
  if (producer) {
    // iterations 0 .. IT-2 prepare the next one; the last prepares nothing
    // and is left out of the loop, which then has no branch inside (a
    // branch around the preparing part would make the compiler see a path
    // on which this pass's loads meet the next pass's with the registers
    // still in flight, and wait for them on every pass)
    for (int it = 0; it + 1 < IT; ++it) {
      const int nxt = (it & 1) ^ 1;
#pragma unroll
      for (int u = 0; u < SUB; ++u) issue_x((it + 1) * SUB + u, nxt * SUB + u);
#pragma unroll
      for (int u = 0; u < SUB; ++u) decode((it + 1) * SUB + u, nxt * SUB + u, u);
      // always issued (the last pass reloads the last step's bytes,
      // unused), so that the count of loads after the x loads is fixed; not
      // moved above the decode, which would need the registers they fill
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < SUB; ++u) dec.issue(min((it + 2) * SUB + u, S - 1), raw[u]);
      // this wave's x loads of iteration it+1 have landed in LDS (only the
      // loads issued after them may still be in flight), its weight stores
      // are done
      __builtin_amdgcn_s_waitcnt(0x0070 | kRawLoads);  // vmcnt(kRawLoads), lgkmcnt(0)
      // every wave is past iteration it: buffer it&1 is free, buffer nxt is full
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    __builtin_amdgcn_s_barrier();  // the multiplying waves' last iteration
    return;
  }
  for (int it = 0; it < IT; ++it) {
    multiply(it & 1);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }

  // D layout of 16x16x32: lane holds rows 4*(lane/16)+v, column lane%16
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + wm * (BM / 2) + 16 * i + 4 * (lane >> 4) + v;
        const int n = n0 + wn * (BN / 2) + 16 * j + (lane & 15);
        if (m < p.M && n < p.N) p.y[(size_t)m * p.N + n] = (half_t)acc[i][j][v];
      }
}


// ---------------------------------------------------------------------------
// The product where one K iteration of a tile is shorter than a memory round
// trip: 32-row tiles (small M), and the larger tiles too, whose iterations
// do not cover a round trip either.  Same work split and LDS layout as
// qmm_kernel, but the loading waves request x and the raw weight bytes D
// iterations ahead, into D register sets, and store an iteration's x to LDS
// (next to its decoded weights) one iteration before it is multiplied.  An
// iteration then waits only for loads issued D - 1 iterations earlier.
//
// The two kinds of waves run separate loops with the same barriers: the
// compiler places the waits for loaded registers from the loads it sees on
// each path, and a loop shared by both kinds would merge the loading
// waves' state with that of waves that never load, which makes every
// register set look freshly requested (a wait for all loads in flight).
// The products and their order are those of qmm_kernel, so the output is
// the same bit for bit.
// ---------------------------------------------------------------------------
constexpr size_t qmm_deep_lds_bytes(int BM, int BN, int lut_words, int SUB) { return qmm_lds_bytes(BM, BN, lut_words, SUB); }

template <int BM, int BN, class Dec, int SUB, int D>
__global__ __launch_bounds__(kQmmThreads) void qmm_deep_kernel(QmmParams p) {
  constexpr int MB = BM / 32;   // 16-row MFMA blocks per wave (wave rows: BM/2)
  constexpr int NB = BN / 32;   // 16-column MFMA blocks per wave (wave columns: BN/2)
  constexpr int NC = Dec::NC;   // codes a thread decodes per step
  constexpr int RPW = 64 / NC;  // spans per weight row (threads per row)
  constexpr int XU = BM / 32;   // 16-byte x units per loading thread per step
  static_assert(NC == BN / 4, "one span of BN/4 codes per producer thread");
  static_assert(RPW * BN == 256, "one span per producer thread");
  static_assert(D >= 2, "use qmm_kernel for one iteration of prefetch");
  extern __shared__ __attribute__((aligned(16))) uint32_t qsmem[];
  half_t* xs = reinterpret_cast<half_t*>(qsmem);                        // [2][SUB][BM*64]
  half_t* ws = xs + 2 * SUB * BM * kQmmBK;                              // [2][SUB][BN*64]
  uint32_t* lut = reinterpret_cast<uint32_t*>(ws + 2 * SUB * BN * kQmmBK);  // [Dec::kLutWords]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: the roles branch on scalars
  const int pw = wave & 3;
  const int wm = (wave >> 1) & 1, wn = wave & 1;
  const int tiles_n = (p.N + BN - 1) / BN;
  // workgroup -> tile and K share: the ksplit shares of a tile are
  // neighbours; share ks walks iterations [itb, itb + IT) (ksplit is at
  // most the iteration count, so every share has one)
  const int S = p.ksplit;
  const int t = (int)blockIdx.x / S;
  const int ks = (int)blockIdx.x - t * S;
  const int m0 = (t / tiles_n) * BM;
  const int n0 = (t % tiles_n) * BN;
  const int IT_all = p.K / (kQmmBK * SUB);
  const int itb = (int)((int64_t)ks * IT_all / S);
  const int IT = (int)((int64_t)(ks + 1) * IT_all / S) - itb;

  // s_waitcnt lgkmcnt(0), the other counters free: this wave's LDS stores
  // are done (barriers here wait for nothing else)
  constexpr int kLdsDone = 0xC07F;
  Dec::init_lut(lut, tid);

  if (wave >= 4) {
    // ---------------- loading and decoding waves ----------------
    const rsrc_t rx = make_rsrc(p.x, p.x_bytes);
    const int pt = tid & 255;
    const int r = pt % BN, h = pt / BN;
    const Dec dec(p, n0 + r, h);
    struct Set {
      u32x4 x[SUB][XU];
      typename Dec::Raw raw[SUB];
    };
    Set set[D];
    // x unit c*64 + lane of a step buffer (c = i*4 + pw) holds row
    // (c*64+lane)/8 of the tile, 16-byte column q XOR row%8
    auto issue = [&](int it, Set& st) {  // it: iteration of this share
#pragma unroll
      for (int u = 0; u < SUB; ++u) {
        const int k0 = ((itb + it) * SUB + u) * kQmmBK;
#pragma unroll
        for (int i = 0; i < XU; ++i) {
          const int un = (i * 4 + pw) * 64 + lane;
          const int row = un >> 3, q = (un & 7) ^ (row & 7);
          const uint32_t off = 2u * ((uint32_t)(m0 + row) * (uint32_t)p.K + (uint32_t)(k0 + q * 8));
          st.x[u][i] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)off, 0, 0);
        }
        dec.issue((itb + it) * SUB + u, st.raw[u]);
      }
    };
    auto put = [&](int it, int buf, const Set& st) {
#pragma unroll
      for (int u = 0; u < SUB; ++u) {
        half_t* xb = xs + (buf * SUB + u) * BM * kQmmBK;
#pragma unroll
        for (int i = 0; i < XU; ++i)
          *reinterpret_cast<u32x4*>(xb + ((i * 4 + pw) * 64 + lane) * 8) = st.x[u][i];
        // every loaded dword stays allocated until here: a register the
        // decode does not read would otherwise be reused while its load is
        // in flight, and the reuse would wait for that load
        keep_loaded(st.raw[u].d);
        uint32_t out[NC / 2];
        dec.decode((itb + it) * SUB + u, st.raw[u], lut, out);
        half_t* wb = ws + (buf * SUB + u) * BN * kQmmBK;
#pragma unroll
        for (int q = 0; q < NC / 8; ++q)
          *reinterpret_cast<u32x4*>(wb + qmm_swz(r, (NC / 8) * h + q) * 8) =
              u32x4{out[4 * q], out[4 * q + 1], out[4 * q + 2], out[4 * q + 3]};
      }
    };
    // requested in the order of the loop below (the waits the compiler
    // places there assume the same count of loads after each set)
#pragma unroll
    for (int j = 0; j < D; ++j) {
      issue(min(j, IT - 1), set[j]);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(kLdsDone);
    __builtin_amdgcn_s_barrier();  // table built
    asm volatile("" ::: "memory");
    put(0, 0, set[0]);
    __builtin_amdgcn_s_waitcnt(kLdsDone);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // whole rounds of D iterations (the multiplying waves skip those past
    // IT): no exit inside the unrolled body, so that the waits the compiler
    // places for each register set see one path through the loop
    for (int it0 = 0; it0 < IT; it0 += D) {
      // iteration it0 + k refills set k (its data went to LDS one iteration
      // ago) and stores set (k+1) % D, iteration it+1
#pragma unroll
      for (int k = 0; k < D; ++k) {
        const int it = it0 + k;
        // the last iterations reload the last one's data and store it again
        // (unused), so that every iteration has the same loads and waits
        issue(min(it + D, IT - 1), set[k]);
        put(min(it + 1, IT - 1), (it + 1) & 1, set[(k + 1) % D]);
        __builtin_amdgcn_s_waitcnt(kLdsDone);
        // every wave is past iteration it: buffers it&1 are free, the x and
        // weights of it+1 are in place
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
    }
    return;
  }

  // ---------------- multiplying waves ----------------
  float4_t acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};

  // MFMA operands of a group are all read before its first MFMA, and the
  // group ends with a VALU read of every accumulator (see qmm_kernel)
  constexpr int KS = kQmmBK / 32;
  constexpr int KG = (MB + NB) <= 6 ? KS : 1;
  auto multiply = [&](int buf) {
#pragma unroll
    for (int u = 0; u < SUB; ++u) {
      const half_t* xb = xs + (buf * SUB + u) * BM * kQmmBK;
      const half_t* wb = ws + (buf * SUB + u) * BN * kQmmBK;
#pragma unroll
      for (int g = 0; g < KS; g += KG) {
        half8_t af[KG][MB], bf[KG][NB];
#pragma unroll
        for (int kk = 0; kk < KG; ++kk) {
          const int q = (g + kk) * 4 + (lane >> 4);
#pragma unroll
          for (int j = 0; j < NB; ++j)
            bf[kk][j] = *reinterpret_cast<const half8_t*>(wb + qmm_swz(wn * (BN / 2) + 16 * j + (lane & 15), q) * 8);
#pragma unroll
          for (int i = 0; i < MB; ++i)
            af[kk][i] = *reinterpret_cast<const half8_t*>(xb + qmm_swz(wm * (BM / 2) + 16 * i + (lane & 15), q) * 8);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk < KG; ++kk)
#pragma unroll
          for (int i = 0; i < MB; ++i)
#pragma unroll
            for (int j = 0; j < NB; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[kk][i], bf[kk][j], acc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        uint32_t done = 0;
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j)
            done |= __builtin_amdgcn_readfirstlane(__builtin_bit_cast(uint32_t, acc[i][j][0]));
        asm volatile("" ::"s"(done) : "memory");
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  __builtin_amdgcn_s_waitcnt(kLdsDone);
  __builtin_amdgcn_s_barrier();  // table built
  __builtin_amdgcn_s_barrier();  // iteration 0 in place
  asm volatile("" ::: "memory");
  const int rounds = (IT + D - 1) / D * D;
  for (int it = 0; it < rounds; ++it) {
    if (it < IT) multiply(it & 1);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }

#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + wm * (BM / 2) + 16 * i + 4 * (lane >> 4) + v;
        const int n = n0 + wn * (BN / 2) + 16 * j + (lane & 15);
        if (m < p.M && n < p.N) {
          if (p.part)
            p.part[(size_t)ks * qmm_part_stride(p.M, p.N) + (size_t)m * p.N + n] = acc[i][j][v];
          else
            p.y[(size_t)m * p.N + n] = (half_t)acc[i][j][v];
        }
      }
}

struct QmmSumParams {
  const float* part;  // S slices of qmm_part_stride(M, N) floats, 16-byte aligned
  half_t* y;          // [M][N]
  size_t MN;          // M * N
  int S;
};

constexpr int kQmmMaxSplit = 8;  // K shares per tile, at most

// y[i] = fp16_rne(part[0][i] + part[1][i] + ... + part[S-1][i]), summed in
// that order, V = 4 elements per thread.  The loads of all slices go out
// before the first add, as straight-line code: slices past S reload slice
// 0 (in bounds, not added).
template <int V>
__global__ __launch_bounds__(256) void qmm_split_sum_kernel(QmmSumParams p) {
  static_assert(V == 4, "one 16-byte vector of each slice per thread");
  const size_t stride = (p.MN + 3) & ~(size_t)3;
  const size_t i0 = ((size_t)blockIdx.x * 256 + threadIdx.x) * V;
  if (i0 >= p.MN) return;
  float4_t v[kQmmMaxSplit];
#pragma unroll
  for (int k = 0; k < kQmmMaxSplit; ++k)
    v[k] = *reinterpret_cast<const float4_t*>(p.part + (size_t)(k < p.S ? k : 0) * stride + i0);
  float4_t a = v[0];
#pragma unroll
  for (int k = 1; k < kQmmMaxSplit; ++k) {
    const float4_t b = a + v[k];
    a = k < p.S ? b : a;
  }
#pragma unroll
  for (int e = 0; e < V; ++e)
    if (i0 + e < p.MN) p.y[i0 + e] = (half_t)a[e];
}

}  // namespace bq
