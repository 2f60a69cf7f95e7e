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
// * A workgroup is 4 waves.  A wave is split into slots of KL lanes (KL = 16,
//   or 8 for t5 with 128-weight groups); the KL lanes of a slot share one
//   output row and split its K range into chunks of CH codes (64, or 128),
//   so one 1024-code K tile is one chunk per lane.  Each slot owns up to
//   RCAP rows, which keeps x in registers across those rows.
// * x is staged tile by tile in LDS (double buffered), permuted into the
//   order in which the unpack below produces code pairs and pre-scaled per
//   code position so that no shift is needed to line codes up (see
//   "scaled codes").  Per-chunk sums of x feed the bias term.
// * Scaled codes: a code masked in place inside a 16-bit half is read as an
//   fp16 subnormal, i.e. q * 2^e * 2^-24 where e is its bit offset in the
//   half.  v_dot2_f32_f16 multiplies it by the staged x*2^-e and adds in
//   fp32, so every product is q*x*2^-24 exactly (up to the fp16 rounding of
//   x*2^-e for |x| < 2^(e-14)); the 2^24 goes into the scale.  2-bit words
//   need one shift per 16 codes, 1-bit words one per 32 codes.
// * t5 bytes go through a 256-entry LDS table that turns a byte into its
//   five base-3 digits laid out as 2-bit fields (digit i at bits 2i); two
//   bytes fill one dword, and each mask then yields a half2 of codes.
// * fp32 accumulation; per chunk: acc += b*X + (s*2^24)*P; a KL-lane
//   butterfly reduces each row at the end and one lane stores fp16 (RNE).
//
// Every K chunk is always processed by the same lane in the same order and
// the reduction tree does not depend on M, so row m of a wide call is
// bit-identical to a call with that row alone.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bq {

typedef _Float16 half_t;
typedef half_t half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
// dword-aligned (not 16-byte aligned) views for t5 rows
typedef uint32_t u32x4a __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x3a __attribute__((ext_vector_type(3), aligned(4)));

enum { FMT_U1 = 1, FMT_U2 = 2, FMT_T5 = 5 };
constexpr int kTile = 1024;       // codes per K tile
constexpr int kWaves = 4;         // waves per workgroup
constexpr int kThreads = 64 * kWaves;

struct QmvParams {
  const half_t* x;       // [M][K]
  const uint8_t* w;      // [N][row_bytes]
  const half_t* s;       // [N][G]
  const half_t* b;       // [N][G] (unused when the bias is implied)
  half_t* y;             // [M][N]
  int N, K, G;           // G = K / group_size
  int row_bytes;
  int rows_per_wg;       // rows of one workgroup (<= slots * RCAP)
  float ratio;           // implied bias = -scale * ratio
};

// --------------------------------------------------------------------------
// Format traits
//   CH  codes per chunk (one lane, one row, one K tile)
//   KL  lanes per slot  (KL * CH = kTile)
//   XD  LDS dwords per staged chunk (padded so that the 16 chunks of a tile
//       start on distinct banks)
//   place(pos) -> staged dword, half and exponent of chunk position pos
// --------------------------------------------------------------------------
template <int FMT, int GS> struct Fmt;

template <int GS> struct Fmt<FMT_U2, GS> {
  static constexpr int CH = 64, KL = 16, XD = 36, XUSED = 32;
  // word i holds codes 16i..16i+15; pair p = (code p, code p+8) of a word;
  // pairs 0..4 are masked in place (offset 2p), pairs 5..7 after >> 10.
  __device__ static inline void place(int pos, int& d, int& h, int& e) {
    int i = pos >> 4, j = pos & 15, pp = j & 7;
    h = j >> 3;
    d = 8 * i + pp;
    e = 2 * (pp < 5 ? pp : pp - 5);
  }
};

template <int GS> struct Fmt<FMT_U1, GS> {
  static constexpr int CH = 64, KL = 16, XD = 36, XUSED = 32;
  // word i holds codes 32i..32i+31; pair p = (code p, code p+16);
  // pairs 0..9 masked in place (offset p), pairs 10..15 after >> 10.
  __device__ static inline void place(int pos, int& d, int& h, int& e) {
    int i = pos >> 5, j = pos & 31, pp = j & 15;
    h = j >> 4;
    d = 16 * i + pp;
    e = pp < 10 ? pp : pp - 10;
  }
};

// t5: byte t of a chunk holds codes 5t..5t+4.  Bytes (2p, 2p+1) form pair p;
// digit i (i < 4) of pair p is staged at dword 4p+i, digit 4 at NP4 + p.
template <> struct Fmt<FMT_T5, 64> {
  static constexpr int CH = 64, KL = 16, XD = 36, XUSED = 34;
  static constexpr int NPAIR = 6;       // bytes 0..11; byte 12 is single
  static constexpr int NP4 = 28;        // first dword of the digit-4 block
  static constexpr int BYTES = 13;
  __device__ static inline void place(int pos, int& d, int& h, int& e) {
    int t = pos / 5, i = pos - 5 * (pos / 5);
    e = 2 * i;
    if (t < 12) {
      int p = t >> 1;
      h = t & 1;
      d = (i < 4) ? 4 * p + i : NP4 + p;
    } else {              // byte 12: codes 60..63 (+ one zero pad digit)
      h = 0;
      d = 24 + i;
    }
  }
};

template <> struct Fmt<FMT_T5, 128> {
  static constexpr int CH = 128, KL = 8, XD = 68, XUSED = 65;
  static constexpr int NPAIR = 13;      // bytes 0..25 (byte 25: 3 digits + 2 pads)
  static constexpr int NP4 = 52;
  static constexpr int BYTES = 26;
  __device__ static inline void place(int pos, int& d, int& h, int& e) {
    int t = pos / 5, i = pos - 5 * (pos / 5);
    int p = t >> 1;
    e = 2 * i;
    h = t & 1;
    d = (i < 4) ? 4 * p + i : NP4 + p;
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

template <int W>
__device__ __forceinline__ float lane_sum(float v) {
#pragma unroll
  for (int off = W / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
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

// Per-lane packed chunk of one row.
template <int FMT, int GS> struct Chunk;
template <int GS> struct Chunk<FMT_U2, GS> { u32x4 v; };
template <int GS> struct Chunk<FMT_U1, GS> { u32x2 v; };
template <> struct Chunk<FMT_T5, 64> { uint32_t d[4]; };
template <> struct Chunk<FMT_T5, 128> { uint32_t d[7]; };

template <int FMT, int GS>
__device__ __forceinline__ void load_chunk(Chunk<FMT, GS>& c, const uint8_t* w, int row, int chunk,
                                           int row_bytes) {
  const uint8_t* rp = w + (size_t)row * row_bytes;
  if constexpr (FMT == FMT_U2) {
    c.v = *reinterpret_cast<const u32x4*>(rp + chunk * 16);
  } else if constexpr (FMT == FMT_U1) {
    c.v = *reinterpret_cast<const u32x2*>(rp + chunk * 8);
  } else if constexpr (GS == 64) {
    // 13 bytes at rp + 13*chunk; rows are whole dwords, so the dword-aligned
    // 16-byte window that holds them never passes the end of the row.
    int off = 13 * chunk;
    const u32x4 v = *reinterpret_cast<const u32x4a*>(rp + (off & ~3));
    c.d[0] = v[0]; c.d[1] = v[1]; c.d[2] = v[2]; c.d[3] = v[3];
  } else {
    // 26 bytes at rp + 26*chunk, dword offset 0 or 2: seven dwords hold them.
    int off = 26 * chunk;
    const uint8_t* p = rp + (off & ~3);
    const u32x4 a = *reinterpret_cast<const u32x4a*>(p);
    const u32x3 b = *reinterpret_cast<const u32x3a*>(p + 16);
    c.d[0] = a[0]; c.d[1] = a[1]; c.d[2] = a[2]; c.d[3] = a[3];
    c.d[4] = b[0]; c.d[5] = b[1]; c.d[6] = b[2];
  }
}

// --------------------------------------------------------------------------
// Staging of one K tile of x into LDS, plus per-chunk sums of x.
// Thread t stages codes 4t..4t+3 of the tile for every row m.
// --------------------------------------------------------------------------
template <int FMT, int GS, int M>
__device__ __forceinline__ void stage_tile(const QmvParams& p, int tile, uint32_t* xs, float* xsum) {
  using F = Fmt<FMT, GS>;
  constexpr int TC = kTile / F::CH;
  const int tid = threadIdx.x;
  const int k0 = tile * kTile + 4 * tid;
  uint16_t* xs16 = reinterpret_cast<uint16_t*>(xs);
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float part = 0.f;
    if (k0 < p.K) {
      const half_t* xr = p.x + (size_t)m * p.K + k0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        half_t v = xr[u];
        float f = h2f(v);
        part += f;
        int pos = (4 * tid + u) % F::CH;
        int c = (4 * tid + u) / F::CH;
        int d, h, e;
        F::place(pos, d, h, e);
        half_t sv = (half_t)__builtin_ldexpf(f, -e);
        xs16[2 * ((m * TC + c) * F::XD + d) + h] = __builtin_bit_cast(uint16_t, sv);
      }
    }
    part = lane_sum<F::CH / 4>(part);
    if ((tid % (F::CH / 4)) == 0) xsum[m * TC + (4 * tid) / F::CH] = part;
  }
}

// --------------------------------------------------------------------------
// Per-chunk multiply: P[r][m] += codes(row r) . xstaged(m), for all rows of
// the slot that are active.
// --------------------------------------------------------------------------
template <int FMT, int GS, int M, int RCAP>
__device__ __forceinline__ void chunk_dot(const Chunk<FMT, GS> (&wc)[RCAP], const uint32_t* xc,
                                          int xstride_m, const uint16_t* lut, int nrows,
                                          uint32_t sh, float (&P)[RCAP][M]) {
  using F = Fmt<FMT, GS>;
  if constexpr (FMT == FMT_U2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x4 xa[M], xb[M];
#pragma unroll
      for (int m = 0; m < M; ++m) {
        xa[m] = *reinterpret_cast<const u32x4*>(xc + m * xstride_m + 8 * i);
        xb[m] = *reinterpret_cast<const u32x4*>(xc + m * xstride_m + 8 * i + 4);
      }
#pragma unroll
      for (int r = 0; r < RCAP; ++r) {
        if (r < nrows) {
          uint32_t wv = wc[r].v[i];
          uint32_t ws = wv >> 10;
          uint32_t q[8];
#pragma unroll
          for (int pp = 0; pp < 5; ++pp) q[pp] = wv & (0x00030003u << (2 * pp));
#pragma unroll
          for (int pp = 5; pp < 8; ++pp) q[pp] = ws & (0x00030003u << (2 * (pp - 5)));
#pragma unroll
          for (int m = 0; m < M; ++m) {
            float a = P[r][m];
            a = dot2(q[0], xa[m][0], a);
            a = dot2(q[1], xa[m][1], a);
            a = dot2(q[2], xa[m][2], a);
            a = dot2(q[3], xa[m][3], a);
            a = dot2(q[4], xb[m][0], a);
            a = dot2(q[5], xb[m][1], a);
            a = dot2(q[6], xb[m][2], a);
            a = dot2(q[7], xb[m][3], a);
            P[r][m] = a;
          }
        }
      }
    }
  } else if constexpr (FMT == FMT_U1) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {  // pairs 8*half .. 8*half+7
        u32x4 xa[M], xb[M];
#pragma unroll
        for (int m = 0; m < M; ++m) {
          xa[m] = *reinterpret_cast<const u32x4*>(xc + m * xstride_m + 16 * i + 8 * half);
          xb[m] = *reinterpret_cast<const u32x4*>(xc + m * xstride_m + 16 * i + 8 * half + 4);
        }
#pragma unroll
        for (int r = 0; r < RCAP; ++r) {
          if (r < nrows) {
            uint32_t wv = wc[r].v[i];
            uint32_t ws = wv >> 10;
            uint32_t q[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              int pp = 8 * half + u;
              q[u] = pp < 10 ? (wv & (0x00010001u << pp)) : (ws & (0x00010001u << (pp - 10)));
            }
#pragma unroll
            for (int m = 0; m < M; ++m) {
              float a = P[r][m];
              a = dot2(q[0], xa[m][0], a);
              a = dot2(q[1], xa[m][1], a);
              a = dot2(q[2], xa[m][2], a);
              a = dot2(q[3], xa[m][3], a);
              a = dot2(q[4], xb[m][0], a);
              a = dot2(q[5], xb[m][1], a);
              a = dot2(q[6], xb[m][2], a);
              a = dot2(q[7], xb[m][3], a);
              P[r][m] = a;
            }
          }
        }
      }
    }
  } else {
    // t5: realign each row's bytes (the chunk starts at byte offset `sh`
    // of its first dword), then look pairs of bytes up in the digit table.
    constexpr int NDW = (GS == 64) ? 4 : 7;
    constexpr int NP = F::NPAIR + ((GS == 64) ? 1 : 0);  // + single byte 12
    uint32_t rb[RCAP][NDW];
#pragma unroll
    for (int r = 0; r < RCAP; ++r) {
#pragma unroll
      for (int j = 0; j < NDW; ++j) {
        const uint32_t lo = wc[r].d[j];
        const uint32_t hi = (j + 1 < NDW) ? wc[r].d[j + 1] : 0u;
        rb[r][j] = __builtin_amdgcn_alignbyte(hi, lo, sh);
      }
    }
#pragma unroll
    for (int pr = 0; pr < NP; ++pr) {
      const bool paired = pr < F::NPAIR;
      u32x4 xq[M], x4[M];
#pragma unroll
      for (int m = 0; m < M; ++m) {
        xq[m] = *reinterpret_cast<const u32x4*>(xc + m * xstride_m + 4 * pr);
        if (paired) x4[m] = *reinterpret_cast<const u32x4*>(xc + m * xstride_m + F::NP4 + 4 * (pr / 4));
      }
#pragma unroll
      for (int r = 0; r < RCAP; ++r) {
        if (r < nrows) {
          const int t0 = 2 * pr, t1 = 2 * pr + 1;
          uint32_t b0 = (rb[r][t0 >> 2] >> (8 * (t0 & 3))) & 0xFFu;
          uint32_t v = lut[b0];
          if (paired) {
            uint32_t b1 = (rb[r][t1 >> 2] >> (8 * (t1 & 3))) & 0xFFu;
            v |= (uint32_t)lut[b1] << 16;
          }
          uint32_t q0 = v & 0x00030003u, q1 = v & 0x000C000Cu, q2 = v & 0x00300030u,
                   q3 = v & 0x00C000C0u, q4 = v & 0x03000300u;
#pragma unroll
          for (int m = 0; m < M; ++m) {
            float a = P[r][m];
            a = dot2(q0, xq[m][0], a);
            a = dot2(q1, xq[m][1], a);
            a = dot2(q2, xq[m][2], a);
            a = dot2(q3, xq[m][3], a);
            if (paired) a = dot2(q4, x4[m][pr & 3], a);
            P[r][m] = a;
          }
        }
      }
    }
  }
}

// --------------------------------------------------------------------------
// The kernel.  Workgroup g owns rows [g*rows_per_wg, ...); slot s of the
// workgroup owns rows base + s + j*SLOTS (j < RCAP).
// --------------------------------------------------------------------------
template <int FMT, int GS, int M, bool IMPLIED, int RCAP>
__global__ __launch_bounds__(kThreads) void qmv_kernel(QmvParams p) {
  using F = Fmt<FMT, GS>;
  constexpr int TC = kTile / F::CH;              // chunks per tile (= KL)
  constexpr int WSLOTS = 64 / F::KL;             // slots per wave
  constexpr int SLOTS = kWaves * WSLOTS;         // slots per workgroup
  constexpr int XT = M * TC * F::XD;             // dwords of one staged tile
  constexpr bool T5 = (FMT == FMT_T5);

  extern __shared__ uint32_t smem[];
  uint32_t* xs = smem;                           // [2][XT]
  float* xsum = reinterpret_cast<float*>(smem + 2 * XT);  // [2][M*TC]
  __shared__ uint16_t lut[256];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int slot = (tid >> 6) * WSLOTS + lane / F::KL;
  const int kl = lane % F::KL;
  const int base = blockIdx.x * p.rows_per_wg;
  const int end = min(base + p.rows_per_wg, p.N);
  int nrows = 0;
#pragma unroll
  for (int r = 0; r < RCAP; ++r)
    if (base + slot + r * SLOTS < end) nrows = r + 1;

  for (int i = tid; i < 2 * XT; i += kThreads) xs[i] = 0u;  // pads stay zero
  if constexpr (T5) lut[tid] = (uint16_t)(tid < 243 ? t5_fields((uint32_t)tid) : 0u);

  const int nchunks = p.K / F::CH;
  const int ntiles = (p.K + kTile - 1) / kTile;
  // byte offset of this lane's t5 chunk inside its first dword
  const uint32_t sh = (GS == 64) ? (uint32_t)(kl & 3) : (uint32_t)((2 * kl) & 3);

  float acc[RCAP][M];
#pragma unroll
  for (int r = 0; r < RCAP; ++r)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[r][m] = 0.f;

  Chunk<FMT, GS> wc[RCAP];
  half_t sc[RCAP], bc[RCAP];

  auto fetch = [&](int tile, Chunk<FMT, GS>(&dst)[RCAP], half_t(&sdst)[RCAP], half_t(&bdst)[RCAP]) {
    const int c = tile * TC + kl;
    if (c < nchunks) {
      const int g = (c * F::CH) / GS;
#pragma unroll
      for (int r = 0; r < RCAP; ++r) {
        if (r < nrows) {
          const int row = base + slot + r * SLOTS;
          load_chunk<FMT, GS>(dst[r], p.w, row, c, p.row_bytes);
          sdst[r] = p.s[(size_t)row * p.G + g];
          if constexpr (!IMPLIED) bdst[r] = p.b[(size_t)row * p.G + g];
        }
      }
    }
  };

  __syncthreads();
  stage_tile<FMT, GS, M>(p, 0, xs, xsum);
  fetch(0, wc, sc, bc);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int cur = t & 1;
    Chunk<FMT, GS> wn[RCAP];
    half_t sn[RCAP], bn[RCAP];
    if (t + 1 < ntiles) {
      stage_tile<FMT, GS, M>(p, t + 1, xs + (cur ^ 1) * XT, xsum + (cur ^ 1) * M * TC);
      fetch(t + 1, wn, sn, bn);
    }
    const int c = t * TC + kl;
    if (c < nchunks) {
      float P[RCAP][M];
#pragma unroll
      for (int r = 0; r < RCAP; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) P[r][m] = 0.f;
      const uint32_t* xc = xs + cur * XT + kl * F::XD;
      chunk_dot<FMT, GS, M, RCAP>(wc, xc, TC * F::XD, lut, nrows, sh, P);
      const float* xsm = xsum + cur * M * TC + kl;
#pragma unroll
      for (int r = 0; r < RCAP; ++r) {
        if (r < nrows) {
          const float s = h2f(sc[r]);
          const float s24 = s * 16777216.0f;
          float b;
          if constexpr (IMPLIED) b = -s * p.ratio;
          else b = h2f(bc[r]);
#pragma unroll
          for (int m = 0; m < M; ++m) {
            float a = __builtin_fmaf(b, xsm[m * TC], acc[r][m]);
            acc[r][m] = __builtin_fmaf(s24, P[r][m], a);
          }
        }
      }
    }
    __syncthreads();
    if (t + 1 < ntiles) {
#pragma unroll
      for (int r = 0; r < RCAP; ++r) {
        wc[r] = wn[r];
        sc[r] = sn[r];
        bc[r] = bn[r];
      }
    }
  }

#pragma unroll
  for (int r = 0; r < RCAP; ++r) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float v = lane_sum<F::KL>(acc[r][m]);
      const int row = base + slot + r * SLOTS;
      if (kl == 0 && r < nrows) p.y[(size_t)m * p.N + row] = (half_t)v;
    }
  }
}

}  // namespace bq
