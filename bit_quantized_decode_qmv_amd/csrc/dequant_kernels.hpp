// Dequantization to fp16: out[n][k] = fp16_rne(scale*q + bias).
//
// Bound: HBM writes (2 bytes per weight against 1/8 .. 1/4 byte read).
// Each thread rounds its group's 2, 3 or 4 possible weights once and then
// picks one per code, so the arithmetic per code is a bit-field extract and
// half a v_perm_b32, and the stores are 16 bytes wide when out allows.
//
// Method: "oMLX Bonsai 自定义内核" article, section 二 path 1 -- for 1-bit
// prefill the weights are dequantized to float16 before a matmul; the same
// expansion is given here for 2-bit words and t5 bytes (path 3).
//
// Rounding: scale*q is exact in fp32 (fp16 scale times a code below 4); the
// sum with the bias is formed in fp32 and rounded to odd (TwoSum gives the
// rounding error), and the fp32 -> fp16 conversion then rounds to nearest
// even.  Rounding to odd with 13 or more spare bits makes the two roundings
// equal to one rounding of the exact value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmv_kernels.hpp"

namespace bq {

struct DequantParams {
  const uint8_t* w;
  const half_t* s;
  const half_t* b;     // null: implied -scale*ratio
  half_t* out;         // [N][K]
  int N, K, G, gs, row_bytes;
  float ratio;
};

__device__ __forceinline__ half_t affine_to_half(float s, uint32_t q, float b) {
  const float a = s * (float)q;
  const float r = a + b;
  const float bb = r - a;
  const float e = (a - (r - bb)) + (b - bb);
  float ro = r;
  if (e != 0.f) {
    uint32_t bits = __builtin_bit_cast(uint32_t, r);
    if ((bits & 1u) == 0u) {
      const bool away = (e > 0.f) == (r > 0.f);
      bits = away ? bits + 1u : bits - 1u;
      ro = __builtin_bit_cast(float, bits);
    }
  }
  return (half_t)ro;
}

// The weights of a group for every code value: table[q] = fp16(s*q + b),
// two per dword (codes 0/1 in the low dword, 2/3 in the high one).
template <int NQ>
__device__ __forceinline__ void weight_table(float s, float b, uint32_t& lo, uint32_t& hi) {
  const uint32_t w0 = __builtin_bit_cast(uint16_t, affine_to_half(s, 0u, b));
  const uint32_t w1 = __builtin_bit_cast(uint16_t, affine_to_half(s, 1u, b));
  lo = w0 | (w1 << 16);
  hi = 0u;
  if constexpr (NQ > 2) {
    const uint32_t w2 = __builtin_bit_cast(uint16_t, affine_to_half(s, 2u, b));
    const uint32_t w3 = NQ > 3 ? (uint32_t)__builtin_bit_cast(uint16_t, affine_to_half(s, 3u, b)) : 0u;
    hi = w2 | (w3 << 16);
  }
}

// The fp16 weights of codes (qa, qb) as one dword: a v_perm_b32 selector
// picking bytes 2q, 2q+1 of the {hi, lo} table for each code.
__device__ __forceinline__ uint32_t pair_weights(uint32_t lo, uint32_t hi, uint32_t qa, uint32_t qb) {
  const uint32_t sel = __umul24(qa | (qb << 16), 0x0202u) + 0x01000100u;
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Stores ND dwords (2*ND fp16) at dst with the widest stores that the
// alignment A of every dst (16, 4 or 2 bytes) allows.
template <int A, int ND>
__device__ __forceinline__ void store_pairs(half_t* dst, const uint32_t (&v)[ND]) {
  if constexpr (A >= 16) {
    static_assert(ND % 4 == 0, "whole 16-byte vectors");
#pragma unroll
    for (int i = 0; i < ND; i += 4)
      *reinterpret_cast<u32x4*>(dst + 2 * i) = u32x4{v[i], v[i + 1], v[i + 2], v[i + 3]};
  } else if constexpr (A >= 4) {
#pragma unroll
    for (int i = 0; i < ND; ++i) *reinterpret_cast<uint32_t*>(dst + 2 * i) = v[i];
  } else {
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      dst[2 * i] = __builtin_bit_cast(half_t, (uint16_t)(v[i] & 0xFFFFu));
      dst[2 * i + 1] = __builtin_bit_cast(half_t, (uint16_t)(v[i] >> 16));
    }
  }
}

// The 256 threads' outputs form one contiguous block (items are in the
// order of the output).  With 16-byte aligned output each thread puts its
// ND dwords in LDS and the block goes out as consecutive 16-byte pieces,
// lane after lane, so every store instruction writes 1 KB of contiguous
// output instead of 64 pieces a thread's width apart.  `live` threads: the
// first `nlive` of the block.
template <int ND>
__device__ __forceinline__ void store_block(half_t* base, const uint32_t (&v)[ND], int nlive) {
  static_assert(ND % 4 == 0, "whole 16-byte pieces");
  constexpr int PT = ND / 4;  // pieces per thread
  __shared__ u32x4 stage[256 * PT];
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < PT; ++i) stage[tid * PT + i] = u32x4{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
  __syncthreads();
  const int npieces = nlive * PT;
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int piece = i * 256 + tid;
    if (piece < npieces) reinterpret_cast<u32x4*>(base)[piece] = stage[piece];
  }
}

// One thread per uint32 word (32/BITS codes, all inside one group).  The
// group's 2^BITS weights are rounded once each; every code then selects
// its weight (one v_perm_b32 per pair of codes).  A: alignment of out.
template <int BITS, bool IMPLIED, int A>
__global__ __launch_bounds__(256) void dequant_words_kernel(DequantParams p) {
  constexpr int CPW = 32 / BITS;
  const int wpr = p.K / CPW;
  const size_t total = (size_t)p.N * wpr;
  const size_t item0 = (size_t)blockIdx.x * blockDim.x;
  const size_t idx = item0 + threadIdx.x;
  const bool live = idx < total;
  if (!live && A < 16) return;  // (the 16-byte path needs every thread at its barrier)
  const int row = live ? (int)(idx / wpr) : 0;
  const int j = (int)(idx % wpr);
  const int k0 = j * CPW;
  const int g = k0 / p.gs;
  const uint32_t word = reinterpret_cast<const uint32_t*>(p.w + (size_t)row * p.row_bytes)[j];
  const float s = (float)p.s[(size_t)row * p.G + g];
  const float b = IMPLIED ? -s * p.ratio : (float)p.b[(size_t)row * p.G + g];
  uint32_t lo, hi;
  weight_table<(1 << BITS)>(s, b, lo, hi);
  constexpr uint32_t mask = (1u << BITS) - 1u;
  uint32_t packed[CPW / 2];
#pragma unroll
  for (int i = 0; i < CPW / 2; ++i)
    packed[i] = pair_weights(lo, hi, (word >> (BITS * (2 * i))) & mask, (word >> (BITS * (2 * i + 1))) & mask);
  if constexpr (A >= 16) {
    store_block<CPW / 2>(p.out + item0 * CPW, packed, (int)min(total - item0, (size_t)256));
  } else {
    store_pairs<A>(p.out + (size_t)row * p.K + k0, packed);
  }
}

// One thread per t5 group: its 13 (gs 64) or 26 (gs 128) bytes come in
// dword-aligned 16-byte windows and are realigned; five base-3 digits per
// byte, least significant first; the pad digits of the last byte are not
// written.  A: alignment of out.
template <int GS, bool IMPLIED, int A>
__global__ __launch_bounds__(256) void dequant_t5_kernel(DequantParams p) {
  constexpr int GB = (GS + 4) / 5;        // bytes per group
  constexpr int NW = GS == 64 ? 4 : 8;    // dwords loaded
  const size_t total = (size_t)p.N * p.G;
  const size_t item0 = (size_t)blockIdx.x * blockDim.x;
  const size_t idx = item0 + threadIdx.x;
  const bool live = idx < total;
  if (!live && A < 16) return;  // (the 16-byte path needs every thread at its barrier)
  const int row = live ? (int)(idx / p.G) : 0;
  const int g = live ? (int)(idx % p.G) : 0;
  const uint32_t a = (uint32_t)row * (uint32_t)p.row_bytes + (uint32_t)(g * GB);
  // whole dwords: the dword holding W's last byte is read in full, later
  // dwords read as zeros
  const rsrc_t rw = make_rsrc(p.w, (int)(((uint32_t)p.N * (uint32_t)p.row_bytes + 3u) & ~3u));
  uint32_t raw[NW + 1];
  {
    const u32x4 v0 = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(a & ~3u), 0, 0);
#pragma unroll
    for (int k = 0; k < 4; ++k) raw[k] = v0[k];
    if constexpr (NW == 8) {
      const u32x4 v1 = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)((a & ~3u) + 16u), 0, 0);
#pragma unroll
      for (int k = 0; k < 4; ++k) raw[4 + k] = v1[k];
    }
    raw[NW] = 0u;
  }
  uint32_t bytes[NW];
#pragma unroll
  for (int k = 0; k < NW; ++k) bytes[k] = __builtin_amdgcn_alignbyte(raw[k + 1], raw[k], a & 3u);
  const float s = (float)p.s[(size_t)row * p.G + g];
  const float b = IMPLIED ? -s * p.ratio : (float)p.b[(size_t)row * p.G + g];
  uint32_t lo, hi;
  if constexpr (IMPLIED) {
    // -s, 0, +s: exact
    const uint32_t sb = __builtin_bit_cast(uint16_t, (half_t)s);
    lo = (sb ^ 0x8000u);
    hi = sb;
  } else {
    weight_table<3>(s, b, lo, hi);
  }
  uint32_t q[GB * 5];
#pragma unroll
  for (int j = 0; j < GB; ++j) {
    uint32_t v = (bytes[j >> 2] >> (8 * (j & 3))) & 0xFFu;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      q[5 * j + i] = v % 3u;
      v /= 3u;
    }
  }
  uint32_t packed[GS / 2];
#pragma unroll
  for (int t = 0; t < GS / 2; ++t) packed[t] = pair_weights(lo, hi, q[2 * t], q[2 * t + 1]);
  if constexpr (A >= 16) {
    store_block<GS / 2>(p.out + item0 * GS, packed, (int)min(total - item0, (size_t)256));
  } else {
    store_pairs<A>(p.out + (size_t)row * p.K + (size_t)g * GS, packed);
  }
}

}  // namespace bq
