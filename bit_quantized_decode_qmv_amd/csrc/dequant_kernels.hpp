// Dequantization to fp16: out[n][k] = fp16_rne(scale*q + bias).
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

__device__ __forceinline__ uint32_t pack2h(half_t lo, half_t hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

// One thread per uint32 word (32/BITS codes, all inside one group).
template <int BITS, bool IMPLIED>
__global__ __launch_bounds__(256) void dequant_words_kernel(DequantParams p) {
  constexpr int CPW = 32 / BITS;
  const int wpr = p.K / CPW;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)p.N * wpr) return;
  const int row = (int)(idx / wpr);
  const int j = (int)(idx % wpr);
  const int k0 = j * CPW;
  const int g = k0 / p.gs;
  const uint32_t word = reinterpret_cast<const uint32_t*>(p.w + (size_t)row * p.row_bytes)[j];
  const float s = (float)p.s[(size_t)row * p.G + g];
  const float b = IMPLIED ? -s * p.ratio : (float)p.b[(size_t)row * p.G + g];
  uint32_t packed[CPW / 2];
#pragma unroll
  for (int i = 0; i < CPW / 2; ++i) {
    const uint32_t q0 = (word >> (BITS * (2 * i))) & ((1u << BITS) - 1u);
    const uint32_t q1 = (word >> (BITS * (2 * i + 1))) & ((1u << BITS) - 1u);
    packed[i] = pack2h(affine_to_half(s, q0, b), affine_to_half(s, q1, b));
  }
  uint32_t* dst = reinterpret_cast<uint32_t*>(p.out + (size_t)row * p.K + k0);
#pragma unroll
  for (int i = 0; i < CPW / 2; i += 4)
    *reinterpret_cast<u32x4*>(dst + i) = u32x4{packed[i], packed[i + 1], packed[i + 2], packed[i + 3]};
}

// One thread per t5 byte: five codes (fewer in the last byte of a group).
template <bool IMPLIED>
__global__ __launch_bounds__(256) void dequant_t5_kernel(DequantParams p) {
  const int gb = (p.gs + 4) / 5;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t total = (size_t)p.N * p.G * gb;
  if (idx >= total) return;
  const int row = (int)(idx / ((size_t)p.G * gb));
  const int rem = (int)(idx % ((size_t)p.G * gb));
  const int g = rem / gb;
  const int j = rem % gb;
  uint32_t v = p.w[(size_t)row * p.row_bytes + rem];
  const float s = (float)p.s[(size_t)row * p.G + g];
  const float b = IMPLIED ? -s * p.ratio : (float)p.b[(size_t)row * p.G + g];
  const int kin = 5 * j;
  half_t* dst = p.out + (size_t)row * p.K + (size_t)g * p.gs + kin;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const uint32_t q = v % 3u;
    v /= 3u;
    if (kin + i < p.gs) dst[i] = affine_to_half(s, q, b);
  }
}

}  // namespace bq
