// Repacking of 1/2-bit affine weights into t5 bytes ("oMLX Bonsai 自定义内核"
// article, section 二, the t5 format: the project ships a tool that repacks
// existing model weights into t5).  A weight s*q + b keeps its scale and bias
// and only changes container: its code q becomes a base-3 digit, so the
// repack is exact when every code is 0, 1 or 2.  A 2-bit code 3 has no digit;
// it is written as 2 (every byte stays a valid t5 byte) and the flag reports
// that the layer was not ternary.
//
// Layout written: t5 row n is (K/gs) groups of ceil(gs/5) bytes; code 5j+i
// of a group is digit i (least significant first) of the group's byte j,
// unused digits 0.  One thread per output dword: its four bytes take twenty
// codes, read from the row's uint32 words (LSB-first codes).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bq {

struct RepackParams {
  const uint32_t* w;  // [N][words_per_row] 1/2-bit codes
  uint32_t* out;      // [N][dwords_per_row] t5 bytes
  int64_t total;      // N * dwords_per_row
  int words_per_row, dwords_per_row;
  int* flag;          // 1 = every code was 0..2, 0 = a code 3 was met
};

__global__ void repack_flag_init_kernel(RepackParams p) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *p.flag = 1;
}

template <int BITS, int GS>
__global__ __launch_bounds__(256) void t5_repack_kernel(RepackParams p) {
  constexpr int GB = (GS + 4) / 5;  // bytes per group
  constexpr uint32_t kMask = (1u << BITS) - 1u;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  bool ternary = true;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < p.total; i += stride) {
    const int n = (int)(i / p.dwords_per_row);
    const int d = (int)(i - (int64_t)n * p.dwords_per_row);
    const uint32_t* row = p.w + (size_t)n * p.words_per_row;
    uint32_t v = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int b = 4 * d + e;  // byte within the row
      const int g = b / GB, j = b - g * GB;
      uint32_t byte = 0, pw = 1;
#pragma unroll
      for (int t = 0; t < 5; ++t) {
        const int c = 5 * j + t;  // code within the group
        if (c < GS) {
          const int k = g * GS + c;
          const uint32_t q = (row[(k * BITS) >> 5] >> ((k * BITS) & 31)) & kMask;
          ternary = ternary && q <= 2u;
          byte += (q > 2u ? 2u : q) * pw;
        }
        pw *= 3u;
      }
      v |= byte << (8 * e);
    }
    p.out[i] = v;
  }
  if (!ternary) *p.flag = 0;
}

}  // namespace bq
