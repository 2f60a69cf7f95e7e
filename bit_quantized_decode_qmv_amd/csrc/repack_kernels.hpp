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
// unused digits 0.  One thread per group: it loads the group's code words
// (2 to 8 dwords), turns the codes 3 of a 2-bit word into 2 all at once
// (the fields with both bits set), forms the group's 13 or 26 bytes in
// registers (Horner's rule over each byte's digits), and the
// workgroup's 256 groups -- a contiguous, dword-aligned run of output bytes
// when K is a multiple of 256 -- go out through LDS as whole dwords.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bq {

struct RepackParams {
  const uint32_t* w;  // [N][words_per_row] 1/2-bit codes
  uint32_t* out;      // [N][dwords_per_row] t5 bytes
  int64_t groups;     // N * (K / gs)
  int words_per_row, groups_per_row;
  int* flag;          // 1 = every code was 0..2, 0 = a code 3 was met
};

__global__ void repack_flag_init_kernel(RepackParams p) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *p.flag = 1;
}

template <int BITS, int GS>
__global__ __launch_bounds__(256) void t5_repack_kernel(RepackParams p) {
  constexpr int GB = (GS + 4) / 5;        // bytes per group
  constexpr int NW = GS * BITS / 32;      // code words per group
  constexpr uint32_t kMask = (1u << BITS) - 1u;
  __shared__ __attribute__((aligned(16))) uint8_t stage[256 * GB];
  const int64_t q0 = (int64_t)blockIdx.x * 256;
  const int64_t q = q0 + threadIdx.x;
  const int nlive = (int)(p.groups - q0 < 256 ? p.groups - q0 : 256);
  bool ternary = true;
  if (q < p.groups) {
    const int n = (int)(q / p.groups_per_row);
    const int g = (int)(q - (int64_t)n * p.groups_per_row);
    const uint32_t* src = p.w + (size_t)n * p.words_per_row + (size_t)g * NW;
    uint32_t wd[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      wd[i] = src[i];
      if constexpr (BITS == 2) {
        // codes 3 (both bits of a field set) become 2, word-wide
        const uint32_t three = wd[i] & (wd[i] >> 1) & 0x55555555u;
        ternary = ternary && three == 0u;
        wd[i] -= three;
      }
    }
#pragma unroll
    for (int j = 0; j < GB; ++j) {
      // Horner from the last digit: byte = sum of q_t * 3^t
      uint32_t byte = 0;
#pragma unroll
      for (int t = 4; t >= 0; --t) {
        const int c = 5 * j + t;  // code within the group
        const uint32_t qc = c < GS ? (wd[(c * BITS) >> 5] >> ((c * BITS) & 31)) & kMask : 0u;
        byte = byte * 3u + qc;
      }
      stage[threadIdx.x * GB + j] = (uint8_t)byte;
    }
  }
  __syncthreads();
  // the live groups' bytes, nlive * GB of them (a multiple of 4: rows hold
  // a multiple of 4 groups of 13 bytes or 2 of 26), as dwords
  const uint32_t* st = reinterpret_cast<const uint32_t*>(stage);
  uint32_t* dst = p.out + q0 * GB / 4;
  const int ndw = nlive * GB / 4;
  for (int i = (int)threadIdx.x; i < ndw; i += 256) dst[i] = st[i];
  if (!ternary) *p.flag = 0;
}

}  // namespace bq
