// t5 prefill product on the matrix cores: y[M][N] = x[M][K] . W^T with W
// unpacked from t5 bytes tile by tile.
//
// Method: "oMLX Bonsai 自定义内核" article, section 二 path 3 -- for prefill
// with more than 16 rows the t5 weights go through a fused "unpack + matrix
// multiply" kernel that reads each t5 byte once.
//
// gfx950 design: a 256-thread workgroup computes a 128x128 tile of y; the
// K loop steps 128 codes at a time.  Per step the x tile (128x128 fp16) is
// copied to LDS and the 128 rows x 26 bytes of t5 weights are read once
// from HBM, decoded through a base-3 digit table and written to LDS as fp16
// weights w = s*(q-1) (exact in fp16 when the bias is -scale) or the
// correctly rounded fp16 of s*q+b.  Each wave then runs 4x4
// v_mfma_f32_16x16x32_f16 tiles (64x64 of y) over the step with fp32
// accumulators.
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
  int M, N, K, G, gs, row_bytes;
};

constexpr int kQmmBM = 128, kQmmBN = 128, kQmmBK = 128;
constexpr int kQmmLd = kQmmBK + 8;  // LDS row stride in halves (272 B)

template <bool IMPLIED>
__global__ __launch_bounds__(256) void t5_qmm_kernel(QmmParams p) {
  __shared__ __attribute__((aligned(16))) half_t xs[kQmmBM * kQmmLd];
  __shared__ __attribute__((aligned(16))) half_t ws[kQmmBN * kQmmLd];
  __shared__ uint32_t raw[kQmmBN * 8];   // 7 dwords of t5 bytes per row (+1 pad)
  __shared__ uint16_t lut[256];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * kQmmBM;
  const int n0 = blockIdx.x * kQmmBN;

  lut[tid] = (uint16_t)(tid < 243 ? t5_fields((uint32_t)tid) : 0u);

  float4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};

  const int nsteps = p.K / kQmmBK;
  const int gb = (p.gs + 4) / 5;             // 13 or 26 bytes per group
  for (int st = 0; st < nsteps; ++st) {
    const int k0 = st * kQmmBK;
    __syncthreads();
    // x tile: 128 rows x 256 B; thread -> (row, 16-byte piece), 8 passes
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int idx = it * 256 + tid;
      const int r = idx >> 4, c = (idx & 15) * 8;
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (m0 + r < p.M) v = *reinterpret_cast<const u32x4*>(p.x + (size_t)(m0 + r) * p.K + k0 + c);
      *reinterpret_cast<u32x4*>(&xs[r * kQmmLd + c]) = v;
    }
    // raw t5 bytes of the step: 26 bytes per row from byte 26*st, read as the
    // 7 dwords that cover them (rows are whole dwords, offset 0 or 2)
    for (int idx = tid; idx < kQmmBN * 7; idx += 256) {
      const int r = idx / 7, d = idx % 7;
      uint32_t v = 0u;
      if (n0 + r < p.N) {
        const uint8_t* rp = p.w + (size_t)(n0 + r) * p.row_bytes + ((26 * st) & ~3);
        v = reinterpret_cast<const uint32_t*>(rp)[d];
      }
      raw[r * 8 + d] = v;
    }
    __syncthreads();
    // decode: thread -> (row, 8-code segment), 8 segments per thread
    const int sh = (26 * st) & 3;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int idx = it * 256 + tid;
      const int r = idx >> 4, seg = idx & 15;
      const int kk0 = seg * 8;
      uint32_t out[4] = {0u, 0u, 0u, 0u};
      if (n0 + r < p.N) {
        const uint8_t* rb = reinterpret_cast<const uint8_t*>(raw + r * 8) + sh;
        const int grp0 = (k0 + kk0) / p.gs;  // a segment never spans two groups
        const float s = (float)p.s[(size_t)(n0 + r) * p.G + grp0];
        const float b = IMPLIED ? -s : (float)p.b[(size_t)(n0 + r) * p.G + grp0];
        const int gbase = (p.gs == 64) ? (kk0 >= 64 ? 13 : 0) : 0;
        const int kg0 = (p.gs == 64) ? (kk0 & 63) : kk0;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int kg = kg0 + u;
          const uint32_t fields = lut[rb[gbase + kg / 5]];
          const uint32_t q = (fields >> (2 * (kg % 5))) & 3u;
          half_t wv;
          if (IMPLIED) wv = (half_t)(s * (float)((int)q - 1));
          else wv = affine_to_half(s, q, b);
          const uint32_t hb = __builtin_bit_cast(uint16_t, wv);
          out[u >> 1] |= hb << (16 * (u & 1));
        }
      }
      *reinterpret_cast<u32x4*>(&ws[r * kQmmLd + kk0]) = u32x4{out[0], out[1], out[2], out[3]};
    }
    (void)gb;
    __syncthreads();
    // MFMA over the step: 4 sub-steps of 32 codes
#pragma unroll
    for (int ks = 0; ks < kQmmBK / 32; ++ks) {
      half8_t af[4], bf[4];
      const int kc = ks * 32 + 8 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const half8_t*>(&xs[(wm * 64 + 16 * i + (lane & 15)) * kQmmLd + kc]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[j] = *reinterpret_cast<const half8_t*>(&ws[(wn * 64 + 16 * j + (lane & 15)) * kQmmLd + kc]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  }

  // D layout of 16x16x32: lane holds rows 4*(lane/16)+v, column lane%16
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + wm * 64 + 16 * i + 4 * (lane >> 4) + v;
        const int n = n0 + wn * 64 + 16 * j + (lane & 15);
        if (m < p.M && n < p.N) p.y[(size_t)m * p.N + n] = (half_t)acc[i][j][v];
      }
}

}  // namespace bq
