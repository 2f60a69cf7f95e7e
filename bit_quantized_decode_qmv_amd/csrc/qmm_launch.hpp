// Host side of the prefill products: tile shape and pipeline depth per
// call.  Included by the per-format translation units.
#pragma once

#include <algorithm>
#include <cmath>
#include <type_traits>

#include "launch_common.hpp"

namespace bq {
namespace {

// the decoder of a format: t5 bytes (bits = BQ_BITS_T5) or 1/2-bit words
template <int BN, int BITS, int GS, bool IMPLIED>
using QmmDecoder = typename std::conditional<BITS == BQ_BITS_T5, T5Decoder<BN, GS, IMPLIED>,
                                             UqDecoder<BN, (BITS == 1 ? 1 : 2), GS, IMPLIED>>::type;

// x staged through LDS by direct loads, requested one iteration ahead
template <int BM, int BN, int BITS, int GS, bool IMPLIED, int SUB>
int launch_qmm_s(const QmmParams& p, void* stream) {
  typedef QmmDecoder<BN, BITS, GS, IMPLIED> Dec;
  const void* fn = reinterpret_cast<const void*>(&qmm_kernel<BM, BN, Dec, SUB>);
  const size_t lds = qmm_lds_bytes(BM, BN, Dec::kLutWords, SUB);
  static const hipError_t attr = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  (void)attr;
  dim3 grid(((p.N + BN - 1) / BN) * ((p.M + BM - 1) / BM));
  QmmParams q = p;
  return launch_kernel(fn, grid, dim3(kQmmThreads), lds, stream, &q);
}

// x and the raw weight bytes requested D iterations ahead into registers;
// p.ksplit workgroups per tile (p.part set when above 1)
template <int BM, int BN, int BITS, int GS, bool IMPLIED, int SUB, int D>
int launch_qmm_deep_s(const QmmParams& p, void* stream) {
  typedef QmmDecoder<BN, BITS, GS, IMPLIED> Dec;
  const void* fn = reinterpret_cast<const void*>(&qmm_deep_kernel<BM, BN, Dec, SUB, D>);
  const size_t lds = qmm_deep_lds_bytes(BM, BN, Dec::kLutWords, SUB);
  static const hipError_t attr = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  (void)attr;
  QmmParams q = p;
  // at most one share per K iteration, and only as many as the workspace holds
  const int iters = p.K / (kQmmBK * SUB);
  if (q.ksplit > iters) q.ksplit = iters;
  if (q.ksplit < 1 || !q.part || (size_t)q.ksplit * qmm_part_stride(q.M, q.N) * sizeof(float) > q.part_cap)
    q.ksplit = 1;
  if (q.ksplit == 1) q.part = nullptr;
  dim3 grid(((p.N + BN - 1) / BN) * ((p.M + BM - 1) / BM) * q.ksplit);
  int st = launch_kernel(fn, grid, dim3(kQmmThreads), lds, stream, &q);
  if (st != BQ_OK || q.ksplit == 1) return st;
  QmmSumParams sp{q.part, q.y, (size_t)q.M * q.N, q.ksplit};
  const size_t vecs = (sp.MN + 3) / 4;
  return launch_kernel(reinterpret_cast<const void*>(&qmm_split_sum_kernel<4>), dim3((unsigned)((vecs + 255) / 256)),
                       dim3(256), 0, stream, &sp);
}

// Small products (M <= 32, 32-row tiles) request x and the weight bytes
// kQmmDepth iterations ahead (measured on MI355X: 4 beats 6 and 8, whose
// register sets cost more than the extra depth brings); larger tiles
// kQmmDepthWide (2: measured no slower than 3 or 4 on any tile, and its
// register sets leave the 128 x 64 tile two workgroups per CU).
constexpr int kQmmDepth = 4;
constexpr int kQmmDepthWide = 2;

// the small-M product as qmm_small_m_choice picks it (split 1 without a
// workspace)
template <int BITS, int GS, bool IMPLIED>
int launch_qmm_small(const QmmParams& p, void* stream) {
  const QmmSmallChoice c = qmm_small_m_choice(p.M, p.N, p.K, p.part ? p.part_cap : 0);
  QmmParams q = p;
  q.ksplit = c.split;
  constexpr int D = kQmmDepth;
  if (c.bn == 64)
    return c.sub == 4 ? launch_qmm_deep_s<32, 64, BITS, GS, IMPLIED, 4, D>(q, stream)
                      : launch_qmm_deep_s<32, 64, BITS, GS, IMPLIED, 1, D>(q, stream);
  return c.sub == 2 ? launch_qmm_deep_s<32, 128, BITS, GS, IMPLIED, 2, D>(q, stream)
                    : launch_qmm_deep_s<32, 128, BITS, GS, IMPLIED, 1, D>(q, stream);
}

template <int BITS, int GS, bool IMPLIED>
int launch_qmm_m(const QmmParams& p, void* stream) {
  const int steps = p.K / kQmmBK;
  if (p.M <= 32) return launch_qmm_small<BITS, GS, IMPLIED>(p, stream);
  // Rules from a measured sweep of seven tiles and prefetch depths 1-4
  // (MI355X; q 6144 x 5120, gate 17408 x 5120, down 5120 x 17408; t5 and
  // 2-bit; M 64 .. 2048), in microseconds per call:
  // * when all 32 x 64 tiles (or else all 64 x 64 tiles) run at once, one
  //   per CU, that tile with 4 steps per iteration and x one iteration
  //   ahead (t5 q M = 64: 32 us, down M = 128: 117 us);
  // * else up to 64 rows: 64 x 64 tiles, two iterations ahead (gate M = 64:
  //   t5 69 -> 63, 2-bit 63 -> 62);
  // * t5: 128 x 64 tiles two iterations ahead (two workgroups per CU): M =
  //   256 q 61 -> 48, M = 512 gate 226 -> 171, M = 2048 down 735 -> 608;
  // * 1/2-bit, whose per-row decode costs more on 64-column tiles: above
  //   512 rows 256 x 128 tiles (M = 2048 q 242 -> 219, gate 601 -> 544,
  //   down 767 -> 709), above 256 rows of at most 8192 columns 256 x 64
  //   (q M = 512: 92 -> 80), else 128 x 64 (q M = 256: 78 -> 55, gate M =
  //   512: 234 -> 198); all two iterations ahead.
  const int t32 = ((p.M + 31) / 32) * ((p.N + 63) / 64);
  const int t64 = ((p.M + 63) / 64) * ((p.N + 63) / 64);
  if (steps % 4 == 0 && t32 <= 256) return launch_qmm_s<32, 64, BITS, GS, IMPLIED, 4>(p, stream);
  if (steps % 4 == 0 && t64 <= 256) return launch_qmm_s<64, 64, BITS, GS, IMPLIED, 4>(p, stream);
  constexpr int D = kQmmDepthWide;
  if (p.M <= 64) return launch_qmm_deep_s<64, 64, BITS, GS, IMPLIED, 1, D>(p, stream);
  if (BITS != BQ_BITS_T5) {
    if (p.M > 512) return launch_qmm_deep_s<256, 128, BITS, GS, IMPLIED, 1, D>(p, stream);
    if (p.M > 256 && p.N <= 8192) return launch_qmm_deep_s<256, 64, BITS, GS, IMPLIED, 1, D>(p, stream);
  }
  return launch_qmm_deep_s<128, 64, BITS, GS, IMPLIED, 1, D>(p, stream);
}

template <int BITS>
int launch_qmm_bits(const QmmParams& p, int group_size, bool implied, void* stream) {
  if (group_size == 64)
    return implied ? launch_qmm_m<BITS, 64, true>(p, stream) : launch_qmm_m<BITS, 64, false>(p, stream);
  return implied ? launch_qmm_m<BITS, 128, true>(p, stream) : launch_qmm_m<BITS, 128, false>(p, stream);
}

}  // namespace
}  // namespace bq
