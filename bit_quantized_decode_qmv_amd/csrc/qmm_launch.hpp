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

// The small-M product (32-row tiles) with x and raw weight bytes requested
// kQmmDepth iterations ahead (measured on MI355X: 4 beats 6 and 8, whose
// register sets cost more than the extra depth brings).
constexpr int kQmmDepth = 4;

template <int BN, int BITS, int GS, bool IMPLIED, int SUB>
int launch_qmm_deep_s(const QmmParams& p, void* stream) {
  typedef QmmDecoder<BN, BITS, GS, IMPLIED> Dec;
  const void* fn = reinterpret_cast<const void*>(&qmm_deep_kernel<32, BN, Dec, SUB, kQmmDepth>);
  const size_t lds = qmm_deep_lds_bytes(32, BN, Dec::kLutWords, SUB);
  static const hipError_t attr = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  (void)attr;
  dim3 grid(((p.N + BN - 1) / BN) * ((p.M + 31) / 32));
  QmmParams q = p;
  return launch_kernel(fn, grid, dim3(kQmmThreads), lds, stream, &q);
}

// sub: K steps per iteration (4, 2 or 1), reduced to what divides the step
// count (and to 2 for 128-column tiles: the LDS of their double buffers)
template <int BN, int BITS, int GS, bool IMPLIED>
int launch_qmm_deep_t(const QmmParams& p, int sub, void* stream) {
  const int steps = p.K / kQmmBK;
  if (BN == 64 && sub >= 4 && steps % 4 == 0) return launch_qmm_deep_s<BN, BITS, GS, IMPLIED, (BN == 64 ? 4 : 2)>(p, stream);
  if (sub >= 2 && steps % 2 == 0) return launch_qmm_deep_s<BN, BITS, GS, IMPLIED, 2>(p, stream);
  return launch_qmm_deep_s<BN, BITS, GS, IMPLIED, 1>(p, stream);
}

// K steps per pipeline iteration of a tile shape: the small tiles (whose
// 64-code step is much shorter than a memory round trip) take 4 (32 x 64,
// 64 x 64) or 2 (32 x 128), as far as the LDS of one workgroup per CU and
// the step count K/64 allow; the others 1.
constexpr int qmm_sub(int BM, int BN) { return (BM <= 64 && BN == 64) ? 4 : (BM == 32 && BN == 128) ? 2 : 1; }

// sub: the K steps per iteration wanted (4, 2 or 1); reduced to what the
// tile's LDS allows (qmm_sub) and what divides the step count
template <int BM, int BN, int BITS, int GS, bool IMPLIED>
int launch_qmm_t(const QmmParams& p, int sub, void* stream) {
  constexpr int SUB = qmm_sub(BM, BN);
  const int steps = p.K / kQmmBK;
  if (sub >= 4 && SUB >= 4 && steps % 4 == 0) return launch_qmm_s<BM, BN, BITS, GS, IMPLIED, (SUB >= 4 ? 4 : 1)>(p, stream);
  if (sub >= 2 && SUB >= 2 && steps % 2 == 0) return launch_qmm_s<BM, BN, BITS, GS, IMPLIED, (SUB >= 2 ? 2 : 1)>(p, stream);
  return launch_qmm_s<BM, BN, BITS, GS, IMPLIED, 1>(p, stream);
}

// Small products (M <= 32, only 32-row tiles) are bound by the time of one
// pipeline iteration, not by the MFMA or memory throughput.  Measured on
// MI355X at M = 32 with one iteration of prefetch, an iteration of SUB steps
// took about 0.57 us plus 0.43 us per step with 64-column tiles and 0.50 us
// per step with 128-column tiles; the deeper prefetch now used cuts both
// by about a third and keeps their order, which is all the choice below
// uses.  Estimated microseconds of (BN, SUB) over `tiles` workgroups (two
// per CU only for 32 x 64 tiles without SUB, whose LDS allows it).
double qmm_small_m_us(int tiles, int steps, int BN, int sub) {
  const int per_cu = (BN == 64 && sub == 1) ? 2 : 1;
  const double rounds = std::ceil((double)tiles / (256.0 * per_cu));
  const double iter = 0.57 + sub * (BN == 64 ? 0.43 : 0.50);
  return rounds * ((double)steps / sub) * iter;
}

// Estimated cycles of one call with BM x BN tiles: per K step the larger of
// the MFMA cycles and the LDS cycles (operand reads, tile writes), plus the
// weight-decoding ALU cycles (measured not to overlap the MFMAs; alu_per_col
// per weight row of the tile), times the rounds of workgroups over 256 CUs;
// against the L2 / last-level-cache traffic of re-reading x once per column
// of tiles and W (w_bytes_per_weight) once per row of tiles at 32 bytes per
// clock per CU.  Only the order of the estimates matters: it picks the tile
// shape.
double qmm_cost(int M, int N, int K, int BM, int BN, int lut_words, double alu_per_col,
                double w_bytes_per_weight) {
  const double mfma = (double)BM * BN / 32.0;
  const double lds = 64.0 * (BM / 32 + BN / 32) + (BM + BN);
  const double alu = alu_per_col * BN;
  const double step = std::max(mfma, lds) + alu;
  const double tiles = (double)((N + BN - 1) / BN) * ((M + BM - 1) / BM);
  const int per_cu = qmm_lds_bytes(BM, BN, lut_words) * 2 <= 160 * 1024 ? 2 : 1;
  const double rounds = std::ceil(tiles / (256.0 * per_cu));
  const double compute = rounds * per_cu * (K / kQmmBK) * step;
  const double traffic = ((double)M * K * 2 * ((N + BN - 1) / BN) +
                          (double)N * K * w_bytes_per_weight * ((M + BM - 1) / BM)) /
                         (256.0 * 32.0);
  return std::max(compute, traffic);
}

template <int BITS, int GS, bool IMPLIED>
int launch_qmm_m(const QmmParams& p, void* stream) {
  typedef int (*Fn)(const QmmParams&, int, void*);
  struct Cand {
    int bm, bn;
    Fn fn;
  };
  // the shapes the estimate picks over M 1..4096, N 256..65536, K 256..17408
  // (128 x 256 tiles, which it picks for a few, do not fit the registers of
  // the two wave kinds)
  static const Cand cands[] = {
      {32, 64, &launch_qmm_t<32, 64, BITS, GS, IMPLIED>},   {32, 128, &launch_qmm_t<32, 128, BITS, GS, IMPLIED>},
      {64, 64, &launch_qmm_t<64, 64, BITS, GS, IMPLIED>},   {64, 256, &launch_qmm_t<64, 256, BITS, GS, IMPLIED>},
      {128, 64, &launch_qmm_t<128, 64, BITS, GS, IMPLIED>}, {256, 64, &launch_qmm_t<256, 64, BITS, GS, IMPLIED>},
      {256, 128, &launch_qmm_t<256, 128, BITS, GS, IMPLIED>},
  };
  const int lut_words = QmmDecoder<64, BITS, GS, IMPLIED>::kLutWords;
  const double alu = BITS == BQ_BITS_T5 ? 2.5 : 1.5;
  const double wbytes = BITS == BQ_BITS_T5 ? 0.2 : BITS / 8.0;
  const int steps = p.K / kQmmBK;
  if (p.M <= 32) {
    // 32 x 64 (SUB 1 or 4) or 32 x 128 (SUB 1 or 2), whichever the measured
    // iteration times say is shortest
    const int t64 = (p.N + 63) / 64, t128 = (p.N + 127) / 128;
    struct Opt {
      int bn, sub;
      double us;
    } opts[] = {{64, 1, qmm_small_m_us(t64, steps, 64, 1)},
                {64, 4, steps % 4 == 0 ? qmm_small_m_us(t64, steps, 64, 4) : 1e30},
                {128, 1, qmm_small_m_us(t128, steps, 128, 1)},
                {128, 2, steps % 2 == 0 ? qmm_small_m_us(t128, steps, 128, 2) : 1e30}};
    const Opt* o = &opts[0];
    for (const Opt& c : opts)
      if (c.us < o->us) o = &c;
    return o->bn == 64 ? launch_qmm_deep_t<64, BITS, GS, IMPLIED>(p, o->sub, stream)
                       : launch_qmm_deep_t<128, BITS, GS, IMPLIED>(p, o->sub, stream);
  }
  // Rules from a measured sweep of every tile (MI355X, gate and down shapes,
  // M 17 .. 2048), where the estimate below falls short:
  // * when all 32 x 64 tiles run at once (one per CU), that tile with 4
  //   steps per iteration (down: M = 48 214 -> 143 us, M = 96 213 -> 143);
  // * else when all 64 x 64 tiles do, that tile with 4 steps per iteration
  //   (down: M = 128 215 -> 156 us);
  // * with 256 to 512 tiles of 128 x 64 (two per CU, all resident) and more
  //   than 64 rows, that tile (down, M = 512: 295 -> 262 us); with fewer
  //   tiles it is slower than the estimate's choice.
  const int t32 = ((p.M + 31) / 32) * ((p.N + 63) / 64);
  const int t64 = ((p.M + 63) / 64) * ((p.N + 63) / 64);
  const int t128 = ((p.M + 127) / 128) * ((p.N + 63) / 64);
  if (steps % 4 == 0 && t32 <= 256) return launch_qmm_t<32, 64, BITS, GS, IMPLIED>(p, 4, stream);
  if (steps % 4 == 0 && t64 <= 256) return launch_qmm_t<64, 64, BITS, GS, IMPLIED>(p, 4, stream);
  if (p.M > 64 && t128 > 256 && t128 <= 512) return launch_qmm_t<128, 64, BITS, GS, IMPLIED>(p, 1, stream);
  const Cand* best = nullptr;
  double best_cost = 0.0;
  for (const Cand& c : cands) {
    if (c.bm > 32 && c.bm / 2 >= p.M) continue;  // a tile at least half full of rows
    const double cost = qmm_cost(p.M, p.N, p.K, c.bm, c.bn, lut_words, alu, wbytes);
    if (!best || cost < best_cost) {
      best = &c;
      best_cost = cost;
    }
  }
  // the 64 x 64 tile iterates over SUB = 4 steps when all its workgroups run
  // at once (one per CU: its LDS then holds no second workgroup)
  const int tiles = ((p.N + best->bn - 1) / best->bn) * ((p.M + best->bm - 1) / best->bm);
  const int sub = (best->bm == 64 && best->bn == 64 && tiles <= 256) ? 4 : 1;
  return best->fn(p, sub, stream);
}

template <int BITS>
int launch_qmm_bits(const QmmParams& p, int group_size, bool implied, void* stream) {
  if (group_size == 64)
    return implied ? launch_qmm_m<BITS, 64, true>(p, stream) : launch_qmm_m<BITS, 64, false>(p, stream);
  return implied ? launch_qmm_m<BITS, 128, true>(p, stream) : launch_qmm_m<BITS, 128, false>(p, stream);
}

}  // namespace
}  // namespace bq
