// Host side of the decode kernels: workgroup geometry and the choice of
// kernel instance per call.  Included by the per-format translation units.
#pragma once

#include <algorithm>

#include "launch_common.hpp"

namespace bq {
namespace {

constexpr int kTargetWorkgroups = 256;
constexpr int kMaxRowsPerWg = 256;
constexpr size_t kLdsBudget = 150 * 1024;


size_t qmv_lds_bytes(int M, int R, int rows_per_wg, int ntiles, int seg_tiles, int G) {
  const size_t U = (size_t)((rows_per_wg + R - 1) / R) * ntiles;
  const size_t cs = (size_t)M * kXD + ((M % 2 == 0) ? 4 : 0);
  return 4 * ((size_t)seg_tiles * kKL * cs + 2 * (size_t)M * seg_tiles * kKL +
              8 * (size_t)sb_entry_dwords(M) * sb_vectors(rows_per_wg, G) + U * R * M);
}

// Workgroup geometry for M activation rows and R rows per unit.  Rows per
// workgroup: a multiple of R, enough for one workgroup per CU.  Segment: as
// many K tiles of x as LDS and the staging tasks (M * tiles * 16 <=
// kStageRounds * kThreads) allow, split evenly.  Returns false if even R rows
// per workgroup do not fit.
bool qmv_geometry(QmvParams& p, int M, int R, int W = kWaves) {
  const int threads = 64 * W;
  p.ntiles = (p.K + kTile - 1) / kTile;
  const int max_st = std::min(p.ntiles, kStageRounds * threads / (kKL * M));
  int rows = R * ((p.N + R * kTargetWorkgroups - 1) / (R * kTargetWorkgroups));
  if (rows > kMaxRowsPerWg) rows = kMaxRowsPerWg;
  for (; rows >= R; rows -= R) {
    if (sb_vectors(rows, p.G) > kSbRounds * threads) continue;
    int st = max_st;
    while (st > 0 && qmv_lds_bytes(M, R, rows, p.ntiles, st, p.G) > kLdsBudget) --st;
    if (st == 0) continue;
    p.nseg = (p.ntiles + st - 1) / st;
    p.seg_tiles = (p.ntiles + p.nseg - 1) / p.nseg;
    p.rows_per_wg = rows;
    p.sb_dwords = 8 * sb_entry_dwords(M) * sb_vectors(rows, p.G);
    return true;
  }
  return false;
}

// Units each slot takes in one segment, at most.
int units_per_slot(const QmvParams& p, int R, int W = kWaves) {
  const int U = ((p.rows_per_wg + R - 1) / R) * p.seg_tiles;
  const int slots = 64 * W / kKL;
  return (U + slots - 1) / slots;
}

template <int FMT, int GS, int M, bool IMPLIED, int P, int R, int W = kWaves>
int launch_qmv_p(const QmvParams& p, void* stream) {
  const void* fn = reinterpret_cast<const void*>(&qmv_kernel<FMT, GS, M, IMPLIED, P, R, W>);
  static const hipError_t attr =
      hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBudget);
  (void)attr;
  const size_t shmem = qmv_lds_bytes(M, R, p.rows_per_wg, p.ntiles, p.seg_tiles, p.G);
  dim3 grid((p.N + p.rows_per_wg - 1) / p.rows_per_wg);
  QmvParams q = p;
  return launch_kernel(fn, grid, dim3(64 * W), shmem, stream, &q);
}

// Rows per unit R and units in flight per slot P never change a row's
// arithmetic.  R = 4 quarters the per-code share of the per-unit work
// (cross-lane sums, scale reads, cursor arithmetic); it is used wherever the
// registers allow it and a 4-row workgroup's scale rows fit one staging
// pass.  Small products (k and v of the decoder, N = 1024) leave most slots
// without a 4-row unit, so one slot's unit is the whole critical path; when
// 1-row units give every slot at most one unit they are used instead (about
// 4x as many slots share the arithmetic).  A shallow ring is faster: with
// every slot of the GPU asking for many units at once, the x and scale
// loads queue behind the weights and the staging barrier comes later, while
// the loop cannot get shorter than its arithmetic.
template <int FMT, int GS, int M, bool IMPLIED>
int launch_qmv_t(QmvParams p, void* stream) {
  {
    QmvParams p1 = p;
    if (qmv_geometry(p1, M, 1) && units_per_slot(p1, 1) <= 1)
      return launch_qmv_p<FMT, GS, M, IMPLIED, 1, 1>(p1, stream);
  }
  if (qmv_geometry(p, M, 4)) {
    if (units_per_slot(p, 4) <= 1) return launch_qmv_p<FMT, GS, M, IMPLIED, 1, 4>(p, stream);
    // several units per slot: three waves per SIMD (measured 3-9% faster at
    // every M than two), on 4-row units for t5 at M >= 3 (1-5% faster than
    // 2-row units on gate, up and down; 2-bit is 1-5% slower on them) and
    // on 2-row units otherwise
    if constexpr (FMT == FMT_T5 && M >= 3) {
      QmvParams p4 = p;
      if (qmv_geometry(p4, M, 4, kWaves3)) return launch_qmv_p<FMT, GS, M, IMPLIED, 2, 4, kWaves3>(p4, stream);
    }
    QmvParams p2 = p;
    if (qmv_geometry(p2, M, 2, kWaves3)) return launch_qmv_p<FMT, GS, M, IMPLIED, 2, 2, kWaves3>(p2, stream);
    return launch_qmv_p<FMT, GS, M, IMPLIED, 2, 4>(p, stream);
  }
  if (!qmv_geometry(p, M, 2)) return BQ_ERR_SHAPE;
  return launch_qmv_p<FMT, GS, M, IMPLIED, 2, 2>(p, stream);
}

template <int FMT, int GS, bool IMPLIED>
QmvLauncher pick_m(int M) {
  switch (M) {
    case 1: return &launch_qmv_t<FMT, GS, 1, IMPLIED>;
    case 2: return &launch_qmv_t<FMT, GS, 2, IMPLIED>;
    case 3: return &launch_qmv_t<FMT, GS, 3, IMPLIED>;
    case 4: return &launch_qmv_t<FMT, GS, 4, IMPLIED>;
    case 5: return &launch_qmv_t<FMT, GS, 5, IMPLIED>;
  }
  return nullptr;
}

}  // namespace
}  // namespace bq
