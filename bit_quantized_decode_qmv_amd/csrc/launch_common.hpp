// Host-side pieces shared by the library's translation units: the launch
// helper, the decode group limit and the per-format launchers.  Each weight
// format's kernel instances live in a translation unit of their own
// (qmv_u1/u2/t5.hip, qmm_u1/u2/t5.hip), so that they compile in parallel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "bq.h"
#include "qmm_kernels.hpp"
#include "qmv_kernels.hpp"

namespace bq {

inline int launch_kernel(const void* fn, dim3 grid, dim3 block, size_t shmem, void* stream, void* params) {
  void* args[] = {params};
  hipError_t err = hipLaunchKernel(fn, grid, block, args, shmem, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? BQ_OK : BQ_ERR_HIP;
}

// 16-byte vectors of a workgroup's scale (or bias) block, at most
constexpr int sb_vectors(int rows_per_wg, int G) { return (int)(((int64_t)rows_per_wg * G * 2 + 15) / 16 + 1); }
// Groups per row the decode kernels take: the scale rows of two rows must
// fit one staging pass.
constexpr int kMaxDecodeGroups = 4092;
static_assert(sb_vectors(kR, kMaxDecodeGroups) <= kSbRounds * kThreads &&
                  sb_vectors(kR, kMaxDecodeGroups + 1) > kSbRounds * kThreads,
              "decode group limit");

// One decode launch of a kernel instance chosen for (format, gs, rows at
// once, implied bias); returns a bq_status.
typedef int (*QmvLauncher)(QmvParams, void*);
QmvLauncher pick_qmv_u1(int gs, int M, bool implied);
QmvLauncher pick_qmv_u2(int gs, int M, bool implied);
QmvLauncher pick_qmv_t5(int gs, int M, bool implied);

// Prefill products with at most 32 rows use 32-row tiles whose loading
// waves request x and the weight bytes four iterations ahead.  The choice
// per call: BN columns per tile (64 or 128), SUB K steps per iteration, and
// SPLIT workgroups per tile, each over 1/SPLIT of the K iterations (SPLIT >
// 1 stores fp32 partial tiles to a workspace of SPLIT *
// qmm_part_stride(M, N) floats and adds them up in a second kernel).
struct QmmSmallChoice {
  int bn, sub, split;
};

// Unsplit: measured on MI355X at M = 32 with one iteration of prefetch, an
// iteration of SUB steps took about 0.57 us plus 0.43 us per step with
// 64-column tiles and 0.50 us per step with 128-column tiles (four
// iterations of prefetch cut both by about a third and keep their order,
// which is all this estimate is used for); workgroups run in rounds of 256,
// 512 for 64-column tiles of one step (their LDS lets two share a CU).
inline double qmm_unsplit_us(int tiles, int iters, int bn, int sub) {
  const int per_cu = (bn == 64 && sub == 1) ? 2 : 1;
  const double rounds = std::ceil((double)tiles / (256.0 * per_cu));
  return rounds * iters * (0.57 + sub * (bn == 64 ? 0.43 : 0.50));
}

// Split: microseconds per call fitted to a sweep on MI355X (t5 and 2-bit;
// 6144 x 5120, 1024 x 5120, 5120 x 6144, 17408 x 5120 and 5120 x 17408;
// M = 17 and 32; every (BN, SUB) with 1 to 8 shares; fit within about 15%):
// 3.4 + 4.0 (the partial sums) + rounds x (3.1 + iterations per share x
// 0.31 / 2.03 / 0.51 / 1.12 for 64 x 1 / 64 x 4 / 128 x 1 / 128 x 2),
// rounds = ceil(workgroups / 256).  On that sweep its pick is within 6% of
// the fastest choice in every case (t5 down at M = 32: 96 -> 35 us).
inline double qmm_split_us(int tiles, int iters, int bn, int sub, int split) {
  const double it = bn == 64 ? (sub == 1 ? 0.31 : 2.03) : (sub == 1 ? 0.51 : 1.12);
  const double rounds = std::ceil((double)tiles * split / 256.0);
  return 3.4 + (split > 1 ? 4.0 : 0.0) + rounds * (3.1 + std::ceil((double)iters / split) * it);
}

// cap: workspace bytes (0: no split); force_split > 0: that many shares only
inline QmmSmallChoice qmm_small_m_choice(int M, int N, int K, size_t cap, int force_split = 0) {
  const int steps = K / kQmmBK;
  const size_t slice = qmm_part_stride(M, N) * sizeof(float);
  const int opts[4][2] = {{64, 1}, {64, 4}, {128, 1}, {128, 2}};
  QmmSmallChoice best{64, 1, 1};
  double best_us = 1e30;
  for (const auto& o : opts) {
    if (steps % o[1] != 0) continue;
    const double us = qmm_unsplit_us((N + o[0] - 1) / o[0], steps / o[1], o[0], o[1]);
    if (us < best_us) {
      best = QmmSmallChoice{o[0], o[1], 1};
      best_us = us;
    }
  }
  if (force_split == 1 || cap < 2 * slice) return best;
  best_us = force_split > 1 ? 1e30 : qmm_split_us((N + best.bn - 1) / best.bn, steps / best.sub, best.bn, best.sub, 1);
  for (const auto& o : opts) {
    if (steps % o[1] != 0) continue;
    const int iters = steps / o[1], tiles = (N + o[0] - 1) / o[0];
    for (int S = 2; S <= kQmmMaxSplit && S <= iters && (size_t)S * slice <= cap; ++S) {
      if (force_split > 1 && S != force_split) continue;
      const double us = qmm_split_us(tiles, iters, o[0], o[1], S);
      if (us < best_us) {
        best = QmmSmallChoice{o[0], o[1], S};
        best_us = us;
      }
    }
  }
  return best;
}

// One prefill product launch (tile shape chosen per call).
int launch_qmm_u1(const QmmParams& p, int gs, bool implied, void* stream);
int launch_qmm_u2(const QmmParams& p, int gs, bool implied, void* stream);
int launch_qmm_t5(const QmmParams& p, int gs, bool implied, void* stream);

}  // namespace bq
