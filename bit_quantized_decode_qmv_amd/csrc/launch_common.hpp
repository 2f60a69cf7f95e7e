// Host-side pieces shared by the library's translation units: the launch
// helper, the decode group limit and the per-format launchers.  Each weight
// format's kernel instances live in a translation unit of their own
// (qmv_u1/u2/t5.hip, qmm_u1/u2/t5.hip), so that they compile in parallel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// One prefill product launch (tile shape chosen per call).
int launch_qmm_u1(const QmmParams& p, int gs, bool implied, void* stream);
int launch_qmm_u2(const QmmParams& p, int gs, bool implied, void* stream);
int launch_qmm_t5(const QmmParams& p, int gs, bool implied, void* stream);

}  // namespace bq
