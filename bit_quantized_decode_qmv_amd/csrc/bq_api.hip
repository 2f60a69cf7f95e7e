// C ABI of the library: argument validation, kernel selection and launch.
// Declarations and the meaning of every argument are in include/bq.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <type_traits>

#include "bq.h"
#include "dequant_kernels.hpp"
#include "qmm_kernels.hpp"
#include "qmv_kernels.hpp"
#include "repack_kernels.hpp"
#include "spec_kernels.hpp"
#include "sym_kernels.hpp"

namespace {

using namespace bq;

// 16-byte vectors of a workgroup's scale (or bias) block, at most
constexpr int sb_vectors(int rows_per_wg, int G) { return (int)(((int64_t)rows_per_wg * G * 2 + 15) / 16 + 1); }
// Groups per row the decode kernels take: the scale rows of two rows must
// fit one staging pass.
constexpr int kMaxDecodeGroups = 4092;
static_assert(sb_vectors(bq::kR, kMaxDecodeGroups) <= bq::kSbRounds * bq::kThreads &&
                  sb_vectors(bq::kR, kMaxDecodeGroups + 1) > bq::kSbRounds * bq::kThreads,
              "decode group limit");

enum Entry { E_QMV, E_WIDE, E_SYM, E_T5, E_T5_WIDE, E_QMM, E_DEQUANT, E_UQMM };

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int row_bytes_of(int bits, int K, int gs) {
  if (bits == BQ_BITS_T5) return (K / gs) * ((gs + 4) / 5);
  return K / 8 * bits;
}

int validate(Entry e, const void* x, const void* w, const void* scales, const void* biases,
             const void* y, int M, int N, int K, int bits, int gs) {
  const bool t5 = (e == E_T5 || e == E_T5_WIDE || e == E_QMM);
  if (!w || !scales || !y) return BQ_ERR_NULL;
  if (e != E_DEQUANT && !x) return BQ_ERR_NULL;
  if ((e == E_QMV || e == E_WIDE) && !biases) return BQ_ERR_NULL;
  if (e == E_DEQUANT) {
    if (bits != 1 && bits != 2 && bits != BQ_BITS_T5) return BQ_ERR_BITS;
  } else if (t5) {
    if (bits != BQ_BITS_T5) return BQ_ERR_BITS;
  } else if (bits != 1 && bits != 2) {
    return BQ_ERR_BITS;
  }
  if (gs != 64 && gs != 128) return BQ_ERR_GROUP;
  if (N <= 0 || K <= 0 || K % gs != 0 || K > (1 << 26)) return BQ_ERR_SHAPE;
  // packed rows and scale rows are addressed with 32-bit offsets
  if ((uint64_t)N * (uint64_t)row_bytes_of(bits == BQ_BITS_T5 ? BQ_BITS_T5 : 2, K, gs) >= (1ull << 30) ||
      (uint64_t)N * (uint64_t)(K / gs) >= (1ull << 29))
    return BQ_ERR_SHAPE;
  const bool mm = (e == E_QMM || e == E_UQMM);
  if (e != E_DEQUANT && !mm && K / gs > kMaxDecodeGroups) return BQ_ERR_SHAPE;
  // qmm addresses x with 32-bit offsets too
  if (mm && M > 0 && (uint64_t)M * (uint64_t)K * 2 >= (1ull << 31)) return BQ_ERR_SHAPE;
  if (e != E_DEQUANT) {
    if (M < 1) return BQ_ERR_M;
    if ((e == E_WIDE || e == E_SYM || e == E_T5_WIDE) && M > BQ_MAX_WIDE_M) return BQ_ERR_M;
  }
  if (!aligned(w, 4) || !aligned(scales, 2) || (biases && !aligned(biases, 2))) return BQ_ERR_ALIGN;
  if (x && !aligned(x, 2)) return BQ_ERR_ALIGN;
  if (!aligned(y, 2)) return BQ_ERR_ALIGN;
  if (bits == BQ_BITS_T5 && K % 256 != 0) return BQ_ERR_ALIGN;
  if (e != E_DEQUANT && !aligned(x, 16)) return BQ_ERR_ALIGN;
  // the decode kernels read scales and biases in 16-byte vectors
  if (e != E_DEQUANT && !mm &&
      (!aligned(scales, 16) || (biases && e != E_SYM && !aligned(biases, 16))))
    return BQ_ERR_ALIGN;
  if (e == E_DEQUANT && bits != BQ_BITS_T5 && !aligned(y, 16)) return BQ_ERR_ALIGN;
  return BQ_OK;
}

// spec verify workspace: row keys, then per-sequence counters
size_t spec_keys_bytes(int B, int L) { return ((size_t)B * (L + 1) * 8 + 255) / 256 * 256; }
size_t spec_workspace_bytes(int B, int L) { return spec_keys_bytes(B, L) + (size_t)B * 4; }

int launch(const void* fn, dim3 grid, dim3 block, size_t shmem, void* stream, void* params) {
  void* args[] = {params};
  hipError_t err = hipLaunchKernel(fn, grid, block, args, shmem, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? BQ_OK : BQ_ERR_HIP;
}

// ---------------------------------------------------------------- qmv family
constexpr int kTargetWorkgroups = 256;
constexpr int kMaxRowsPerWg = 256;
constexpr size_t kLdsBudget = 150 * 1024;


size_t qmv_lds_bytes(int M, int R, int rows_per_wg, int ntiles, int seg_tiles, int G) {
  const size_t U = (size_t)((rows_per_wg + R - 1) / R) * ntiles;
  const size_t cs = (size_t)M * kXD + ((M % 2 == 0) ? 4 : 0);
  return 4 * ((size_t)seg_tiles * kKL * cs + (size_t)M * seg_tiles * kKL +
              8 * (size_t)sb_entry_dwords(M) * sb_vectors(rows_per_wg, G) + U * R * M);
}

// Workgroup geometry for M activation rows and R rows per unit.  Rows per
// workgroup: a multiple of R, enough for one workgroup per CU.  Segment: as
// many K tiles of x as LDS and the staging tasks (M * tiles * 16 <=
// kStageRounds * kThreads) allow, split evenly.  Returns false if even R rows
// per workgroup do not fit.
bool qmv_geometry(QmvParams& p, int M, int R) {
  p.ntiles = (p.K + kTile - 1) / kTile;
  const int max_st = std::min(p.ntiles, kStageRounds * kThreads / (kKL * M));
  int rows = R * ((p.N + R * kTargetWorkgroups - 1) / (R * kTargetWorkgroups));
  if (rows > kMaxRowsPerWg) rows = kMaxRowsPerWg;
  for (; rows >= R; rows -= R) {
    if (sb_vectors(rows, p.G) > kSbRounds * kThreads) continue;
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
int units_per_slot(const QmvParams& p, int R) {
  const int U = ((p.rows_per_wg + R - 1) / R) * p.seg_tiles;
  return (U + kSlots - 1) / kSlots;
}

template <int FMT, int GS, int M, bool IMPLIED, int P, int R>
int launch_qmv_p(const QmvParams& p, void* stream) {
  const void* fn = reinterpret_cast<const void*>(&qmv_kernel<FMT, GS, M, IMPLIED, P, R>);
  static const hipError_t attr =
      hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBudget);
  (void)attr;
  const size_t shmem = qmv_lds_bytes(M, R, p.rows_per_wg, p.ntiles, p.seg_tiles, p.G);
  dim3 grid((p.N + p.rows_per_wg - 1) / p.rows_per_wg);
  QmvParams q = p;
  return launch(fn, grid, dim3(kThreads), shmem, stream, &q);
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
    return launch_qmv_p<FMT, GS, M, IMPLIED, 2, 4>(p, stream);
  }
  if (!qmv_geometry(p, M, 2)) return BQ_ERR_SHAPE;
  return launch_qmv_p<FMT, GS, M, IMPLIED, 2, 2>(p, stream);
}

typedef int (*QmvLauncher)(QmvParams, void*);

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

QmvLauncher pick_qmv(int fmt, int gs, int M, bool implied) {
  if (fmt == FMT_U1) {
    if (gs == 64) return implied ? pick_m<FMT_U1, 64, true>(M) : pick_m<FMT_U1, 64, false>(M);
    return implied ? pick_m<FMT_U1, 128, true>(M) : pick_m<FMT_U1, 128, false>(M);
  }
  if (fmt == FMT_U2) {
    if (gs == 64) return implied ? pick_m<FMT_U2, 64, true>(M) : pick_m<FMT_U2, 64, false>(M);
    return implied ? pick_m<FMT_U2, 128, true>(M) : pick_m<FMT_U2, 128, false>(M);
  }
  if (gs == 64) return implied ? pick_m<FMT_T5, 64, true>(M) : pick_m<FMT_T5, 64, false>(M);
  return implied ? pick_m<FMT_T5, 128, true>(M) : pick_m<FMT_T5, 128, false>(M);
}

// rows_at_once: M for the wide entry points, 1 for the per-row ones.
int run_qmv(Entry e, const void* x, const void* w, const void* scales, const void* biases, void* y,
            int M, int N, int K, int bits, int gs, void* stream) {
  int st = validate(e, x, w, scales, biases, y, M, N, K, bits, gs);
  if (st != BQ_OK) return st;
  const bool t5 = (bits == BQ_BITS_T5);
  const int fmt = t5 ? FMT_T5 : (bits == 1 ? FMT_U1 : FMT_U2);
  const bool implied = (e == E_SYM) || (t5 && biases == nullptr);
  QmvParams p{};
  p.w = static_cast<const uint8_t*>(w);
  p.s = static_cast<const half_t*>(scales);
  p.b = implied ? nullptr : static_cast<const half_t*>(biases);
  p.N = N;
  p.K = K;
  p.G = K / gs;
  p.row_bytes = row_bytes_of(bits, K, gs);
  p.ratio = t5 ? 1.0f : (bits == 1 ? 0.5f : 1.5f);
  p.x_bytes = 0;  // per launch, below
  p.w_bytes = (int)((size_t)N * p.row_bytes);
  p.sb_bytes = (int)((size_t)N * p.G * 2);
  const bool per_row = (e == E_QMV || e == E_T5);
  const int rows_at_once = per_row ? 1 : M;
  QmvLauncher fn = pick_qmv(fmt, gs, rows_at_once, implied);
  if (!fn) return BQ_ERR_M;
  p.x_bytes = rows_at_once * K * 2;
  for (int m0 = 0; m0 < M; m0 += rows_at_once) {
    p.x = static_cast<const half_t*>(x) + (size_t)m0 * K;
    p.y = static_cast<half_t*>(y) + (size_t)m0 * N;
    st = fn(p, stream);
    if (st != BQ_OK) return st;
  }
  return BQ_OK;
}

// ---------------------------------------------------------------- qmm
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
  return launch(fn, grid, dim3(kQmmThreads), lds, stream, &q);
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
// pipeline iteration, not by the MFMA or memory throughput: measured on
// MI355X at M = 32, an iteration of SUB steps takes about 0.57 us plus
// 0.43 us per step with 64-column tiles and 0.50 us per step with 128-column
// tiles.  Estimated microseconds of (BN, SUB) over `tiles` workgroups (two
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
    return o->bn == 64 ? launch_qmm_t<32, 64, BITS, GS, IMPLIED>(p, o->sub, stream)
                       : launch_qmm_t<32, 128, BITS, GS, IMPLIED>(p, o->sub, stream);
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

int launch_qmm(const void* x, const void* w, const void* scales, const void* biases, void* y, int M, int N,
               int K, int bits, int group_size, void* stream) {
  QmmParams p{};
  p.x = static_cast<const half_t*>(x);
  p.w = static_cast<const uint8_t*>(w);
  p.s = static_cast<const half_t*>(scales);
  p.b = static_cast<const half_t*>(biases);
  p.y = static_cast<half_t*>(y);
  p.M = M;
  p.N = N;
  p.K = K;
  p.G = K / group_size;
  p.row_bytes = row_bytes_of(bits, K, group_size);
  p.x_bytes = (int)((size_t)M * K * 2);
  p.w_bytes = (int)((size_t)N * p.row_bytes);
  p.sb_bytes = (int)((size_t)N * p.G * 2);
  const bool implied = biases == nullptr;
  if (bits == BQ_BITS_T5) return launch_qmm_bits<BQ_BITS_T5>(p, group_size, implied, stream);
  if (bits == 1) return launch_qmm_bits<1>(p, group_size, implied, stream);
  return launch_qmm_bits<2>(p, group_size, implied, stream);
}

}  // namespace

extern "C" {

int bq_abi_version(void) { return BQ_ABI_VERSION; }

const char* bq_strerror(int status) {
  switch (status) {
    case BQ_OK: return "success";
    case BQ_ERR_NULL: return "a required pointer is NULL";
    case BQ_ERR_BITS:
      return "bits (1, 2, or BQ_BITS_T5 = 0) or the logits dtype is not valid for this entry point";
    case BQ_ERR_GROUP: return "group_size must be 64 or 128";
    case BQ_ERR_SHAPE:
      return "N and K must be positive, K a multiple of group_size, and the sizes within the limits of bq.h";
    case BQ_ERR_M: return "M is outside the range this entry point accepts";
    case BQ_ERR_ALIGN:
      return "a pointer is misaligned (x, and for the decode calls scales and biases, need 16 bytes), or a t5 "
             "call has K not a multiple of 256";
    case BQ_ERR_FLAGS: return "flags holds bits this entry point does not define";
    case BQ_ERR_HIP: return "the HIP runtime rejected the kernel launch";
    case BQ_ERR_WORKSPACE: return "the workspace is NULL or smaller than bq_spec_verify_workspace reports";
  }
  return "unknown bq status";
}

int bq_qmv(const void* x, const void* w, const void* scales, const void* biases, void* y, int M,
           int N, int K, int bits, int group_size, void* stream) {
  return run_qmv(E_QMV, x, w, scales, biases, y, M, N, K, bits, group_size, stream);
}

int bq_qmv_wide(const void* x, const void* w, const void* scales, const void* biases, void* y,
                int M, int N, int K, int bits, int group_size, void* stream) {
  return run_qmv(E_WIDE, x, w, scales, biases, y, M, N, K, bits, group_size, stream);
}

int bq_qmv_sym(const void* x, const void* w, const void* scales, const void* biases, void* y, int M,
               int N, int K, int bits, int group_size, void* stream) {
  return run_qmv(E_SYM, x, w, scales, biases, y, M, N, K, bits, group_size, stream);
}

int bq_t5_qmv(const void* x, const void* w, const void* scales, const void* biases, void* y, int M,
              int N, int K, int bits, int group_size, void* stream) {
  return run_qmv(E_T5, x, w, scales, biases, y, M, N, K, bits, group_size, stream);
}

int bq_t5_qmv_wide(const void* x, const void* w, const void* scales, const void* biases, void* y,
                   int M, int N, int K, int bits, int group_size, void* stream) {
  return run_qmv(E_T5_WIDE, x, w, scales, biases, y, M, N, K, bits, group_size, stream);
}

int bq_qmm(const void* x, const void* w, const void* scales, const void* biases, void* y, int M, int N,
           int K, int bits, int group_size, void* stream) {
  int st = validate(E_UQMM, x, w, scales, biases, y, M, N, K, bits, group_size);
  if (st != BQ_OK) return st;
  return launch_qmm(x, w, scales, biases, y, M, N, K, bits, group_size, stream);
}

int bq_t5_qmm(const void* x, const void* w, const void* scales, const void* biases, void* y, int M,
              int N, int K, int bits, int group_size, void* stream) {
  int st = validate(E_QMM, x, w, scales, biases, y, M, N, K, bits, group_size);
  if (st != BQ_OK) return st;
  return launch_qmm(x, w, scales, biases, y, M, N, K, BQ_BITS_T5, group_size, stream);
}

int bq_dequant(const void* x, const void* w, const void* scales, const void* biases, void* y, int M,
               int N, int K, int bits, int group_size, void* stream) {
  int st = validate(E_DEQUANT, x, w, scales, biases, y, M, N, K, bits, group_size);
  if (st != BQ_OK) return st;
  DequantParams p{};
  p.w = static_cast<const uint8_t*>(w);
  p.s = static_cast<const half_t*>(scales);
  p.b = static_cast<const half_t*>(biases);
  p.out = static_cast<half_t*>(y);
  p.N = N;
  p.K = K;
  p.G = K / group_size;
  p.gs = group_size;
  p.row_bytes = row_bytes_of(bits, K, group_size);
  p.ratio = bits == BQ_BITS_T5 ? 1.0f : (bits == 1 ? 0.5f : 1.5f);
  const bool implied = (biases == nullptr);
  size_t items;
  const void* fn;
  if (bits == BQ_BITS_T5) {
    items = (size_t)N * p.G * ((group_size + 4) / 5);
    fn = implied ? reinterpret_cast<const void*>(&dequant_t5_kernel<true>)
                 : reinterpret_cast<const void*>(&dequant_t5_kernel<false>);
  } else {
    items = (size_t)N * (K / (32 / bits));
    if (bits == 1)
      fn = implied ? reinterpret_cast<const void*>(&dequant_words_kernel<1, true>)
                   : reinterpret_cast<const void*>(&dequant_words_kernel<1, false>);
    else
      fn = implied ? reinterpret_cast<const void*>(&dequant_words_kernel<2, true>)
                   : reinterpret_cast<const void*>(&dequant_words_kernel<2, false>);
  }
  const size_t blocks = (items + 255) / 256;
  if (blocks > 0x7FFFFFFF) return BQ_ERR_SHAPE;
  return launch(fn, dim3((unsigned)blocks), dim3(256), 0, stream, &p);
}

int bq_linear_route(int M, int N, int bits, int flags, int* passes) {
  if (M < 1) return BQ_ERR_M;
  if (N < 1) return BQ_ERR_SHAPE;
  if (bits != 1 && bits != 2 && bits != BQ_BITS_T5) return BQ_ERR_BITS;
  int route, n = 1;
  // the fused product needs enough output tiles to occupy the GPU: with
  // fewer, passes of up to five rows are faster (measured on the down
  // shape, N = 5120, t5 at M = 17: about 88 us in four passes against
  // 145 us fused)
  const bool tiles = (int64_t)((N + 63) / 64) * ((M + 31) / 32) >= BQ_QMM_MIN_TILES;
  if (bits == BQ_BITS_T5 && M >= BQ_T5_QMM_MIN_M && tiles) {
    route = BQ_ROUTE_T5_QMM;
  } else if (bits != BQ_BITS_T5 && M >= BQ_QMM_MIN_M && tiles) {
    route = BQ_ROUTE_QMM;
  } else {
    route = bits == BQ_BITS_T5 ? BQ_ROUTE_T5_WIDE : ((flags & BQ_LINEAR_SYM) ? BQ_ROUTE_QMV_SYM : BQ_ROUTE_QMV_WIDE);
    n = (M + BQ_MAX_WIDE_M - 1) / BQ_MAX_WIDE_M;
  }
  if (passes) *passes = n;
  return route;
}

int bq_linear(const void* x, const void* w, const void* scales, const void* biases, void* y, int M, int N,
              int K, int bits, int group_size, int flags, void* stream) {
  if ((flags & ~BQ_LINEAR_SYM) != 0) return BQ_ERR_FLAGS;
  int passes = 0;
  const int route = bq_linear_route(M, N, bits, flags, &passes);
  if (route < 0) return route;
  // symmetric: the bias is implied and never read (t5: -scale)
  const void* b = (flags & BQ_LINEAR_SYM) ? nullptr : biases;
  if (route == BQ_ROUTE_T5_QMM) return bq_t5_qmm(x, w, scales, b, y, M, N, K, bits, group_size, stream);
  if (route == BQ_ROUTE_QMM) {
    // without the symmetric flag the stored biases are required, as for the wide route
    if (!b && !(flags & BQ_LINEAR_SYM)) return BQ_ERR_NULL;
    return bq_qmm(x, w, scales, b, y, M, N, K, bits, group_size, stream);
  }
  const Entry e = route == BQ_ROUTE_T5_WIDE ? E_T5_WIDE : (route == BQ_ROUTE_QMV_SYM ? E_SYM : E_WIDE);
  // every pass is validated in full before it launches; the first check
  // also covers the arguments common to all passes
  for (int m0 = 0; m0 < M; m0 += BQ_MAX_WIDE_M) {
    const int mc = M - m0 < BQ_MAX_WIDE_M ? M - m0 : BQ_MAX_WIDE_M;
    const void* xm = x ? static_cast<const void*>(static_cast<const half_t*>(x) + (size_t)m0 * K) : nullptr;
    void* ym = y ? static_cast<void*>(static_cast<half_t*>(y) + (size_t)m0 * N) : nullptr;
    const int st = run_qmv(e, xm, w, scales, b, ym, mc, N, K, bits, group_size, stream);
    if (st != BQ_OK) return st;
  }
  return BQ_OK;
}

int bq_sym_check(const void* scales, const void* biases, int N, int K, int bits, int group_size, int* flag,
                 void* stream) {
  if (!scales || !biases || !flag) return BQ_ERR_NULL;
  if (bits != 1 && bits != 2 && bits != BQ_BITS_T5) return BQ_ERR_BITS;
  if (group_size != 64 && group_size != 128) return BQ_ERR_GROUP;
  if (N <= 0 || K <= 0 || K % group_size != 0) return BQ_ERR_SHAPE;
  if (!aligned(scales, 2) || !aligned(biases, 2) || !aligned(flag, 4)) return BQ_ERR_ALIGN;
  SymCheckParams p{};
  p.s = static_cast<const _Float16*>(scales);
  p.b = static_cast<const _Float16*>(biases);
  p.n = (int64_t)N * (K / group_size);
  p.ratio = bits == BQ_BITS_T5 ? 1.0f : (bits == 1 ? 0.5f : 1.5f);
  p.flag = flag;
  int st = launch(reinterpret_cast<const void*>(&sym_flag_init_kernel), dim3(1), dim3(64), 0, stream, &p);
  if (st != BQ_OK) return st;
  const int64_t blocks = std::min<int64_t>((p.n + 255) / 256, 2048);
  return launch(reinterpret_cast<const void*>(&sym_check_kernel), dim3((unsigned)blocks), dim3(256), 0, stream, &p);
}

int bq_t5_repack(const void* w, void* w_t5, int N, int K, int bits, int group_size, int* flag, void* stream) {
  if (!w || !w_t5 || !flag) return BQ_ERR_NULL;
  if (bits != 1 && bits != 2) return BQ_ERR_BITS;
  if (group_size != 64 && group_size != 128) return BQ_ERR_GROUP;
  if (N <= 0 || K <= 0 || K % group_size != 0 || K > (1 << 26)) return BQ_ERR_SHAPE;
  if ((uint64_t)N * (uint64_t)row_bytes_of(2, K, group_size) >= (1ull << 30)) return BQ_ERR_SHAPE;
  if (K % 256 != 0) return BQ_ERR_ALIGN;
  if (!aligned(w, 4) || !aligned(w_t5, 4) || !aligned(flag, 4)) return BQ_ERR_ALIGN;
  RepackParams p{};
  p.w = static_cast<const uint32_t*>(w);
  p.out = static_cast<uint32_t*>(w_t5);
  p.words_per_row = K / 32 * bits;
  p.dwords_per_row = row_bytes_of(BQ_BITS_T5, K, group_size) / 4;
  p.total = (int64_t)N * p.dwords_per_row;
  p.flag = flag;
  int st = launch(reinterpret_cast<const void*>(&repack_flag_init_kernel), dim3(1), dim3(64), 0, stream, &p);
  if (st != BQ_OK) return st;
  const void* fn;
  if (bits == 1) {
    fn = group_size == 64 ? reinterpret_cast<const void*>(&t5_repack_kernel<1, 64>)
                          : reinterpret_cast<const void*>(&t5_repack_kernel<1, 128>);
  } else {
    fn = group_size == 64 ? reinterpret_cast<const void*>(&t5_repack_kernel<2, 64>)
                          : reinterpret_cast<const void*>(&t5_repack_kernel<2, 128>);
  }
  const int64_t blocks = std::min<int64_t>((p.total + 255) / 256, 8192);
  return launch(fn, dim3((unsigned)blocks), dim3(256), 0, stream, &p);
}

int bq_spec_verify_workspace(int B, int L, int V, size_t* bytes) {
  if (!bytes) return BQ_ERR_NULL;
  if (B < 1 || L < 0 || L > BQ_SPEC_MAX_DRAFT || V < 1) return BQ_ERR_SHAPE;
  *bytes = spec_workspace_bytes(B, L);
  return BQ_OK;
}

int bq_spec_decode_verify(const void* logits, int logits_dtype, const int* draft, int B, int L, int V,
                          int* accepted, int* next_token, int* target_tokens, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (!logits || (L > 0 && !draft) || !accepted || !next_token) return BQ_ERR_NULL;
  if (logits_dtype != BQ_DTYPE_F16 && logits_dtype != BQ_DTYPE_F32) return BQ_ERR_BITS;
  if (B < 1 || L < 0 || L > BQ_SPEC_MAX_DRAFT || V < 1) return BQ_ERR_SHAPE;
  const int64_t chunks = (V + kSpecChunk - 1) / kSpecChunk;
  if ((int64_t)B * (L + 1) * chunks >= (1ll << 31)) return BQ_ERR_SHAPE;
  if (!workspace || workspace_bytes < spec_workspace_bytes(B, L)) return BQ_ERR_WORKSPACE;
  const size_t esz = logits_dtype == BQ_DTYPE_F16 ? 2 : 4;
  if (!aligned(logits, esz) || (draft && !aligned(draft, 4)) || !aligned(accepted, 4) ||
      !aligned(next_token, 4) || (target_tokens && !aligned(target_tokens, 4)) || !aligned(workspace, 8))
    return BQ_ERR_ALIGN;
  SpecParams p{};
  p.logits = logits;
  p.draft = draft;
  p.accepted = accepted;
  p.next_token = next_token;
  p.target = target_tokens;
  p.keys = static_cast<unsigned long long*>(workspace);
  p.counters = reinterpret_cast<unsigned int*>(static_cast<char*>(workspace) + spec_keys_bytes(B, L));
  p.B = B;
  p.L = L;
  p.V = V;
  p.chunks = (int)chunks;
  const void* fn = logits_dtype == BQ_DTYPE_F16 ? reinterpret_cast<const void*>(&spec_verify_kernel<_Float16>)
                                                : reinterpret_cast<const void*>(&spec_verify_kernel<float>);
  return launch(fn, dim3((unsigned)((int64_t)B * (L + 1) * chunks)), dim3(kSpecThreads), 0, stream, &p);
}

}  // extern "C"
