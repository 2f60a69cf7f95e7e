// C ABI of the library: argument validation, kernel selection and launch.
// Declarations and the meaning of every argument are in include/bq.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <type_traits>

#include "bq.h"
#include "dequant_kernels.hpp"
#include "launch_common.hpp"
#include "repack_kernels.hpp"
#include "spec_kernels.hpp"
#include "sym_kernels.hpp"

namespace {

using namespace bq;

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
  // Alignment: W and, for the decode calls, x, scales and biases (read as
  // dwords) 4 bytes; the prefill products stage x with 16-byte loads that
  // write LDS directly and need x 16-byte aligned; fp16 arrays read or
  // written element by element 2 bytes.  A symmetric call never reads its
  // biases, so their alignment does not matter there.
  const bool decode = (e != E_DEQUANT && !mm);
  const uintptr_t sb_align = decode ? 4 : 2;
  if (!aligned(w, 4) || !aligned(scales, sb_align) || (biases && e != E_SYM && !aligned(biases, sb_align)))
    return BQ_ERR_ALIGN;
  if (x && !aligned(x, mm ? 16 : (decode ? 4 : 2))) return BQ_ERR_ALIGN;
  if (!aligned(y, 2)) return BQ_ERR_ALIGN;
  return BQ_OK;
}

// spec verify workspace: row keys, then per-sequence counters

// Scratch of the allocation-free verify entry point: a file-scope device
// array, one copy per GPU, held until the process ends.  Host code never
// passes its name to a kernel (on the host the name is only a stand-in):
// it takes the device address from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = BQ_SPEC_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BQ_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return BQ_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BQ_OK;
}

// zeroes n bytes (a multiple of 4) of device memory with vector stores
__global__ __launch_bounds__(256) void zero_fill_kernel(uint32_t* p, size_t n_words) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

int launch(const void* fn, dim3 grid, dim3 block, size_t shmem, void* stream, void* params) {
  return launch_kernel(fn, grid, block, shmem, stream, params);
}

// dequant kernel instances by output alignment (16, 4 or 2 bytes)
template <int BITS>
const void* pick_dequant_words(bool implied, int A) {
  if (implied)
    return A == 16 ? reinterpret_cast<const void*>(&dequant_words_kernel<BITS, true, 16>)
         : A == 4  ? reinterpret_cast<const void*>(&dequant_words_kernel<BITS, true, 4>)
                   : reinterpret_cast<const void*>(&dequant_words_kernel<BITS, true, 2>);
  return A == 16 ? reinterpret_cast<const void*>(&dequant_words_kernel<BITS, false, 16>)
       : A == 4  ? reinterpret_cast<const void*>(&dequant_words_kernel<BITS, false, 4>)
                 : reinterpret_cast<const void*>(&dequant_words_kernel<BITS, false, 2>);
}
template <int GS>
const void* pick_dequant_t5(bool implied, int A) {
  if (implied)
    return A == 16 ? reinterpret_cast<const void*>(&dequant_t5_kernel<GS, true, 16>)
         : A == 4  ? reinterpret_cast<const void*>(&dequant_t5_kernel<GS, true, 4>)
                   : reinterpret_cast<const void*>(&dequant_t5_kernel<GS, true, 2>);
  return A == 16 ? reinterpret_cast<const void*>(&dequant_t5_kernel<GS, false, 16>)
       : A == 4  ? reinterpret_cast<const void*>(&dequant_t5_kernel<GS, false, 4>)
                 : reinterpret_cast<const void*>(&dequant_t5_kernel<GS, false, 2>);
}

// ---------------------------------------------------------------- qmv family
QmvLauncher pick_qmv(int fmt, int gs, int M, bool implied) {
  if (M < 1 || M > BQ_MAX_WIDE_M) return nullptr;
  if (fmt == FMT_U1) return pick_qmv_u1(gs, M, implied);
  if (fmt == FMT_U2) return pick_qmv_u2(gs, M, implied);
  return pick_qmv_t5(gs, M, implied);
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
int launch_qmm(const void* x, const void* w, const void* scales, const void* biases, void* y, int M, int N,
               int K, int bits, int group_size, void* stream, void* workspace = nullptr, size_t ws_bytes = 0) {
  QmmParams p{};
  p.ksplit = 1;
  p.part = static_cast<float*>(workspace);
  p.part_cap = workspace ? ws_bytes : 0;
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
  if (bits == BQ_BITS_T5) return launch_qmm_t5(p, group_size, implied, stream);
  if (bits == 1) return launch_qmm_u1(p, group_size, implied, stream);
  return launch_qmm_u2(p, group_size, implied, stream);
}

// checks of bq_spec_decode_verify's arguments other than the workspace
int spec_validate(const void* logits, int logits_dtype, const int* draft, int B, int L, int V, const int* accepted,
                  const int* next_token, const int* target_tokens) {
  if (!logits || (L > 0 && !draft) || !accepted || !next_token) return BQ_ERR_NULL;
  if (logits_dtype != BQ_DTYPE_F16 && logits_dtype != BQ_DTYPE_F32) return BQ_ERR_BITS;
  if (B < 1 || L < 0 || L > BQ_SPEC_MAX_DRAFT || V < 1) return BQ_ERR_SHAPE;
  const size_t esz = logits_dtype == BQ_DTYPE_F16 ? 2 : 4;
  if ((int64_t)B * (L + 1) * spec_chunks(V, (int)esz) >= (1ll << 31)) return BQ_ERR_SHAPE;
  if (!aligned(logits, esz) || (draft && !aligned(draft, 4)) || !aligned(accepted, 4) || !aligned(next_token, 4) ||
      (target_tokens && !aligned(target_tokens, 4)))
    return BQ_ERR_ALIGN;
  return BQ_OK;
}

int spec_launch(const void* logits, int logits_dtype, const int* draft, int B, int L, int V, int* accepted,
                int* next_token, int* target_tokens, void* workspace, void* stream) {
  SpecParams p{};
  p.logits = logits;
  p.draft = draft;
  p.accepted = accepted;
  p.next_token = next_token;
  p.target = target_tokens;
  p.keys = static_cast<unsigned long long*>(workspace);
  char* ws = static_cast<char*>(workspace);
  p.row_counts = reinterpret_cast<unsigned int*>(ws + spec_keys_bytes(B, L));
  p.counters = reinterpret_cast<unsigned int*>(ws + spec_keys_bytes(B, L) + spec_row_counts_bytes(B, L));
  p.B = B;
  p.L = L;
  p.V = V;
  p.chunks = (int)spec_chunks(V, logits_dtype == BQ_DTYPE_F16 ? 2 : 4);
  const void* fn = logits_dtype == BQ_DTYPE_F16 ? reinterpret_cast<const void*>(&spec_verify_kernel<_Float16>)
                                                : reinterpret_cast<const void*>(&spec_verify_kernel<float>);
  return launch(fn, dim3((unsigned)((int64_t)B * (L + 1) * p.chunks)), dim3(kSpecThreads), 0, stream, &p);
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
      return "a pointer is misaligned (W 4 bytes; x, scales and biases of the decode calls 4 bytes; x and the "
             "workspace of the prefill products 16 bytes; fp16 outputs 2 bytes), or a t5 repack has K not a "
             "multiple of 256";
    case BQ_ERR_FLAGS: return "flags holds bits this entry point does not define";
    case BQ_ERR_HIP: return "the HIP runtime rejected the kernel launch";
    case BQ_ERR_WORKSPACE: return "the workspace is NULL or smaller than bq_spec_verify_workspace reports";
    case BQ_ERR_SCRATCH:
      return "the call needs more scratch than the allocation-free entry point's static array "
             "(BQ_SPEC_NOALLOC_SCRATCH_BYTES) holds";
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

int bq_qmm_workspace(int M, int N, int K, int bits, int group_size, size_t* bytes) {
  if (!bytes) return BQ_ERR_NULL;
  *bytes = 0;
  if (bits != 1 && bits != 2 && bits != BQ_BITS_T5) return BQ_ERR_BITS;
  if (group_size != 64 && group_size != 128) return BQ_ERR_GROUP;
  if (N <= 0 || K <= 0 || K % group_size != 0 || K > (1 << 26)) return BQ_ERR_SHAPE;
  if (M < 1) return BQ_ERR_M;
  if (M > 32) return BQ_OK;
  const QmmSmallChoice c = qmm_small_m_choice(M, N, K, SIZE_MAX);
  if (c.split > 1) *bytes = (size_t)c.split * qmm_part_stride(M, N) * sizeof(float);
  return BQ_OK;
}

int bq_qmm_ws(const void* x, const void* w, const void* scales, const void* biases, void* y, int M, int N,
              int K, int bits, int group_size, void* workspace, size_t workspace_bytes, void* stream) {
  int st = validate(E_UQMM, x, w, scales, biases, y, M, N, K, bits, group_size);
  if (st != BQ_OK) return st;
  if (workspace && !aligned(workspace, 16)) return BQ_ERR_ALIGN;
  return launch_qmm(x, w, scales, biases, y, M, N, K, bits, group_size, stream, workspace, workspace_bytes);
}

int bq_t5_qmm_ws(const void* x, const void* w, const void* scales, const void* biases, void* y, int M,
                 int N, int K, int bits, int group_size, void* workspace, size_t workspace_bytes, void* stream) {
  int st = validate(E_QMM, x, w, scales, biases, y, M, N, K, bits, group_size);
  if (st != BQ_OK) return st;
  if (workspace && !aligned(workspace, 16)) return BQ_ERR_ALIGN;
  return launch_qmm(x, w, scales, biases, y, M, N, K, BQ_BITS_T5, group_size, stream, workspace, workspace_bytes);
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
  // widest stores the output's alignment allows
  const int A = aligned(y, 16) ? 16 : (aligned(y, 4) ? 4 : 2);
  size_t items;
  const void* fn;
  if (bits == BQ_BITS_T5) {
    items = (size_t)N * p.G;  // one thread per group
    fn = group_size == 64 ? pick_dequant_t5<64>(implied, A) : pick_dequant_t5<128>(implied, A);
  } else {
    items = (size_t)N * (K / (32 / bits));  // one thread per word
    fn = bits == 1 ? pick_dequant_words<1>(implied, A) : pick_dequant_words<2>(implied, A);
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
  // fewer, passes of up to five rows are faster.  Measured on MI355X (gs
  // 128, graph launches): 2-bit down (80 tiles) at M = 17 takes 87 us in
  // four passes against 147 us fused; t5 fused at M = 17 takes 31 / 37 /
  // 95 us on q / o / down (96 / 80 / 80 tiles) against 44 / 45 / 102 us in
  // passes, and on k (16 tiles) 31 us against 28 us at M = 17 but 37 us
  // in passes at M = 24.
  const int64_t ntiles = (int64_t)((N + 63) / 64) * ((M + 31) / 32);
  const bool tiles = ntiles >= BQ_QMM_MIN_TILES;
  const bool t5_tiles = ntiles >= BQ_T5_QMM_MIN_TILES || (M >= BQ_T5_QMM_FEW_MIN_M && ntiles >= BQ_T5_QMM_FEW_TILES);
  if (bits == BQ_BITS_T5 && M >= BQ_T5_QMM_MIN_M && t5_tiles) {
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

int bq_linear_ws(const void* x, const void* w, const void* scales, const void* biases, void* y, int M, int N,
                 int K, int bits, int group_size, int flags, void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace) return bq_linear(x, w, scales, biases, y, M, N, K, bits, group_size, flags, stream);
  if ((flags & ~BQ_LINEAR_SYM) != 0) return BQ_ERR_FLAGS;
  const bool t5 = bits == BQ_BITS_T5;
  if (M < (t5 ? BQ_T5_QMM_MIN_M : BQ_QMM_MIN_M))
    return bq_linear(x, w, scales, biases, y, M, N, K, bits, group_size, flags, stream);
  const void* b = (flags & BQ_LINEAR_SYM) ? nullptr : biases;
  if (t5) return bq_t5_qmm_ws(x, w, scales, b, y, M, N, K, bits, group_size, workspace, workspace_bytes, stream);
  if (!b && !(flags & BQ_LINEAR_SYM)) return BQ_ERR_NULL;
  return bq_qmm_ws(x, w, scales, b, y, M, N, K, bits, group_size, workspace, workspace_bytes, stream);
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
  p.groups_per_row = K / group_size;
  p.groups = (int64_t)N * p.groups_per_row;
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
  const int64_t blocks = (p.groups + 255) / 256;
  if (blocks > 0x7FFFFFFF) return BQ_ERR_SHAPE;
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
  int st = spec_validate(logits, logits_dtype, draft, B, L, V, accepted, next_token, target_tokens);
  if (st != BQ_OK) return st;
  if (!workspace || workspace_bytes < spec_workspace_bytes(B, L)) return BQ_ERR_WORKSPACE;
  if (!aligned(workspace, 8)) return BQ_ERR_ALIGN;
  return spec_launch(logits, logits_dtype, draft, B, L, V, accepted, next_token, target_tokens, workspace, stream);
}

int bq_spec_decode_verify_noalloc(const void* logits, int logits_dtype, const int* draft, int B, int L, int V,
                                  int* accepted, int* next_token, int* target_tokens, void* stream) {
  int st = spec_validate(logits, logits_dtype, draft, B, L, V, accepted, next_token, target_tokens);
  if (st != BQ_OK) return st;
  const size_t need = spec_workspace_bytes(B, L);
  if (need > kScratchBytes) return BQ_ERR_SCRATCH;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != BQ_OK) return st;
  // the verify kernel needs its keys and counters zero; the array keeps the
  // last call's contents, so they are cleared first (a kernel, not a
  // memset: graph-capture safe)
  const size_t words = (need + 3) / 4;
  const unsigned blocks = (unsigned)std::min<size_t>((words + 255) / 256, 256);
  size_t nw = words;
  void* args[] = {&ws, &nw};
  if (hipLaunchKernel(reinterpret_cast<const void*>(&zero_fill_kernel), dim3(blocks), dim3(256), args, 0,
                      static_cast<hipStream_t>(stream)) != hipSuccess)
    return BQ_ERR_HIP;
  return spec_launch(logits, logits_dtype, draft, B, L, V, accepted, next_token, target_tokens, ws, stream);
}

}  // extern "C"
