/*
 * bq.h -- C ABI of the low-bit weight-quantized decode QMV library (gfx950).
 *
 * Source of the method: the web article "oMLX Bonsai 自定义内核: Qwen 系列快速
 * QMV 路径完整解析" (cnnetsun.cn), section 二 (three kernel paths: qmv_fast,
 * qmv_wide with its symmetric variant, the t5 ternary format with its qmv,
 * qmv_wide and fused unpack+matmul qmm) and section 三 (an ABI probe guards
 * the native extension).
 *
 * Shared conventions of every entry point
 * ---------------------------------------
 *   x       fp16 [M][K] row-major activations (device memory).
 *   w       packed weights [N][row_bytes] (device memory), W[n][k] is the
 *           weight from input k to output n:
 *             bits = 1 or 2: uint32 words [N][K*bits/32]; code k of a row is
 *             bits (k*bits)%32 .. +bits-1 of word (k*bits)/32 (LSB first).
 *             bits = BQ_BITS_T5: uint8 [N][(K/gs)*ceil(gs/5)]; each group of
 *             gs weights owns ceil(gs/5) bytes (13 for gs=64, 26 for 128);
 *             code 5j+i of a group is base-3 digit i (least significant
 *             first) of the group's byte j; unused digits are 0; a byte
 *             above 242 is invalid (the result is then unspecified).
 *   scales  fp16 [N][K/gs], one per (output row, group along K).
 *   biases  fp16 [N][K/gs], or NULL where the call says so.  The weight is
 *           w = scale*q + bias (group-wise affine quantization).
 *   y       fp16 [M][N] row-major output, y[m][n] = sum_k x[m][k]*W[n][k],
 *           accumulated in fp32 and rounded to fp16 (nearest even) once.
 *           y is overwritten, never accumulated into.
 *   M, N, K sizes; K must be a positive multiple of group_size; N > 0.
 *   bits    1, 2, or BQ_BITS_T5 for the ternary format.
 *   group_size  64 or 128.
 *   stream  a hipStream_t (NULL = the default stream).  Every call only
 *           enqueues work on it and returns; there is no synchronization.
 *
 * Ownership: all pointers are device pointers owned by the caller.  The
 * library allocates nothing per call and keeps no mutable global state,
 * so calls from several host threads are safe.
 *
 * Errors: each entry point validates every argument before it launches
 * anything and returns BQ_OK (0) or a negative bq_status; bq_strerror()
 * names it.  A failed launch returns BQ_ERR_HIP.  Nothing aborts or throws
 * across this interface.
 *
 * Alignment: w needs 4-byte alignment (uint32 words for bits 1/2; dword
 * loads for t5).  The decode calls (qmv, qmv_wide, qmv_sym, t5_qmv,
 * t5_qmv_wide) read x, scales and biases as dwords and need them 4-byte
 * aligned (qmv_sym ignores the bias pointer).  bq_qmm and bq_t5_qmm stage x
 * with 16-byte loads that write LDS directly and need x 16-byte aligned,
 * scales and biases 2-byte aligned.  y needs 2-byte alignment everywhere
 * (bq_dequant uses 16-byte or dword stores when y allows them).  Fresh
 * allocations from hipMalloc or torch meet all of these.  t5 weights need
 * K to be a multiple of group_size only; rows need not be whole dwords
 * (bq_t5_repack alone needs K to be a multiple of 256).
 */
#ifndef BQ_H
#define BQ_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BQ_ABI_VERSION 10
#define BQ_BITS_T5 0
#define BQ_MAX_WIDE_M 5

typedef enum bq_status {
  BQ_OK = 0,
  BQ_ERR_NULL = -1,       /* a required pointer is NULL */
  BQ_ERR_BITS = -2,       /* bits (or the logits dtype) not valid for this entry point */
  BQ_ERR_GROUP = -3,      /* group_size not 64 or 128 */
  BQ_ERR_SHAPE = -4,      /* N or K not positive, K % group_size != 0, K > 2^26,
                             or N * (packed row bytes) >= 2^30, or
                             N * (K / group_size) >= 2^29 (32-bit offsets), or
                             a decode call with K / group_size > 4092 (a
                             workgroup's scales must fit its LDS) */
  BQ_ERR_M = -5,          /* M outside the range this entry point accepts */
  BQ_ERR_ALIGN = -6,      /* a pointer is misaligned, or a t5 repack with K % 256 != 0 */
  BQ_ERR_HIP = -7,        /* the HIP runtime rejected a launch */
  BQ_ERR_FLAGS = -8,      /* bq_linear: flags holds undefined bits */
  BQ_ERR_WORKSPACE = -9,  /* bq_spec_decode_verify: workspace NULL or too small */
  BQ_ERR_SCRATCH = -10    /* bq_spec_decode_verify_noalloc: the call needs more than
                             BQ_SPEC_NOALLOC_SCRATCH_BYTES of scratch */
} bq_status;

/* bq_linear flags */
#define BQ_LINEAR_SYM 1   /* bias implied (-scale*ratio; t5: -scale), biases never read */
/* t5 calls of bq_linear with M >= BQ_T5_QMM_MIN_M take the fused qmm path
 * when the product has at least BQ_T5_QMM_MIN_TILES tiles of 32 x 64
 * outputs, or from BQ_T5_QMM_FEW_MIN_M rows at least BQ_T5_QMM_FEW_TILES
 * tiles (the small-M t5 product keeps four iterations of loads in flight,
 * which makes it faster than passes of five rows on fewer tiles than the
 * 1/2-bit product) */
#define BQ_T5_QMM_MIN_M 17
#define BQ_T5_QMM_MIN_TILES 64
#define BQ_T5_QMM_FEW_MIN_M 24
#define BQ_T5_QMM_FEW_TILES 16
/* 1/2-bit calls of bq_linear take bq_qmm when M >= BQ_QMM_MIN_M and the
 * product has at least BQ_QMM_MIN_TILES tiles of 32 x 64 outputs
 * (ceil(N/64)*ceil(M/32)), enough to occupy half the CUs */
#define BQ_QMM_MIN_M 17
#define BQ_QMM_MIN_TILES 128

typedef enum bq_route {
  BQ_ROUTE_QMV_WIDE = 1,  /* bits 1/2, stored bias: bq_qmv_wide per pass of <= 5 rows */
  BQ_ROUTE_QMV_SYM = 2,   /* bits 1/2, implied bias: bq_qmv_sym per pass of <= 5 rows */
  BQ_ROUTE_T5_WIDE = 3,   /* t5: bq_t5_qmv_wide per pass of <= 5 rows */
  BQ_ROUTE_T5_QMM = 4,    /* t5, M >= BQ_T5_QMM_MIN_M and tiles as below: one bq_t5_qmm */
  BQ_ROUTE_QMM = 5        /* bits 1/2, M and tiles as above: one bq_qmm */
} bq_route;

/* ABI version of the loaded library; callers must refuse to use a library
 * whose version differs from BQ_ABI_VERSION (the probe of section 三, but a
 * mismatch is an error here, never a silent fallback). */
int bq_abi_version(void);

/* Static, NUL-terminated description of a bq_status value. */
const char* bq_strerror(int status);

/* qmv -- section 二 path 1 (qmv_fast): bits 1 or 2, biases required, any
 * M >= 1.  Each activation row is an independent pass over W (W is read M
 * times); row m gives the same bits as a call with M = 1 on that row. */
int bq_qmv(const void* x, const void* w, const void* scales, const void* biases, void* y,
           int M, int N, int K, int bits, int group_size, void* stream);

/* qmv_wide -- section 二 path 2: bits 1 or 2, biases required,
 * 1 <= M <= 5; one read of W serves all M rows.  Row m gives the same
 * bits as bq_qmv on that row alone. */
int bq_qmv_wide(const void* x, const void* w, const void* scales, const void* biases, void* y,
                int M, int N, int K, int bits, int group_size, void* stream);

/* qmv_sym -- section 二 path 2, symmetric variant: bits 1 or 2,
 * 1 <= M <= 5; the bias is implied as -scale*(2^bits-1)/2 and the biases
 * argument is ignored and never read (it may be NULL).  Bit-identical to
 * bq_qmv_wide with an explicit fp16 bias equal to -scale*(2^bits-1)/2
 * whenever that value is exact in fp16. */
int bq_qmv_sym(const void* x, const void* w, const void* scales, const void* biases, void* y,
               int M, int N, int K, int bits, int group_size, void* stream);

/* t5_qmv -- section 二 path 3: bits must be BQ_BITS_T5, any M >= 1 (each
 * row an independent pass over W).  biases == NULL implies bias = -scale
 * (weights in {-s, 0, +s}) and no bias is read; non-NULL biases are read. */
int bq_t5_qmv(const void* x, const void* w, const void* scales, const void* biases, void* y,
              int M, int N, int K, int bits, int group_size, void* stream);

/* t5_qmv_wide -- section 二 path 3: as bq_t5_qmv with 1 <= M <= 5 and one
 * read of W for all rows. */
int bq_t5_qmv_wide(const void* x, const void* w, const void* scales, const void* biases, void* y,
                   int M, int N, int K, int bits, int group_size, void* stream);

/* t5_qmm -- section 二 path 3 (prefill, M > 16 intended; any M >= 1):
 * fused t5 unpack + matrix-core (MFMA, fp16 x fp16 -> fp32) product.  Each
 * t5 byte is unpacked once per weight tile; biases as in bq_t5_qmv. */
int bq_t5_qmm(const void* x, const void* w, const void* scales, const void* biases, void* y,
              int M, int N, int K, int bits, int group_size, void* stream);

/* qmm -- section 二 path 1 (1-bit prefill dequantizes to float16 and then
 * multiplies) and path 3 (the fused unpack + matrix multiply of t5): the
 * fused product for the uint32 formats, bits 1 or 2, any M >= 1 (prefill,
 * M > 16 intended).  Each code word is unpacked once per weight tile;
 * fp16 x fp16 -> fp32 on the matrix cores.  biases == NULL implies
 * -scale*(2^bits-1)/2 and no bias is read; non-NULL biases are read.  Each
 * weight enters the product as fp16_rne(scale*q + bias), as bq_dequant
 * writes it. */
int bq_qmm(const void* x, const void* w, const void* scales, const void* biases, void* y,
           int M, int N, int K, int bits, int group_size, void* stream);

/* K-split prefill -- section 二 path 3 (and path 1 for bits 1/2): the
 * products of bq_t5_qmm and bq_qmm with a caller-owned workspace.  At most
 * 32 rows give few output tiles (a 5120-column product has 80) for the
 * 256 CUs, so the K iterations of each tile are shared by up to 8
 * workgroups: each stores its fp32 partial tile to the workspace and a
 * second kernel adds the partials in a fixed order (same result every
 * call) and rounds once to fp16.  The sum order differs from the unsplit
 * product, so results may differ from bq_t5_qmm / bq_qmm in the last
 * bits (both are within the decode tolerance of the exact product).
 *
 * bq_qmm_workspace: *bytes := the workspace the split the library would
 * choose for (M, N, K, bits, group_size) needs; 0 when it would not split
 * (M > 32, or enough tiles).  bits 1, 2 or BQ_BITS_T5.  Host-only.
 *
 * bq_t5_qmm_ws / bq_qmm_ws: arguments as bq_t5_qmm / bq_qmm, plus
 * workspace (device memory, 16-byte aligned, or NULL) of workspace_bytes
 * bytes.  The split is taken only as far as the workspace holds its
 * partials; NULL or too small a workspace gives the unsplit product (no
 * error).  The workspace needs no initial contents; concurrent calls on
 * different streams must not share one.  BQ_ERR_ALIGN for a misaligned
 * workspace, else the errors of bq_t5_qmm / bq_qmm. */
int bq_qmm_workspace(int M, int N, int K, int bits, int group_size, size_t* bytes);
int bq_t5_qmm_ws(const void* x, const void* w, const void* scales, const void* biases, void* y,
                 int M, int N, int K, int bits, int group_size, void* workspace, size_t workspace_bytes,
                 void* stream);
int bq_qmm_ws(const void* x, const void* w, const void* scales, const void* biases, void* y,
              int M, int N, int K, int bits, int group_size, void* workspace, size_t workspace_bytes,
              void* stream);

/* dequant -- section 二 path 1 (1-bit prefill dequantizes to float16
 * before a matmul): y := fp16 [N][K], y[n][k] = fp16_rne(scale*q + bias)
 * computed exactly and rounded once.  x is ignored (may be NULL) and so is
 * M.  bits 1, 2 or BQ_BITS_T5.  biases == NULL implies -scale*(2^bits-1)/2
 * for bits 1/2 and -scale for t5. */
int bq_dequant(const void* x, const void* w, const void* scales, const void* biases, void* y,
               int M, int N, int K, int bits, int group_size, void* stream);

/* linear -- the routing of section 二 (the kernels are chosen by bits and
 * by the number of activation rows M) and section 三 (1/2-bit affine layers
 * in decode take the fast kernels): y = x * W^T for any M >= 1.
 *   bits 1/2: one bq_qmm when M >= BQ_QMM_MIN_M and the product has
 *             BQ_QMM_MIN_TILES tiles, else passes of up to 5 rows through
 *             bq_qmv_wide, or bq_qmv_sym when flags has BQ_LINEAR_SYM (each
 *             pass reads W once; M > 5 reads it ceil(M/5) times);
 *   t5:       bq_t5_qmm when M >= BQ_T5_QMM_MIN_M (the article's prefill
 *             rule, M > 16) and the product has BQ_T5_QMM_MIN_TILES tiles
 *             (or, from BQ_T5_QMM_FEW_MIN_M rows, BQ_T5_QMM_FEW_TILES
 *             tiles), else passes of up to 5 rows through bq_t5_qmv_wide.
 * Arguments as for the entry point a pass goes to; with BQ_LINEAR_SYM the
 * biases argument is ignored (may be NULL) and the bias is implied.
 * Results are those of the entry points the passes take; each pass is
 * validated before it launches, so an invalid argument fails before
 * anything runs.  Undefined flag bits: BQ_ERR_FLAGS. */
int bq_linear(const void* x, const void* w, const void* scales, const void* biases, void* y,
              int M, int N, int K, int bits, int group_size, int flags, void* stream);

/* linear with a workspace -- the routing of bq_linear, where a
 * workspace lets the fused prefill product split K (bq_t5_qmm_ws /
 * bq_qmm_ws): from BQ_T5_QMM_MIN_M (t5) or BQ_QMM_MIN_M (bits 1/2) rows
 * every product takes the fused route whatever its tile count, with
 * the workspace; fewer rows take the passes of bq_linear.  workspace ==
 * NULL: exactly bq_linear.  The fused route needs bq_qmm_workspace bytes
 * for its full split (less: a smaller split or none, see bq_qmm_ws);
 * workspace 16-byte aligned.  Arguments and errors otherwise as
 * bq_linear. */
int bq_linear_ws(const void* x, const void* w, const void* scales, const void* biases, void* y,
                 int M, int N, int K, int bits, int group_size, int flags, void* workspace,
                 size_t workspace_bytes, void* stream);

/* The route bq_linear takes for (M, N, bits, flags), a bq_route value, and
 * the number of kernel passes in *passes (may be NULL); BQ_ERR_M,
 * BQ_ERR_SHAPE (N < 1) or BQ_ERR_BITS for invalid arguments.  Host-only:
 * launches nothing. */
int bq_linear_route(int M, int N, int bits, int flags, int* passes);

/* sym detection -- section 二 path 2 (the symmetric variant applies when
 * bias = -scale * ratio holds): writes 1 to the device int *flag when every
 * stored fp16 bias equals -scale * ratio exactly (ratio (2^bits-1)/2, t5: 1),
 * else 0, asynchronously on stream.  scales and biases: fp16 [N][K/gs],
 * 2-byte aligned; flag: a caller-owned device int, 4-byte aligned.  A NaN
 * anywhere gives 0.  When it is 1, bq_qmv_sym (bq_linear with
 * BQ_LINEAR_SYM) gives the same bits as the affine call and skips the
 * bias read. */
int bq_sym_check(const void* scales, const void* biases, int N, int K, int bits, int group_size, int* flag,
                 void* stream);

/* t5 repack -- section 二, the t5 format (existing 1/2-bit weights are
 * repacked into t5 bytes): w holds uint32 code words [N][K*bits/32] (bits 1
 * or 2, the layout above); w_t5 receives t5 bytes [N][(K/gs)*ceil(gs/5)]
 * (the layout above).  Scales and biases stay as they are: s*q + b is the
 * same weight in both formats.  Writes 1 to the device int *flag when every
 * code is 0, 1 or 2 (the repack is exact), else 0; a code 3 is written as
 * digit 2.  K must be a multiple of 256 (whole dwords per t5 row); w, w_t5
 * and flag need 4-byte alignment.  Asynchronous on stream. */
int bq_t5_repack(const void* w, void* w_t5, int N, int K, int bits, int group_size, int* flag, void* stream);

/* speculative-decoding verification -- section 三 (spec_decode_verify:
 * comparing the draft tokens, counting the accepted length and producing the
 * correction token, fused into one kernel).  For each sequence b:
 *   t[i] = argmax over v of logits[b][i][v], i = 0..L (the largest value;
 *          equal values: the lowest v; -0 equals +0; a NaN is larger than
 *          every number and the first NaN wins);
 *   accepted[b] = the first i < L with draft[b][i] != t[i], else L;
 *   next_token[b] = t[accepted[b]] (the correction token, or the bonus token
 *          when every draft token is accepted);
 *   target_tokens[b][i] = t[i] when target_tokens is not NULL.
 * logits: [B][L+1][V] row-major, fp16 (BQ_DTYPE_F16) or fp32 (BQ_DTYPE_F32),
 * aligned to its element size; draft: int32 [B][L] (may be NULL when L = 0);
 * accepted, next_token: int32 [B]; target_tokens: int32 [B][L+1] or NULL;
 * all device memory owned by the caller, int arrays 4-byte aligned.
 * 1 <= B, 0 <= L <= BQ_SPEC_MAX_DRAFT, 1 <= V.
 * workspace: device memory of at least bq_spec_verify_workspace() bytes,
 * 8-byte aligned, all zero before its first use (e.g. hipMemset once);
 * every call leaves it zero again.  Calls that overlap in time on one
 * workspace race; give concurrent streams their own.  The library
 * allocates nothing.  Asynchronous on stream; one kernel launch. */
#define BQ_DTYPE_F16 1
#define BQ_DTYPE_F32 2
#define BQ_SPEC_MAX_DRAFT 1024

/* Workspace bytes bq_spec_decode_verify needs for B sequences of L draft
 * tokens (into *bytes).  Host-only. */
int bq_spec_verify_workspace(int B, int L, int V, size_t* bytes);

int bq_spec_decode_verify(const void* logits, int logits_dtype, const int* draft, int B, int L, int V,
                          int* accepted, int* next_token, int* target_tokens, void* workspace,
                          size_t workspace_bytes, void* stream);

/* bq_spec_decode_verify for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments and results without a workspace.  Its
 * scratch is a static device array of BQ_SPEC_NOALLOC_SCRATCH_BYTES inside
 * the library, one per GPU, held until the process ends; the call clears
 * what it uses (a kernel, no memset), then runs the verify kernel: two
 * launches, no allocation of any kind.  A call whose scratch,
 * bq_spec_verify_workspace(B, L), exceeds the array returns BQ_ERR_SCRATCH
 * before launching anything (e.g. B = 256 sequences of L = 15 draft tokens
 * need about 1.1 MB: 256 bytes per verified position, 128 per sequence).  Every call on a GPU shares that GPU's array: calls
 * that overlap in time on one GPU (several streams, several host threads)
 * race and give wrong results; serialize them.  Other errors as
 * bq_spec_decode_verify; BQ_ERR_HIP if the array's address cannot be
 * taken. */
#define BQ_SPEC_NOALLOC_SCRATCH_BYTES (2 * 1024 * 1024)
int bq_spec_decode_verify_noalloc(const void* logits, int logits_dtype, const int* draft, int B, int L, int V,
                                  int* accepted, int* next_token, int* target_tokens, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BQ_H */
