// Speculative-decoding verification in one kernel ("oMLX Bonsai 自定义内核"
// article, section 三: spec_decode_verify fuses comparing the draft tokens,
// counting the accepted length and producing the correction token).
//
// Reading (greedy verification): for sequence b with L draft tokens d[0..L-1]
// and target logits for L+1 positions, t[i] = argmax_v logits[b][i][v]
// (largest value; among equal values the lowest v; -0 equals +0; any NaN
// counts as larger than every number and the first NaN wins), the accepted
// length a = the first i < L with d[i] != t[i], else L, and the next token
// is t[a]: the correction when a draft token was rejected, the bonus token
// when all were accepted.
//
// gfx950 design: the argmax is an HBM-bound scan of B*(L+1)*V logits.  The
// grid splits every logits row into chunks of kSpecChunk values, one
// 256-thread workgroup per chunk, so even one sequence spreads over many
// CUs.  A workgroup reduces its chunk to one 64-bit key (order-preserving
// 16/32-bit key of the value above, complement of the index below) and
// merges it into the row's slot with a 64-bit atomic max.  Then it counts
// itself done on the sequence's counter; the workgroup that completes the
// count reads the L+1 row keys, writes the outputs and clears the slots and
// the counter, so the workspace is zero again for the next call.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bq.h"

namespace bq {

constexpr int kSpecChunk = 8192;   // logits per workgroup
constexpr int kSpecThreads = 256;

struct SpecParams {
  const void* logits;       // [B][L+1][V], fp16 or fp32
  const int* draft;         // [B][L]
  int* accepted;            // [B]
  int* next_token;          // [B]
  int* target;              // [B][L+1] or null
  unsigned long long* keys; // workspace: [B][L+1] row keys, zero between calls
  unsigned int* counters;   // workspace: [B], zero between calls
  int B, L, V, chunks;      // chunks per row
};

// Order-preserving keys: a larger value gets a larger key, -0 and +0 the
// same key, NaN the largest key.
__device__ __forceinline__ uint32_t spec_key(uint16_t h) {
  if ((h & 0x7FFFu) > 0x7C00u) return 0xFFFFu;            // NaN
  if (h == 0x8000u) return 0x8000u;                        // -0 as +0
  return (h & 0x8000u) ? 0x7FFFu - (h & 0x7FFFu) : (0x8000u | h);
}
__device__ __forceinline__ uint32_t spec_key(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0xFFFFFFFFu;  // NaN
  if (u == 0x80000000u) return 0x80000000u;                 // -0 as +0
  return (u & 0x80000000u) ? 0x7FFFFFFFu - (u & 0x7FFFFFFFu) : (0x80000000u | u);
}

__device__ __forceinline__ unsigned long long spec_pack(uint32_t key, int v) {
  return ((unsigned long long)key << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)v);
}

template <typename T>
__global__ __launch_bounds__(kSpecThreads) void spec_verify_kernel(SpecParams p) {
  __shared__ unsigned long long red[kSpecThreads / 64];
  __shared__ int last;
  const int rows = p.L + 1;
  const int wg = (int)blockIdx.x;
  const int chunk = wg % p.chunks;
  const int row = (wg / p.chunks) % rows;
  const int b = wg / (p.chunks * rows);
  const int v0 = chunk * kSpecChunk;
  const int v1 = min(v0 + kSpecChunk, p.V);
  const T* lg = static_cast<const T*>(p.logits) + ((size_t)b * rows + row) * (size_t)p.V;

  // chunk maximum: consecutive threads read consecutive values (a wave
  // instruction reads 64 consecutive values); all of a thread's loads are
  // issued before the first comparison, and a thread keeps its largest key
  // with the first index that has it (its values come in increasing v)
  constexpr int NL = kSpecChunk / kSpecThreads;
  T val[NL];
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    const int v = v0 + j * kSpecThreads + (int)threadIdx.x;
    val[j] = v < v1 ? lg[v] : T(0);
  }
  uint32_t bk = 0;
  int bv = v0;
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    const int v = v0 + j * kSpecThreads + (int)threadIdx.x;
    uint32_t k;
    if constexpr (sizeof(T) == 2) k = spec_key(__builtin_bit_cast(uint16_t, val[j]));
    else k = spec_key(val[j]);
    k = v < v1 ? k : 0u;
    if (k > bk) {
      bk = k;
      bv = v;
    }
  }
  unsigned long long best = bk ? spec_pack(bk, bv) : 0ull;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long c = __shfl_xor(best, o, 64);
    best = c > best ? c : best;
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long m = red[0];
#pragma unroll
    for (int w = 1; w < kSpecThreads / 64; ++w) m = red[w] > m ? red[w] : m;
    // the row's key, then the count: the count is taken only after the max
    // has returned, i.e. has been performed where device-scope atomics are
    // (a device-scope fence here would write back and invalidate this XCD's
    // L2 once per workgroup, which dominated the call's time)
    const unsigned long long old =
        __hip_atomic_fetch_max(&p.keys[(size_t)b * rows + row], m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" ::"v"(old) : "memory");
    const unsigned int done = __hip_atomic_fetch_add(&p.counters[b], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = done == (unsigned int)(rows * p.chunks - 1);
  }
  __syncthreads();
  if (!last) return;
  // the last workgroup of sequence b: every row key is final (each was
  // performed before its count, and the keys are read with device-scope
  // atomic loads).  Its threads take the rows in parallel (one round trip
  // per row, not one per row in sequence): each reads its row's key, writes
  // the target token, notes a draft mismatch, and clears the key.
  __shared__ int tl[BQ_SPEC_MAX_DRAFT + 1];
  __shared__ int first_bad;
  if (threadIdx.x == 0) first_bad = p.L;
  __syncthreads();
  unsigned long long* keys = p.keys + (size_t)b * rows;
  for (int i = (int)threadIdx.x; i < rows; i += kSpecThreads) {
    const unsigned long long k = __hip_atomic_load(&keys[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int t = (int)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull));
    tl[i] = t;
    if (p.target) p.target[(size_t)b * rows + i] = t;
    if (i < p.L && p.draft[(size_t)b * p.L + i] != t) atomicMin(&first_bad, i);
    __hip_atomic_store(&keys[i], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int a = first_bad;
    p.accepted[b] = a;
    p.next_token[b] = tl[a];
    __hip_atomic_store(&p.counters[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace bq
