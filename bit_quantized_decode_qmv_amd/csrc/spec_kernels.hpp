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
// grid splits every logits row into chunks of kSpecChunkBytes, one
// 256-thread workgroup each, so even one sequence spreads over many CUs.  A
// thread reads its share of the chunk with 16-byte loads, all issued before
// the first comparison; the loads are aligned to 16 bytes in memory, so a
// row that does not start on a 16-byte boundary has its first and last
// blocks partly outside it (those values are replaced by the most negative
// finite value, the fill; an aligned 16-byte block holding one byte of the
// row lies in the row's pages).  A workgroup reduces its chunk to one
// 64-bit key (order-preserving 16/32-bit key of the value above, complement
// of the index below): with the hardware max when that decides alone (a
// finite normal maximum other than the fill), else by comparing every
// value's key.  It merges the key into the row's slot with a 64-bit atomic
// max.  Then it counts itself done on the
// row's counter, and the workgroup that completes a row counts the row done
// on the sequence's counter; the workgroup that completes that count reads
// the L+1 row keys, writes the outputs and clears the slots and counters, so
// the workspace is zero again for the next call.  Every key slot and counter
// has a line of its own: atomics on one address, or on one line, are
// performed one after another.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bq.h"

namespace bq {

constexpr int kSpecThreads = 256;
constexpr int kSpecLoads = 4;                                  // 16-byte loads per thread
constexpr int kSpecChunkBytes = kSpecThreads * kSpecLoads * 16;  // logits bytes per workgroup
constexpr int kSpecKeyStride = 16;                             // 8-byte words between row keys
constexpr int kSpecCountStride = 32;                           // 4-byte words between counters

// workspace: [B][L+1] row keys, [B][L+1] row counters, [B] sequence
// counters, each on a 128-byte line
inline size_t spec_keys_bytes(int B, int L) { return (size_t)B * (L + 1) * kSpecKeyStride * 8; }
inline size_t spec_row_counts_bytes(int B, int L) { return (size_t)B * (L + 1) * kSpecCountStride * 4; }
inline size_t spec_workspace_bytes(int B, int L) {
  return spec_keys_bytes(B, L) + spec_row_counts_bytes(B, L) + (size_t)B * kSpecCountStride * 4;
}
// chunks per row: enough for a row of V values starting anywhere in a
// 16-byte block
inline int64_t spec_chunks(int V, int esz) { return ((int64_t)V * esz + 15 + kSpecChunkBytes - 1) / kSpecChunkBytes; }

struct SpecParams {
  const void* logits;       // [B][L+1][V], fp16 or fp32
  const int* draft;         // [B][L]
  int* accepted;            // [B]
  int* next_token;          // [B]
  int* target;              // [B][L+1] or null
  unsigned long long* keys; // workspace: row keys, zero between calls
  unsigned int* row_counts; // workspace: chunks done per row, zero between calls
  unsigned int* counters;   // workspace: rows done per sequence, zero between calls
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

// Bit patterns per logits type: the fill that stands for values outside
// the row (the most negative finite value), the smallest normal magnitude,
// the magnitude mask, and value_of: the value bits a key other than the NaN
// key stands for (spec_key inverted; zero comes back as +0).
template <typename T> struct SpecBits;
template <> struct SpecBits<_Float16> {
  static constexpr uint32_t kFill = 0xFBFFu, kMinNormal = 0x0400u, kAbs = 0x7FFFu;
  __device__ static uint32_t value_of(uint32_t k) { return k >= 0x8000u ? (k & 0x7FFFu) : (0x8000u | (0x7FFFu - k)); }
};
template <> struct SpecBits<float> {
  static constexpr uint32_t kFill = 0xFF7FFFFFu, kMinNormal = 0x00800000u, kAbs = 0x7FFFFFFFu;
  __device__ static uint32_t value_of(uint32_t k) {
    return k >= 0x80000000u ? (k & 0x7FFFFFFFu) : (0x80000000u | (0x7FFFFFFFu - k));
  }
};

template <typename T>
__device__ __forceinline__ uint32_t spec_elem(const uint4& r, int e) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
  if constexpr (sizeof(T) == 2) return (w[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
  else return w[e];
}

template <typename T>
__device__ __forceinline__ uint32_t spec_key_bits(uint32_t bits) {
  if constexpr (sizeof(T) == 2) return spec_key((uint16_t)bits);
  else return spec_key(__builtin_bit_cast(float, bits));
}

template <typename T>
__global__ __launch_bounds__(kSpecThreads) void spec_verify_kernel(SpecParams p) {
  using Bits = SpecBits<T>;
  constexpr int EPV = 16 / (int)sizeof(T);  // values per 16-byte block
  __shared__ unsigned long long red[kSpecThreads / 64];
  __shared__ uint32_t red32[kSpecThreads / 64];
  __shared__ int last;
  const int rows = p.L + 1;
  const int wg = (int)blockIdx.x;
  const int chunk = wg % p.chunks;
  const int row = (wg / p.chunks) % rows;
  const int b = wg / (p.chunks * rows);
  const char* rp = static_cast<const char*>(p.logits) + ((size_t)b * rows + row) * (size_t)p.V * sizeof(T);
  // the row in aligned 16-byte blocks: block q holds values q*EPV - lead ..
  const int lead = (int)(((uintptr_t)rp & 15) / sizeof(T));
  const uint4* blk = reinterpret_cast<const uint4*>(rp - lead * (int)sizeof(T));
  const int nblk = (int)(((int64_t)lead + p.V + EPV - 1) / EPV);
  const int q0 = chunk * (kSpecThreads * kSpecLoads) + (int)threadIdx.x;

  // a wave instruction reads 1 KiB of consecutive blocks; all of a
  // thread's loads are issued before the first comparison
  uint4 raw[kSpecLoads];
#pragma unroll
  for (int j = 0; j < kSpecLoads; ++j) {
    const int q = q0 + j * kSpecThreads;
    raw[j] = q < nblk ? blk[q] : make_uint4(0, 0, 0, 0);
  }
  // values outside the row (the first and last blocks of an unaligned row,
  // blocks past its end) become the fill
#pragma unroll
  for (int j = 0; j < kSpecLoads; ++j) {
    const int vb = (q0 + j * kSpecThreads) * EPV - lead;
    if (vb < 0 || vb + EPV > p.V) {
      uint32_t w[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        if (vb + e >= 0 && vb + e < p.V) continue;
        if constexpr (sizeof(T) == 2) {
          const int sh = (e & 1) * 16;
          w[e >> 1] = (w[e >> 1] & ~(0xFFFFu << sh)) | (Bits::kFill << sh);
        } else {
          w[e] = Bits::kFill;
        }
      }
      raw[j] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }

  // Fast path: the chunk maximum with the hardware max (packed for fp16)
  // and a flag for NaN or infinity (x*0 is NaN only for them).  It decides
  // alone when the maximum is a finite normal number other than the fill:
  // then equal values have equal bits, and only threads holding the maximum
  // look for its first index.  Otherwise (NaN, infinity, a zero or subnormal
  // maximum, the fill) every value's order key is compared.
  uint32_t tk;
  if constexpr (sizeof(T) == 2) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    h2 mx = __builtin_bit_cast(h2, (Bits::kFill << 16) | Bits::kFill), z = {0, 0};
#pragma unroll
    for (int j = 0; j < kSpecLoads; ++j) {
      const uint32_t w[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const h2 x = __builtin_bit_cast(h2, w[d]);
        mx = __builtin_elementwise_max(mx, x);
        z = __builtin_elementwise_fma(x, h2{0, 0}, z);
      }
    }
    const _Float16 m = mx.x > mx.y ? mx.x : mx.y;
    const bool bad = z.x != z.x || z.y != z.y;
    tk = bad ? 0xFFFFFFFFu : spec_key(__builtin_bit_cast(uint16_t, m));
  } else {
    float mx = __builtin_bit_cast(float, Bits::kFill), z = 0.f;
#pragma unroll
    for (int j = 0; j < kSpecLoads; ++j) {
      const uint32_t w[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float x = __builtin_bit_cast(float, w[d]);
        mx = __builtin_fmaxf(mx, x);
        z = __builtin_fmaf(x, 0.f, z);
      }
    }
    tk = z != z ? 0xFFFFFFFFu : spec_key(mx);
  }
  uint32_t K = tk;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t c = __shfl_xor(K, o, 64);
    K = c > K ? c : K;
  }
  if ((threadIdx.x & 63) == 0) red32[threadIdx.x >> 6] = K;
  __syncthreads();
  K = red32[0];
#pragma unroll
  for (int w = 1; w < kSpecThreads / 64; ++w) K = red32[w] > K ? red32[w] : K;
  // a NaN/infinity flag has the key of every NaN; no finite value has it
  const uint32_t mbits = Bits::value_of(K);
  const bool fast = K != 0xFFFFFFFFu && (mbits & Bits::kAbs) >= Bits::kMinNormal && mbits != Bits::kFill;

  unsigned long long best = 0;
  if (fast) {
    if (tk == K) {
      // a thread's values come in increasing v: scanning backwards, the
      // last match is the first index (fills never match: they differ
      // from the maximum)
      int bv = 0;
#pragma unroll
      for (int j = kSpecLoads - 1; j >= 0; --j) {
#pragma unroll
        for (int e = EPV - 1; e >= 0; --e) {
          if (spec_elem<T>(raw[j], e) == mbits) bv = (q0 + j * kSpecThreads) * EPV + e - lead;
        }
      }
      best = spec_pack(K, bv);
    }
  } else {
    // every value's order key; a thread keeps its largest key with the
    // first index that has it
    uint32_t bk = 0;
    int bv = 0;
#pragma unroll
    for (int j = 0; j < kSpecLoads; ++j) {
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const int v = (q0 + j * kSpecThreads) * EPV + e - lead;
        uint32_t k = spec_key_bits<T>(spec_elem<T>(raw[j], e));
        k = (v >= 0 && v < p.V) ? k : 0u;
        if (k > bk) {
          bk = k;
          bv = v;
        }
      }
    }
    best = bk ? spec_pack(bk, bv) : 0ull;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long c = __shfl_xor(best, o, 64);
    best = c > best ? c : best;
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = best;
  __syncthreads();
  unsigned long long* keys = p.keys + (size_t)b * rows * kSpecKeyStride;
  unsigned int* row_counts = p.row_counts + (size_t)b * rows * kSpecCountStride;
  unsigned int* counter = p.counters + (size_t)b * kSpecCountStride;
  if (threadIdx.x == 0) {
    unsigned long long m = red[0];
#pragma unroll
    for (int w = 1; w < kSpecThreads / 64; ++w) m = red[w] > m ? red[w] : m;
    // the row's key, then the row's count, then (by the row's last
    // chunk) the sequence's count: each is taken only after the one before
    // has returned, i.e. has been performed where device-scope atomics are
    // (a device-scope fence here would write back and invalidate this XCD's
    // L2 once per workgroup, which dominated the call's time).  Counting in
    // two levels keeps the atomics on any one line to a row's chunks or a
    // sequence's rows.
    const unsigned long long old =
        __hip_atomic_fetch_max(&keys[(size_t)row * kSpecKeyStride], m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" ::"v"(old) : "memory");
    const unsigned int c = __hip_atomic_fetch_add(&row_counts[(size_t)row * kSpecCountStride], 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
    bool l = false;
    if (c == (unsigned int)(p.chunks - 1))
      l = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (unsigned int)(rows - 1);
    last = l;
  }
  __syncthreads();
  if (!last) return;
  // the last workgroup of sequence b: every row key is final (each was
  // performed before its counts, and the keys are read with device-scope
  // atomic loads).  Its threads take the rows in parallel (one round trip
  // per row, not one per row in sequence): each reads its row's key, writes
  // the target token, notes a draft mismatch, and clears the key and the
  // row's count.
  __shared__ int tl[BQ_SPEC_MAX_DRAFT + 1];
  __shared__ int first_bad;
  if (threadIdx.x == 0) first_bad = p.L;
  __syncthreads();
  for (int i = (int)threadIdx.x; i < rows; i += kSpecThreads) {
    unsigned long long* slot = &keys[(size_t)i * kSpecKeyStride];
    const unsigned long long k = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int t = (int)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull));
    tl[i] = t;
    if (p.target) p.target[(size_t)b * rows + i] = t;
    if (i < p.L && p.draft[(size_t)b * p.L + i] != t) atomicMin(&first_bad, i);
    __hip_atomic_store(slot, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&row_counts[(size_t)i * kSpecCountStride], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int a = first_bad;
    p.accepted[b] = a;
    p.next_token[b] = tl[a];
    __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace bq
