// Top-K selection per row: the producer of the teacher cache (the page
// "Making Knowledge Distillation Cheap Enough to Run at Scale", section "Two
// systems changes": the K most likely tokens per position are computed once
// and cached).  For every row of X[T,V] (bf16): the ids of its K largest
// values in descending order, equal values by ascending id, and the values.
//
// One 512-thread workgroup per row, values compared as 16-bit
// order-preserving keys:
//   1. one pass over the row: each thread keeps the two largest keys of its
//      even-indexed and of its odd-indexed elements, both pairs in the two
//      16-bit halves of two registers (packed 16-bit min / max, about four
//      ALU operations per element), and the vector where each half's largest
//      key first appeared; theta, the K-th largest of those 2048
//      keys, is a lower bound of the row's K-th largest (K distinct elements
//      reach it), found bit by bit;
//   2. every (key, id) with key >= theta goes to LDS: a thread's best key
//      per half (its position found again in the noted vector) is all it
//      holds at or above theta unless its second key reaches theta too; only such
//      threads' shares of the row (one in 512 vectors each) are scanned
//      again, one share per wave with a vector per lane (for ordinary rows a
//      few shares);
//   3. the order is descending key, then ascending id: up to 512 candidates
//      each count the candidates ahead of them and the first K go straight to
//      their places; larger sets are sorted in LDS (bitonic) first.
// The pass ranks -0 just below +0 (raw keys); a theta at either zero is
// lowered to the -0 key, so that every zero is a candidate, and the
// candidates carry keys on which -0 equals +0.
// Rows where more than kTopkCand keys reach theta (e.g. long runs of equal
// values) take an exact slow path: the K-th largest key and the cut among
// its ties are found bit by bit with a pass over the row per bit, then
// exactly K entries are collected.
#pragma once
#include "kd_common.hpp"

namespace kd {

constexpr int kTopkThreads = 512;
constexpr int kTopkMaxK = 1024;
constexpr int kTopkCand = 4096;

// order-preserving 16-bit key of a bf16 bit pattern (-0 taken as +0)
__device__ __forceinline__ uint32_t bf16_key(uint32_t b) {
  b = (b == 0x8000u) ? 0u : b;
  return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u);
}
// the raw order-preserving keys of a packed bf16 pair, both halves at once
// (x ^ 0x8000 for a clear sign bit, ~x for a set one; -0 sits just below +0)
__device__ __forceinline__ uint32_t raw_key2(uint32_t x) {
  return x ^ (((x >> 15) & 0x00010001u) * 0x7FFFu + 0x80008000u);
}
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t,
                            __builtin_elementwise_max(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b)));
}
__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t,
                            __builtin_elementwise_min(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b)));
}
__device__ __forceinline__ float key_bf16_value(uint32_t k) {
  const uint32_t b = (k & 0x8000u) ? (k & 0x7FFFu) : (~k & 0xFFFFu);
  return __uint_as_float(b << 16);
}

struct TopkArgs {
  const uint16_t* X;  // [T, V] bf16, V % 8 == 0
  int32_t* idx;       // [T, K]
  float* val;         // [T, K]
  int64_t V;
  int K;
  int id_bits;        // bits of the largest id (V - 1)
};

// workgroup-wide sum of one int per thread; red: kTopkThreads / 64 ints of
// LDS, alternated by the caller between consecutive calls so that one
// barrier per call suffices
__device__ __forceinline__ int block_count(int v, int* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  int s = 0;
#pragma unroll
  for (int q = 0; q < kTopkThreads / 64; ++q) s += red[q];
  return s;
}

// the 8 keys of vector i of the row (a streaming read: nontemporal)
__device__ __forceinline__ void load_keys(const uint16_t* row, int64_t i, uint32_t (&k)[8]) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row) + i);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    k[2 * q] = bf16_key(v[q] & 0xFFFFu);
    k[2 * q + 1] = bf16_key(v[q] >> 16);
  }
}

// Sorts n entries (n a power of two, <= capacity) of (key, id) in LDS:
// larger key first, then smaller id.
__device__ __forceinline__ void lds_sort(uint32_t* key, int32_t* id, int n) {
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < n; i += kTopkThreads) {
        const int j = i ^ stride;
        if (j > i) {
          const uint32_t ki = key[i], kj = key[j];
          const int32_t ii = id[i], ij = id[j];
          const bool j_first = kj > ki || (kj == ki && ij < ii);
          if ((i & size) == 0 ? j_first : !j_first) {
            key[i] = kj;
            key[j] = ki;
            id[i] = ij;
            id[j] = ii;
          }
        }
      }
      __syncthreads();
    }
  }
}

__global__ void __launch_bounds__(kTopkThreads) k_topk(TopkArgs a) {
  __shared__ uint32_t ck[kTopkCand];
  __shared__ int32_t ci[kTopkCand];
  __shared__ int red[2][kTopkThreads / 64];
  __shared__ int16_t shares[kTopkThreads];
  __shared__ int ncand, nshares;
  const int tid = threadIdx.x;
  const int64_t t = blockIdx.x;
  const int64_t V = a.V, nvec = V >> 3;
  const int K = a.K;
  const uint16_t* row = a.X + t * V;
  int rb = 0;
  // 1. per half (even / odd elements): m1 = largest raw key, m2 = second
  uint32_t m1 = 0, m2 = 0;  // key 0 (the pattern 0xFFFF, a NaN) is the floor
  // vector of the thread's share (its n-th: row vector tid + 512 n) where
  // each half's m1 was first seen; the word inside it is found again later
  int p_lo = 0, p_hi = 0;
  constexpr int kAhead = 4;  // vectors in flight per thread
  int pos = 0;
  auto fold = [&](const u32x4 (&v)[kAhead]) {
#pragma unroll
    for (int u = 0; u < kAhead; ++u, ++pos) {
      const uint32_t before = m1;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t k = raw_key2(v[u][q]);
        const uint32_t lo = pk_min_u16(k, m1);
        m1 = pk_max_u16(k, m1);
        m2 = pk_max_u16(lo, m2);
      }
      const uint32_t ch = m1 ^ before;  // a half changes only for a strictly larger key
      p_lo = (ch & 0xFFFFu) ? pos : p_lo;
      p_hi = (ch >> 16) ? pos : p_hi;
    }
  };
  const u32x4* rv = reinterpret_cast<const u32x4*>(row);
  int64_t i0 = tid;
  // whole groups of kAhead vectors: no bounds tests
  for (; i0 + (int64_t)(kAhead - 1) * kTopkThreads < nvec; i0 += (int64_t)kAhead * kTopkThreads) {
    u32x4 v[kAhead];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) v[u] = __builtin_nontemporal_load(rv + i0 + (int64_t)u * kTopkThreads);
    fold(v);
  }
  // the last, partial group: past the row the floor pattern, which changes no kept key
  if (i0 < nvec) {
    u32x4 v[kAhead];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      const int64_t i = i0 + (int64_t)u * kTopkThreads;
      v[u] = i < nvec ? __builtin_nontemporal_load(rv + i) : u32x4{~0u, ~0u, ~0u, ~0u};
    }
    fold(v);
  }
  if (tid == 0) {
    ncand = 0;
    nshares = 0;
  }
  uint32_t theta = 0;
  for (int b = 15; b >= 0; --b) {
    const uint32_t cand = theta | (1u << b);
    const int n = ((m1 & 0xFFFFu) >= cand) + ((m1 >> 16) >= cand) + ((m2 & 0xFFFFu) >= cand) + ((m2 >> 16) >= cand);
    if (block_count(n, red[rb]) >= K) theta = cand;
    rb ^= 1;
  }
  // the elements behind the 2048 kept keys are distinct, so at least K keys
  // of the row are >= theta; at a zero theta both zeros become candidates
  if (theta == 0x7FFFu || theta == 0x8000u) theta = 0x7FFFu;
  // 2. candidates: every element with key >= theta.  A half whose second key
  // is below theta holds at most its best element there (known with its
  // position); a thread with a second key >= theta may have dropped some, and
  // its share is scanned again
  if ((m2 & 0xFFFFu) >= theta || (m2 >> 16) >= theta) {
    shares[atomicAdd(&nshares, 1)] = (int16_t)tid;
  } else {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const uint32_t rk = hf ? (m1 >> 16) : (m1 & 0xFFFFu);
      if (rk >= theta) {
        // the vector where the key first appeared: its first word whose half
        // holds the key (earlier words of the vector hold smaller keys)
        const int64_t gi = (int64_t)tid + (int64_t)kTopkThreads * (hf ? p_hi : p_lo);
        const u32x4 v = rv[gi];
        int q = 3;
#pragma unroll
        for (int qq = 2; qq >= 0; --qq) {
          const uint32_t k = raw_key2(v[qq]);
          if ((hf ? (k >> 16) : (k & 0xFFFFu)) == rk) q = qq;
        }
        const int p = atomicAdd(&ncand, 1);
        if (p < kTopkCand) {
          ck[p] = rk == 0x7FFFu ? 0x8000u : rk;  // -0 as +0
          ci[p] = (int32_t)(8 * gi + 2 * q + hf);
        }
      }
    }
  }
  __syncthreads();
  {
    const int lane = tid & 63, nsh = nshares;
    for (int sh = tid >> 6; sh < nsh; sh += kTopkThreads / 64) {
      const int64_t r = shares[sh];
      for (int64_t i = r + (int64_t)kTopkThreads * lane; i < nvec; i += (int64_t)kTopkThreads * 64) {
        uint32_t k[8];
        load_keys(row, i, k);  // keys with -0 == +0: the same test against theta
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (k[q] >= theta) {
            const int p = atomicAdd(&ncand, 1);
            if (p < kTopkCand) {
              ck[p] = k[q];
              ci[p] = (int32_t)(8 * i + q);
            }
          }
      }
    }
  }
  __syncthreads();
  const int nc = ncand;
  int ns;  // entries to sort
  if (nc <= kTopkCand) {
    ns = nc;
  } else {
    // exact slow path: x = K-th largest key; r of its ties, the smallest ids
    uint32_t x = 0;
    for (int b = 15; b >= 0; --b) {
      const uint32_t cand = x | (1u << b);
      int n = 0;
      for (int64_t i = tid; i < nvec; i += kTopkThreads) {
        uint32_t k[8];
        load_keys(row, i, k);
#pragma unroll
        for (int q = 0; q < 8; ++q) n += k[q] >= cand;
      }
      if (block_count(n, red[rb]) >= K) x = cand;
      rb ^= 1;
    }
    int ngt = 0;
    for (int64_t i = tid; i < nvec; i += kTopkThreads) {
      uint32_t k[8];
      load_keys(row, i, k);
#pragma unroll
      for (int q = 0; q < 8; ++q) ngt += k[q] > x;
    }
    const int r = K - block_count(ngt, red[rb]);
    rb ^= 1;
    // largest y with #{key == x, id < y} < r; the ties with id <= y are taken
    uint32_t y = 0;
    for (int b = a.id_bits - 1; b >= 0; --b) {
      const uint32_t cand = y | (1u << b);
      int n = 0;
      for (int64_t i = tid; i < nvec; i += kTopkThreads) {
        uint32_t k[8];
        load_keys(row, i, k);
#pragma unroll
        for (int q = 0; q < 8; ++q) n += k[q] == x && (uint32_t)(8 * i + q) < cand;
      }
      if (block_count(n, red[rb]) < r) y = cand;
      rb ^= 1;
    }
    if (tid == 0) ncand = 0;
    __syncthreads();
    for (int64_t i = tid; i < nvec; i += kTopkThreads) {
      uint32_t k[8];
      load_keys(row, i, k);
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (k[q] > x || (k[q] == x && (uint32_t)(8 * i + q) <= y)) {
          const int p = atomicAdd(&ncand, 1);
          if (p < kTopkCand) {
            ck[p] = k[q];
            ci[p] = (int32_t)(8 * i + q);
          }
        }
    }
    __syncthreads();
    ns = K;
  }
  if (ns <= kTopkThreads) {
    // at most one candidate per thread: its place in the order (larger key
    // first, then smaller id) is the number of candidates ahead of it (all
    // (key, id) pairs differ), and the first K places are written directly
    if (tid < ns) {
      const uint32_t ki = ck[tid];
      const int32_t ii = ci[tid];
      int rank = 0;
      for (int j = 0; j < ns; ++j) {
        const uint32_t kj = ck[j];
        const int32_t ij = ci[j];
        rank += (kj > ki) | ((kj == ki) & (ij < ii));
      }
      if (rank < K) {
        a.idx[t * K + rank] = ii;
        a.val[t * K + rank] = key_bf16_value(ki);
      }
    }
    return;
  }
  int np = 1;
  while (np < ns) np <<= 1;
  for (int i = ns + tid; i < np; i += kTopkThreads) {
    ck[i] = 0u;
    ci[i] = INT32_MAX;
  }
  __syncthreads();
  lds_sort(ck, ci, np);
  for (int k = tid; k < K; k += kTopkThreads) {
    a.idx[t * K + k] = ci[k];
    a.val[t * K + k] = key_bf16_value(ck[k]);
  }
}

}  // namespace kd
