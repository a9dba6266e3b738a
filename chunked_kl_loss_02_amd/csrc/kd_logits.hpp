// Forward-chunked KL on materialised student logits (the second of the three
// loss variants on the page "Making Knowledge Distillation Cheap Enough to
// Run at Scale", section "Two systems changes": the teacher stays sparse, the
// student's logits Z[T,V] exist in full).  One workgroup per token row:
//   pass A  streams the row once: running (max, sum 2^(c z - max)) per
//           thread, merged across the workgroup -> lse2[t]; the student logits
//           at the cached teacher ids are gathered for the loss;
//   pass B  streams the row again (the rows in flight fit the last-level
//           cache, so this read mostly misses HBM) and writes
//           dZ = coef 2^(c z - lse2), then patches the teacher ids with
//           coef (q - mass).
// HBM-bound: about 2 (read) + 2 (write) bytes per bf16 logit, plus the
// second read where it misses the cache.  bf16 rows of up to 512 * 8 * 50
// logits take k_lrow_reg, which keeps the row in registers and reads it once.
#pragma once
#include <algorithm>

#include "kd_common.hpp"

namespace kd {

struct LrowArgs {
  const void* Z;         // [T, V] bf16 or fp32
  void* dZ;              // [T, V] same type (nullable: loss only)
  int64_t T, V;
  int K;
  const int32_t* idx;    // [T, K]
  const float* pm;       // [T, K] merged teacher mass
  const uint8_t* mask;   // [T] (nullable)
  const float* scal_f;   // [0] gradient coefficient
  float* lse2;           // [T] out
  float* s_out;          // [T, K] out: student logit at each teacher id
  float c;               // log2(e) / tau
};

template <class E>
struct ElemIO;
template <>
struct ElemIO<uint16_t> {  // bf16 bit patterns, 8 per 16-byte vector
  static constexpr int kN = 8;
  static __device__ __forceinline__ void unpack(const u32x4& v, float (&x)[8]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      x[2 * q] = __uint_as_float(v[q] << 16);
      x[2 * q + 1] = __uint_as_float(v[q] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ u32x4 pack(const float (&x)[8]) {
    u32x4 v;
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = pack_bf16x2(x[2 * q], x[2 * q + 1]);
    return v;
  }
  static __device__ __forceinline__ float load1(const void* p, int64_t i) {
    return __uint_as_float((uint32_t)static_cast<const uint16_t*>(p)[i] << 16);
  }
  static __device__ __forceinline__ void store1(void* p, int64_t i, float x) {
    static_cast<uint16_t*>(p)[i] = __builtin_bit_cast(uint16_t, (__bf16)x);
  }
};
template <>
struct ElemIO<float> {  // fp32, 4 per 16-byte vector
  static constexpr int kN = 4;
  static __device__ __forceinline__ void unpack(const u32x4& v, float (&x)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) x[q] = __uint_as_float(v[q]);
  }
  static __device__ __forceinline__ u32x4 pack(const float (&x)[4]) {
    u32x4 v;
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = __float_as_uint(x[q]);
    return v;
  }
  static __device__ __forceinline__ float load1(const void* p, int64_t i) { return static_cast<const float*>(p)[i]; }
  static __device__ __forceinline__ void store1(void* p, int64_t i, float x) { static_cast<float*>(p)[i] = x; }
};

constexpr int kLrowThreads = 512;

// (m, l) <- (m, l) merged with 2^(y - m) over the values y (log2 units)
template <int N>
__device__ __forceinline__ void lse_fold(float& m, float& l, const float (&y)[N]) {
  float cm = y[0];
#pragma unroll
  for (int j = 1; j < N; ++j) cm = fmaxf(cm, y[j]);
  const float nm = fmaxf(m, cm);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < N; ++j) s += fast_exp2(y[j] - nm);
  l = (m == -INFINITY ? 0.f : l * fast_exp2(m - nm)) + s;
  m = nm;
}

// kVec: rows are 16-byte aligned (V * sizeof(E) % 16 == 0): 16-byte vector
// accesses; otherwise element by element.
template <class E, bool kVec>
__global__ void __launch_bounds__(kLrowThreads) k_lrow(LrowArgs a) {
  using IO = ElemIO<E>;
  constexpr int N = IO::kN;
  __shared__ float red_m[kLrowThreads / 64], red_l[kLrowThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t t = blockIdx.x;
  const int64_t V = a.V;
  const E* row = static_cast<const E*>(a.Z) + t * V;
  E* drow = a.dZ ? static_cast<E*>(a.dZ) + t * V : nullptr;
  const bool keep = a.mask ? a.mask[t] != 0 : true;
  const int64_t nvec = kVec ? V / N : 0;
  if (!keep) {
    // masked row: zero gradient, no loss contribution
    if (drow) {
      for (int64_t i = tid; i < nvec; i += kLrowThreads)
        __builtin_nontemporal_store(u32x4{0u, 0u, 0u, 0u}, reinterpret_cast<u32x4*>(drow) + i);
      for (int64_t i = nvec * N + tid; i < V; i += kLrowThreads) IO::store1(drow, i, 0.f);
    }
    for (int k = tid; k < a.K; k += kLrowThreads) a.s_out[t * a.K + k] = 0.f;
    if (tid == 0) a.lse2[t] = 0.f;
    return;
  }
  // pass A: log-sum-exp of c z over the row
  float m = -INFINITY, l = 0.f;
  for (int64_t i = tid; i < nvec; i += kLrowThreads) {
    const u32x4 v = reinterpret_cast<const u32x4*>(row)[i];
    float x[N];
    IO::unpack(v, x);
#pragma unroll
    for (int j = 0; j < N; ++j) x[j] *= a.c;
    lse_fold<N>(m, l, x);
  }
  for (int64_t i = nvec * N + tid; i < V; i += kLrowThreads) {
    const float y[1] = {IO::load1(row, i) * a.c};
    lse_fold<1>(m, l, y);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float om = __shfl_xor(m, o, 64), ol = __shfl_xor(l, o, 64);
    const float nm = fmaxf(m, om);
    l = (nm == -INFINITY) ? 0.f : l * fast_exp2(m - nm) + ol * fast_exp2(om - nm);
    m = nm;
  }
  if (lane == 0) {
    red_m[w] = m;
    red_l[w] = l;
  }
  __syncthreads();
  float M = red_m[0], Lsum = 0.f;
#pragma unroll
  for (int q = 1; q < kLrowThreads / 64; ++q) M = fmaxf(M, red_m[q]);
#pragma unroll
  for (int q = 0; q < kLrowThreads / 64; ++q) Lsum += red_l[q] * fast_exp2(red_m[q] - M);
  const float lse2 = M + fast_log2(Lsum);
  if (tid == 0) a.lse2[t] = lse2;
  // student logits at the cached teacher ids
  for (int k = tid; k < a.K; k += kLrowThreads) {
    const int32_t v = a.idx[t * a.K + k];
    a.s_out[t * a.K + k] = (v >= 0 && (int64_t)v < V) ? IO::load1(row, v) : 0.f;
  }
  if (!drow) return;
  // pass B: dZ = coef 2^(c z - lse2), then the teacher ids
  const float coef = a.scal_f[0];
  for (int64_t i = tid; i < nvec; i += kLrowThreads) {
    const u32x4 v = reinterpret_cast<const u32x4*>(row)[i];
    float x[N];
    IO::unpack(v, x);
#pragma unroll
    for (int j = 0; j < N; ++j) x[j] = coef * fast_exp2(fmaf(x[j], a.c, -lse2));
    __builtin_nontemporal_store(IO::pack(x), reinterpret_cast<u32x4*>(drow) + i);
  }
  for (int64_t i = nvec * N + tid; i < V; i += kLrowThreads)
    IO::store1(drow, i, coef * fast_exp2(fmaf(IO::load1(row, i), a.c, -lse2)));
  __syncthreads();  // the dense values of this row are written before the patches
  for (int k = tid; k < a.K; k += kLrowThreads) {
    const int32_t v = a.idx[t * a.K + k];
    if (v < 0 || (int64_t)v >= V) continue;
    const float q = fast_exp2(fmaf(IO::load1(row, v), a.c, -lse2));
    IO::store1(drow, v, coef * (q - a.pm[t * a.K + k]));
  }
}

// Register-resident variant for bf16 rows of V = 8 * nvec logits with
// nvec <= 512 * PER: one 512-thread workgroup (two waves per SIMD, up to 256
// registers each) holds its row in registers (PER 16-byte chunks per thread,
// chunk c of thread i = vector c * 512 + i), so the row is read from HBM
// once and dZ written once: 4 bytes per logit.
constexpr int kLrowRegThreads = 512;
// cache policy of the row's streaming loads and stores: nontemporal (each
// byte of Z and dZ moves once)
constexpr int kNT = 2;
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

template <int PER>
__global__ void __launch_bounds__(kLrowRegThreads) k_lrow_reg(LrowArgs a) {
  using IO = ElemIO<uint16_t>;
  __shared__ float red_m[kLrowRegThreads / 64], red_l[kLrowRegThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t t = blockIdx.x;
  const int64_t V = a.V, nvec = V >> 3;
  const uint16_t* row = static_cast<const uint16_t*>(a.Z) + t * V;
  uint16_t* drow = a.dZ ? static_cast<uint16_t*>(a.dZ) + t * V : nullptr;
  // Buffer resources over the row: one lane offset (tid * 16) and a scalar
  // offset per chunk.  The hardware range check covers the lane offset only,
  // so a chunk that would run past the row is shifted back to end at its
  // last vector (base(c) = clamp(c * 512, 0, nvec - 512)): every load stays
  // in the row, and lanes whose vector an earlier chunk already holds (or,
  // for nvec < 512, past the row: those read 0) are left out by in_row.
  const __amdgpu_buffer_rsrc_t rz = make_rsrc(row, (uint64_t)V * 2);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(drow ? drow : row, drow ? (uint64_t)V * 2 : 0);
  const int voff = tid * 16;
  auto base = [&](int c) -> int {
    const int64_t b = std::min<int64_t>((int64_t)c * kLrowRegThreads, nvec - kLrowRegThreads);
    return (int)std::max<int64_t>(b, 0);
  };
  auto in_row = [&](int c) {
    const int64_t i = (int64_t)base(c) + tid;
    return i >= (int64_t)c * kLrowRegThreads && i < nvec;
  };
  const bool keep = a.mask ? a.mask[t] != 0 : true;
  if (!keep) {
    if (drow) {
#pragma unroll
      for (int c = 0; c < PER; ++c)
        if (in_row(c))
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, u32x4{0u, 0u, 0u, 0u}), rd, voff,
                                                 base(c) * 16, kNT);
    }
    for (int k = tid; k < a.K; k += kLrowRegThreads) a.s_out[t * a.K + k] = 0.f;
    if (tid == 0) a.lse2[t] = 0.f;
    return;
  }
  u32x4 v[PER];
#pragma unroll
  for (int c = 0; c < PER; ++c)
    v[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rz, voff, base(c) * 16, kNT));
  float m = -INFINITY, l = 0.f;
#pragma unroll
  for (int c = 0; c < PER; ++c) {
    if (in_row(c)) {
      float x[8];
      IO::unpack(v[c], x);
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] *= a.c;
      lse_fold<8>(m, l, x);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float om = __shfl_xor(m, o, 64), ol = __shfl_xor(l, o, 64);
    const float nm = fmaxf(m, om);
    l = (nm == -INFINITY) ? 0.f : l * fast_exp2(m - nm) + ol * fast_exp2(om - nm);
    m = nm;
  }
  if (lane == 0) {
    red_m[w] = m;
    red_l[w] = l;
  }
  __syncthreads();
  float M = red_m[0], Lsum = 0.f;
#pragma unroll
  for (int q = 1; q < kLrowRegThreads / 64; ++q) M = fmaxf(M, red_m[q]);
#pragma unroll
  for (int q = 0; q < kLrowRegThreads / 64; ++q) Lsum += red_l[q] * fast_exp2(red_m[q] - M);
  const float lse2 = M + fast_log2(Lsum);
  if (tid == 0) a.lse2[t] = lse2;
  for (int k = tid; k < a.K; k += kLrowRegThreads) {
    const int32_t vi = a.idx[t * a.K + k];
    a.s_out[t * a.K + k] = (vi >= 0 && (int64_t)vi < V) ? IO::load1(row, vi) : 0.f;
  }
  if (!drow) return;
  const float coef = a.scal_f[0];
  // keep the packed row live, not pass A's unpacked floats (twice the registers)
#pragma unroll
  for (int c = 0; c < PER; ++c) asm volatile("" : "+v"(v[c]));
#pragma unroll
  for (int c = 0; c < PER; ++c) {
    float x[8];
    IO::unpack(v[c], x);
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = coef * fast_exp2(fmaf(x[j], a.c, -lse2));
    if (in_row(c)) __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, IO::pack(x)), rd, voff, base(c) * 16, kNT);
  }
  __syncthreads();  // the dense values of this row are written before the patches
  for (int k = tid; k < a.K; k += kLrowRegThreads) {
    const int32_t vi = a.idx[t * a.K + k];
    if (vi < 0 || (int64_t)vi >= V) continue;
    const float q = fast_exp2(fmaf(IO::load1(row, vi), a.c, -lse2));
    IO::store1(drow, vi, coef * (q - a.pm[t * a.K + k]));
  }
}

}  // namespace kd
