// gfx950 kernels of the fused chunked top-K KL distillation loss.
//
// The loss (page "Efficient Knowledge Distillation for LLMs: Offline Top-K
// Logits and a Fused Chunked KL Loss", abstract; page "Making Knowledge
// Distillation Cheap Enough to Run at Scale", section "Two systems changes"):
// the student's logits S = h W^T are projected one block at a time, folded
// into a running log-sum-exp per token and discarded; the teacher is its
// cached top-K logits, renormalised over those K entries; the backward pass
// recomputes each block.  With c = log2(e)/tau all exponentials run in base 2.
//
//   pass 1 : k_pass1   S^T tile = W_tile h_tile^T (MFMA), per token the
//                      tile's (max, sum 2^(c S - max))
//            k_lse     merges the per-tile partials -> lse2[t] (log2 units)
//            (and, through the teacher entries bucketed by tile, the logit
//            s[t,k] = S[t, idx[t,k]] at each cached id, read out of the tile)
//   teacher: k_teacher p = softmax_K(u/tau), merged mass of duplicate ids,
//                      sum_k p log(mass) per row
//   loss   : k_rows / k_sum   KL_t = sum p log p - sum p s / tau + LSE_t
//   pass 2 : k_pass2   recomputes the S^T tile, writes the logit gradient
//                      G = coef * 2^(c S - lse2) (bf16) for one (token block,
//                      vocabulary chunk), with the per-token offsets of
//                      k_offsets, the bucketed teacher entries written in
//                      place (coef * (q - mass) at the cached ids); k_bwd
//                      contracts G into dH (over the chunk's vocabulary) and
//                      dW (over the block's tokens, with h^T from
//                      k_transpose_h); k_bwd_pass2 runs one unit's
//                      contractions with the next unit's pass 2.
//   sequence-chunk schedule: k_pass1<true> also stores a token block's S^T;
//            k_gather_s reads the logits at the cached ids out of it,
//            k_sgrad forms the gradient tiles from it (entries in place),
//            k_bwd_sgrad runs one chunk's contractions with the next
//            chunk's gradient tiles.
#pragma once
#include "kd_gemm.hpp"

namespace kd {

// ----------------------------------------------------------------- small ops
// N = number of kept tokens; scal_f[0] = g / (N tau) (gradient coefficient,
// g = *grad or 1), scal_f[1] = 1 / N (0 when N = 0).
__global__ void __launch_bounds__(1024) k_count(const uint8_t* __restrict__ mask, int64_t T, float tau,
                                                const float* __restrict__ grad, float* __restrict__ scal_f,
                                                int64_t* __restrict__ scal_i) {
  __shared__ int64_t part[1024];
  int64_t c = 0;
  for (int64_t t = threadIdx.x; t < T; t += 1024) c += mask ? (mask[t] != 0) : 1;
  part[threadIdx.x] = c;
  __syncthreads();
  for (int s = 512; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) part[threadIdx.x] += part[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int64_t N = part[0];
    scal_i[0] = N;
    const double g = grad ? (double)grad[0] : 1.0;
    scal_f[0] = N > 0 ? (float)(g / ((double)N * (double)tau)) : 0.0f;  // gradient coefficient
    scal_f[1] = N > 0 ? (float)(1.0 / (double)N) : 0.0f;
  }
}

__global__ void k_fill(float* __restrict__ p, int64_t n, float v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}

// dst (bf16) = RNE(src) or RNE(dst + src) (accumulate); n a multiple of 4,
// both 8-byte aligned.
__global__ void k_to_bf16(const float* __restrict__ src, uint16_t* __restrict__ dst, int64_t n, int accumulate) {
  const int64_t n4 = n >> 2;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
    float4 v = reinterpret_cast<const float4*>(src)[i];
    u32x2* d = reinterpret_cast<u32x2*>(dst) + i;
    if (accumulate) {
      const u32x2 o = *d;
      v.x += __uint_as_float(o[0] << 16);
      v.y += __uint_as_float(o[0] & 0xFFFF0000u);
      v.z += __uint_as_float(o[1] << 16);
      v.w += __uint_as_float(o[1] & 0xFFFF0000u);
    }
    u32x2 r;
    r[0] = pack_bf16x2(v.x, v.y);
    r[1] = pack_bf16x2(v.z, v.w);
    *d = r;
  }
}

// (m, l) <- (m, l) merged with (om, ol), l = sum 2^(x - m); (-inf, 0) is empty.
__device__ __forceinline__ void lse_merge(float& m, float& l, float om, float ol) {
  const float nm = fmaxf(m, om);
  if (nm == -INFINITY) return;
  // one rounding order wherever this is inlined: an explicit fma, not a
  // contraction the compiler may place on either product
  l = fmaf(l, fast_exp2(m - nm), ol * fast_exp2(om - nm));
  m = nm;
}

// Teacher side, one wave per token: p = softmax over the K cached logits at
// temperature tau; pm[k] = total mass on id idx[k] (duplicates add);
// negent[t] = sum_k p_k log pm_k (= sum_v P log P on the vocabulary).
constexpr int kTeacherMaxK = 1024;
__global__ void __launch_bounds__(256) k_teacher(const int32_t* __restrict__ idx, const float* __restrict__ logit,
                                                 const uint8_t* __restrict__ mask, int64_t T, int K, int64_t V,
                                                 float inv_tau, float* __restrict__ p_out, float* __restrict__ pm_out,
                                                 float* __restrict__ negent, uint32_t* __restrict__ status, int validate) {
  __shared__ int32_t sid[4][kTeacherMaxK];
  __shared__ float sp[4][kTeacherMaxK];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + w;
  if (t >= T) return;
  const int32_t* ir = idx + t * K;
  const float* lr = logit + t * K;
  float* pr = p_out + t * K;
  float* pmr = pm_out + t * K;
  const bool keep = mask ? mask[t] != 0 : true;
  if (!keep) {
    for (int k = lane; k < K; k += 64) { pr[k] = 0.f; pmr[k] = 0.f; }
    if (lane == 0) negent[t] = 0.f;
    return;
  }
  float mx = -INFINITY;
  uint32_t bad = 0;
  for (int k = lane; k < K; k += 64) {
    const float u = lr[k] * inv_tau;
    mx = fmaxf(mx, u);
    if (validate) {
      const int32_t v = ir[k];
      if (v < 0 || (int64_t)v >= V) bad |= 1u;
      if (__builtin_isnan(lr[k]) || lr[k] == INFINITY) bad |= 2u;
    }
  }
  mx = wave_max(mx);
  if (validate) {
    if (mx == -INFINITY) bad |= 2u;
    if (bad) atomicOr(status, bad);
  }
  float z = 0.f;
  for (int k = lane; k < K; k += 64) z += expf(lr[k] * inv_tau - mx);
  z = wave_sum(z);
  const float iz = 1.0f / z;
  for (int k = lane; k < K; k += 64) {
    const float p = expf(lr[k] * inv_tau - mx) * iz;
    pr[k] = p;
    sp[w][k] = p;
    sid[w][k] = ir[k];
  }
  // make this wave's LDS writes visible to its other lanes
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  __builtin_amdgcn_wave_barrier();
  float ne = 0.f;
  for (int k = lane; k < K; k += 64) {
    const int32_t v = sid[w][k];
    float m = 0.f;
    for (int j = 0; j < K; ++j) m += (sid[w][j] == v) ? sp[w][j] : 0.f;
    pmr[k] = m;
    const float p = sp[w][k];
    if (p > 0.f) ne += p * logf(m);
  }
  ne = wave_sum(ne);
  if (lane == 0) negent[t] = ne;
}

// ----------------------------------------------------------------- pass 1
// Grid: padded to a multiple of 8; work id -> (token tile, vocabulary tile),
// both of 256.  Each workgroup writes one (max, sum) pair per token of its
// tile:  part[vt * ldp + t] = (m, l) with l = sum_v 2^(c S[t,v] - m) over the
// tile's vocabulary rows.
struct Pass1Args {
  const uint16_t* W;     // [V, H]
  const uint16_t* h;     // token block origin [rows, H]
  float2* part;          // [nvt, ldp]: (max, sum) per vocabulary tile and token
  int64_t V, H, rows;    // rows = valid tokens in the block
  int ntt, nvt, gt, gv, total, ldp;  // gv > 0: group vocabulary tiles instead
  float c;               // log2(e) / tau
  float* St;             // kStore: S^T of the block, [V rows, lds] fp32 (row v, column t)
  int64_t lds;
  // !kStore: the teacher entries by tile (nullable: no gather), and where
  // the gathered logits go (s_out[t * K + k], t global)
  const uint32_t* bstart;
  const uint32_t* bbase;
  const uint32_t* ent;
  float* s_out;
  int ldk, gtt0, K;
};

// Writes the raw logits S^T[v, t] of the tile's valid vocabulary rows (the
// sequence-chunk schedule reads them back instead of recomputing).  The
// tile leaves in two halves of 128 vocabulary rows through the four free
// LDS stages (32 rows of 256 fp32 each): the owning waves scatter their
// accumulators (16-byte chunk c of row r at c ^ 8((r >> 2) & 1), which
// keeps the two lane halves, 4 rows apart, on different banks), then every
// thread copies whole 1-KiB row segments to HBM with 16-byte stores.
__device__ __forceinline__ void store_tile_t(const Pass1Args& a, const Stages& st, const f32x16 (&acc)[4][4], int vt,
                                             int tt, int wm, int wn, int lane) {
  auto row = [&](int r) -> float* {
    uint16_t* b = r < 32 ? st.a0 : r < 64 ? st.a1 : r < 96 ? st.b0 : st.b1;
    return reinterpret_cast<float*>(b) + (r & 31) * 256;
  };
  const int tid = threadIdx.x;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (wm == half) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int r = acc_row(i, e, lane);
          float* rp = row(r);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int t = wn * 128 + acc_col(j, lane);
            rp[(((t >> 2) ^ (8 * ((r >> 2) & 1))) << 2) | (t & 3)] = acc[i][j][e];
          }
        }
    }
    __syncthreads();
    const int64_t v0 = (int64_t)vt * 256 + half * 128;
#pragma unroll 4
    for (int k = 0; k < 32; ++k) {
      const int r = (tid >> 6) + 4 * k, c = tid & 63;
      if (v0 + r < a.V) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(row(r) + ((c ^ (8 * ((r >> 2) & 1))) << 2));
        __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(a.St + (v0 + r) * a.lds + tt * 256) + c);
      }
    }
    __syncthreads();
  }
}

// The student logits at the cached teacher ids of this tile (its bucket of
// entries [e0, e1), entry = t | v << 8 | k << 16 within the tile): the
// tile's fp32 S^T passes through the four free LDS stages in two halves of
// 128 vocabulary rows, laid out as in store_tile_t, and each entry of a
// half reads its logit there and stores it at (t, k).  ent0 is the
// workgroup's first entries, loaded earlier (one per thread).
__device__ __forceinline__ void gather_tile_t(const Pass1Args& a, Stages st, const f32x16 (&acc)[4][4],
                                              int tt, int wm, int wn, int lane, uint32_t e0, uint32_t e1,
                                              uint32_t ent0) {
  auto row = [&](int r) -> float* {
    uint16_t* b = r < 32 ? st.a0 : r < 64 ? st.a1 : r < 96 ? st.b0 : st.b1;
    return reinterpret_cast<float*>(b) + (r & 31) * 256;
  };
  const int tid = threadIdx.x;
  const int64_t t0 = ((int64_t)a.gtt0 + tt) * 256;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (wm == half) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int r = acc_row(i, e, lane);
          float* rp = row(r);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int t = wn * 128 + acc_col(j, lane);
            rp[(((t >> 2) ^ (8 * ((r >> 2) & 1))) << 2) | (t & 3)] = acc[i][j][e];
          }
        }
    }
    __syncthreads();
    auto take = [&](uint32_t x) {
      const int tl = x & 255, vr = (x >> 8) & 255, k = (int)(x >> 16);
      if ((vr >> 7) != half) return;
      const int r = vr & 127;
      a.s_out[(t0 + tl) * a.K + k] = row(r)[(((tl >> 2) ^ (8 * ((r >> 2) & 1))) << 2) | (tl & 3)];
    };
    if (e0 + (uint32_t)tid < e1) take(ent0);
    for (uint32_t e = e0 + 256 + tid; e < e1; e += 256) take(a.ent[e]);
    __syncthreads();
  }
}

// One (token tile, vocabulary tile) per workgroup: S^T of the tile, then per
// token the tile's max m and sum l of 2^(c S - m) (base-2 log-sum-exp parts),
// folded across tiles by k_lse.  Nothing but the loaders lives across the K
// loop.  kStore additionally writes the tile's logits (store_tile_t).
template <bool kStore>
__global__ void __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) k_pass1(Pass1Args a) {
  KD_DECLARE_STAGES(st, 256, 256);
  __shared__ float2 red[2][128];
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  if (id >= a.total) return;
  int tt, vt;
  if (a.gv > 0)
    grouped(id, a.nvt, a.ntt, a.gv, vt, tt);
  else
    grouped(id, a.ntt, a.nvt, a.gt, tt, vt);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w & 1, wn = w >> 1;
  // this tile's teacher entries: [e0, e1) of a.ent
  uint32_t e0 = 0, e1 = 0;
  if (!kStore && a.ent) {
    const int gtt = a.gtt0 + tt;
    const int64_t key = (int64_t)gtt * a.ldk + vt;
    const uint32_t bb = a.bbase[gtt];
    e0 = bb + a.bstart[key];
    e1 = bb + a.bstart[key + 1];
  }
  f32x16 acc[4][4];
  {
    LoaderKC<256> la, lb;
    la.init(a.W + (int64_t)vt * 256 * a.H, a.V - (int64_t)vt * 256, a.H);
    lb.init(a.h + (int64_t)tt * 256 * a.H, a.rows - (int64_t)tt * 256, a.H);
    gemm_tile<4, 4>(la, lb, (int)(a.H / kBK), st, acc);
  }
  // first entries now: their latency hides under the exponentials below
  const uint32_t ent0 = e0 + threadIdx.x < e1 ? a.ent[e0 + threadIdx.x] : 0u;
  // vocabulary rows of this lane: vt*256 + wm*128 + acc_row(i, e)
  const int64_t vbase = (int64_t)vt * 256 + wm * 128;
  if constexpr (kStore) store_tile_t(a, st, acc, vt, tt, wm, wn, lane);
  float rm[4], rl[4];
  if (vbase + 128 <= a.V) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, acc[i][j][e]);
      const float m = mx * a.c;
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) sum += fast_exp2(fmaf(acc[i][j][e], a.c, -m));
      rm[j] = m;
      rl[j] = sum;
    }
  } else {
    // the vocabulary's last tile: rows of this wave at or past V count as
    // absent (row r of the wave's block is valid iff r < lim)
    const int lim = (int)(a.V - vbase);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (acc_row(i, e, lane) < lim) mx = fmaxf(mx, acc[i][j][e]);
      const float m = mx * a.c;
      const float ref = m == -INFINITY ? 0.f : m;  // rows of this lane all past V
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (acc_row(i, e, lane) < lim) sum += fast_exp2(fmaf(acc[i][j][e], a.c, -ref));
      rm[j] = m;
      rl[j] = sum;
    }
  }
  // merge the two lane halves (same token, other vocabulary rows)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float om = __shfl_xor(rm[j], 32, 64);
    const float ol = __shfl_xor(rl[j], 32, 64);
    lse_merge(rm[j], rl[j], om, ol);
  }
  // merge the two M waves through LDS
  if (wm == 1 && lane < 32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) red[wn][acc_col(j, lane)] = make_float2(rm[j], rl[j]);
  }
  __syncthreads();
  if (wm == 0 && lane < 32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float2 o = red[wn][acc_col(j, lane)];
      lse_merge(rm[j], rl[j], o.x, o.y);
      const int t = tt * 256 + wn * 128 + acc_col(j, lane);
      a.part[(int64_t)vt * a.ldp + t] = make_float2(rm[j], rl[j]);
    }
  }
  if constexpr (!kStore) {
    if (e1 > e0) gather_tile_t(a, st, acc, tt, wm, wn, lane, e0, e1, ent0);
  }
}

// lse2[t] = log2 sum_v 2^(c S[t,v]) from the per-tile partials.  A block
// handles 16 tokens; its 16 thread groups each fold every 16th tile (four
// loads in flight), then the 16 partial results are folded in a fixed order
// (deterministic).
constexpr int kLseTok = 16, kLseGroups = 16;
__global__ void __launch_bounds__(256) k_lse(const float2* __restrict__ part, int nranges, int ldp, int64_t rows,
                                             float* __restrict__ lse2) {
  __shared__ float2 red[kLseGroups][kLseTok];
  const int tx = threadIdx.x % kLseTok, g = threadIdx.x / kLseTok;
  const int64_t t = (int64_t)blockIdx.x * kLseTok + tx;
  float m = -INFINITY, l = 0.f;
  if (t < rows) {
    float m2 = -INFINITY, l2 = 0.f;
    int r = g;
    for (; r + 3 * kLseGroups < nranges; r += 4 * kLseGroups) {
      float2 q[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) q[u] = part[(int64_t)(r + u * kLseGroups) * ldp + t];
      lse_merge(m, l, q[0].x, q[0].y);
      lse_merge(m2, l2, q[1].x, q[1].y);
      lse_merge(m, l, q[2].x, q[2].y);
      lse_merge(m2, l2, q[3].x, q[3].y);
    }
    for (; r < nranges; r += kLseGroups) {
      const float2 q = part[(int64_t)r * ldp + t];
      lse_merge(m, l, q.x, q.y);
    }
    lse_merge(m, l, m2, l2);
  }
  red[g][tx] = make_float2(m, l);
  __syncthreads();
  if (g == 0 && t < rows) {
#pragma unroll
    for (int k = 1; k < kLseGroups; ++k) lse_merge(m, l, red[k][tx].x, red[k][tx].y);
    lse2[t] = m + log2f(l);
  }
}

// Per-row KL and per-block partial sums (fp64, fixed order).
__global__ void __launch_bounds__(256) k_rows(const float* __restrict__ p, const float* __restrict__ s,
                                              const float* __restrict__ negent, const float* __restrict__ lse2,
                                              const uint8_t* __restrict__ mask, int64_t T, int K, float inv_tau,
                                              float* __restrict__ row_loss, double* __restrict__ bsum) {
  __shared__ double red[256];
  const int64_t t = blockIdx.x * (int64_t)256 + threadIdx.x;
  double v = 0.0;
  if (t < T && (mask ? mask[t] != 0 : true)) {
    float g = 0.f;
    for (int k = 0; k < K; ++k) g = fmaf(p[t * K + k], s[t * K + k], g);
    v = (double)negent[t] - (double)g * (double)inv_tau + (double)lse2[t] * (double)kLn2;
  }
  if (t < T) row_loss[t] = (float)v;
  red[threadIdx.x] = v;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) bsum[blockIdx.x] = red[0];
}

__global__ void __launch_bounds__(1024) k_sum(const double* __restrict__ bsum, int64_t nb,
                                              const float* __restrict__ scal_f, float* __restrict__ loss) {
  __shared__ double red[1024];
  double v = 0.0;
  for (int64_t i = threadIdx.x; i < nb; i += 1024) v += bsum[i];
  red[threadIdx.x] = v;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss[0] = (float)(red[0] * (double)scal_f[1]);
}

// --------------------------------------------- teacher entries by tile
// The cached teacher entries of kept tokens, grouped by the (token tile,
// vocabulary tile) of 256 x 256 they fall in (the per-chunk bucketing of
// the teacher ids).  The pass-1 workgroup of a tile reads the student logit
// at each of its entries out of its own logit tile; then every entry gets
// its final logit-gradient value bf16(coef * (q - mass)), q = 2^(c s - lse2),
// which the pass-2 workgroup of that tile writes into its staged tile.
// Bucket (tt, vt) is slot tt * ldk + vt, ldk = nvt + 1; after the scans slot
// (tt, vt) holds the bucket's start relative to the token tile's first
// entry, slot (tt, nvt) the token tile's count, and base[tt] the token
// tile's first entry.  Before pass 1 an entry is (t & 255) | (v & 255) << 8
// | k << 16 (token and id within the tile, cached slot); after,
// (t & 255) | (v & 255) << 8 | bits << 16.
__global__ void k_bucket_count(const int32_t* __restrict__ idx, const uint8_t* __restrict__ mask, int64_t T, int K,
                               int64_t V, int ldk, uint32_t* __restrict__ cnt) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= T * K) return;
  const int64_t t = i / K;
  if (mask && mask[t] == 0) return;
  const int32_t v = idx[i];
  if (v < 0 || (int64_t)v >= V) return;
  atomicAdd(cnt + (t >> 8) * ldk + (v >> 8), 1u);
}

// Exclusive scan of n counts in place, one workgroup per row of `data`
// (stride ld); data[n] of the row receives the row's total.  Thread j
// scans a contiguous share of the row.
__global__ void __launch_bounds__(1024) k_scan_rows(uint32_t* __restrict__ data, int n, int64_t ld) {
  __shared__ uint32_t part[1024];
  uint32_t* row = data + (int64_t)blockIdx.x * ld;
  const int per = (n + 1023) / 1024;
  const int j = threadIdx.x;
  const int b0 = min(n, j * per), b1 = min(n, b0 + per);
  uint32_t sum = 0;
  for (int i = b0; i < b1; ++i) sum += row[i];
  part[j] = sum;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // inclusive scan of the shares
    const uint32_t v = j >= o ? part[j - o] : 0u;
    __syncthreads();
    part[j] += v;
    __syncthreads();
  }
  uint32_t run = j ? part[j - 1] : 0u;
  for (int i = b0; i < b1; ++i) {
    const uint32_t c = row[i];
    row[i] = run;
    run += c;
  }
  if (j == 1023) row[n] = part[1023];
}

// base[tt] = first entry of token tile tt (exclusive scan of the tile
// totals that k_scan_rows left in slot nvt of each row), base[ntt] = the
// number of entries; one workgroup.
__global__ void __launch_bounds__(1024) k_scan_tiles(const uint32_t* __restrict__ start, int ntt, int ldk, int nvt,
                                                      uint32_t* __restrict__ base) {
  __shared__ uint32_t part[1024];
  const int per = (ntt + 1023) / 1024;
  const int j = threadIdx.x;
  const int b0 = min(ntt, j * per), b1 = min(ntt, b0 + per);
  uint32_t sum = 0;
  for (int i = b0; i < b1; ++i) sum += start[(int64_t)i * ldk + nvt];
  part[j] = sum;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const uint32_t v = j >= o ? part[j - o] : 0u;
    __syncthreads();
    part[j] += v;
    __syncthreads();
  }
  uint32_t run = j ? part[j - 1] : 0u;
  for (int i = b0; i < b1; ++i) {
    base[i] = run;
    run += start[(int64_t)i * ldk + nvt];
  }
  if (j == 1023) base[ntt] = part[1023];
}

// Places every kept entry in its bucket (order inside a bucket is free) as
// t | v << 8 | k << 16 (token and id within their tiles, cached slot), and
// its flat index t * K + k beside it: pass 1 gathers the logits through
// these, then k_bucket_value turns them into the pass-2 entries.
__global__ void k_bucket_index(const int32_t* __restrict__ idx, const uint8_t* __restrict__ mask, int64_t T, int K,
                               int64_t V, int ldk, const uint32_t* __restrict__ start,
                               const uint32_t* __restrict__ base, uint32_t* __restrict__ cur,
                               uint32_t* __restrict__ ent, uint32_t* __restrict__ ent_i) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= T * K) return;
  const int64_t t = i / K;
  if (mask && mask[t] == 0) return;
  const int32_t v = idx[i];
  if (v < 0 || (int64_t)v >= V) return;
  const int64_t key = (t >> 8) * ldk + (v >> 8);
  const uint32_t pos = base[t >> 8] + start[key] + atomicAdd(cur + key, 1u);
  ent[pos] = (uint32_t)(t & 255) | ((uint32_t)(v & 255) << 8) | ((uint32_t)(i - t * K) << 16);
  ent_i[pos] = (uint32_t)i;
}

// Each placed entry at a position p in [lo[0], hi[0]) (the whole call:
// base[0] .. base[ntt], the number placed; one token block: the bases of its
// first and one-past-last token tiles) gets its final logit-gradient value
// bf16(coef * (q - mass)), q = 2^(c s - lse2) from the gathered logit, in
// place of its slot: t | v << 8 | bits << 16.  Both schedules write these
// entries into their staged gradient tiles (pass 2, or the stored logits'
// gradient tiles of the sequence-chunk schedule).
__global__ void k_bucket_value(const float* __restrict__ s, const float* __restrict__ pm,
                               const float* __restrict__ lse2, const float* __restrict__ scal_f, int K, float c,
                               const uint32_t* __restrict__ lo, const uint32_t* __restrict__ hi,
                               const uint32_t* __restrict__ ent_i, uint32_t* __restrict__ ent) {
  const int64_t p = (int64_t)lo[0] + blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (p >= (int64_t)hi[0]) return;
  const uint32_t i = ent_i[p];
  const uint32_t t = i / (uint32_t)K;
  const float q = fast_exp2(fmaf(s[i], c, -lse2[t]));
  const float g = scal_f[0] * (q - pm[i]);
  const uint32_t bits = __builtin_bit_cast(uint16_t, (__bf16)g);
  ent[p] = (ent[p] & 0xFFFFu) | (bits << 16);
}

// ----------------------------------------------------------------- pass 2
// One (token block, vocabulary chunk): G[t, v] = coef_t 2^(c S[t,v] - lse2[t])
// in bf16 for every (t, v) of the padded tile grid (zero outside the valid
// range or on masked tokens).
// off[t] = lse2[t] - log2 |coef| for a kept token, +inf for a masked token,
// for t past T (up to the 256-aligned end) and for coef = 0: pass 2 forms
// |G| = |coef| 2^(c S - lse2) as 2^(c S - off), so the dropped tokens get
// exact zeros.
__global__ void __launch_bounds__(256) k_offsets(const float* __restrict__ lse2, const uint8_t* __restrict__ mask,
                                                 int64_t T, int64_t Tp, const float* __restrict__ scal_f,
                                                 float* __restrict__ off) {
  const int64_t t = blockIdx.x * (int64_t)256 + threadIdx.x;
  if (t >= Tp) return;
  const float cs = scal_f[0];
  const bool kept = t < T && (mask ? mask[t] != 0 : true) && cs != 0.f;
  off[t] = kept ? lse2[t] - log2f(fabsf(cs)) : INFINITY;
}

struct Pass2Args {
  const uint16_t* W;      // chunk origin [V - v0, H]
  const uint16_t* h;      // block origin
  const float* off;       // block origin (k_offsets), 256-aligned length
  const float* scal_f;
  uint16_t* G;            // [ntt*256, ldg]
  int64_t vrows, H, rows; // valid vocabulary rows in chunk / tokens in block
  int ntt, nvt, gt, gv, total, ldg;  // gv > 0: group vocabulary tiles instead
  float c;
  // teacher entries by tile (k_bucket_*; nullable: none written): bucket
  // starts [*, ldk], token-tile bases, entries; global tile index of this
  // launch's first token / vocabulary tile
  const uint32_t* bstart;
  const uint32_t* bbase;
  const uint32_t* ent;
  int ldk, gtt0, gvt0;
};

// One pass-2 tile, work id `id` < a.total, in the four stages `st`.
__device__ __forceinline__ void pass2_tile(const Pass2Args& a, int id, Stages st) {
  int tt, vt;
  if (a.gv > 0)
    grouped(id, a.nvt, a.ntt, a.gv, vt, tt);
  else
    grouped(id, a.ntt, a.nvt, a.gt, tt, vt);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w & 1, wn = w >> 1;
  LoaderKC<256> la, lb;
  la.init(a.W + (int64_t)vt * 256 * a.H, a.vrows - (int64_t)vt * 256, a.H);
  lb.init(a.h + (int64_t)tt * 256 * a.H, a.rows - (int64_t)tt * 256, a.H);
  // The tile's 256 token offsets (|G| = 2^(c S - off), k_offsets) go global
  // -> LDS with one 4-byte-per-lane buffer load per wave: no registers held
  // and no wait before the K loop, whose final wait and barrier cover them.
  __shared__ __attribute__((aligned(16))) float s_off[256];
  {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.off + (int64_t)tt * 256, 256 * 4);
    const int wv = __builtin_amdgcn_readfirstlane(w);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(s_off + 64 * wv), 4, (uint32_t)threadIdx.x * 4u, 0, 0,
                                             0);
  }
  const float cs = a.scal_f[0];
  // this tile's teacher entries: [e0, e1) of a.ent
  uint32_t e0 = 0, e1 = 0;
  if (a.ent) {
    const int gtt = a.gtt0 + tt;
    const int64_t key = (int64_t)gtt * a.ldk + a.gvt0 + vt;
    const uint32_t bb = a.bbase[gtt];
    e0 = bb + a.bstart[key];
    e1 = bb + a.bstart[key + 1];
  }
  f32x16 acc[4][4];
  gemm_tile<4, 4>(la, lb, (int)(a.H / kBK), st, acc);
  const int tid = threadIdx.x;
  // first entries now: their latency hides under the exponentials below
  const uint32_t ent0 = e0 + (uint32_t)tid < e1 ? a.ent[e0 + tid] : 0u;
  const uint32_t sgn = cs < 0.f ? 0x80008000u : 0u;  // sign bits of a negative coefficient
  // The bf16 tile goes through LDS (the four stages, 4 x 32 KiB, are free
  // after gemm_tile; 64 token rows each) as [256 tokens][256 vocab] rows of
  // 32 16-byte chunks, chunk c of row t at position c ^ (t & 31), then leaves
  // as full 512-byte row segments of G.
  auto row = [&](int tl) -> uint16_t* {
    uint16_t* b = tl < 64 ? st.a0 : tl < 128 ? st.a1 : tl < 192 ? st.b0 : st.b1;
    return b + (tl & 63) * 256;
  };
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tl = wn * 128 + acc_col(j, lane);  // token row inside the tile
    const float off = s_off[tl];
    uint16_t* trow = row(tl);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int vr = wm * 128 + acc_row(i, 4 * q, lane);  // 4 consecutive vocabulary rows
        float g[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) g[r] = fast_exp2(fmaf(acc[i][j][4 * q + r], a.c, -off));
        u32x2 pk;
        pk[0] = pack_bf16x2(g[0], g[1]) ^ sgn;
        pk[1] = pack_bf16x2(g[2], g[3]) ^ sgn;
        const int pos = ((vr >> 3) ^ (tl & 31)) * 8 + (vr & 7);
        *reinterpret_cast<u32x2*>(trow + pos) = pk;
      }
  }
  __syncthreads();
  // the teacher entries replace the dense values at their (token, id)
  if (e1 > e0) {
    auto put = [&](uint32_t x) {
      const int tl = x & 255, vr = (x >> 8) & 255;
      row(tl)[((vr >> 3) ^ (tl & 31)) * 8 + (vr & 7)] = (uint16_t)(x >> 16);
    };
    if (e0 + (uint32_t)tid < e1) put(ent0);
    for (uint32_t e = e0 + 256 + tid; e < e1; e += 256) put(a.ent[e]);
    __syncthreads();
  }
  // vocabulary columns past the chunk's valid rows leave as zeros (only in
  // the chunk's last tile)
  const int lim = (int)min<int64_t>(256, a.vrows - (int64_t)vt * 256);
  if (lim == 256) {
#pragma unroll 4
    for (int e = tid; e < 256 * 32; e += 256) {
      const int tl = e >> 5, c = e & 31;
      const u32x4 v = *reinterpret_cast<const u32x4*>(row(tl) + ((c ^ (tl & 31)) * 8));
      *reinterpret_cast<u32x4*>(a.G + (int64_t)(tt * 256 + tl) * a.ldg + vt * 256 + c * 8) = v;
    }
  } else {
    for (int e = tid; e < 256 * 32; e += 256) {
      const int tl = e >> 5, c = e & 31;
      u32x4 v = *reinterpret_cast<const u32x4*>(row(tl) + ((c ^ (tl & 31)) * 8));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = c * 8 + 2 * q;
        if (col >= lim) v[q] = 0u;
        else if (col + 1 >= lim) v[q] &= 0xFFFFu;
      }
      *reinterpret_cast<u32x4*>(a.G + (int64_t)(tt * 256 + tl) * a.ldg + vt * 256 + c * 8) = v;
    }
  }
}

__global__ void __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) k_pass2(Pass2Args a) {
  KD_DECLARE_STAGES(st, 256, 256);
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  if (id >= a.total) return;
  pass2_tile(a, id, st);
}

// Sequence-chunk schedule: s[t,k] = S[t, idx[t,k]] read from the stored
// S^T of the block (0 on masked rows); the recompute schedule reads them out
// of pass 1's tiles instead (gather_tile_t).
__global__ void k_gather_s(const float* __restrict__ St, int64_t lds, const int32_t* __restrict__ idx,
                           const uint8_t* __restrict__ mask, int64_t rows, int K, int64_t V,
                           float* __restrict__ s_out) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= rows * K) return;
  const int64_t t = i / K;
  const int32_t v = idx[i];
  const bool keep = (mask ? mask[t] != 0 : true) && v >= 0 && (int64_t)v < V;
  s_out[i] = keep ? St[(int64_t)v * lds + t] : 0.f;
}

// Sequence-chunk schedule: the logit gradient of one (token block,
// vocabulary chunk) from the block's stored fp32 S^T, one 256 (token) x 256
// (vocabulary) tile per work id: G = coef * 2^(c S - lse2) on kept tokens,
// the tile's bucketed teacher entries written in place, bf16.  HBM-bound:
// 256 KiB read and 128 KiB written per tile.
struct SgradArgs {
  const float* St;        // block's S^T, chunk origin (row v0): [*, lds]
  int64_t lds;
  const float* lse2;      // block origin
  const uint8_t* mask;    // block origin (nullable)
  const float* scal_f;
  uint16_t* G;            // [ntt * 256, ldg]
  int64_t vrows, rows;    // valid vocabulary rows in the chunk / tokens in the block
  int ntt, nvt, total, ldg;
  float c;
  // teacher entries by tile (k_bucket_*): bucket starts [*, ldk], token-tile
  // bases, entries; global index of the block's first token tile and of the
  // chunk's first vocabulary tile
  const uint32_t* bstart;
  const uint32_t* bbase;
  const uint32_t* ent;
  int ldk, gtt0, gvt0;
};

// One tile, work id `id` < a.total, staged in the four LDS stages (free in
// either kernel that runs it) as pass 2 stages its tile: [256 tokens][256
// vocabulary] bf16 rows, 16-byte chunk c of row t at position c ^ (t & 31).
// The tile's S^T is read 64 tokens at a time (256 rows x 256 bytes), the
// next group's loads issued before the current group's exponentials; a
// thread takes 4 tokens of 8 pairs of vocabulary rows and writes the pairs
// packed.
__device__ __forceinline__ void sgrad_tile(const SgradArgs& a, int id, Stages st) {
  const int tt = id / a.nvt, vt = id - tt * a.nvt;
  const int th = threadIdx.x;
  const int q = th & 15, rp = th >> 4;  // tokens 4q .. 4q+3 of a group; pairs rp + 16 j
  auto row = [&](int tl) -> uint16_t* {
    uint16_t* b = tl < 64 ? st.a0 : tl < 128 ? st.a1 : tl < 192 ? st.b0 : st.b1;
    return b + (tl & 63) * 256;
  };
  const float cf = a.scal_f[0];
  const int64_t tb = (int64_t)tt * 256;   // first token of the tile in the block
  const int64_t vb = (int64_t)vt * 256;   // first vocabulary row of the tile in the chunk
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.St + vb * a.lds, (uint64_t)max<int64_t>(0, min<int64_t>(256, a.vrows - vb)) * (uint64_t)a.lds * 4u);
  // this tile's teacher entries: [e0, e1) of a.ent
  const int gtt = a.gtt0 + tt;
  const int64_t key = (int64_t)gtt * a.ldk + a.gvt0 + vt;
  const uint32_t bb = a.bbase[gtt];
  const uint32_t e0 = bb + a.bstart[key], e1 = bb + a.bstart[key + 1];
  f32x4 x[2][16];
  auto load = [&](int g, f32x4 (&dst)[16]) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int v = 2 * (rp + 16 * j) + r;  // vocabulary row in the tile (rows past vrows read as zero)
        const uint32_t off = ((uint32_t)v * (uint32_t)a.lds + (uint32_t)(tb + 64 * g + 4 * q)) * 4u;
        dst[2 * j + r] = __builtin_bit_cast(f32x4, buf_load16(rs, off));
      }
  };
  load(0, x[0]);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    if (g < 3) load(g + 1, x[(g + 1) & 1]);
    float l2[4];
    bool keep[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t t = tb + 64 * g + 4 * q + k;
      keep[k] = t < a.rows && (a.mask ? a.mask[t] != 0 : true);
      l2[k] = keep[k] ? a.lse2[t] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int pi = rp + 16 * j;  // pair: vocabulary rows 2 pi, 2 pi + 1 of the tile
      const bool v0ok = vb + 2 * pi < a.vrows, v1ok = vb + 2 * pi + 1 < a.vrows;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int tl = 64 * g + 4 * q + k;
        const float g0 = keep[k] && v0ok ? cf * fast_exp2(fmaf(x[g & 1][2 * j][k], a.c, -l2[k])) : 0.f;
        const float g1 = keep[k] && v1ok ? cf * fast_exp2(fmaf(x[g & 1][2 * j + 1][k], a.c, -l2[k])) : 0.f;
        const int pos = ((((pi >> 2) ^ (tl & 31)) << 2) | (pi & 3)) * 2;  // bf16 offset of the pair
        *reinterpret_cast<uint32_t*>(row(tl) + pos) = pack_bf16x2(g0, g1);
      }
    }
  }
  __syncthreads();
  // the teacher entries replace the dense values at their (token, id)
  if (e1 > e0) {
    for (uint32_t e = e0 + (uint32_t)th; e < e1; e += 256) {
      const uint32_t xe = a.ent[e];
      const int tl = xe & 255, vr = (xe >> 8) & 255;
      row(tl)[((vr >> 3) ^ (tl & 31)) * 8 + (vr & 7)] = (uint16_t)(xe >> 16);
    }
    __syncthreads();
  }
#pragma unroll 4
  for (int e = th; e < 256 * 32; e += 256) {
    const int tl = e >> 5, c = e & 31;
    const u32x4 v = *reinterpret_cast<const u32x4*>(row(tl) + ((c ^ (tl & 31)) * 8));
    *reinterpret_cast<u32x4*>(a.G + (tb + tl) * a.ldg + vb + c * 8) = v;
  }
}

// The tiles of one (block, chunk) alone (the first chunk of a block, and
// every chunk in the one-gradient-buffer plan).  Grid: total padded to 8.
__global__ void __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) k_sgrad(SgradArgs a) {
  KD_DECLARE_STAGES(st, 256, 256);
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  if (id >= a.total) return;
  sgrad_tile(a, id, st);
}

// h^T of one token block: hT[m, t] = h[t0 + t, m] for t < rows, zero for
// rows <= t < ldt (the padded block), so that the dW contraction reads its h
// operand k-contiguous.  A workgroup moves a 64 (token) x 64 (hidden) tile
// through LDS: 16-byte reads along the hidden axis, 4-byte writes (two
// tokens) along the token axis.  Grid: (ldt / 64, H / 64).
__global__ void __launch_bounds__(256) k_transpose_h(const uint16_t* __restrict__ h, int64_t rows, int64_t H,
                                                      uint16_t* __restrict__ hT, int64_t ldt) {
  __shared__ uint16_t tile[64][66];  // [token][hidden], two spare columns of bank skew
  const int64_t t0 = (int64_t)blockIdx.x * 64, m0 = (int64_t)blockIdx.y * 64;
  const int tid = threadIdx.x;
#pragma unroll
  for (int e = tid; e < 64 * 8; e += 256) {
    const int t = e >> 3, c = e & 7;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (t0 + t < rows) v = *reinterpret_cast<const u32x4*>(h + (t0 + t) * H + m0 + c * 8);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      tile[t][c * 8 + 2 * q] = (uint16_t)(v[q] & 0xFFFFu);
      tile[t][c * 8 + 2 * q + 1] = (uint16_t)(v[q] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int e = tid; e < 64 * 32; e += 256) {
    const int m = e >> 5, q = e & 31;  // hidden row, token pair
    const uint32_t x = (uint32_t)tile[2 * q][m] | ((uint32_t)tile[2 * q + 1][m] << 16);
    *reinterpret_cast<uint32_t*>(hT + (m0 + m) * ldt + t0 + 2 * q) = x;
  }
}

// dH (over the chunk's vocabulary) and dW (over the block's tokens) from G.
// Work ids [0, ndh) are dH tiles (hidden tile x token tile, K = vocabulary);
// the rest are dW tiles (hidden tile x vocabulary tile, K = tokens).  Both
// are computed transposed so that a lane stores 4 consecutive hidden units:
//   dH^T[m, t] = sum_v W[v, m] G[t, v]      (W rows read with transposed LDS reads)
//   dW^T[m, v] = sum_t hT[m, t] G[t, v]     (G rows read with transposed LDS reads)
struct BwdArgs {
  const uint16_t* W;      // chunk origin [vrows, H]
  const uint16_t* hT;     // the block's h^T [H, ldt] (k_transpose_h)
  int64_t ldt;
  const uint16_t* G;      // [*, ldg]
  float* dH;              // block origin [rows, H] (nullable)
  float* dW;              // chunk origin [vrows, H] (nullable)
  int64_t vrows, H, rows; // valid rows
  int nht, ntt, nvt, ndh, ndw, ldg, grows;  // grows = allocated rows of G
  int ndh_pad, ndw_pad;   // segment sizes rounded up to multiples of 8
  int gm_dh, gm_dw;       // hidden-tile group sizes of the two rasters
  int acc_dh, acc_dw;     // accumulate (1) or overwrite (0)
  // The last hidden tile when H % 256 is 64 or 128: rem_mi (1 or 2) 32-row
  // subtiles per wave instead of 4 (a 64 or 128-row tile, all rows valid),
  // else 0 (a full 256-row tile, its rows past H computed and dropped).  Its
  // dH tiles read W's last 64 rem_mi columns from WTr, a k-contiguous copy
  // ([64 rem_mi, ldwr], chunk origin, zero past V; k_transpose_h of W).
  int rem_mi;
  const uint16_t* WTr;
  int64_t ldwr;
};

// One gradient-contraction tile: hidden tile mt (rows mt * 256 ...) by token
// tile (dH) or vocabulary tile (dW) nt, 64 MI hidden rows (MI = 4: the full
// 256; fewer for the last tile of an H that is not a multiple of 256).
// (At H = 2880, 192-row tiles throughout, 2880 = 15 x 192, gave bitwise the
// same results but ran slower: a fourth more fragment reads and loads per
// flop.)
template <int MI>
__device__ __forceinline__ void bwd_contract(const BwdArgs& a, bool dh, int mt, int nt, Stages st) {
  constexpr int BM = 256;  // hidden-tile pitch
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w & 1, wn = w >> 1;
  f32x16 acc[MI][4];
  float* out;
  int64_t nvalid;
  int acc_mode;
  if (dh) {
    LoaderKC<256> lb;
    lb.init(a.G + (int64_t)nt * 256 * a.ldg, (int64_t)a.grows - (int64_t)nt * 256, a.ldg);
    const int nk = (int)((a.vrows + kBK - 1) / kBK);
    if constexpr (MI == 4) {
      LoaderTR la;
      la.init(a.W, a.vrows, a.H, mt * BM);
      gemm_tile<MI, 4>(la, lb, nk, st, acc);
    } else {
      LoaderKC<64 * MI> la;
      la.init(a.WTr, a.H - (int64_t)mt * BM, a.ldwr);
      gemm_tile<MI, 4>(la, lb, nk, st, acc);
    }
    out = a.dH;
    nvalid = a.rows;
    acc_mode = a.acc_dh;
  } else {
    LoaderKC<64 * MI> la;
    LoaderTR lb;
    la.init(a.hT + (int64_t)mt * BM * a.ldt, a.H - (int64_t)mt * BM, a.ldt);
    lb.init(a.G, a.grows, a.ldg, nt * 256);
    gemm_tile<MI, 4>(la, lb, (int)((a.rows + kBK - 1) / kBK), st, acc);
    out = a.dW;
    nvalid = a.vrows;
    acc_mode = a.acc_dw;
  }
  // The wave's (32 MI) (m) x 128 (n) block leaves through a private 32 KiB
  // LDS stage (free after gemm_tile), 64 columns n at a time: each lane
  // writes its 4 consecutive m of one n (16-byte chunk m/4 of row n stored
  // at position (m/4) ^ (n & 31), so the 32 columns of one write land in
  // different banks), then every row n leaves as one segment of up to 512
  // bytes (32 lanes x 16 bytes, the first 8 MI lanes holding the wave's m)
  // instead of 32-byte pieces of 32 rows per store.  Accumulating reads the
  // old values the same coalesced way (range-checked: zeros past the
  // output's rows; lanes past the wave's m or past H read and store nothing).
  {
    const int w = threadIdx.x >> 6;
    float* stg = reinterpret_cast<float*>(w == 0 ? st.a0 : w == 1 ? st.a1 : w == 2 ? st.b0 : st.b1);
    const int64_t m0 = (int64_t)mt * BM + wm * (32 * MI);  // the wave's first m
    const int64_t n0 = (int64_t)nt * 256 + wn * 128;       // the wave's first n
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(out, (uint64_t)nvalid * (uint64_t)a.H * 4u);
    const int c = lane & 31;  // 16-byte chunk of a row: m = m0 + 4c .. 4c+3
    // H % 64 == 0: a chunk is all in or all out
    const bool m_ok = c < 8 * MI && m0 + 4 * c < a.H;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int j = 2 * half + jj;
        const int nl = 32 * jj + (lane & 31);  // row of the stage
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int ml = acc_row(i, 4 * q, lane);  // 4-aligned m within the wave's block
            const f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
            *reinterpret_cast<f32x4*>(stg + nl * 128 + (((ml >> 2) ^ (nl & 31)) << 2)) = v;
          }
      }
      __builtin_amdgcn_wave_barrier();
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      // rows r = 2k + (lane >> 5) of this half, k = 0..31; a lane with no m
      // reads at an offset past every output (range check: zeros, no traffic)
      f32x4 old[32];
      if (acc_mode) {
#pragma unroll
        for (int k = 0; k < 32; ++k) {
          const int64_t n = n0 + 64 * half + 2 * k + (lane >> 5);
          const uint32_t off = m_ok ? (uint32_t)((n * a.H + m0 + 4 * c) * 4) : 0xFFFFFFF0u;
          old[k] = __builtin_bit_cast(f32x4, buf_load16(ro, off));
        }
      }
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        const int nl = 2 * k + (lane >> 5);
        const int64_t n = n0 + 64 * half + nl;
        f32x4 v = *reinterpret_cast<const f32x4*>(stg + nl * 128 + ((c ^ (nl & 31)) << 2));
        if (acc_mode) v += old[k];
        if (n < nvalid && m_ok) *reinterpret_cast<f32x4*>(out + n * a.H + m0 + 4 * c) = v;
      }
      __builtin_amdgcn_wave_barrier();
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
  }
}

// The gradient-contraction workgroup with linear id L of the k_bwd grid.
__device__ __forceinline__ void bwd_tile(const BwdArgs& a, int L, Stages st) {
  int mt, nt;
  bool dh;
  if (L < a.ndh_pad) {
    const int id = xcd_remap(L, a.ndh_pad);
    if (id >= a.ndh) return;
    grouped(id, a.nht, a.ntt, a.gm_dh, mt, nt);
    dh = true;
  } else {
    const int id = xcd_remap(L - a.ndh_pad, a.ndw_pad);
    if (id >= a.ndw) return;
    grouped(id, a.nht, a.nvt, a.gm_dw, mt, nt);
    dh = false;
  }
  const int mi = mt == a.nht - 1 ? a.rem_mi : 0;
  if (mi == 1)
    bwd_contract<1>(a, dh, mt, nt, st);
  else if (mi == 2)
    bwd_contract<2>(a, dh, mt, nt, st);
  else
    bwd_contract<4>(a, dh, mt, nt, st);
}

// Grid: [0, ndh_pad) dH work, then [ndh_pad, ndh_pad + ndw_pad) dW work;
// inside each segment the 8 XCDs get contiguous work ranges (idle padding
// workgroups exit at once).  dH tiles come first: their K loop (the chunk's
// vocabulary) is the longer one.
__global__ void __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) k_bwd(BwdArgs a) {
  KD_DECLARE_STAGES(st, 256, 256);
  bwd_tile(a, blockIdx.x, st);
}

// The contractions of one (token block, vocabulary chunk) and the pass-2
// tiles of the next one, into the other gradient buffer, in one launch:
// grid = k_bwd's grid, then p_pad (a multiple of 8) pass-2 workgroups.  The
// dH tiles (longest) are dispatched first and the short pass-2 tiles last,
// so they fill the contractions' uneven end instead of a launch boundary.
__global__ void __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
k_bwd_pass2(BwdArgs g, Pass2Args p, int p_pad) {
  KD_DECLARE_STAGES(st, 256, 256);
  const int nb = g.ndh_pad + g.ndw_pad;
  if ((int)blockIdx.x < nb) {
    bwd_tile(g, blockIdx.x, st);
  } else {
    const int id = xcd_remap((int)blockIdx.x - nb, p_pad);
    if (id < p.total) pass2_tile(p, id, st);
  }
}

// Sequence-chunk schedule: the contractions of one chunk of a token block and
// the gradient tiles of the block's next chunk, into the other gradient
// buffer, in one launch.  Grid: the dH work (ndh_pad ids), then the gradient
// tiles (s_pad, a multiple of 8), then the dW work (ndw_pad).  The long dH
// tiles fill 3/4 of the CUs; the HBM-bound gradient tiles stream on the rest
// beside them (a few CUs get far more bandwidth each than all CUs at once),
// and the dW tiles follow.
__global__ void __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
k_bwd_sgrad(BwdArgs g, SgradArgs sg, int s_pad) {
  KD_DECLARE_STAGES(st, 256, 256);
  const int L = blockIdx.x;
  if (L < g.ndh_pad) {
    bwd_tile(g, L, st);
  } else if (L < g.ndh_pad + s_pad) {
    const int id = xcd_remap(L - g.ndh_pad, s_pad);
    if (id < sg.total) sgrad_tile(sg, id, st);
  } else {
    bwd_tile(g, L - s_pad, st);
  }
}

}  // namespace kd
