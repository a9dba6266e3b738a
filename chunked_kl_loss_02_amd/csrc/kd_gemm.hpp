// Tile engine for the bf16 MFMA contractions of the fused chunked KL loss.
//
// One workgroup = 256 threads = 4 wave64s arranged 2 (M) x 2 (N).  A wave
// owns a (32*MI) x (32*NI) block of the output tile, held in MI*NI
// v_mfma_f32_32x32x16_bf16 accumulators (16 fp32 per lane each).  K advances
// 64 at a time (four MFMA sub-steps of 16) through two LDS stages per
// operand, with one barrier per step, in the middle: each sub-step has its
// own set of fragment registers, sub-steps 2 and 3 read theirs under the
// MFMAs of sub-steps 0 and 1, and after the barrier the MFMAs of sub-steps 2
// and 3 cover the fetch of the next stage's first two sub-steps.  The
// barrier also frees the stage just consumed, and the loads of the step
// after next go into it right away, so global data has a full step of MFMAs
// to arrive.
//
// Operands are loaded with raw buffer loads whose range ends exactly at the
// last valid row: out-of-range rows read as zero, which covers the ragged
// vocabulary, token and chunk edges without branches in the main loop.
//
// LDS layout of an operand stage: rows (M or N index) of 64 bf16 = 8 chunks
// of 16 B; chunk c of row r lives at chunk position c ^ swz(r) with
// swz(r) = (r & 7) ^ ((r >> 3) & 3).  The ds_read_b128 of 16 consecutive rows
// (one MFMA operand fetch) then touches 16 distinct 16-byte bank groups, and
// swz does not depend on bits >= 5 of r, so the fragment reads of the 32-row
// subtiles of a wave differ only by an immediate offset.  The four stages
// (A0, A1, B0, B1) are distinct LDS objects so the compiler may move the
// loads into one stage across the fragment reads of the other.
//
// Two operand layouts are supported, both loaded global -> LDS directly
// (buffer_load_dwordx4 ... lds):
//   KC : element (row, k) at base + row*ld + k   (k contiguous; e.g. W, h for S = W h^T)
//   TR : element (row, k) at base + k*ld + row   (row contiguous; e.g. W in dH = G W),
//        read out of LDS with transposing fragment reads.
#pragma once
#include "kd_common.hpp"

namespace kd {

constexpr int kBK = 64;
constexpr int kThreads = 256;

__device__ __forceinline__ int lds_swz(int r) { return (r & 7) ^ ((r >> 3) & 3); }
// offset in bf16 elements of chunk `c` of row `r` in a [rows][64] stage
__device__ __forceinline__ int lds_off(int r, int c) { return (r << 6) + ((c ^ lds_swz(r)) << 3); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Loader for a tile of R rows x 64 k of a k-contiguous operand, global ->
// LDS without registers.  One wave instruction fills 8 consecutive LDS rows
// (1 KiB, lane l at row 8q + l/8, chunk position l%8), so each lane fetches
// the logical chunk that the swizzle maps to its slot.  Completion is
// tracked by vmcnt.
template <int R>
struct LoaderKC {
  static constexpr int NQ = R / 32;  // wave instructions per wave per k-step
  static constexpr int kVmem = NQ;   // vector-memory instructions per k-step
  static constexpr int kReads = 1;   // LDS read instructions per MFMA fragment
  __amdgpu_buffer_rsrc_t rs;
  uint32_t voff[NQ];
  int w;

  // base: address of (row 0 of the tile, k = 0); rows_left: valid rows from base
  __device__ __forceinline__ void init(const uint16_t* base, int64_t rows_left, int64_t ld) {
    const int lane = threadIdx.x & 63;
    w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t ldb = (uint32_t)(ld * 2);
    rs = make_rsrc(base, rows_left > 0 ? (uint64_t)rows_left * (uint64_t)ldb : 0);
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int q = w * NQ + j;
      const int r = 8 * q + (lane >> 3);
      voff[j] = (uint32_t)r * ldb + (uint32_t)((lane & 7) ^ lds_swz(r)) * 16u;
    }
  }
  // k-step kt into stage `s` ([R][64] bf16)
  __device__ __forceinline__ void issue(int kt, uint16_t* s) const {
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      uint16_t* dst = s + (w * NQ + j) * 8 * kBK;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)dst, 16, voff[j],
                                               __builtin_amdgcn_readfirstlane(kt * (kBK * 2)), 0, 0);
    }
  }
  // MFMA fragment of sub-step s: row rbase + lane % 32, k = 16 s + 8 (lane / 32) + 0..7
  static __device__ __forceinline__ bf16x8 frag(const uint16_t* st, int rbase, int s, int lane) {
    return __builtin_bit_cast(bf16x8,
                              *reinterpret_cast<const u32x4*>(st + lds_off(rbase + (lane & 31), 2 * s + (lane >> 5))));
  }
};

// Loader for a tile of 256 rows x 64 k of a row-contiguous operand (element
// (row, k) at base + k*ld + row: W or h or G contracted over their leading
// index), global -> LDS without registers and without a transpose: the stage
// holds the 64 k-rows as they are in memory ([64][256] bf16, 512 B per row),
// and the MFMA fragments are read with ds_read_b64_tr_b16, which hands lane
// i of each 16-lane group 4 consecutive k of column i from the 4 rows its
// group addresses.  16-byte chunk c of k-row r sits at position
// c ^ kTrMask[r & 3]; the masks {0, 6, 10, 12} put the 4 rows x 2 (or 4)
// chunks of one transposed read in distinct bank groups.
struct LoaderTR {
  static constexpr int NQ = 8;       // 64 rows x 512 B = 32 KiB = 8 x 1 KiB per wave
  static constexpr int kVmem = NQ;
  static constexpr int kReads = 2;
  __amdgpu_buffer_rsrc_t rs;
  uint32_t voff[NQ];
  uint32_t step_bytes;  // 64 k-rows
  int w;

  static __device__ __forceinline__ int trm(int r) { return (0xCA60 >> (4 * (r & 3))) & 15; }

  // base: address of (row 0, k = 0) of the operand's k-origin; rows are the
  // contiguous dimension; row0: first row of the tile; k_left: valid k rows.
  __device__ __forceinline__ void init(const uint16_t* base, int64_t k_left, int64_t ld, int row0) {
    const int lane = threadIdx.x & 63;
    w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t ldb = (uint32_t)(ld * 2);
    step_bytes = (uint32_t)kBK * ldb;
    rs = make_rsrc(base, k_left > 0 ? (uint64_t)k_left * (uint64_t)ldb : 0);
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int r = 2 * (w * NQ + j) + (lane >> 5);  // k-row of the stage
      const int c = (lane & 31) ^ trm(r);           // logical chunk landing in this lane's slot
      voff[j] = (uint32_t)r * ldb + (uint32_t)row0 * 2u + (uint32_t)c * 16u;
    }
  }
  // the k-step offset goes into the per-lane offset: rows past k_left must
  // fail the range check, which covers the per-lane offset only
  __device__ __forceinline__ void issue(int kt, uint16_t* st) const {
    const uint32_t o = (uint32_t)kt * step_bytes;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      uint16_t* dst = st + (w * NQ + j) * 512;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)dst, 16, voff[j] + o, 0, 0, 0);
    }
  }
  static __device__ __forceinline__ bf16x8 frag(const uint16_t* st, int rbase, int s, int lane) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    const int g = lane >> 4, i = lane & 15;
    const int col = rbase + 16 * (g & 1) + 4 * (i & 3);  // first of the 4 columns this lane addresses
    const int kb = 16 * s + 8 * (g >> 1) + (i >> 2);
    v4i16 v[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = kb + 4 * h;
      const int pos = (((col >> 3) ^ trm(r)) << 3) + (col & 7);
      v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16*)(st + r * 256 + pos));
    }
    const short __attribute__((ext_vector_type(8))) x = {v[0][0], v[0][1], v[0][2], v[0][3],
                                                         v[1][0], v[1][1], v[1][2], v[1][3]};
    return __builtin_bit_cast(bf16x8, x);
  }
};

// The four operand stages of one workgroup.
struct Stages {
  uint16_t *a0, *a1, *b0, *b1;
};

template <int MI, int NI, class LA, class LB>
__device__ __forceinline__ void load_frags(const uint16_t* __restrict__ As, const uint16_t* __restrict__ Bs,
                                           bf16x8 (&a)[MI], bf16x8 (&b)[NI], int arow0, int brow0, int lane, int s) {
#pragma unroll
  for (int i = 0; i < MI; ++i) a[i] = LA::frag(As, arow0 + 32 * i, s, lane);
#pragma unroll
  for (int j = 0; j < NI; ++j) b[j] = LB::frag(Bs, brow0 + 32 * j, s, lane);
}

template <int MI, int NI>
__device__ __forceinline__ void mfma_substep(f32x16 (&acc)[MI][NI], const bf16x8 (&a)[MI], const bf16x8 (&b)[NI]) {
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
}

// Instruction-order hints spread evenly over a region of NM MFMAs: its NR
// fragment reads and NV global loads follow the MFMAs at evenly spaced
// positions (16 reads and 16 loads over 32 MFMAs alternate; 24 reads take 3
// of every 4).  Bunched instead (the reads one per MFMA from the start, the
// loads one per MFMA in the first half) pass 1 ran 4 %, pass 2 5 % and k_bwd
// 1-5 % slower: many memory instructions issued back to back hold up the
// MFMAs behind them.
template <int NM, int NR, int NV, int Q = 0, int TM = NM, int TR = NR, int TV = NV>
__device__ __forceinline__ void sched_even() {
  if constexpr (NM > 0) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    // Bresenham: the q-th MFMA is followed by the reads and loads whose even
    // share of the region ends there (loads offset by half a slot)
    constexpr int r = (Q + 1) * TR / TM - Q * TR / TM;
    constexpr int v = ((2 * Q + 2) * TV + TM) / (2 * TM) - ((2 * Q) * TV + TM) / (2 * TM);
    if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);
    if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x010, v, 0);
    sched_even<NM - 1, NR - r, NV - v, Q + 1, TM, TR, TV>();
  }
}

__device__ __forceinline__ void wait_all() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory"); }

// One k-step over stage (ca, cb), whose successor (na, nb) is already in
// flight; fragment set s (a[s], b[s]) holds sub-step s:
//   region 1: the MFMAs of sub-steps 0 and 1 interleaved with the fragment
//             reads of sub-steps 2 and 3; then wait for this wave's loads
//             into (na, nb) and its LDS reads, and meet the other waves;
//   region 2: (ca, cb) is free: the loads of step kn go into it, and the
//             fragments of sub-steps 0 and 1 of (na, nb) load, under the
//             MFMAs of sub-steps 2 and 3.
// On entry sets 0 and 1 hold sub-steps 0 and 1 of (ca, cb); on exit of (na, nb).
template <int MI, int NI, class LA, class LB>
__device__ __forceinline__ void kstep(LA& la, LB& lb, int kn, uint16_t* ca, uint16_t* cb, const uint16_t* na,
                                      const uint16_t* nb, f32x16 (&acc)[MI][NI], bf16x8 (&a)[4][MI],
                                      bf16x8 (&b)[4][NI], int arow0, int brow0, int lane) {
  constexpr int NM = MI * NI, NR = MI * LA::kReads + NI * LB::kReads;
  constexpr int NVM = LA::kVmem + LB::kVmem;
  load_frags<MI, NI, LA, LB>(ca, cb, a[2], b[2], arow0, brow0, lane, 2);
  load_frags<MI, NI, LA, LB>(ca, cb, a[3], b[3], arow0, brow0, lane, 3);
  mfma_substep<MI, NI>(acc, a[0], b[0]);
  mfma_substep<MI, NI>(acc, a[1], b[1]);
  sched_even<2 * NM, 2 * NR, 0>();
  wait_all();
  __syncthreads();
  la.issue(kn, ca);
  lb.issue(kn, cb);
  load_frags<MI, NI, LA, LB>(na, nb, a[0], b[0], arow0, brow0, lane, 0);
  load_frags<MI, NI, LA, LB>(na, nb, a[1], b[1], arow0, brow0, lane, 1);
  mfma_substep<MI, NI>(acc, a[2], b[2]);
  mfma_substep<MI, NI>(acc, a[3], b[3]);
  sched_even<2 * NM, 2 * NR, NVM>();
}

// Full K loop for one output tile: acc = A_tile * B_tile^T over nk steps,
// alternating between the stage pairs (a0, b0) and (a1, b1).  Ends with
// every wave past a barrier that follows its last reads of the stages, so
// the LDS can be reused (or the next tile started) right after.  The last
// two steps re-fetch step nk - 1 into the stage they free (never consumed),
// which keeps every step identical.
template <int MI, int NI, class LA, class LB>
__device__ __forceinline__ void gemm_tile(LA& la, LB& lb, int nk, const Stages& st, f32x16 (&acc)[MI][NI]) {
  constexpr int NVM = LA::kVmem + LB::kVmem;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int arow0 = (w & 1) * 32 * MI;
  const int brow0 = (w >> 1) * 32 * NI;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = f32x16{};
  if (nk <= 0) return;
  bf16x8 a[4][MI], b[4][NI];
  // an odd step count starts in the second half of the loop body (step 0 in
  // stage 1), so that one loop body, with no separate tail, runs every step
  const bool odd = nk & 1;
  uint16_t* sa = odd ? st.a1 : st.a0;
  uint16_t* sb = odd ? st.b1 : st.b0;
  la.issue(0, sa);
  lb.issue(0, sb);
  la.issue(nk > 1 ? 1 : 0, odd ? st.a0 : st.a1);
  lb.issue(nk > 1 ? 1 : 0, odd ? st.b0 : st.b1);
  // step 0 has landed once at most step 1's loads are outstanding
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(NVM) : "memory");
  __syncthreads();
  load_frags<MI, NI, LA, LB>(sa, sb, a[0], b[0], arow0, brow0, lane, 0);
  load_frags<MI, NI, LA, LB>(sa, sb, a[1], b[1], arow0, brow0, lane, 1);
  const int last = nk - 1;
  for (int kt = odd ? -1 : 0; kt < last; kt += 2) {
    if (kt >= 0) kstep<MI, NI>(la, lb, kt + 2 < nk ? kt + 2 : last, st.a0, st.b0, st.a1, st.b1, acc, a, b, arow0, brow0, lane);
    kstep<MI, NI>(la, lb, kt + 3 < nk ? kt + 3 : last, st.a1, st.b1, st.a0, st.b0, acc, a, b, arow0, brow0, lane);
  }
  // the last region read the idle stage's first fragments and loaded into the
  // stage it freed: let every wave finish both before anyone reuses the stages
  wait_all();
  __syncthreads();
}

// Declares the four stages of a (BM x 64) + (BN x 64) workgroup in LDS.
#define KD_DECLARE_STAGES(name, BM, BN)                                   \
  __shared__ __attribute__((aligned(16))) uint16_t name##_a0[(BM) * kBK]; \
  __shared__ __attribute__((aligned(16))) uint16_t name##_a1[(BM) * kBK]; \
  __shared__ __attribute__((aligned(16))) uint16_t name##_b0[(BN) * kBK]; \
  __shared__ __attribute__((aligned(16))) uint16_t name##_b1[(BN) * kBK]; \
  Stages name{name##_a0, name##_a1, name##_b0, name##_b1}

// Position of accumulator element e of subtile (i, j) for this lane, relative
// to the wave's block: row (M) = 32 i + 8 (e >> 2) + 4 (lane >> 5) + (e & 3),
// column (N) = 32 j + (lane & 31).
__device__ __forceinline__ int acc_row(int i, int e, int lane) { return 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3); }
__device__ __forceinline__ int acc_col(int j, int lane) { return 32 * j + (lane & 31); }

// Maps a linear workgroup id to a work id so that each of the 8 XCDs (which
// receive workgroups round-robin) gets a contiguous range of work ids.
__device__ __forceinline__ int xcd_remap(int L, int padded_total) {
  const int per = padded_total >> 3;
  return (L & 7) * per + (L >> 3);
}

// Grouped raster over an (nt x nu) grid of tiles: consecutive ids cover gt
// tiles of the first index before moving to the next unit of the second, so
// workgroups running together share both operand tiles through L2.
__device__ __forceinline__ void grouped(int id, int nt, int nu, int gt, int& t, int& u) {
  const int gsz = gt * nu;
  const int g = id / gsz;
  const int first = g * gt;
  const int span = min(nt - first, gt);
  const int w = id - g * gsz;
  t = first + w % span;
  u = w / span;
}

}  // namespace kd
