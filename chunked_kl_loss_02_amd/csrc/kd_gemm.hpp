// Tile engine for the bf16 MFMA contractions of the fused chunked KL loss.
//
// One workgroup = 256 threads = 4 wave64s arranged 2 (M) x 2 (N).  A wave
// owns a (32*MI) x (32*NI) block of the output tile, held in MI*NI
// v_mfma_f32_32x32x16_bf16 accumulators (16 fp32 per lane each).  K advances
// 64 at a time through a two-stage LDS ring; global loads for step k+1 are in
// flight while the MFMAs of step k run, so one barrier per step suffices.
//
// Operands are loaded with raw buffer loads whose range ends exactly at the
// last valid row: out-of-range rows read as zero, which covers the ragged
// vocabulary, token and chunk edges without branches in the main loop.
//
// LDS layout of a stage: rows (M or N index) of 64 bf16 = 8 chunks of 16 B;
// chunk c of row r lives at chunk position c ^ (r & 7) ^ ((r >> 3) & 7), so
// the ds_read_b128 of eight consecutive rows (one MFMA operand fetch) and the
// row-wise / transposed ds_write_b128 of the loaders hit distinct banks.
//
// Two operand layouts are supported:
//   KC : element (row, k) at base + row*ld + k   (k contiguous; e.g. W, h for S = W h^T)
//   RC : element (row, k) at base + k*ld + row   (row contiguous; e.g. W in dH = G W)
// RC tiles are loaded as 8x8 bf16 blocks and transposed in registers
// (v_perm_b32) before the LDS write, so MFMA always reads k-contiguous LDS.
#pragma once
#include "kd_common.hpp"

namespace kd {

constexpr int kBK = 64;
constexpr int kThreads = 256;

__device__ __forceinline__ int lds_swz(int r) { return (r & 7) ^ ((r >> 3) & 7); }
// offset in bf16 elements of chunk `c` of row `r` in a [rows][64] stage
__device__ __forceinline__ int lds_off(int r, int c) { return (r << 6) + ((c ^ lds_swz(r)) << 3); }

// Loader for a tile of R rows x 64 k of a k-contiguous operand.
template <int R>
struct LoaderKC {
  static constexpr int NV = R / 32;  // 16-byte loads per thread
  u32x4 v[NV];
  __amdgpu_buffer_rsrc_t rs;
  uint32_t off0;    // per-thread byte offset at k-step 0
  uint32_t ldb;     // leading dimension in bytes
  int r0, c0;

  // base: address of (row 0 of the tile, k = 0); rows_left: valid rows from base
  __device__ __forceinline__ void init(const uint16_t* base, int64_t rows_left, int64_t ld) {
    const int tid = threadIdx.x;
    ldb = (uint32_t)(ld * 2);
    rs = make_rsrc(base, rows_left > 0 ? (uint64_t)rows_left * (uint64_t)ldb : 0);
    c0 = tid & 7;
    r0 = tid >> 3;
    off0 = (uint32_t)r0 * ldb + (uint32_t)c0 * 16u;
  }
  __device__ __forceinline__ void load(int kt) {
    const uint32_t o = off0 + (uint32_t)kt * (kBK * 2);
#pragma unroll
    for (int j = 0; j < NV; ++j) v[j] = buf_load16(rs, o + (uint32_t)j * 32u * ldb);
  }
  __device__ __forceinline__ void store(uint16_t* s) const {
#pragma unroll
    for (int j = 0; j < NV; ++j)
      *reinterpret_cast<u32x4*>(s + lds_off(r0 + 32 * j, c0)) = v[j];
  }
};

// Loader for a tile of R rows x 64 k of a row-contiguous operand (transposed
// in registers).  R must be a multiple of 8 and R/8 * 8 <= 256 threads.
template <int R>
struct LoaderRC {
  static constexpr int NB = R / 8;  // 8-row blocks across the tile
  u32x4 v[8];
  __amdgpu_buffer_rsrc_t rs;
  uint32_t off0;
  uint32_t ldb;
  int mb, kb;
  bool active;

  // base: address of (row 0, k = 0) of the operand's k-origin; rows are the
  // contiguous dimension; row0: first row of the tile; k_left: valid k rows.
  __device__ __forceinline__ void init(const uint16_t* base, int64_t k_left, int64_t ld, int row0) {
    const int tid = threadIdx.x;
    ldb = (uint32_t)(ld * 2);
    rs = make_rsrc(base, k_left > 0 ? (uint64_t)k_left * (uint64_t)ldb : 0);
    mb = tid % NB;
    kb = tid / NB;
    active = kb < 8;
    off0 = (uint32_t)(kb * 8) * ldb + (uint32_t)(row0 + mb * 8) * 2u;
  }
  __device__ __forceinline__ void load(int kt) {
    if (!active) return;
    const uint32_t o = off0 + (uint32_t)kt * (uint32_t)kBK * ldb;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = buf_load16(rs, o + (uint32_t)j * ldb);
  }
  __device__ __forceinline__ void store(uint16_t* s) const {
    if (!active) return;
    // v[kk].d[q] holds elements (2q, 2q+1) of k-row kk.  Output row mm holds
    // k = 0..7 of column mm: dword p = (elem mm of k-row 2p, elem mm of 2p+1).
#pragma unroll
    for (int mm = 0; mm < 8; ++mm) {
      const uint32_t sel = (mm & 1) ? 0x07060302u : 0x05040100u;
      u32x4 y;
#pragma unroll
      for (int p = 0; p < 4; ++p) y[p] = __builtin_amdgcn_perm(v[2 * p + 1][mm >> 1], v[2 * p][mm >> 1], sel);
      *reinterpret_cast<u32x4*>(s + lds_off(mb * 8 + mm, kb)) = y;
    }
  }
};

template <bool KC, int R> struct LoaderSel;
template <int R> struct LoaderSel<true, R> { using type = LoaderKC<R>; };
template <int R> struct LoaderSel<false, R> { using type = LoaderRC<R>; };

// MFMAs of one 64-deep LDS stage.  As: [BM][64], Bs: [BN][64].
template <int MI, int NI>
__device__ __forceinline__ void mma_stage(const uint16_t* __restrict__ As, const uint16_t* __restrict__ Bs,
                                          f32x16 (&acc)[MI][NI], int arow0, int brow0, int lane) {
  const int lr = lane & 31;
  const int hk = lane >> 5;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    bf16x8 a[MI], b[NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
      a[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(As + lds_off(arow0 + 32 * i + lr, 2 * s + hk)));
#pragma unroll
    for (int j = 0; j < NI; ++j)
      b[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(Bs + lds_off(brow0 + 32 * j + lr, 2 * s + hk)));
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

// Full K loop for one output tile: acc += A_tile * B_tile^T over nk steps.
// lds must hold 2 * (BM + BN) * 64 bf16.  Ends with a barrier, so the LDS
// can be reused (or the next tile started) immediately after.
template <int MI, int NI, class LA, class LB>
__device__ __forceinline__ void gemm_tile(LA& la, LB& lb, int nk, uint16_t* lds, f32x16 (&acc)[MI][NI]) {
  constexpr int BM = 64 * MI, BN = 64 * NI;
  constexpr int STAGE = (BM + BN) * kBK;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int arow0 = (w & 1) * 32 * MI;
  const int brow0 = (w >> 1) * 32 * NI;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = f32x16{};
  if (nk <= 0) return;
  la.load(0);
  lb.load(0);
  la.store(lds);
  lb.store(lds + BM * kBK);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    uint16_t* cur = lds + (kt & 1) * STAGE;
    uint16_t* nxt = lds + ((kt + 1) & 1) * STAGE;
    const bool more = kt + 1 < nk;
    if (more) {
      la.load(kt + 1);
      lb.load(kt + 1);
    }
    mma_stage<MI, NI>(cur, cur + BM * kBK, acc, arow0, brow0, lane);
    if (more) {
      la.store(nxt);
      lb.store(nxt + BM * kBK);
    }
    __syncthreads();
  }
}

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
// token tiles before moving to the next unit, so workgroups running together
// share both operand tiles through L2.
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
