// Host side of libkdkl: argument checks, workspace plan, launch sequence and
// the optional event timing.  Everything here is synchronous argument work
// plus asynchronous launches on the caller's stream; no device allocation.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/kdkl.h"
#include "kd_kernels.hpp"
#include "kd_logits.hpp"
#include "kd_topk.hpp"

namespace {

// Default tiling (measured at H = 2880, V = 201088): token blocks of 8192;
// vocabulary chunks of 12288 for a block of at most 4096 tokens, else 8192,
// so the bf16 gradient buffer (block x chunk) stays near 100-130 MB and, with
// the chunk's W rows, inside the last-level cache; the sequence-chunk
// schedule keeps blocks of 4096 and chunks of 16384.
constexpr int kDefaultChunkV = 12288;
constexpr int kDefaultChunkVLargeBlock = 8192;
constexpr int kDefaultSeqChunkV = 16384;
constexpr int kDefaultBlockT = 8192;
constexpr int kDefaultSeqBlockT = 4096;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  if (!s || !*s) return dflt;
  return atoi(s);
}

struct Plan {
  int64_t T, H, V;
  int K;
  float tau;
  int chunk_v, block_t;
  int64_t Tb;        // tokens per block
  int ntt_max;       // token tiles in a full block
  int64_t nvt;       // vocabulary tiles of 256
  int nranges;       // pass 1: partial (max, sum) rows, one per vocabulary tile
  int gt1, gt2;      // token-tile group sizes of pass 1 / pass 2
  int gv1, gv2;      // vocabulary group sizes (take precedence when > 0)
  int gm_dh, gm_dw;  // hidden-tile group sizes of the gradient contractions
  int bm;            // hidden rows of a gradient-contraction tile
  // the last hidden tile's height in 64-row units when H % 256 is 64 or 128
  // (else 0: a full tile), and the pitch of the copy of W's last columns
  // that its dH tiles read
  int rem_mi;
  int64_t ldwr;
  int64_t ldp;       // leading dim of the pass-1 partials
  int64_t grows;     // rows of the gradient buffer
  int64_t nunits;    // (token block, vocabulary chunk) units of the gradient pass
  int ngbuf;         // gradient buffers (2: alternating between units)
  // workspace offsets (bytes); o_G, o_dhs, o_dws are meaningful only in a
  // plan made with the gradient pass (o_dhs / o_dws: fp32 staging of bf16
  // gradient outputs)
  bool seq;          // sequence-chunk schedule (stored logits of a token block)
  size_t o_S;        // seq: S^T of one block, [V, Tb] fp32
  size_t o_hT;       // h^T of one token block, [H, Tb] bf16 (gradient pass)
  size_t o_wtr;      // W's last 64 rem_mi columns, [64 rem_mi, ldwr] bf16 (gradient pass)
  size_t o_off;      // per-token pass-2 offsets [Tp] (gradient pass)
  // teacher entries by (token tile, vocabulary tile): counts / starts
  // [ntt_all, ldk] then fill cursors [ntt_all, ldk] (contiguous, cleared
  // together), token-tile bases [ntt_all + 1], entries and their flat
  // indices [T*K]
  int ntt_all, ldk;
  size_t o_bcnt, o_bcur, o_bbase, o_ent, o_enti;
  size_t o_G, o_dhs, o_dws, o_part, o_lse2, o_p, o_pm, o_s, o_neg, o_row, o_bsum, o_scal_f, o_scal_i, o_status, total;
};

constexpr uint32_t kAllFlags =
    KD_FLAG_VALIDATE | KD_FLAG_ACCUMULATE_DH | KD_FLAG_ACCUMULATE_DW | KD_FLAG_GRAD_BF16 | KD_FLAG_SEQ_CHUNK;

// Token block and vocabulary chunk a call uses (the caller's, else the
// defaults above).  seq: the sequence-chunk schedule (gradient pass only).
void tiling(const kd_problem* p, bool seq, int64_t* Tb, int64_t* cv) {
  const int64_t bt = p->block_t ? p->block_t : seq ? kDefaultSeqBlockT : kDefaultBlockT;
  int64_t tb = p->T < bt ? align256(p->T) : bt;
  if (tb == 0) tb = 256;
  *Tb = tb;
  *cv = p->chunk_v ? p->chunk_v : seq ? kDefaultSeqChunkV : tb <= 4096 ? kDefaultChunkV : kDefaultChunkVLargeBlock;
}

kd_status check(const kd_problem* p) {
  if (!p) return KD_ERR_ARG;
  if (p->T < 0 || p->H <= 0 || p->V <= 0 || p->K <= 0) return KD_ERR_ARG;
  if (!(p->tau > 0.f) || !isfinite(p->tau)) return KD_ERR_ARG;
  if ((int64_t)p->K > p->V) return KD_ERR_ARG;
  if (p->chunk_v < 0 || p->block_t < 0) return KD_ERR_ARG;
  if (p->flags & ~kAllFlags) return KD_ERR_ARG;
  if (p->H % 64 != 0) return KD_ERR_UNSUPPORTED;
  if (p->K > kd::kTeacherMaxK) return KD_ERR_UNSUPPORTED;
  if (p->chunk_v % 256 != 0 || p->block_t % 256 != 0) return KD_ERR_UNSUPPORTED;
  // Launch grids stay under 2^32 work-items (the limit of a dispatch): 64
  // per token in k_teacher, one per teacher entry in the bucket kernels
  // (whose positions are 32-bit too), and pass 1 below.
  if (p->V > (int64_t)INT32_MAX || p->T > ((int64_t)1 << 26) - 256) return KD_ERR_UNSUPPORTED;
  if (p->T * (int64_t)p->K > (int64_t)UINT32_MAX - 255) return KD_ERR_UNSUPPORTED;
  // Every kernel addresses one chunk or block operand through 32-bit buffer
  // offsets: the bf16 chunk of W and the token block of h (and its h^T), the
  // bf16 gradient buffer (block x chunk), and the fp32 gradient targets the
  // contractions read back and add to (the block's rows of dH, the chunk's
  // rows of dW, or their fp32 staging for bf16 outputs), 4 bytes an element.
  int64_t bt, cv;
  tiling(p, (p->flags & KD_FLAG_SEQ_CHUNK) != 0, &bt, &cv);
  const int64_t lim = (int64_t)UINT32_MAX;
  if (cv * p->H * 4 > lim || bt * p->H * 4 > lim || bt * cv * 2 > lim) return KD_ERR_UNSUPPORTED;
  if (256 * p->H * 2 > lim / 2) return KD_ERR_UNSUPPORTED;
  // the sequence-chunk schedule's gradient tiles read 256 stored fp32 logit
  // rows of one token block (bt columns each) through one 32-bit range
  if ((p->flags & KD_FLAG_SEQ_CHUNK) && 256 * bt * 4 > lim) return KD_ERR_UNSUPPORTED;
  // pass 1: 256 work-items per (token tile, vocabulary tile) of one block
  if (cdiv(cdiv(bt, 256) * cdiv(p->V, 256), 8) * 8 * 256 > lim) return KD_ERR_UNSUPPORTED;
  return KD_OK;
}

// Workspace plan.  with_grad: room for the gradient pass (the bf16 gradient
// tile buffer, and fp32 staging when the gradient outputs are bf16).
Plan make_plan(const kd_problem* p, bool with_grad = true, bool one_gbuf = false) {
  Plan P{};
  P.T = p->T;
  P.H = p->H;
  P.V = p->V;
  P.K = p->K;
  P.tau = p->tau;
  P.seq = with_grad && (p->flags & KD_FLAG_SEQ_CHUNK);
  int64_t tb, cv;
  tiling(p, P.seq, &tb, &cv);
  P.Tb = tb;
  P.block_t = (int)(p->block_t ? p->block_t : P.seq ? kDefaultSeqBlockT : kDefaultBlockT);
  P.chunk_v = (int)cv;
  P.ntt_max = (int)(P.Tb / 256);
  P.nvt = cdiv(P.V, 256);
  P.nranges = (int)P.nvt;
  P.gt1 = env_int("KDKL_GROUP_T1", 4);
  P.gt2 = env_int("KDKL_GROUP_T2", 4);
  P.gv1 = env_int("KDKL_GROUP_V1", 8);
  P.gv2 = env_int("KDKL_GROUP_V2", 8);
  P.gm_dh = std::max(1, env_int("KDKL_GROUP_MDH", 6));
  P.gm_dw = std::max(1, env_int("KDKL_GROUP_MDW", 4));
  P.bm = 256;
  // a 64- or 128-row last hidden tile (the copy's 32-bit offsets permitting;
  // not in the allocation-free entry point's plan, which keeps full-height
  // tiles and no copy: the results are bitwise the same, the k order of
  // every dot product being unchanged)
  P.ldwr = (P.V + 63) / 64 * 64;
  const int64_t rem = P.H % 256;
  P.rem_mi = !one_gbuf && (rem == 64 || rem == 128) && rem * P.ldwr * 2 <= (int64_t)UINT32_MAX ? (int)(rem / 64) : 0;
  if (P.gt1 < 1) P.gt1 = 1;
  if (P.gt2 < 1) P.gt2 = 1;
  P.ldp = (int64_t)P.ntt_max * 256;
  P.grows = (int64_t)P.ntt_max * 256;
  const int64_t Tp = align256(P.T);
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o += (bytes + 255) & ~size_t(255); return r; };
  // the recompute schedule alternates two gradient buffers when a call has
  // several (block, chunk) units (the next unit's pass 2 runs beside the
  // current unit's contractions)
  P.nunits = cdiv(P.T, P.Tb) * cdiv(P.V, P.chunk_v);
  P.ngbuf = !one_gbuf && (P.seq ? P.V > P.chunk_v : P.nunits > 1) ? 2 : 1;
  P.o_G = with_grad ? take((size_t)P.ngbuf * P.grows * P.chunk_v * 2) : 0;
  P.o_hT = with_grad ? take((size_t)P.H * P.Tb * 2) : 0;
  P.o_wtr = with_grad && P.rem_mi ? take((size_t)64 * P.rem_mi * P.ldwr * 2) : 0;
  P.o_off = with_grad ? take((size_t)Tp * 4) : 0;
  P.ntt_all = (int)cdiv(P.T, 256);
  P.ldk = (int)P.nvt + 1;
  const size_t nkeys = (size_t)P.ntt_all * P.ldk;
  P.o_bcnt = take(nkeys * 8);  // counts then cursors: one region
  P.o_bcur = P.o_bcnt + nkeys * 4;
  P.o_bbase = take((size_t)P.ntt_all * 4 + 4);
  P.o_ent = take((size_t)P.T * P.K * 4);
  P.o_enti = take((size_t)P.T * P.K * 4);
  P.o_S = P.seq ? take((size_t)P.V * P.Tb * 4) : 0;
  const bool stage = with_grad && (p->flags & KD_FLAG_GRAD_BF16);
  // both schedules walk token blocks in the outer loop: a block's dH is
  // final after its last chunk (staged one block at a time), a dW chunk only
  // after the last block (with several blocks its staging holds all of dW)
  const bool whole_dw = P.T > P.Tb;
  P.o_dhs = stage ? take((size_t)(P.seq ? Tp : P.Tb) * P.H * 4) : 0;
  P.o_dws = stage ? take((size_t)(whole_dw ? P.V : P.chunk_v) * P.H * 4) : 0;
  P.o_part = take((size_t)P.nranges * P.ldp * 8);
  P.o_lse2 = take((size_t)Tp * 4);
  P.o_p = take((size_t)P.T * P.K * 4);
  P.o_pm = take((size_t)P.T * P.K * 4);
  P.o_s = take((size_t)P.T * P.K * 4);
  P.o_neg = take((size_t)Tp * 4);
  P.o_row = take((size_t)Tp * 4);
  P.o_bsum = take((size_t)cdiv(Tp, 256) * 8 + 8);
  P.o_scal_f = take(64);
  P.o_scal_i = take(64);
  P.o_status = take(64);
  P.total = o;
  return P;
}

// ------------------------------------------------------------------ timing
struct TimedLaunch {
  int cls;
  hipEvent_t a, b;
};
// The optional timing facility's state, shared by every caller thread:
// g_timing / g_timing_mask are read without the lock on each launch (a
// torn read only times a launch more or less), the event lists under it.
std::atomic<bool> g_timing{false};
std::atomic<uint32_t> g_timing_mask{~0u};
std::mutex g_timing_mu;
constexpr int kTimingClasses = 12;
std::vector<TimedLaunch> g_launches;
std::vector<hipEvent_t> g_pool;

hipEvent_t pool_get() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

struct Launcher {
  hipStream_t s;
  hipError_t err = hipSuccess;
  template <class F>
  void run(int cls, F&& f) {
    if (err != hipSuccess) return;
    hipEvent_t a = nullptr, b = nullptr;
    const bool timed = g_timing.load(std::memory_order_relaxed) &&
                       ((g_timing_mask.load(std::memory_order_relaxed) >> cls) & 1u);
    if (timed) {
      std::lock_guard<std::mutex> lock(g_timing_mu);
      a = pool_get();
      b = pool_get();
      if (a) (void)hipEventRecord(a, s);
    }
    f();
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) err = e;
    if (timed && a && b) {
      (void)hipEventRecord(b, s);
      std::lock_guard<std::mutex> lock(g_timing_mu);
      g_launches.push_back({cls, a, b});
    }
  }
};

int grid_fill(int64_t n, int block) { return (int)std::max<int64_t>(1, std::min<int64_t>(cdiv(n, block), 65536)); }

struct Inputs {
  const uint16_t* h;
  const uint16_t* W;
  const int32_t* idx;
  const float* logit;
  const uint8_t* mask;
};

// Device pointers of one call: workspace regions plus where the saved
// per-token state (lse2, gathered logits) lives.
struct Bufs {
  uint16_t* G;
  uint16_t* hT;  // h^T of one token block (gradient pass)
  uint16_t* wtr;  // W's last columns, k-contiguous (gradient pass, nullable)
  float* off;    // pass-2 offsets (gradient pass)
  uint32_t *bcnt, *bcur, *bbase, *ent, *enti;  // teacher entries by tile
  float* dhs;   // fp32 staging of a bf16 dH (nullable)
  float* dws;   // fp32 staging of one chunk of a bf16 dW (nullable)
  float2* part;
  float* lse2;
  float* p;
  float* pm;
  float* s;
  float* neg;
  float* rows;
  double* bsum;
  float* scal_f;
  int64_t* scal_i;
  uint32_t* status;
};

Bufs carve(const Plan& P, void* workspace, bool with_grad) {
  char* ws = static_cast<char*>(workspace);
  Bufs b{};
  b.G = with_grad ? reinterpret_cast<uint16_t*>(ws + P.o_G) : nullptr;
  b.hT = with_grad ? reinterpret_cast<uint16_t*>(ws + P.o_hT) : nullptr;
  b.wtr = with_grad && P.rem_mi ? reinterpret_cast<uint16_t*>(ws + P.o_wtr) : nullptr;
  b.off = with_grad ? reinterpret_cast<float*>(ws + P.o_off) : nullptr;
  b.bcnt = reinterpret_cast<uint32_t*>(ws + P.o_bcnt);
  b.bcur = reinterpret_cast<uint32_t*>(ws + P.o_bcur);
  b.bbase = reinterpret_cast<uint32_t*>(ws + P.o_bbase);
  b.ent = reinterpret_cast<uint32_t*>(ws + P.o_ent);
  b.enti = reinterpret_cast<uint32_t*>(ws + P.o_enti);
  b.dhs = with_grad && P.o_dhs ? reinterpret_cast<float*>(ws + P.o_dhs) : nullptr;
  b.dws = with_grad && P.o_dws ? reinterpret_cast<float*>(ws + P.o_dws) : nullptr;
  b.part = reinterpret_cast<float2*>(ws + P.o_part);
  b.lse2 = reinterpret_cast<float*>(ws + P.o_lse2);
  b.p = reinterpret_cast<float*>(ws + P.o_p);
  b.pm = reinterpret_cast<float*>(ws + P.o_pm);
  b.s = reinterpret_cast<float*>(ws + P.o_s);
  b.neg = reinterpret_cast<float*>(ws + P.o_neg);
  b.rows = reinterpret_cast<float*>(ws + P.o_row);
  b.bsum = reinterpret_cast<double*>(ws + P.o_bsum);
  b.scal_f = reinterpret_cast<float*>(ws + P.o_scal_f);
  b.scal_i = reinterpret_cast<int64_t*>(ws + P.o_scal_i);
  b.status = reinterpret_cast<uint32_t*>(ws + P.o_status);
  return b;
}

// The saved state of the split entry points: lse2 [T] then s [T, K].
size_t saved_lse2_bytes(const Plan& P) { return (size_t)align256(align256(P.T) * 4); }
size_t saved_bytes(const Plan& P) { return saved_lse2_bytes(P) + (size_t)align256(P.T * P.K * 4) + 256; }

bool misaligned(const void* q, uintptr_t a) { return q && (reinterpret_cast<uintptr_t>(q) & (a - 1)); }

kd_status check_common(const kd_problem* p, const uint16_t* h, const uint16_t* W, const int32_t* idx,
                       const float* logit, const void* workspace) {
  const kd_status st = check(p);
  if (st != KD_OK) return st;
  if (!W || !workspace) return KD_ERR_ARG;
  if (p->T > 0 && (!h || !idx || !logit)) return KD_ERR_ARG;
  if (misaligned(h, 16) || misaligned(W, 16) || misaligned(workspace, 256) || misaligned(idx, 4) ||
      misaligned(logit, 4))
    return KD_ERR_UNSUPPORTED;
  return KD_OK;
}

// Status clear, N and the gradient coefficient, teacher distribution.
void launch_prep(Launcher& L, const Plan& P, const Inputs& in, const Bufs& b, bool validate, const float* grad) {
  hipStream_t s = L.s;
  using namespace kd;
  const int64_t T = P.T;
  if (validate) L.run(8, [&] { k_fill<<<1, 64, 0, s>>>(reinterpret_cast<float*>(b.status), 1, 0.f); });
  L.run(4, [&] { k_count<<<1, 1024, 0, s>>>(in.mask, T, P.tau, grad, b.scal_f, b.scal_i); });
  L.run(0, [&] {
    k_teacher<<<(unsigned)cdiv(T, 4), 256, 0, s>>>(in.idx, in.logit, in.mask, T, P.K, P.V, 1.0f / P.tau, b.p, b.pm,
                                                    b.neg, b.status, validate ? 1 : 0);
  });
}

// Teacher entries of kept tokens bucketed by (token tile, vocabulary tile):
// counts, the two scans, placement with their cached slots.
void launch_bucket_index(Launcher& L, const Plan& P, const Inputs& in, const Bufs& b) {
  hipStream_t s = L.s;
  using namespace kd;
  const int64_t T = P.T, n = T * P.K;
  const int64_t nkeys = (int64_t)P.ntt_all * P.ldk;
  L.run(6, [&] {
    k_fill<<<grid_fill(2 * nkeys, 256), 256, 0, s>>>(reinterpret_cast<float*>(b.bcnt), 2 * nkeys, 0.f);
  });
  L.run(6, [&] {
    k_bucket_count<<<(unsigned)cdiv(n, 256), 256, 0, s>>>(in.idx, in.mask, T, P.K, P.V, P.ldk, b.bcnt);
  });
  L.run(6, [&] { k_scan_rows<<<(unsigned)P.ntt_all, 1024, 0, s>>>(b.bcnt, (int)P.nvt, P.ldk); });
  L.run(6, [&] { k_scan_tiles<<<1, 1024, 0, s>>>(b.bcnt, P.ntt_all, P.ldk, (int)P.nvt, b.bbase); });
  L.run(6, [&] {
    k_bucket_index<<<(unsigned)cdiv(n, 256), 256, 0, s>>>(in.idx, in.mask, T, P.K, P.V, P.ldk, b.bcnt, b.bbase,
                                                          b.bcur, b.ent, b.enti);
  });
}

// The placed entries' logit-gradient values (after pass 1 and the gather).
void launch_bucket_value(Launcher& L, const Plan& P, const Bufs& b) {
  hipStream_t s = L.s;
  using namespace kd;
  const int64_t n = P.T * P.K;
  L.run(6, [&] {
    k_bucket_value<<<(unsigned)cdiv(n, 256), 256, 0, s>>>(b.s, b.pm, b.lse2, b.scal_f, P.K, kLog2e / P.tau, b.bbase,
                                                          b.bbase + P.ntt_all, b.enti, b.ent);
  });
}

// Teacher entries bucketed by tile, pass 1 (per-token log-sum-exp, and the
// logits at the cached ids), per-row loss and the mean.
void launch_forward(Launcher& L, const Plan& P, const Inputs& in, const Bufs& b, float* loss, float* row_loss) {
  hipStream_t s = L.s;
  using namespace kd;
  const int64_t T = P.T, H = P.H, V = P.V;
  const int K = P.K;
  const float c = kLog2e / P.tau;
  // the student logits at the cached ids come out of pass 1's own tiles,
  // through the entries bucketed by tile (slots of masked tokens and
  // out-of-range ids read 0)
  L.run(1, [&] { k_fill<<<grid_fill(T * K, 256), 256, 0, s>>>(b.s, T * K, 0.f); });
  launch_bucket_index(L, P, in, b);
  for (int64_t t0 = 0; t0 < T; t0 += P.Tb) {
    const int64_t rows = std::min<int64_t>(P.Tb, T - t0);
    Pass1Args a{};
    a.W = in.W;
    a.h = in.h + t0 * H;
    a.part = b.part;
    a.V = V;
    a.H = H;
    a.rows = rows;
    a.ntt = (int)cdiv(rows, 256);
    a.nvt = (int)P.nvt;
    a.gt = std::min(P.gt1, a.ntt);
    a.gv = std::min(P.gv1, a.nvt);
    a.total = a.ntt * a.nvt;
    a.ldp = (int)P.ldp;
    a.c = c;
    a.bstart = b.bcnt;
    a.bbase = b.bbase;
    a.ent = b.ent;
    a.s_out = b.s;
    a.ldk = P.ldk;
    a.gtt0 = (int)(t0 / 256);
    a.K = K;
    const int grid = (int)(cdiv(a.total, 8) * 8);
    L.run(2, [&] { k_pass1<false><<<grid, 256, 0, s>>>(a); });
    L.run(3, [&] {
      k_lse<<<(unsigned)cdiv(rows, kLseTok), 256, 0, s>>>(b.part, P.nranges, (int)P.ldp, rows, b.lse2 + t0);
    });
  }
  const int64_t nb = cdiv(T, 256);
  float* rows_out = row_loss ? row_loss : b.rows;
  L.run(4, [&] {
    k_rows<<<(unsigned)nb, 256, 0, s>>>(b.p, b.s, b.neg, b.lse2, in.mask, T, K, 1.0f / P.tau, rows_out, b.bsum);
  });
  L.run(4, [&] { k_sum<<<1, 1024, 0, s>>>(b.bsum, nb, b.scal_f, loss); });
}

// h^T of the token block [t0, t0 + rows) into the workspace (the dW
// contraction's operand), zero-padded to the block width.
void launch_transpose_h(Launcher& L, const Plan& P, const Inputs& in, const Bufs& b, int64_t t0, int64_t rows) {
  hipStream_t s = L.s;
  const dim3 grid((unsigned)(P.Tb / 64), (unsigned)(P.H / 64));
  L.run(8, [&] { kd::k_transpose_h<<<grid, 256, 0, s>>>(in.h + t0 * P.H, rows, P.H, b.hT, P.Tb); });
}

// The k-contiguous copy of W's last 64 rem_mi columns that the dH tiles of
// the last hidden tile read: wtr[j, v] = W[v, H - 64 rem_mi + j], zero for
// V <= v < ldwr (k_transpose_h over those columns).
void launch_transpose_wrem(Launcher& L, const Plan& P, const Inputs& in, const Bufs& b) {
  hipStream_t s = L.s;
  const int64_t c0 = P.H - 64 * P.rem_mi;
  const dim3 grid((unsigned)(P.ldwr / 64), (unsigned)P.rem_mi);
  L.run(8, [&] { kd::k_transpose_h<<<grid, 256, 0, s>>>(in.W + c0, P.V, P.H, b.wtr, P.ldwr); });
}

// The gradient contractions of one unit alone (k_bwd at the plan's tile height).
void launch_bwd(Launcher& L, const Plan& P, const kd::BwdArgs& g, int grid) {
  hipStream_t s = L.s;
  L.run(7, [&] { kd::k_bwd<<<grid, 256, 0, s>>>(g); });
}

// Pass 2: for each token block (outer) and vocabulary chunk (inner),
// recompute the logits, form the logit gradient (teacher entries included)
// and contract it into dH / dW (fp32 or bf16 per the flags).  Unit i's
// contractions and unit i + 1's pass 2 share one launch (k_bwd_pass2), the
// two units' gradient tiles in alternate buffers.  A block's h^T is made
// once; its dH rows are final after its last chunk, a dW chunk after the
// last block.
void launch_backward(Launcher& L, const Plan& P, uint32_t flags, const Inputs& in, const Bufs& b, void* dH_out,
                     void* dW_out, bool have_index) {
  hipStream_t s = L.s;
  using namespace kd;
  const int64_t T = P.T, H = P.H, V = P.V;
  const float c = kLog2e / P.tau;
  const bool bf16 = (flags & KD_FLAG_GRAD_BF16) != 0;
  const bool acc_dh_in = (flags & KD_FLAG_ACCUMULATE_DH) != 0;
  const bool acc_dw_in = (flags & KD_FLAG_ACCUMULATE_DW) != 0;
  const bool whole_dw = T > P.Tb;  // bf16 dW staging holds all of dW
  const int nht = (int)cdiv(H, P.bm);
  const int64_t Tp = align256(T);
  const size_t gbuf = (size_t)P.grows * P.chunk_v;  // elements of one gradient buffer
  L.run(8, [&] {
    k_offsets<<<(unsigned)cdiv(Tp, 256), 256, 0, s>>>(b.lse2, in.mask, T, Tp, b.scal_f, b.off);
  });
  if (!have_index) launch_bucket_index(L, P, in, b);
  launch_bucket_value(L, P, b);
  if (dH_out && P.rem_mi) launch_transpose_wrem(L, P, in, b);
  struct Unit {
    int64_t t0, rows, v0, vrows;
    int bi, ci;
    Pass2Args p;
    BwdArgs g;
  };
  std::vector<Unit> units;
  int bi = 0;
  for (int64_t t0 = 0; t0 < T; t0 += P.Tb, ++bi) {
    const int64_t rows = std::min<int64_t>(P.Tb, T - t0);
    const int ntt = (int)cdiv(rows, 256);
    float* dH = dH_out ? (bf16 ? b.dhs : static_cast<float*>(dH_out) + t0 * H) : nullptr;
    int ci = 0;
    for (int64_t v0 = 0; v0 < V; v0 += P.chunk_v, ++ci) {
      Unit u{};
      u.t0 = t0;
      u.rows = rows;
      u.v0 = v0;
      u.vrows = std::min<int64_t>(P.chunk_v, V - v0);
      u.bi = bi;
      u.ci = ci;
      const int nvt_c = (int)cdiv(u.vrows, 256);
      uint16_t* G = b.G + (units.size() % P.ngbuf) * gbuf;
      Pass2Args& a = u.p;
      a.W = in.W + v0 * H;
      a.h = in.h + t0 * H;
      a.off = b.off + t0;
      a.scal_f = b.scal_f;
      a.G = G;
      a.vrows = u.vrows;
      a.H = H;
      a.rows = rows;
      a.ntt = ntt;
      a.nvt = nvt_c;
      a.gt = std::min(P.gt2, ntt);
      a.gv = std::min(P.gv2, nvt_c);
      a.total = ntt * nvt_c;
      a.ldg = P.chunk_v;
      a.c = c;
      a.bstart = b.bcnt;
      a.bbase = b.bbase;
      a.ent = b.ent;
      a.ldk = P.ldk;
      a.gtt0 = (int)(t0 / 256);
      a.gvt0 = (int)(v0 / 256);
      BwdArgs& g = u.g;
      g.W = in.W + v0 * H;
      g.hT = b.hT;
      g.ldt = P.Tb;
      g.G = G;
      g.dH = dH;
      g.dW = dW_out ? (bf16 ? (whole_dw ? b.dws + v0 * H : b.dws) : static_cast<float*>(dW_out) + v0 * H) : nullptr;
      g.vrows = u.vrows;
      g.H = H;
      g.rows = rows;
      g.nht = nht;
      g.ntt = ntt;
      g.nvt = nvt_c;
      g.ndh = g.dH ? nht * ntt : 0;
      g.ndw = g.dW ? nht * nvt_c : 0;
      g.ndh_pad = (int)(cdiv(g.ndh, 8) * 8);
      g.ndw_pad = (int)(cdiv(g.ndw, 8) * 8);
      g.gm_dh = std::min(P.gm_dh, nht);
      g.gm_dw = std::min(P.gm_dw, nht);
      g.ldg = P.chunk_v;
      g.grows = (int)P.grows;
      g.rem_mi = P.rem_mi;
      g.WTr = b.wtr ? b.wtr + v0 : nullptr;
      g.ldwr = P.ldwr;
      // the first contribution overwrites, later ones add; a caller's
      // accumulate flag makes every fp32 contribution add (bf16 outputs add
      // in the final rounding instead)
      g.acc_dh = ci > 0 || (acc_dh_in && !bf16);
      g.acc_dw = bi > 0 || (acc_dw_in && !bf16);
      units.push_back(u);
    }
  }
  const int64_t nchunks = cdiv(V, P.chunk_v);
  auto pad8 = [](int n) { return (int)(cdiv(n, 8) * 8); };
  // one gradient buffer (the allocation-free entry point): pass 2 and the
  // contractions of each unit in launches of their own
  const bool merged = P.ngbuf == 2;
  if (merged) L.run(5, [&] { k_pass2<<<pad8(units[0].p.total), 256, 0, s>>>(units[0].p); });
  for (size_t i = 0; i < units.size(); ++i) {
    const Unit& u = units[i];
    if (dW_out && u.ci == 0) launch_transpose_h(L, P, in, b, u.t0, u.rows);
    const int nb = u.g.ndh_pad + u.g.ndw_pad;
    if (!merged) {
      L.run(5, [&] { k_pass2<<<pad8(u.p.total), 256, 0, s>>>(u.p); });
      launch_bwd(L, P, u.g, nb);
    } else if (i + 1 < units.size()) {
      const Pass2Args& pn = units[i + 1].p;
      const int p_pad = pad8(pn.total);
      L.run(11, [&] { k_bwd_pass2<<<nb + p_pad, 256, 0, s>>>(u.g, pn, p_pad); });
    } else {
      launch_bwd(L, P, u.g, nb);
    }
    if (dW_out && bf16 && !whole_dw) {
      const int64_t n = u.vrows * H;
      uint16_t* dst = static_cast<uint16_t*>(dW_out) + u.v0 * H;
      L.run(8, [&] { k_to_bf16<<<grid_fill(n / 4, 256), 256, 0, s>>>(b.dws, dst, n, acc_dw_in ? 1 : 0); });
    }
    if (dH_out && bf16 && u.ci == nchunks - 1) {
      const int64_t n = u.rows * H;
      uint16_t* dst = static_cast<uint16_t*>(dH_out) + u.t0 * H;
      L.run(8, [&] { k_to_bf16<<<grid_fill(n / 4, 256), 256, 0, s>>>(b.dhs, dst, n, acc_dh_in ? 1 : 0); });
    }
  }
  if (dW_out && bf16 && whole_dw) {
    const int64_t n = V * H;
    L.run(8, [&] {
      k_to_bf16<<<grid_fill(n / 4, 256), 256, 0, s>>>(b.dws, static_cast<uint16_t*>(dW_out), n, acc_dw_in ? 1 : 0);
    });
  }
}

// Sequence-chunk schedule of kd_topk_kl_fwd_bwd: per token block, pass 1
// also stores the block's logits; the gradient of each vocabulary chunk is
// then formed from them (k_sgrad) instead of recomputed, and contracted as in
// the recompute schedule.  The loss rows are reduced after the last block.
void launch_seq(Launcher& L, const Plan& P, uint32_t flags, const Inputs& in, const Bufs& b, float* St, float* loss,
                float* row_loss, void* dH_out, void* dW_out) {
  hipStream_t s = L.s;
  using namespace kd;
  const int64_t T = P.T, H = P.H, V = P.V;
  const int K = P.K;
  const float c = kLog2e / P.tau;
  const bool bf16 = (flags & KD_FLAG_GRAD_BF16) != 0;
  const bool acc_dh_in = (flags & KD_FLAG_ACCUMULATE_DH) != 0;
  const bool acc_dw_in = (flags & KD_FLAG_ACCUMULATE_DW) != 0;
  float* dH = dH_out ? (bf16 ? b.dhs : static_cast<float*>(dH_out)) : nullptr;
  const bool whole_dw = T > P.Tb;  // bf16 staging holds all of dW
  const int nht = (int)cdiv(H, P.bm);
  const int64_t lds = P.Tb;
  if (dH_out || dW_out) launch_bucket_index(L, P, in, b);
  if (dH_out && P.rem_mi) launch_transpose_wrem(L, P, in, b);
  int bi = 0;
  for (int64_t t0 = 0; t0 < T; t0 += P.Tb, ++bi) {
    const int64_t rows = std::min<int64_t>(P.Tb, T - t0);
    const int ntt = (int)cdiv(rows, 256);
    Pass1Args a{};
    a.W = in.W;
    a.h = in.h + t0 * H;
    a.part = b.part;
    a.V = V;
    a.H = H;
    a.rows = rows;
    a.ntt = ntt;
    a.nvt = (int)P.nvt;
    a.gt = std::min(P.gt1, a.ntt);
    a.gv = std::min(P.gv1, a.nvt);
    a.total = a.ntt * a.nvt;
    a.ldp = (int)P.ldp;
    a.c = c;
    a.St = St;
    a.lds = lds;
    const int grid = (int)(cdiv(a.total, 8) * 8);
    L.run(2, [&] { k_pass1<true><<<grid, 256, 0, s>>>(a); });
    L.run(3, [&] {
      k_lse<<<(unsigned)cdiv(rows, kLseTok), 256, 0, s>>>(b.part, P.nranges, (int)P.ldp, rows, b.lse2 + t0);
    });
    L.run(1, [&] {
      k_gather_s<<<(unsigned)cdiv(rows * K, 256), 256, 0, s>>>(St, lds, in.idx + t0 * K,
                                                               in.mask ? in.mask + t0 : nullptr, rows, K, V,
                                                               b.s + t0 * K);
    });
    if (!dH_out && !dW_out) continue;
    // the block's teacher entries get their gradient values (its logits
    // at the cached ids and its lse2 are final now)
    L.run(6, [&] {
      k_bucket_value<<<(unsigned)cdiv(rows * K, 256), 256, 0, s>>>(b.s, b.pm, b.lse2, b.scal_f, K, c,
                                                                   b.bbase + t0 / 256, b.bbase + t0 / 256 + ntt,
                                                                   b.enti, b.ent);
    });
    if (dW_out) launch_transpose_h(L, P, in, b, t0, rows);
    // the block's chunks: gradient tiles (k_sgrad, or inside the previous
    // chunk's contraction launch with two gradient buffers), contractions
    const int64_t nch = cdiv(V, P.chunk_v);
    auto sgrad_args = [&](int64_t ci) {
      const int64_t v0 = ci * P.chunk_v;
      const int64_t vrows = std::min<int64_t>(P.chunk_v, V - v0);
      SgradArgs sg{};
      sg.St = St + v0 * lds;
      sg.lds = lds;
      sg.lse2 = b.lse2 + t0;
      sg.mask = in.mask ? in.mask + t0 : nullptr;
      sg.scal_f = b.scal_f;
      sg.G = b.G + (size_t)(ci % P.ngbuf) * P.grows * P.chunk_v;
      sg.vrows = vrows;
      sg.rows = rows;
      sg.ntt = ntt;
      sg.nvt = (int)cdiv(vrows, 256);
      sg.total = sg.ntt * sg.nvt;
      sg.ldg = P.chunk_v;
      sg.c = c;
      sg.bstart = b.bcnt;
      sg.bbase = b.bbase;
      sg.ent = b.ent;
      sg.ldk = P.ldk;
      sg.gtt0 = (int)(t0 / 256);
      sg.gvt0 = (int)(v0 / 256);
      return sg;
    };
    auto pad8 = [](int n) { return (int)(cdiv(n, 8) * 8); };
    const bool merged = P.ngbuf == 2;
    {
      const SgradArgs sg0 = sgrad_args(0);
      L.run(5, [&] { k_sgrad<<<pad8(sg0.total), 256, 0, s>>>(sg0); });
    }
    for (int64_t ci = 0; ci < nch; ++ci) {
      const int64_t v0 = ci * P.chunk_v;
      const int64_t vrows = std::min<int64_t>(P.chunk_v, V - v0);
      const int nvt_c = (int)cdiv(vrows, 256);
      float* dW = nullptr;
      if (dW_out) dW = bf16 ? (whole_dw ? b.dws + v0 * H : b.dws) : static_cast<float*>(dW_out) + v0 * H;
      BwdArgs g{};
      g.W = in.W + v0 * H;
      g.hT = b.hT;
      g.ldt = P.Tb;
      g.G = b.G + (size_t)(ci % P.ngbuf) * P.grows * P.chunk_v;
      g.dH = dH ? dH + t0 * H : nullptr;
      g.dW = dW;
      g.vrows = vrows;
      g.H = H;
      g.rows = rows;
      g.nht = nht;
      g.ntt = ntt;
      g.nvt = nvt_c;
      g.ndh = dH ? nht * ntt : 0;
      g.ndw = dW ? nht * nvt_c : 0;
      g.ndh_pad = (int)(cdiv(g.ndh, 8) * 8);
      g.ndw_pad = (int)(cdiv(g.ndw, 8) * 8);
      g.gm_dh = std::min(P.gm_dh, nht);
      g.gm_dw = std::min(P.gm_dw, nht);
      g.ldg = P.chunk_v;
      g.grows = (int)P.grows;
      g.rem_mi = P.rem_mi;
      g.WTr = b.wtr ? b.wtr + v0 : nullptr;
      g.ldwr = P.ldwr;
      g.acc_dh = ci > 0 || (acc_dh_in && !bf16);
      g.acc_dw = bi > 0 || (acc_dw_in && !bf16);
      const int nb = g.ndh_pad + g.ndw_pad;
      if (ci + 1 < nch && merged) {
        const SgradArgs sn = sgrad_args(ci + 1);
        const int s_pad = pad8(sn.total);
        L.run(11, [&] { k_bwd_sgrad<<<nb + s_pad, 256, 0, s>>>(g, sn, s_pad); });
      } else {
        launch_bwd(L, P, g, nb);
        if (ci + 1 < nch) {
          const SgradArgs sn = sgrad_args(ci + 1);
          L.run(5, [&] { k_sgrad<<<pad8(sn.total), 256, 0, s>>>(sn); });
        }
      }
      if (dW_out && bf16 && !whole_dw) {
        const int64_t n = vrows * H;
        uint16_t* dst = static_cast<uint16_t*>(dW_out) + v0 * H;
        L.run(8, [&] { k_to_bf16<<<grid_fill(n / 4, 256), 256, 0, s>>>(b.dws, dst, n, acc_dw_in ? 1 : 0); });
      }
    }
  }
  if (dW_out && bf16 && whole_dw) {
    const int64_t n = V * H;
    L.run(8, [&] {
      k_to_bf16<<<grid_fill(n / 4, 256), 256, 0, s>>>(b.dws, static_cast<uint16_t*>(dW_out), n, acc_dw_in ? 1 : 0);
    });
  }
  if (dH_out && bf16) {
    const int64_t n = T * H;
    L.run(8, [&] {
      k_to_bf16<<<grid_fill(n / 4, 256), 256, 0, s>>>(b.dhs, static_cast<uint16_t*>(dH_out), n, acc_dh_in ? 1 : 0);
    });
  }
  const int64_t nb = cdiv(T, 256);
  float* rows_out = row_loss ? row_loss : b.rows;
  L.run(4, [&] {
    k_rows<<<(unsigned)nb, 256, 0, s>>>(b.p, b.s, b.neg, b.lse2, in.mask, T, K, 1.0f / P.tau, rows_out, b.bsum);
  });
  L.run(4, [&] { k_sum<<<1, 1024, 0, s>>>(b.bsum, nb, b.scal_f, loss); });
}

// Gradient outputs of an empty batch: zero dW (unless accumulating).
void launch_empty_grads(Launcher& L, const Plan& P, uint32_t flags, void* dW_out) {
  hipStream_t s = L.s;
  if (!dW_out || (flags & KD_FLAG_ACCUMULATE_DW)) return;
  const int64_t words = (flags & KD_FLAG_GRAD_BF16) ? P.V * P.H / 2 : P.V * P.H;
  L.run(8, [&] { kd::k_fill<<<grid_fill(words, 256), 256, 0, s>>>(static_cast<float*>(dW_out), words, 0.f); });
}

kd_status finish(Launcher& L, bool validate, const uint32_t* status) {
  if (L.err != hipSuccess) return KD_ERR_HIP;
  if (validate) {
    uint32_t host_status = 0;
    if (hipMemcpyAsync(&host_status, status, 4, hipMemcpyDeviceToHost, L.s) != hipSuccess) return KD_ERR_HIP;
    if (hipStreamSynchronize(L.s) != hipSuccess) return KD_ERR_HIP;
    if (host_status & 1u) return KD_ERR_INDEX;
    if (host_status & 2u) return KD_ERR_NONFINITE;
  }
  return KD_OK;
}

// Argument checks of the fused call that need no workspace: synchronous,
// before anything touches the device.
kd_status fwd_bwd_args(const kd_problem* p, const uint16_t* h, const uint16_t* W, const int32_t* idx,
                       const float* logit, const float* loss, const void* dH, const void* dW,
                       const float* row_loss) {
  const kd_status st = check(p);
  if (st != KD_OK) return st;
  if (!W || !loss) return KD_ERR_ARG;
  if (p->T > 0 && (!h || !idx || !logit)) return KD_ERR_ARG;
  if (misaligned(h, 16) || misaligned(W, 16) || misaligned(idx, 4) || misaligned(logit, 4) ||
      misaligned(dH, 16) || misaligned(dW, 16) || misaligned(loss, 4) || misaligned(row_loss, 4))
    return KD_ERR_UNSUPPORTED;
  return KD_OK;
}

// The fused call's launches over a checked problem and a workspace of at
// least make_plan(p).total bytes.
kd_status fwd_bwd_run(const kd_problem* p, const uint16_t* h, const uint16_t* W, const int32_t* teacher_idx,
                      const float* teacher_logit, const uint8_t* mask, float* loss, void* dH, void* dW,
                      float* row_loss, void* workspace, hipStream_t stream, bool one_gbuf) {
  const Plan P = make_plan(p, true, one_gbuf);
  Launcher L{stream};
  const Inputs in{h, W, teacher_idx, teacher_logit, mask};
  const Bufs b = carve(P, workspace, true);
  const bool validate = (p->flags & KD_FLAG_VALIDATE) != 0;
  if (P.T == 0) {
    L.run(8, [&] { kd::k_fill<<<1, 64, 0, L.s>>>(loss, 1, 0.f); });
    launch_empty_grads(L, P, p->flags, dW);
    return finish(L, false, nullptr);
  }
  launch_prep(L, P, in, b, validate, nullptr);
  if (P.seq) {
    float* St = reinterpret_cast<float*>(static_cast<char*>(workspace) + P.o_S);
    launch_seq(L, P, p->flags, in, b, St, loss, row_loss, dH, dW);
    return finish(L, validate, b.status);
  }
  launch_forward(L, P, in, b, loss, row_loss);
  if (dH || dW) launch_backward(L, P, p->flags, in, b, dH, dW, true);
  return finish(L, validate, b.status);
}

}  // namespace

// Scratch of kd_topk_kl_fwd_bwd_noalloc, in place of a caller's workspace:
// one copy per GPU, resident from the library's first use on that GPU until
// the process ends.  On the host this name is only a stand-in for the
// symbol; the device address of each GPU's copy comes from
// hipGetSymbolAddress (scratch_for) and is what the kernels receive.
static __device__ __align__(256) uint8_t scratch[KD_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];  // device address of `scratch` on each GPU

// The scratch address on the current device, looked up once per device with
// that device current.  The stream (NULL = the current device's null
// stream) must belong to the current device.
kd_status scratch_for(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return KD_ERR_HIP;
  if (dev >= kMaxDevices) return KD_ERR_UNSUPPORTED;
  if (stream) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return KD_ERR_HIP;
    if (sdev != dev) return KD_ERR_ARG;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return KD_ERR_HIP;
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return KD_OK;
}

}  // namespace

extern "C" {

int kd_abi_version(void) { return 5; }

const char* kd_status_string(kd_status s) {
  switch (s) {
    case KD_OK: return "ok";
    case KD_ERR_ARG: return "invalid argument";
    case KD_ERR_UNSUPPORTED: return "unsupported problem (H % 64, K > 1024, chunk/block not multiples of 256, size limits or alignment)";
    case KD_ERR_WORKSPACE: return "workspace too small";
    case KD_ERR_INDEX: return "teacher index out of range";
    case KD_ERR_NONFINITE: return "teacher logits NaN/+inf or all -inf in a kept row";
    case KD_ERR_HIP: return "HIP runtime error";
    default: break;
  }
  return "unknown status";
}

kd_status kd_topk_kl_tiling(const kd_problem* p, int64_t* block_t, int64_t* chunk_v, int32_t* gbufs) {
  if (!block_t || !chunk_v || !gbufs) return KD_ERR_ARG;
  const kd_status st = check(p);
  if (st != KD_OK) return st;
  const Plan P = make_plan(p);
  *block_t = P.Tb;
  *chunk_v = P.chunk_v;
  *gbufs = P.ngbuf;
  return KD_OK;
}

kd_status kd_topk_kl_workspace_size(const kd_problem* p, size_t* bytes) {
  if (!bytes) return KD_ERR_ARG;
  const kd_status st = check(p);
  if (st != KD_OK) return st;
  *bytes = make_plan(p).total;
  return KD_OK;
}

const float* kd_topk_kl_workspace_lse2(const kd_problem* p, const void* workspace) {
  if (check(p) != KD_OK || !workspace) return nullptr;
  const Plan P = make_plan(p);
  return reinterpret_cast<const float*>(static_cast<const char*>(workspace) + P.o_lse2);
}

kd_status kd_timing_enable(int on) {
  g_timing.store(on != 0);
  return KD_OK;
}

kd_status kd_timing_classes(uint32_t mask) {
  g_timing_mask.store(mask);
  return KD_OK;
}

kd_status kd_timing_collect(double* ms, int64_t* launches) {
  std::lock_guard<std::mutex> lock(g_timing_mu);
  kd_status st = KD_OK;
  for (auto& l : g_launches) {
    if (hipEventSynchronize(l.b) != hipSuccess) st = KD_ERR_HIP;
    float t = 0.f;
    if (hipEventElapsedTime(&t, l.a, l.b) != hipSuccess) st = KD_ERR_HIP;
    if (l.cls >= 0 && l.cls < kTimingClasses) {
      if (ms) ms[l.cls] += t;
      if (launches) launches[l.cls] += 1;
    }
    g_pool.push_back(l.a);
    g_pool.push_back(l.b);
  }
  g_launches.clear();
  return st;
}

kd_status kd_topk_kl_fwd_bwd(const kd_problem* p, const uint16_t* h, const uint16_t* W,
                             const int32_t* teacher_idx, const float* teacher_logit, const uint8_t* mask,
                             float* loss, void* dH, void* dW, float* row_loss, void* workspace,
                             size_t workspace_bytes, void* stream) {
  kd_status st = fwd_bwd_args(p, h, W, teacher_idx, teacher_logit, loss, dH, dW, row_loss);
  if (st != KD_OK) return st;
  if (!workspace) return KD_ERR_ARG;
  if (misaligned(workspace, 256)) return KD_ERR_UNSUPPORTED;
  if (workspace_bytes < make_plan(p).total) return KD_ERR_WORKSPACE;
  return fwd_bwd_run(p, h, W, teacher_idx, teacher_logit, mask, loss, dH, dW, row_loss, workspace,
                     static_cast<hipStream_t>(stream), false);
}

kd_status kd_topk_kl_fwd_bwd_noalloc(const kd_problem* p, const uint16_t* h, const uint16_t* W,
                                     const int32_t* teacher_idx, const float* teacher_logit, const uint8_t* mask,
                                     float* loss, void* dH, void* dW, float* row_loss, void* stream) {
  kd_status st = fwd_bwd_args(p, h, W, teacher_idx, teacher_logit, loss, dH, dW, row_loss);
  if (st != KD_OK) return st;
  if (make_plan(p, true, true).total > (size_t)KD_NOALLOC_SCRATCH_BYTES) return KD_ERR_WORKSPACE;
  void* ws = nullptr;
  st = scratch_for(static_cast<hipStream_t>(stream), &ws);
  if (st != KD_OK) return st;
  return fwd_bwd_run(p, h, W, teacher_idx, teacher_logit, mask, loss, dH, dW, row_loss, ws,
                     static_cast<hipStream_t>(stream), true);
}

kd_status kd_topk_kl_saved_size(const kd_problem* p, size_t* bytes) {
  if (!bytes) return KD_ERR_ARG;
  const kd_status st = check(p);
  if (st != KD_OK) return st;
  *bytes = saved_bytes(make_plan(p, false));
  return KD_OK;
}

kd_status kd_topk_kl_fwd_workspace_size(const kd_problem* p, size_t* bytes) {
  if (!bytes) return KD_ERR_ARG;
  const kd_status st = check(p);
  if (st != KD_OK) return st;
  *bytes = make_plan(p, false).total;
  return KD_OK;
}

kd_status kd_topk_kl_fwd(const kd_problem* p, const uint16_t* h, const uint16_t* W, const int32_t* teacher_idx,
                         const float* teacher_logit, const uint8_t* mask, float* loss, float* row_loss, void* saved,
                         void* workspace, size_t workspace_bytes, void* stream) {
  kd_status st = check_common(p, h, W, teacher_idx, teacher_logit, workspace);
  if (st != KD_OK) return st;
  if (!loss || !saved) return KD_ERR_ARG;
  if (misaligned(saved, 256) || misaligned(loss, 4) || misaligned(row_loss, 4)) return KD_ERR_UNSUPPORTED;
  const Plan P = make_plan(p, false);
  if (workspace_bytes < P.total) return KD_ERR_WORKSPACE;
  Launcher L{static_cast<hipStream_t>(stream)};
  const Inputs in{h, W, teacher_idx, teacher_logit, mask};
  Bufs b = carve(P, workspace, false);
  b.lse2 = static_cast<float*>(saved);
  b.s = reinterpret_cast<float*>(static_cast<char*>(saved) + saved_lse2_bytes(P));
  const bool validate = (p->flags & KD_FLAG_VALIDATE) != 0;
  if (P.T == 0) {
    L.run(8, [&] { kd::k_fill<<<1, 64, 0, L.s>>>(loss, 1, 0.f); });
    return finish(L, false, nullptr);
  }
  launch_prep(L, P, in, b, validate, nullptr);
  launch_forward(L, P, in, b, loss, row_loss);
  return finish(L, validate, b.status);
}

kd_status kd_topk_kl_bwd(const kd_problem* p, const uint16_t* h, const uint16_t* W, const int32_t* teacher_idx,
                         const float* teacher_logit, const uint8_t* mask, const void* saved, const float* grad_loss,
                         void* dH, void* dW, void* workspace, size_t workspace_bytes, void* stream) {
  if (!p) return KD_ERR_ARG;
  // the split backward always recomputes: the sequence-chunk flag, which
  // would change the default tiling, is ignored
  kd_problem q = *p;
  q.flags &= ~KD_FLAG_SEQ_CHUNK;
  p = &q;
  kd_status st = check_common(p, h, W, teacher_idx, teacher_logit, workspace);
  if (st != KD_OK) return st;
  if (!saved) return KD_ERR_ARG;
  if (misaligned(saved, 256) || misaligned(dH, 16) || misaligned(dW, 16) || misaligned(grad_loss, 4))
    return KD_ERR_UNSUPPORTED;
  const Plan P = make_plan(p);
  if (workspace_bytes < P.total) return KD_ERR_WORKSPACE;
  Launcher L{static_cast<hipStream_t>(stream)};
  const Inputs in{h, W, teacher_idx, teacher_logit, mask};
  Bufs b = carve(P, workspace, true);
  b.lse2 = const_cast<float*>(static_cast<const float*>(saved));
  b.s = reinterpret_cast<float*>(const_cast<char*>(static_cast<const char*>(saved)) + saved_lse2_bytes(P));
  const bool validate = (p->flags & KD_FLAG_VALIDATE) != 0;
  if (P.T == 0) {
    launch_empty_grads(L, P, p->flags, dW);
    return finish(L, false, nullptr);
  }
  if (!dH && !dW) return KD_OK;
  launch_prep(L, P, in, b, validate, grad_loss);
  launch_backward(L, P, p->flags, in, b, dH, dW, false);
  return finish(L, validate, b.status);
}

}  // extern "C"

// ------------------------------------------------ KL on given student logits
namespace {

struct LogitsPlan {
  int64_t T, V, Tp;
  int K;
  size_t o_p, o_pm, o_s, o_neg, o_lse2, o_row, o_bsum, o_scal_f, o_scal_i, o_status, total;
};

kd_status check_logits(const kd_logits_problem* p) {
  if (!p) return KD_ERR_ARG;
  if (p->T < 0 || p->V <= 0 || p->K <= 0 || (int64_t)p->K > p->V) return KD_ERR_ARG;
  if (!(p->tau > 0.f) || !isfinite(p->tau)) return KD_ERR_ARG;
  if (p->flags & ~(KD_FLAG_VALIDATE | KD_FLAG_LOGITS_F32)) return KD_ERR_ARG;
  if (p->K > kd::kTeacherMaxK) return KD_ERR_UNSUPPORTED;
  // one workgroup of kLrowThreads per row, under 2^32 work-items a launch
  if (p->V > (int64_t)INT32_MAX || p->T > (int64_t)UINT32_MAX / std::max(kd::kLrowThreads, kd::kLrowRegThreads))
    return KD_ERR_UNSUPPORTED;
  return KD_OK;
}

LogitsPlan logits_plan(const kd_logits_problem* p) {
  LogitsPlan P{};
  P.T = p->T;
  P.V = p->V;
  P.K = p->K;
  P.Tp = align256(std::max<int64_t>(P.T, 1));
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o += (bytes + 255) & ~size_t(255); return r; };
  P.o_p = take((size_t)P.T * P.K * 4);
  P.o_pm = take((size_t)P.T * P.K * 4);
  P.o_s = take((size_t)P.T * P.K * 4);
  P.o_neg = take((size_t)P.Tp * 4);
  P.o_lse2 = take((size_t)P.Tp * 4);
  P.o_row = take((size_t)P.Tp * 4);
  P.o_bsum = take((size_t)cdiv(P.Tp, 256) * 8 + 8);
  P.o_scal_f = take(64);
  P.o_scal_i = take(64);
  P.o_status = take(64);
  P.total = o;
  return P;
}

}  // namespace

extern "C" {

kd_status kd_topk_kl_logits_workspace_size(const kd_logits_problem* p, size_t* bytes) {
  if (!bytes) return KD_ERR_ARG;
  const kd_status st = check_logits(p);
  if (st != KD_OK) return st;
  *bytes = logits_plan(p).total;
  return KD_OK;
}

kd_status kd_topk_kl_logits(const kd_logits_problem* p, const void* Z, const int32_t* teacher_idx,
                            const float* teacher_logit, const uint8_t* mask, float* loss, void* dZ,
                            float* row_loss, void* workspace, size_t workspace_bytes, void* stream) {
  const kd_status st = check_logits(p);
  if (st != KD_OK) return st;
  if (!loss || !workspace) return KD_ERR_ARG;
  if (p->T > 0 && (!Z || !teacher_idx || !teacher_logit)) return KD_ERR_ARG;
  if (misaligned(Z, 16) || misaligned(dZ, 16) || misaligned(workspace, 256) || misaligned(teacher_idx, 4) ||
      misaligned(teacher_logit, 4) || misaligned(loss, 4) || misaligned(row_loss, 4))
    return KD_ERR_UNSUPPORTED;
  const LogitsPlan P = logits_plan(p);
  if (workspace_bytes < P.total) return KD_ERR_WORKSPACE;
  Launcher L{static_cast<hipStream_t>(stream)};
  hipStream_t s = L.s;
  char* ws = static_cast<char*>(workspace);
  float* tp = reinterpret_cast<float*>(ws + P.o_p);
  float* tpm = reinterpret_cast<float*>(ws + P.o_pm);
  float* ts = reinterpret_cast<float*>(ws + P.o_s);
  float* neg = reinterpret_cast<float*>(ws + P.o_neg);
  float* lse2 = reinterpret_cast<float*>(ws + P.o_lse2);
  float* rows_out = row_loss ? row_loss : reinterpret_cast<float*>(ws + P.o_row);
  double* bsum = reinterpret_cast<double*>(ws + P.o_bsum);
  float* scal_f = reinterpret_cast<float*>(ws + P.o_scal_f);
  int64_t* scal_i = reinterpret_cast<int64_t*>(ws + P.o_scal_i);
  uint32_t* status = reinterpret_cast<uint32_t*>(ws + P.o_status);
  const bool validate = (p->flags & KD_FLAG_VALIDATE) != 0;
  const bool f32 = (p->flags & KD_FLAG_LOGITS_F32) != 0;
  const int64_t T = P.T, V = P.V;
  const int K = P.K;
  using namespace kd;
  if (T == 0) {
    L.run(8, [&] { k_fill<<<1, 64, 0, s>>>(loss, 1, 0.f); });
    return finish(L, false, nullptr);
  }
  if (validate) L.run(8, [&] { k_fill<<<1, 64, 0, s>>>(reinterpret_cast<float*>(status), 1, 0.f); });
  L.run(4, [&] { k_count<<<1, 1024, 0, s>>>(mask, T, p->tau, nullptr, scal_f, scal_i); });
  L.run(0, [&] {
    k_teacher<<<(unsigned)cdiv(T, 4), 256, 0, s>>>(teacher_idx, teacher_logit, mask, T, K, V, 1.0f / p->tau, tp, tpm,
                                                    neg, status, validate ? 1 : 0);
  });
  LrowArgs a{};
  a.Z = Z;
  a.dZ = dZ;
  a.T = T;
  a.V = V;
  a.K = K;
  a.idx = teacher_idx;
  a.pm = tpm;
  a.mask = mask;
  a.scal_f = scal_f;
  a.lse2 = lse2;
  a.s_out = ts;
  a.c = kLog2e / p->tau;
  const bool vec = (V * (f32 ? 4 : 2)) % 16 == 0;
  // bf16 rows that fit 512 threads x PER 16-byte chunks stay in registers
  const int64_t need = cdiv(V / 8, kLrowRegThreads);
  static const int kPer[] = {1, 2, 4, 8, 16, 24, 32, 40, 50};
  int per = 0;
  if (!f32 && vec)
    for (int c : kPer)
      if (c >= need) {
        per = c;
        break;
      }
  L.run(9, [&] {
    if (per) {
      const unsigned g = (unsigned)T;
      switch (per) {
        case 1: k_lrow_reg<1><<<g, kLrowRegThreads, 0, s>>>(a); break;
        case 2: k_lrow_reg<2><<<g, kLrowRegThreads, 0, s>>>(a); break;
        case 4: k_lrow_reg<4><<<g, kLrowRegThreads, 0, s>>>(a); break;
        case 8: k_lrow_reg<8><<<g, kLrowRegThreads, 0, s>>>(a); break;
        case 16: k_lrow_reg<16><<<g, kLrowRegThreads, 0, s>>>(a); break;
        case 24: k_lrow_reg<24><<<g, kLrowRegThreads, 0, s>>>(a); break;
        case 32: k_lrow_reg<32><<<g, kLrowRegThreads, 0, s>>>(a); break;
        case 40: k_lrow_reg<40><<<g, kLrowRegThreads, 0, s>>>(a); break;
        default: k_lrow_reg<50><<<g, kLrowRegThreads, 0, s>>>(a); break;
      }
    } else if (f32) {
      if (vec) k_lrow<float, true><<<(unsigned)T, kLrowThreads, 0, s>>>(a);
      else k_lrow<float, false><<<(unsigned)T, kLrowThreads, 0, s>>>(a);
    } else {
      if (vec) k_lrow<uint16_t, true><<<(unsigned)T, kLrowThreads, 0, s>>>(a);
      else k_lrow<uint16_t, false><<<(unsigned)T, kLrowThreads, 0, s>>>(a);
    }
  });
  const int64_t nb = cdiv(T, 256);
  L.run(4, [&] {
    k_rows<<<(unsigned)nb, 256, 0, s>>>(tp, ts, neg, lse2, mask, T, K, 1.0f / p->tau, rows_out, bsum);
  });
  L.run(4, [&] { k_sum<<<1, 1024, 0, s>>>(bsum, nb, scal_f, loss); });
  return finish(L, validate, status);
}

kd_status kd_topk_select(const kd_topk_problem* p, const uint16_t* X, int32_t* idx, float* values,
                         void* stream) {
  if (!p) return KD_ERR_ARG;
  if (p->T < 0 || p->V <= 0 || p->K <= 0 || (int64_t)p->K > p->V || p->flags != 0) return KD_ERR_ARG;
  if (p->T > 0 && (!X || !idx || !values)) return KD_ERR_ARG;
  using namespace kd;
  // one workgroup of kTopkThreads per row, under 2^32 work-items a launch
  if (p->K > kTopkMaxK || p->V % 8 != 0 || p->V > (int64_t)INT32_MAX / 2 || p->T > (int64_t)UINT32_MAX / kTopkThreads)
    return KD_ERR_UNSUPPORTED;
  if (misaligned(X, 16) || misaligned(idx, 4) || misaligned(values, 4)) return KD_ERR_UNSUPPORTED;
  Launcher L{static_cast<hipStream_t>(stream)};
  if (p->T == 0) return finish(L, false, nullptr);
  hipStream_t s = L.s;
  TopkArgs a{};
  a.X = X;
  a.idx = idx;
  a.val = values;
  a.V = p->V;
  a.K = p->K;
  int bits = 0;
  while (((int64_t)1 << bits) < p->V) ++bits;
  a.id_bits = bits;
  L.run(10, [&] { k_topk<<<(unsigned)p->T, kTopkThreads, 0, s>>>(a); });
  return finish(L, false, nullptr);
}

}  // extern "C"
