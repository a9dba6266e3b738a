// Host side of libkdkl: argument checks, workspace plan, launch sequence and
// the optional event timing.  Everything here is synchronous argument work
// plus asynchronous launches on the caller's stream; no device allocation.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "../../include/kdkl.h"
#include "kd_kernels.hpp"

namespace {

constexpr int kDefaultChunkV = 16384;
constexpr int kDefaultBlockT = 16384;

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
  int per, nranges;  // pass 1: vocabulary tiles per workgroup, ranges
  int gt1, gt2;      // token-tile group sizes of pass 1 / pass 2
  int gv1, gv2;      // vocabulary group sizes (take precedence when > 0)
  int gm_dh, gm_dw;  // hidden-tile group sizes of the gradient contractions
  int64_t ldp;       // leading dim of the pass-1 partials
  int64_t grows;     // rows of the gradient buffer
  // workspace offsets (bytes)
  size_t o_G, o_part, o_lse2, o_p, o_pm, o_s, o_neg, o_row, o_bsum, o_scal_f, o_scal_i, o_status, total;
};

kd_status check(const kd_problem* p) {
  if (!p) return KD_ERR_ARG;
  if (p->T < 0 || p->H <= 0 || p->V <= 0 || p->K <= 0) return KD_ERR_ARG;
  if (!(p->tau > 0.f) || !isfinite(p->tau)) return KD_ERR_ARG;
  if ((int64_t)p->K > p->V) return KD_ERR_ARG;
  if (p->chunk_v < 0 || p->block_t < 0) return KD_ERR_ARG;
  if (p->flags & ~KD_FLAG_VALIDATE) return KD_ERR_ARG;
  if (p->H % 64 != 0) return KD_ERR_UNSUPPORTED;
  if (p->K > kd::kTeacherMaxK) return KD_ERR_UNSUPPORTED;
  if (p->chunk_v % 256 != 0 || p->block_t % 256 != 0) return KD_ERR_UNSUPPORTED;
  if (p->V > (int64_t)INT32_MAX || p->T > ((int64_t)1 << 40)) return KD_ERR_UNSUPPORTED;
  const int64_t cv = p->chunk_v ? p->chunk_v : kDefaultChunkV;
  const int64_t bt = p->block_t ? p->block_t : kDefaultBlockT;
  // 32-bit buffer offsets inside one chunk / block operand
  const int64_t lim = (int64_t)UINT32_MAX;
  if (cv * p->H * 2 > lim || bt * p->H * 2 > lim || bt * cv * 2 > lim) return KD_ERR_UNSUPPORTED;
  if (256 * p->H * 2 > lim / 2) return KD_ERR_UNSUPPORTED;
  return KD_OK;
}

Plan make_plan(const kd_problem* p) {
  Plan P{};
  P.T = p->T;
  P.H = p->H;
  P.V = p->V;
  P.K = p->K;
  P.tau = p->tau;
  P.chunk_v = p->chunk_v ? p->chunk_v : kDefaultChunkV;
  P.block_t = p->block_t ? p->block_t : kDefaultBlockT;
  P.Tb = P.T < P.block_t ? align256(P.T) : P.block_t;
  if (P.Tb == 0) P.Tb = 256;
  P.ntt_max = (int)(P.Tb / 256);
  P.nvt = cdiv(P.V, 256);
  P.per = env_int("KDKL_PASS1_PER", 1);
  if (P.per < 1) P.per = 1;
  P.nranges = (int)cdiv(P.nvt, P.per);
  P.gt1 = env_int("KDKL_GROUP_T1", 4);
  P.gt2 = env_int("KDKL_GROUP_T2", 4);
  P.gv1 = env_int("KDKL_GROUP_V1", 8);
  P.gv2 = env_int("KDKL_GROUP_V2", 8);
  P.gm_dh = std::max(1, env_int("KDKL_GROUP_MDH", 4));
  P.gm_dw = std::max(1, env_int("KDKL_GROUP_MDW", 2));
  if (P.gt1 < 1) P.gt1 = 1;
  if (P.gt2 < 1) P.gt2 = 1;
  P.ldp = (int64_t)P.ntt_max * 256;
  P.grows = (int64_t)P.ntt_max * 256;
  const int64_t Tp = align256(P.T);
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o += (bytes + 255) & ~size_t(255); return r; };
  P.o_G = take((size_t)P.grows * P.chunk_v * 2);
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
bool g_timing = false;
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
    if (g_timing) {
      a = pool_get();
      b = pool_get();
      if (a) (void)hipEventRecord(a, s);
    }
    f();
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) err = e;
    if (g_timing && a && b) {
      (void)hipEventRecord(b, s);
      g_launches.push_back({cls, a, b});
    }
  }
};

int grid_fill(int64_t n, int block) { return (int)std::max<int64_t>(1, std::min<int64_t>(cdiv(n, block), 65536)); }

}  // namespace

extern "C" {

int kd_abi_version(void) { return 1; }

const char* kd_status_string(kd_status s) {
  switch (s) {
    case KD_OK: return "ok";
    case KD_ERR_ARG: return "invalid argument";
    case KD_ERR_UNSUPPORTED: return "unsupported problem (H % 64, K > 1024, chunk/block not multiples of 256, size or alignment)";
    case KD_ERR_WORKSPACE: return "workspace too small";
    case KD_ERR_INDEX: return "teacher index out of range";
    case KD_ERR_NONFINITE: return "teacher logits NaN/+inf or all -inf in a kept row";
    case KD_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
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
  g_timing = on != 0;
  return KD_OK;
}

kd_status kd_timing_collect(double* ms, int64_t* launches) {
  kd_status st = KD_OK;
  for (auto& l : g_launches) {
    if (hipEventSynchronize(l.b) != hipSuccess) st = KD_ERR_HIP;
    float t = 0.f;
    if (hipEventElapsedTime(&t, l.a, l.b) != hipSuccess) st = KD_ERR_HIP;
    if (l.cls >= 0 && l.cls < 9) {
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
                             float* loss, float* dH, float* dW, float* row_loss, void* workspace,
                             size_t workspace_bytes, void* stream) {
  const kd_status st = check(p);
  if (st != KD_OK) return st;
  if (!W || !loss || !workspace) return KD_ERR_ARG;
  if (p->T > 0 && (!h || !teacher_idx || !teacher_logit)) return KD_ERR_ARG;
  auto misaligned = [](const void* q, uintptr_t a) { return q && (reinterpret_cast<uintptr_t>(q) & (a - 1)); };
  if (misaligned(h, 16) || misaligned(W, 16) || misaligned(dH, 16) || misaligned(dW, 16) ||
      misaligned(workspace, 256) || misaligned(teacher_idx, 4) || misaligned(teacher_logit, 4) ||
      misaligned(loss, 4) || misaligned(row_loss, 4))
    return KD_ERR_UNSUPPORTED;
  const Plan P = make_plan(p);
  if (workspace_bytes < P.total) return KD_ERR_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  uint16_t* G = reinterpret_cast<uint16_t*>(ws + P.o_G);
  float2* part = reinterpret_cast<float2*>(ws + P.o_part);
  float* lse2 = reinterpret_cast<float*>(ws + P.o_lse2);
  float* tp = reinterpret_cast<float*>(ws + P.o_p);
  float* tpm = reinterpret_cast<float*>(ws + P.o_pm);
  float* ts = reinterpret_cast<float*>(ws + P.o_s);
  float* neg = reinterpret_cast<float*>(ws + P.o_neg);
  float* rows_out = row_loss ? row_loss : reinterpret_cast<float*>(ws + P.o_row);
  double* bsum = reinterpret_cast<double*>(ws + P.o_bsum);
  float* scal_f = reinterpret_cast<float*>(ws + P.o_scal_f);
  int64_t* scal_i = reinterpret_cast<int64_t*>(ws + P.o_scal_i);
  uint32_t* status = reinterpret_cast<uint32_t*>(ws + P.o_status);
  const bool validate = (p->flags & KD_FLAG_VALIDATE) != 0;
  const int64_t T = P.T, H = P.H, V = P.V;
  const int K = P.K;
  const float inv_tau = 1.0f / P.tau;
  const float c = kd::kLog2e / P.tau;

  Launcher L{s};
  using namespace kd;
  if (T == 0) {
    L.run(8, [&] { k_fill<<<1, 64, 0, s>>>(loss, 1, 0.f); });
    if (dW) L.run(8, [&] { k_fill<<<grid_fill(V * H, 256), 256, 0, s>>>(dW, V * H, 0.f); });
    return L.err == hipSuccess ? KD_OK : KD_ERR_HIP;
  }
  if (validate) L.run(8, [&] { k_fill<<<1, 64, 0, s>>>(reinterpret_cast<float*>(status), 1, 0.f); });
  L.run(4, [&] { k_count<<<1, 1024, 0, s>>>(mask, T, P.tau, scal_f, scal_i); });
  L.run(0, [&] {
    k_teacher<<<(unsigned)cdiv(T, 4), 256, 0, s>>>(teacher_idx, teacher_logit, mask, T, K, V, inv_tau, tp, tpm, neg,
                                                    status, validate ? 1 : 0);
  });
  L.run(1, [&] { k_gather<<<(unsigned)T, 256, 0, s>>>(h, W, teacher_idx, mask, T, H, V, K, ts); });

  // pass 1: per-token log-sum-exp over the whole vocabulary, block by block
  for (int64_t t0 = 0; t0 < T; t0 += P.Tb) {
    const int64_t rows = std::min<int64_t>(P.Tb, T - t0);
    kd::Pass1Args a{};
    a.W = W;
    a.h = h + t0 * H;
    a.part = part;
    a.V = V;
    a.H = H;
    a.rows = rows;
    a.ntt = (int)cdiv(rows, 256);
    a.nvt = (int)P.nvt;
    a.per = P.per;
    a.nranges = P.nranges;
    a.gt = std::min(P.gt1, a.ntt);
    a.gv = std::min(P.gv1, a.nranges);
    a.total = a.ntt * a.nranges;
    a.ldp = (int)P.ldp;
    a.c = c;
    const int grid = (int)(cdiv(a.total, 8) * 8);
    L.run(2, [&] { k_pass1<<<grid, 256, 0, s>>>(a); });
    L.run(3, [&] {
      k_lse<<<(unsigned)cdiv(rows, 32), 256, 0, s>>>(part, P.nranges, (int)P.ldp, rows, lse2 + t0);
    });
  }
  const int64_t nb = cdiv(T, 256);
  L.run(4, [&] {
    k_rows<<<(unsigned)nb, 256, 0, s>>>(tp, ts, neg, lse2, mask, T, K, inv_tau, rows_out, bsum);
  });
  L.run(4, [&] { k_sum<<<1, 1024, 0, s>>>(bsum, nb, scal_f, loss); });

  // pass 2: recompute every (block, chunk), form the logit gradient, contract it
  if (dH || dW) {
    const int nht = (int)cdiv(H, 256);
    int ci = 0;
    for (int64_t v0 = 0; v0 < V; v0 += P.chunk_v, ++ci) {
      const int64_t vrows = std::min<int64_t>(P.chunk_v, V - v0);
      const int nvt_c = (int)cdiv(vrows, 256);
      int bi = 0;
      for (int64_t t0 = 0; t0 < T; t0 += P.Tb, ++bi) {
        const int64_t rows = std::min<int64_t>(P.Tb, T - t0);
        const int ntt = (int)cdiv(rows, 256);
        kd::Pass2Args a{};
        a.W = W + v0 * H;
        a.h = h + t0 * H;
        a.lse2 = lse2 + t0;
        a.mask = mask ? mask + t0 : nullptr;
        a.scal_f = scal_f;
        a.G = G;
        a.vrows = vrows;
        a.H = H;
        a.rows = rows;
        a.ntt = ntt;
        a.nvt = nvt_c;
        a.gt = std::min(P.gt2, ntt);
        a.gv = std::min(P.gv2, nvt_c);
        a.total = ntt * nvt_c;
        a.ldg = P.chunk_v;
        a.c = c;
        const int grid = (int)(cdiv(a.total, 8) * 8);
        L.run(5, [&] { k_pass2<<<grid, 256, 0, s>>>(a); });
        L.run(6, [&] {
          k_fixup<<<(unsigned)cdiv(rows * K, 256), 256, 0, s>>>(
              teacher_idx + t0 * K, ts + t0 * K, tpm + t0 * K, lse2 + t0, mask ? mask + t0 : nullptr, scal_f, rows, K,
              v0, vrows, c, G, P.chunk_v);
        });
        kd::BwdArgs b{};
        b.W = W + v0 * H;
        b.h = h + t0 * H;
        b.G = G;
        b.dH = dH ? dH + t0 * H : nullptr;
        b.dW = dW ? dW + v0 * H : nullptr;
        b.vrows = vrows;
        b.H = H;
        b.rows = rows;
        b.nht = nht;
        b.ntt = ntt;
        b.nvt = nvt_c;
        b.ndh = dH ? nht * ntt : 0;
        b.ndw = dW ? nht * nvt_c : 0;
        b.ndh_pad = (int)(cdiv(b.ndh, 8) * 8);
        b.ndw_pad = (int)(cdiv(b.ndw, 8) * 8);
        b.gm_dh = std::min(P.gm_dh, nht);
        b.gm_dw = std::min(P.gm_dw, nht);
        b.ldg = P.chunk_v;
        b.grows = (int)P.grows;
        b.acc_dh = ci > 0;
        b.acc_dw = bi > 0;
        L.run(7, [&] { k_bwd<<<b.ndh_pad + b.ndw_pad, 256, 0, s>>>(b); });
      }
    }
  }
  if (L.err != hipSuccess) return KD_ERR_HIP;
  if (validate) {
    uint32_t host_status = 0;
    if (hipMemcpyAsync(&host_status, status, 4, hipMemcpyDeviceToHost, s) != hipSuccess) return KD_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return KD_ERR_HIP;
    if (host_status & 1u) return KD_ERR_INDEX;
    if (host_status & 2u) return KD_ERR_NONFINITE;
  }
  return KD_OK;
}

}  // extern "C"
