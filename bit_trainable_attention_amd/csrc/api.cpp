// C ABI of the SageBwd-style INT8 attention (declared in include/sagebwd.h).
// Validates arguments without touching the HIP runtime, then enqueues the kernels.
#include "sagebwd.h"

#include <stdio.h>

#include <hip/hip_runtime.h>

#include "launch.hpp"

namespace {

using sagebwd::BackwardArgs;
using sagebwd::ForwardArgs;
using sagebwd::PrologueArgs;

constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape / option checks shared by every entry point.
sagebwd_status check_params(const sagebwd_params* p) {
  if (!p) return SAGEBWD_ERR_NULL;
  if (p->B < 0 || p->H < 0 || p->N < 0) return SAGEBWD_ERR_SHAPE;
  if (p->d != 64 && p->d != 128) return SAGEBWD_ERR_UNSUPPORTED;
  if (p->blk != 64 && p->blk != 128) return SAGEBWD_ERR_UNSUPPORTED;
  if (p->dtype != SAGEBWD_FP16 && p->dtype != SAGEBWD_BF16) return SAGEBWD_ERR_UNSUPPORTED;
  if (p->dq_mode < SAGEBWD_DQ_AUTO || p->dq_mode > SAGEBWD_DQ_ATOMIC) return SAGEBWD_ERR_UNSUPPORTED;
  if (!(p->eps >= 0.0f)) return SAGEBWD_ERR_UNSUPPORTED;
  if (p->layout != SAGEBWD_LAYOUT_BHND && p->layout != SAGEBWD_LAYOUT_BNHD) return SAGEBWD_ERR_UNSUPPORTED;
  if (p->qk_gain && !p->qk_norm) return SAGEBWD_ERR_UNSUPPORTED;
  if (p->normed_grads && (!p->qk_norm || p->qk_gain)) return SAGEBWD_ERR_UNSUPPORTED;
  if (p->fmt != SAGEBWD_FMT_INT8 && p->fmt != SAGEBWD_FMT_FP8) return SAGEBWD_ERR_UNSUPPORTED;
  if (p->fmt == SAGEBWD_FMT_FP8 && p->q_smooth) return SAGEBWD_ERR_UNSUPPORTED;
  if (p->split != SAGEBWD_SPLIT_SAGEBWD && p->split != SAGEBWD_SPLIT_QATTN) return SAGEBWD_ERR_UNSUPPORTED;
  if (p->split == SAGEBWD_SPLIT_QATTN && p->q_smooth) return SAGEBWD_ERR_UNSUPPORTED;
  // index arithmetic inside the kernels: byte offsets inside one head's arrays fit in 31 bits
  // (Np * d * 4 < 2^31), grids in 2^31 workgroups
  if ((long long)p->B * p->H > (1LL << 24) || p->N > (1 << 22)) return SAGEBWD_ERR_SHAPE;
  if ((long long)p->B * p->H * ((p->N + p->blk - 1) / p->blk) * 3 >= (1LL << 31)) return SAGEBWD_ERR_SHAPE;
  return SAGEBWD_OK;
}

bool empty(const sagebwd_params* p) { return p->B == 0 || p->H == 0 || p->N == 0; }

// Tokens per head of the library's own arrays: N rounded up to whole quantisation blocks.
int padded_n(const sagebwd_params* p) { return (p->N + p->blk - 1) / p->blk * p->blk; }

// The parameters with N replaced by the padded length (for sizes and grids).
sagebwd_params padded(const sagebwd_params* p) {
  sagebwd_params q = *p;
  q.N = padded_n(p);
  return q;
}

sagebwd::Strides16 strides16(const sagebwd_params* p) {
  const long long d = p->d, N = p->N, H = p->H;
  if (p->layout == SAGEBWD_LAYOUT_BNHD) return {N * H * d, d, (int)(H * d), p->H};
  return {H * N * d, N * d, (int)d, p->H};
}

size_t elems(const sagebwd_params* p) { return (size_t)p->B * p->H * padded_n(p) * p->d; }

float sm_scale_of(const sagebwd_params* p) {
  return p->sm_scale > 0.0f ? p->sm_scale : 1.0f / __builtin_sqrtf((float)p->d);
}

template <typename... Ptrs>
sagebwd_status check_ptrs(Ptrs... ptrs) {
  const void* arr[] = {static_cast<const void*>(ptrs)...};
  for (const void* q : arr)
    if (!q) return SAGEBWD_ERR_NULL;
  for (const void* q : arr)
    if (!aligned16(q)) return SAGEBWD_ERR_ALIGN;
  return SAGEBWD_OK;
}

struct BwdLayout {
  bool spill;
  bool spill_fits;  // one head's dS tiles stay below 4 GiB
  long long tiles;  // dS tiles per head (spill mode)
  size_t pk, dq, ktp, dsp, dsm, gq, gk, total;
};

BwdLayout bwd_layout(const sagebwd_params* praw) {
  const sagebwd_params pp = padded(praw);
  const sagebwd_params* p = &pp;
  BwdLayout L{};
  const size_t bh = (size_t)p->B * p->H;
  L.pk = 0;
  const size_t after_pk = round_up(bh * (p->N / 64) * sagebwd::packet_bytes(p->d));
  L.tiles = sagebwd::spill_tiles_per_head(p->N, p->blk, p->causal != 0);
  const size_t ktp_bytes = round_up(bh * (p->N / p->blk) * (size_t)p->d * p->blk);
  const size_t dsp_bytes = round_up(bh * (size_t)L.tiles * 64 * p->blk);
  const size_t dsm_bytes = round_up(bh * (size_t)L.tiles * (p->blk / 64) * 4);
  const size_t spill_bytes = ktp_bytes + dsp_bytes + dsm_bytes;
  // the dQ pass addresses one head's dS tiles with 32-bit buffer offsets
  L.spill_fits = (size_t)L.tiles * 64 * p->blk < (1ull << 32);
  L.spill = L.spill_fits && (p->dq_mode == SAGEBWD_DQ_SPILL ||
                             (p->dq_mode == SAGEBWD_DQ_AUTO && spill_bytes <= SAGEBWD_DQ_AUTO_SPILL_LIMIT));
  if (L.spill) {
    L.ktp = after_pk;
    L.dsp = L.ktp + ktp_bytes;
    L.dsm = L.dsp + dsp_bytes;
    L.total = L.dsm + dsm_bytes;
  } else {
    L.dq = after_pk;
    L.total = L.dq + round_up(4 * elems(p));
  }
  if (p->qk_gain) {
    // partial sums of the gains' gradients: per (head, 64-query tile) and per (head, key block)
    L.gq = L.total;
    L.gk = L.gq + round_up(4 * bh * (p->N / 64) * (size_t)p->d);
    L.total = L.gk + round_up(4 * bh * (p->N / p->blk) * (size_t)p->d);
  }
  return L;
}

// Prologue scratch: the keys' per-block channel sums (K-smoothing), then the queries'
// (Q-smoothing), each 256-byte aligned.
size_t prologue_part_bytes(const sagebwd_params* p) {
  return round_up(4 * (size_t)p->B * p->H * (padded_n(p) / p->blk) * p->d);
}

}  // namespace

extern "C" {

const char* sagebwd_status_string(sagebwd_status s) {
  switch (s) {
    case SAGEBWD_OK: return "ok";
    case SAGEBWD_ERR_NULL: return "null pointer argument";
    case SAGEBWD_ERR_SHAPE: return "invalid shape (negative size, N > 2^22, B*H > 2^24, or too many quantisation blocks)";
    case SAGEBWD_ERR_UNSUPPORTED: return "unsupported option (d, blk, dtype, dq_mode, layout, fmt, split, eps or gains)";
    case SAGEBWD_ERR_ALIGN: return "pointer not 16-byte aligned";
    case SAGEBWD_ERR_WORKSPACE: return "workspace too small";
    case SAGEBWD_ERR_HIP: return "HIP kernel launch failed";
    case SAGEBWD_ERR_SCRATCH: return "problem exceeds the allocation-free entry point's static scratch";
  }
  return "unknown status";
}

// Text of the last HIP failure on this host thread ("" if none since the thread started).
static thread_local char g_last_error[192];

static sagebwd_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return SAGEBWD_OK;
  snprintf(g_last_error, sizeof g_last_error, "%s: %s (%s)", what, hipGetErrorName(e), hipGetErrorString(e));
  return SAGEBWD_ERR_HIP;
}

const char* sagebwd_last_error(void) { return g_last_error; }

size_t sagebwd_prologue_workspace_bytes(const sagebwd_params* p) {
  if (check_params(p) != SAGEBWD_OK) return 0;
  if (empty(p)) return 0;
  return (p->k_smooth ? prologue_part_bytes(p) : 0) + (p->q_smooth ? prologue_part_bytes(p) : 0);
}

size_t sagebwd_backward_workspace_bytes(const sagebwd_params* p) {
  if (check_params(p) != SAGEBWD_OK) return 0;
  if (empty(p)) return 0;
  const BwdLayout L = bwd_layout(p);
  if (p->dq_mode == SAGEBWD_DQ_SPILL && !L.spill_fits) return 0;
  return L.total;
}

// noalloc: the workspace is the current device's static scratch (looked up after every
// argument check), never the caller's.
static sagebwd_status prologue_impl(const sagebwd_params* p, const void* Q, const void* K, const void* V,
                                    int8_t* Qc, int8_t* Kc, int8_t* Vtc, float* Qs, float* Ks, float* Vs,
                                    float* q_rstd, float* k_rstd, float* k_mean, float* q_mean, float* kbias,
                                    const float* q_gain, const float* k_gain, void* workspace,
                                    size_t workspace_bytes, void* stream, bool noalloc) {
  const char* who = noalloc ? "sagebwd_quant_prologue_noalloc" : "sagebwd_quant_prologue";
  sagebwd_status st = check_params(p);
  if (st != SAGEBWD_OK) return st;
  if (empty(p)) return SAGEBWD_OK;
  st = check_ptrs(Q, K, V, Qc, Kc, Vtc, Qs, Ks, Vs, q_rstd, k_rstd, k_mean);
  if (st != SAGEBWD_OK) return st;
  if (p->q_smooth && (st = check_ptrs(q_mean, kbias)) != SAGEBWD_OK) return st;
  if (p->qk_gain && (st = check_ptrs(q_gain, k_gain)) != SAGEBWD_OK) return st;
  const size_t need = sagebwd_prologue_workspace_bytes(p);
  if (noalloc) {
    if (need > SAGEBWD_NOALLOC_SCRATCH_BYTES) return SAGEBWD_ERR_SCRATCH;
    workspace = nullptr;
    workspace_bytes = 0;
    if (need > 0) {
      const hipError_t e = sagebwd::noalloc_scratch(static_cast<hipStream_t>(stream), &workspace);
      if (e != hipSuccess) return hip_status(e, who);
      workspace_bytes = SAGEBWD_NOALLOC_SCRATCH_BYTES;
    }
  } else if (need > 0) {
    if (!workspace) return SAGEBWD_ERR_NULL;
    if (!aligned16(workspace)) return SAGEBWD_ERR_ALIGN;
    if (workspace_bytes < need) return SAGEBWD_ERR_WORKSPACE;
  }
  PrologueArgs a{};
  a.Q = static_cast<const unsigned short*>(Q);
  a.K = static_cast<const unsigned short*>(K);
  a.V = static_cast<const unsigned short*>(V);
  a.Qc = Qc; a.Kc = Kc; a.Vtc = Vtc;
  a.Qs = Qs; a.Ks = Ks; a.Vs = Vs;
  a.q_rstd = q_rstd; a.k_rstd = k_rstd; a.k_mean = k_mean;
  if (p->qk_gain) {
    a.q_gain = q_gain;
    a.k_gain = k_gain;
  }
  char* ws = static_cast<char*>(workspace);
  a.kpart = p->k_smooth ? reinterpret_cast<float*>(ws) : nullptr;
  if (p->q_smooth) {
    a.q_mean = q_mean;
    a.kbias = kbias;
    a.qpart = reinterpret_cast<float*>(ws + (p->k_smooth ? prologue_part_bytes(p) : 0));
  }
  a.BH = p->B * p->H; a.N = padded_n(p); a.Nv = p->N; a.D = p->d; a.BLK = p->blk; a.dtype = p->dtype;
  a.fmt = p->fmt;
  a.x16 = strides16(p);
  a.qk_norm = p->qk_norm != 0; a.k_smooth = p->k_smooth != 0; a.q_smooth = p->q_smooth != 0;
  a.eps = p->eps;
  return hip_status(sagebwd::launch_prologue(a, static_cast<hipStream_t>(stream)), who);
}

sagebwd_status sagebwd_quant_prologue(const sagebwd_params* p, const void* Q, const void* K, const void* V,
                                      int8_t* Qc, int8_t* Kc, int8_t* Vtc, float* Qs, float* Ks, float* Vs,
                                      float* q_rstd, float* k_rstd, float* k_mean, float* q_mean,
                                      float* kbias, const float* q_gain, const float* k_gain, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  return prologue_impl(p, Q, K, V, Qc, Kc, Vtc, Qs, Ks, Vs, q_rstd, k_rstd, k_mean, q_mean, kbias, q_gain, k_gain,
                       workspace, workspace_bytes, stream, false);
}

sagebwd_status sagebwd_quant_prologue_noalloc(const sagebwd_params* p, const void* Q, const void* K,
                                              const void* V, int8_t* Qc, int8_t* Kc, int8_t* Vtc, float* Qs,
                                              float* Ks, float* Vs, float* q_rstd, float* k_rstd, float* k_mean,
                                              float* q_mean, float* kbias, const float* q_gain,
                                              const float* k_gain, void* stream) {
  return prologue_impl(p, Q, K, V, Qc, Kc, Vtc, Qs, Ks, Vs, q_rstd, k_rstd, k_mean, q_mean, kbias, q_gain, k_gain,
                       nullptr, 0, stream, true);
}

sagebwd_status sagebwd_forward(const sagebwd_params* p, const int8_t* Qc, const int8_t* Kc, const int8_t* Vtc,
                               const float* Qs, const float* Ks, const float* Vs, const float* kbias,
                               const void* V, void* O, float* lse, void* stream) {
  sagebwd_status st = check_params(p);
  if (st != SAGEBWD_OK) return st;
  if (empty(p)) return SAGEBWD_OK;
  const bool qattn = p->split == SAGEBWD_SPLIT_QATTN;
  st = qattn ? check_ptrs(Qc, Kc, Qs, Ks, V, O, lse) : check_ptrs(Qc, Kc, Vtc, Qs, Ks, Vs, O, lse);
  if (st != SAGEBWD_OK) return st;
  if (p->q_smooth && (st = check_ptrs(kbias)) != SAGEBWD_OK) return st;
  ForwardArgs a{};
  a.Qc = Qc; a.Kc = Kc; a.Qs = Qs; a.Ks = Ks;
  a.qattn = qattn;
  if (qattn) {
    a.V = static_cast<const unsigned short*>(V);
  } else {
    a.Vtc = Vtc;
    a.Vs = Vs;
  }
  a.q_smooth = p->q_smooth != 0;
  a.kbias = a.q_smooth ? kbias : nullptr;
  a.O = static_cast<unsigned short*>(O); a.lse = lse;
  a.BH = p->B * p->H; a.N = padded_n(p); a.Nv = p->N; a.D = p->d; a.BLK = p->blk; a.dtype = p->dtype;
  a.fmt = p->fmt;
  a.x16 = strides16(p);
  a.causal = p->causal != 0; a.sm_scale = sm_scale_of(p);
  return hip_status(sagebwd::launch_forward(a, static_cast<hipStream_t>(stream)), "sagebwd_forward");
}

static sagebwd_status backward_impl(const sagebwd_params* p, int part, const void* Q, const void* K,
                                    const void* V, const int8_t* Qc, const int8_t* Kc, const float* Qs,
                                    const float* Ks, const float* q_rstd, const float* k_rstd,
                                    const float* q_mean, const float* kbias, const float* q_gain,
                                    const float* k_gain, const void* O, const float* lse, const void* dO,
                                    void* dQ, void* dK, void* dV, float* dq_gain, float* dk_gain,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  sagebwd_status st = check_params(p);
  if (st != SAGEBWD_OK) return st;
  if (part < -1 || part > 2) return SAGEBWD_ERR_UNSUPPORTED;
  if (empty(p)) return SAGEBWD_OK;
  st = check_ptrs(Q, K, V, Qc, Kc, Qs, Ks, q_rstd, k_rstd, O, lse, dO, dQ, dK, dV);
  if (st != SAGEBWD_OK) return st;
  if (p->q_smooth && (st = check_ptrs(q_mean, kbias)) != SAGEBWD_OK) return st;
  if (p->qk_gain && (st = check_ptrs(q_gain, k_gain, dq_gain, dk_gain)) != SAGEBWD_OK) return st;
  if (!workspace) return SAGEBWD_ERR_NULL;
  if (!aligned16(workspace)) return SAGEBWD_ERR_ALIGN;
  const BwdLayout L = bwd_layout(p);
  if (p->dq_mode == SAGEBWD_DQ_SPILL && !L.spill_fits) return SAGEBWD_ERR_UNSUPPORTED;
  if (workspace_bytes < L.total) return SAGEBWD_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  BackwardArgs a{};
  a.Q = static_cast<const unsigned short*>(Q);
  a.K = static_cast<const unsigned short*>(K);
  a.V = static_cast<const unsigned short*>(V);
  a.O = static_cast<const unsigned short*>(O);
  a.dO = static_cast<const unsigned short*>(dO);
  a.Qc = Qc; a.Kc = Kc; a.Qs = Qs; a.Ks = Ks;
  a.q_rstd = q_rstd; a.k_rstd = k_rstd; a.lse = lse;
  a.q_smooth = p->q_smooth != 0;
  if (a.q_smooth) {
    a.q_mean = q_mean;
    a.kbias = kbias;
  }
  a.dQ = static_cast<unsigned short*>(dQ);
  a.dK = static_cast<unsigned short*>(dK);
  a.dV = static_cast<unsigned short*>(dV);
  if (p->qk_gain) {
    a.q_gain = q_gain;
    a.k_gain = k_gain;
    a.dq_gain = dq_gain;
    a.dk_gain = dk_gain;
    a.gq_part = reinterpret_cast<float*>(ws + L.gq);
    a.gk_part = reinterpret_cast<float*>(ws + L.gk);
  }
  a.pk = reinterpret_cast<int8_t*>(ws + L.pk);
  a.spill = L.spill;
  if (L.spill) {
    a.ktp = reinterpret_cast<int8_t*>(ws + L.ktp);
    a.dsp = reinterpret_cast<int8_t*>(ws + L.dsp);
    a.dsm = reinterpret_cast<float*>(ws + L.dsm);
    a.spill_tiles = L.tiles;
  } else {
    a.dq_acc = reinterpret_cast<float*>(ws + L.dq);
  }
  a.BH = p->B * p->H; a.N = padded_n(p); a.Nv = p->N; a.D = p->d; a.BLK = p->blk; a.dtype = p->dtype;
  a.fmt = p->fmt;
  a.x16 = strides16(p);
  // normed_grads: the epilogues stop before the RMSNorm backward
  a.causal = p->causal != 0; a.qk_norm = p->qk_norm != 0 && !p->normed_grads; a.sm_scale = sm_scale_of(p);
  a.qattn = p->split == SAGEBWD_SPLIT_QATTN;
  return hip_status(sagebwd::launch_backward(a, part, static_cast<hipStream_t>(stream)), "sagebwd_backward");
}

sagebwd_status sagebwd_backward(const sagebwd_params* p, const void* Q, const void* K, const void* V,
                                const int8_t* Qc, const int8_t* Kc, const float* Qs, const float* Ks,
                                const float* q_rstd, const float* k_rstd, const float* q_mean,
                                const float* kbias, const float* q_gain, const float* k_gain, const void* O,
                                const float* lse, const void* dO, void* dQ, void* dK, void* dV, float* dq_gain,
                                float* dk_gain, void* workspace, size_t workspace_bytes, void* stream) {
  return backward_impl(p, -1, Q, K, V, Qc, Kc, Qs, Ks, q_rstd, k_rstd, q_mean, kbias, q_gain, k_gain, O, lse, dO,
                       dQ, dK, dV, dq_gain, dk_gain, workspace, workspace_bytes, stream);
}

sagebwd_status sagebwd_backward_part(const sagebwd_params* p, int32_t part, const void* Q, const void* K,
                                     const void* V, const int8_t* Qc, const int8_t* Kc, const float* Qs,
                                     const float* Ks, const float* q_rstd, const float* k_rstd,
                                     const float* q_mean, const float* kbias, const float* q_gain,
                                     const float* k_gain, const void* O, const float* lse, const void* dO,
                                     void* dQ, void* dK, void* dV, float* dq_gain, float* dk_gain,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  if (part < 0) return check_params(p) != SAGEBWD_OK ? check_params(p) : SAGEBWD_ERR_UNSUPPORTED;
  return backward_impl(p, part, Q, K, V, Qc, Kc, Qs, Ks, q_rstd, k_rstd, q_mean, kbias, q_gain, k_gain, O, lse,
                       dO, dQ, dK, dV, dq_gain, dk_gain, workspace, workspace_bytes, stream);
}

}  // extern "C"
