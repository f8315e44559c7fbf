// Kernel argument blocks and launch entry points (host side of the HIP kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>

#include "sagebwd.h"

namespace sagebwd {

// Element strides of the 16-bit tensors (Q, K, V, O, dO, dQ, dK, dV): element (b, h, n, c)
// sits at b*sb + h*sh + n*sn + c (channels contiguous). [B,H,N,d]: sb = H*N*d, sh = N*d,
// sn = d; [B,N,H,d]: sb = N*H*d, sh = d, sn = H*d.
struct Strides16 {
  long long sb, sh;
  int sn, H;
  __host__ __device__ size_t head(int bh) const { return (size_t)(bh / H) * sb + (size_t)(bh % H) * sh; }
  __host__ __device__ size_t row(int bh, int n) const { return head(bh) + (size_t)n * sn; }
};

struct PrologueArgs {
  const unsigned short *Q, *K, *V;   // 16-bit [BH, N, D]
  int8_t *Qc, *Kc, *Vtc;             // [BH, N, D], [BH, N, D], [BH, D, N]
  float *Qs, *Ks, *Vs;               // [BH, N/BLK]
  float *q_rstd, *k_rstd;            // [BH, N]
  float* k_mean;                     // [BH, D]
  float* kpart;                      // [BH, N/BLK, D] (K-smoothing only)
  float* q_mean;                     // [BH, D] (Q-smoothing only)
  float* kbias;                      // [BH, N] (Q-smoothing only)
  float* qpart;                      // [BH, N/BLK, D] (Q-smoothing only)
  const float *q_gain, *k_gain;      // QK-norm gains [H, D] (NULL: gain 1)
  int BH, N, D, BLK, dtype;
  int qk_norm, k_smooth, q_smooth;
  float eps;
  int Nv;                            // valid tokens per head (N = Nv rounded up to blk)
  int fmt;                           // code format: FMT_INT8 or FMT_FP8
  Strides16 x16;                     // layout of the 16-bit tensors
};

struct ForwardArgs {
  const int8_t *Qc, *Kc, *Vtc;
  const float *Qs, *Ks, *Vs;
  const float* kbias;                // [BH, N] (Q-smoothing only)
  const unsigned short* V;           // 16-bit V, layout x16 (Q-Attn split only)
  int qattn;                         // Q-Attn split: PV in 16 bits from V
  unsigned short* O;                 // [BH, N, D]
  float* lse;                        // [BH, N]
  int BH, N, D, BLK, dtype;
  int causal, q_smooth;
  float sm_scale;
  int Nv;                            // valid tokens per head (N = Nv rounded up to blk)
  int fmt;                           // code format: FMT_INT8 or FMT_FP8
  Strides16 x16;                     // layout of the 16-bit tensors
};

struct BackwardArgs {
  const unsigned short *Q, *K, *V, *O, *dO;  // 16-bit [BH, N, D]
  const int8_t *Qc, *Kc;                     // [BH, N, D]
  const float *Qs, *Ks;                      // [BH, N/BLK]
  const float *q_rstd, *k_rstd, *lse;        // [BH, N]
  const float *q_mean, *kbias;               // [BH, D], [BH, N] (Q-smoothing only)
  const float *q_gain, *k_gain;              // QK-norm gains [H, D] (NULL: gain 1)
  float *dq_gain, *dk_gain;                  // their gradients [H, D] (with the gains)
  float *gq_part, *gk_part;                  // gain-gradient partials [BH, N/64, D], [BH, N/BLK, D]
  unsigned short *dQ, *dK, *dV;              // [BH, N, D]
  // workspace regions
  int8_t* pk;                                // [BH, N/64] tile packets
  float* dq_acc;                             // atomic mode: [BH, N, D]
  int8_t* ktp;                               // spill mode: K^T packets [BH, N/BLK][D*BLK]
  int8_t* dsp;                               // spill mode: dS tiles [BH, spill_tiles][64*BLK]
  float* dsm;                                // spill mode: dQ multipliers [BH, spill_tiles]
  long long spill_tiles;                     // dS tiles per head
  int spill;
  int BH, N, D, BLK, dtype;
  int causal, qk_norm, q_smooth;
  float sm_scale;
  int Nv;                            // valid tokens per head (N = Nv rounded up to blk)
  int fmt;                           // code format: FMT_INT8 or FMT_FP8
  Strides16 x16;                     // layout of the 16-bit tensors
  int qattn;                         // Q-Attn split: dV = P^T dO in 16 bits
};

// Enqueue one kernel and return the status of this launch itself (hipLaunchKernel reports
// it directly, so an error left pending by an unrelated runtime call is not picked up).
template <typename Args>
hipError_t launch_kernel(void (*kernel)(Args), dim3 grid, dim3 block, hipStream_t st, const Args& a) {
  Args copy = a;
  void* params[] = {&copy};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, params, 0, st);
}

hipError_t launch_prologue(const PrologueArgs& a, hipStream_t st);
// Bytes of the static device scratch of the allocation-free prologue entry point, and the
// device address of the current device's copy (looked up on the first call per device; the
// stream, if not null, must belong to the current device).
constexpr size_t kNoAllocScratchBytes = SAGEBWD_NOALLOC_SCRATCH_BYTES;
hipError_t noalloc_scratch(hipStream_t st, void** out);
hipError_t launch_forward(const ForwardArgs& a, hipStream_t st);
hipError_t launch_backward(const BackwardArgs& a, int part, hipStream_t st);  // part -1 = all
size_t packet_bytes(int d);  // bytes of one 64-query backward tile packet
long long spill_tiles_per_head(int N, int blk, int causal);

// Calls f(dtype, d, blk) with std::integral_constant arguments for the supported
// combinations (dtype in {fp16, bf16}, d in {64, 128}, blk in {64, 128}).
template <typename F>
hipError_t dispatch_dt_d_blk(int dtype, int d, int blk, F&& f) {
#define SAGEBWD_CASE(DTV, DV, BV)                                                    \
  if (dtype == DTV && d == DV && blk == BV)                                          \
    return f(std::integral_constant<int, DTV>{}, std::integral_constant<int, DV>{},  \
             std::integral_constant<int, BV>{});
  SAGEBWD_CASE(0, 64, 64) SAGEBWD_CASE(0, 64, 128) SAGEBWD_CASE(0, 128, 64) SAGEBWD_CASE(0, 128, 128)
  SAGEBWD_CASE(1, 64, 64) SAGEBWD_CASE(1, 64, 128) SAGEBWD_CASE(1, 128, 64) SAGEBWD_CASE(1, 128, 128)
#undef SAGEBWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace sagebwd
