// Quantisation prologue: QK-norm -> K-smoothing -> per-block INT8 codes.
// SageBwd article (aitrends.kr 8227): QK-norm paragraph (per-token RMSNorm, gain 1),
// K-smoothing paragraph (subtract the keys' per-channel mean right before quantising),
// per-block kernels paragraph (one scale per block of tokens).
//
// The results are specified bit for bit (include/sagebwd.h): every float32 operation
// below is one IEEE operation with round-to-nearest-even, no contraction into FMA,
// sums in ascending index order, correctly rounded division and square root.
//
// Pass 1, one workgroup per (head, token block, tensor):
//   Q: rstd per token, Q^ = Q*rstd, block absmax, codes (token-major).
//   K: rstd per token; with smoothing, the block's per-channel sums of K^ (pass 2
//      quantises); without smoothing, codes of K^ as for Q.
//   V: block absmax, codes written channel-major (V^T), as the forward's PV product reads it.
// Pass 2 (smoothing only), one workgroup per (head, token block): mean = sum of the block
//   sums / N, K~ = K^ - mean, block absmax, codes.
// Each block is staged once through LDS as float32 rows of D+1 words, so that a thread
// walking its own token row and a thread walking a channel column both hit distinct banks.
#pragma clang fp contract(off)

#include "common.hpp"
#include "launch.hpp"

namespace sagebwd {

namespace {

constexpr int kThreads = 256;

template <int D, int BLK>
struct ProLds {
  float x[BLK][D + 1];
  float rstd[BLK];
  float red[kThreads / 64];
  float mu[D];
};

// Block absmax over the whole workgroup (exact: max is order independent).
__device__ __forceinline__ float block_absmax(float v, float* red) {
  v = wave_max(v);
  if (lane_id() == 0) red[wave_id()] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

// Coalesced load of a BLK x D block of 16-bit values into LDS as float32.
template <int DT, int D, int BLK>
__device__ __forceinline__ void load_block(const unsigned short* __restrict__ src, ProLds<D, BLK>& s) {
  constexpr int kChunks = BLK * D / 8;  // 8 values (16 bytes) per chunk
#pragma unroll
  for (int ch = threadIdx.x; ch < kChunks; ch += kThreads) {
    u16x8 v = *reinterpret_cast<const u16x8*>(src + (size_t)ch * 8);
    const int t = (ch * 8) / D, c = (ch * 8) % D;
#pragma unroll
    for (int i = 0; i < 8; ++i) s.x[t][c + i] = to_f32<DT>(v[i]);
  }
}

// rstd of every token row of s.x (threads t < BLK), ascending channel order.
template <int D, int BLK>
__device__ __forceinline__ void token_rstd(ProLds<D, BLK>& s, float eps, float* __restrict__ rstd_out) {
  const int t = threadIdx.x;
  if (t < BLK) {
    float ss = 0.0f;
    for (int c = 0; c < D; ++c) {
      const float v = s.x[t][c];
      ss = ss + v * v;
    }
    const float ms = ss / (float)D;
    const float r = 1.0f / __builtin_sqrtf(ms + eps);
    s.rstd[t] = r;
    rstd_out[t] = r;
  }
}

// Quantise s.x (already the values to quantise) as one block; codes token-major.
template <int D, int BLK>
__device__ __forceinline__ void quant_token_major(ProLds<D, BLK>& s, int8_t* __restrict__ codes,
                                                  float* __restrict__ scale_out) {
  constexpr int kWords = BLK * D / 4;
  float m = 0.0f;
  for (int w = threadIdx.x; w < kWords; w += kThreads) {
    const int t = (w * 4) / D, c = (w * 4) % D;
#pragma unroll
    for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(s.x[t][c + i]));
  }
  const float a = block_absmax(m, s.red);
  const float inv = a > 0.0f ? 127.0f / a : 0.0f;
  if (threadIdx.x == 0) *scale_out = a > 0.0f ? a / 127.0f : 0.0f;
  for (int w = threadIdx.x; w < kWords; w += kThreads) {
    const int t = (w * 4) / D, c = (w * 4) % D;
    const unsigned word = pack4_lo_bytes(quant_word(s.x[t][c], inv), quant_word(s.x[t][c + 1], inv),
                                         quant_word(s.x[t][c + 2], inv), quant_word(s.x[t][c + 3], inv));
    reinterpret_cast<unsigned*>(codes)[w] = word;
  }
}

}  // namespace

template <int DT, int D, int BLK>
__global__ __launch_bounds__(kThreads) void prologue_pass1(PrologueArgs a) {
  __shared__ ProLds<D, BLK> s;
  const int nb = a.N / BLK;
  const int tensor = blockIdx.x % 3;          // 0 = Q, 1 = K, 2 = V
  const int blk_id = (blockIdx.x / 3) % nb;
  const int bh = (blockIdx.x / 3) / nb;
  const size_t tok0 = (size_t)bh * a.N + (size_t)blk_id * BLK;   // first token row of the block
  const size_t sidx = (size_t)bh * nb + blk_id;                    // scale index

  const unsigned short* src = (tensor == 0 ? a.Q : tensor == 1 ? a.K : a.V) + tok0 * D;
  load_block<DT, D, BLK>(src, s);
  __syncthreads();

  if (tensor == 2) {
    // V: quantise the raw values; codes stored channel-major: Vtc[bh][c][token].
    constexpr int kWords = BLK * D / 4;
    float m = 0.0f;
    for (int w = threadIdx.x; w < kWords; w += kThreads) {
      const int t = (w * 4) / D, c = (w * 4) % D;
#pragma unroll
      for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(s.x[t][c + i]));
    }
    const float amax = block_absmax(m, s.red);
    const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
    if (threadIdx.x == 0) a.Vs[sidx] = amax > 0.0f ? amax / 127.0f : 0.0f;
    for (int w = threadIdx.x; w < kWords; w += kThreads) {
      const int c = w / (BLK / 4), t = 4 * (w % (BLK / 4));
      const unsigned word = pack4_lo_bytes(quant_word(s.x[t][c], inv), quant_word(s.x[t + 1][c], inv),
                                           quant_word(s.x[t + 2][c], inv), quant_word(s.x[t + 3][c], inv));
      int8_t* dst = a.Vtc + ((size_t)bh * D + c) * a.N + (size_t)blk_id * BLK + t;
      *reinterpret_cast<unsigned*>(dst) = word;
    }
    return;
  }

  float* rstd_out = (tensor == 0 ? a.q_rstd : a.k_rstd) + tok0;
  if (a.qk_norm) {
    token_rstd<D, BLK>(s, a.eps, rstd_out);
    __syncthreads();
    for (int e = threadIdx.x; e < BLK * D; e += kThreads) {
      const int t = e / D, c = e % D;
      s.x[t][c] = s.x[t][c] * s.rstd[t];
    }
  } else {
    if (threadIdx.x < BLK) rstd_out[threadIdx.x] = 1.0f;
  }
  __syncthreads();

  if (tensor == 1 && a.k_smooth) {
    // Per-channel sum of the block's normalised keys, tokens in ascending order.
    for (int c = threadIdx.x; c < D; c += kThreads) {
      float part = 0.0f;
      for (int t = 0; t < BLK; ++t) part = part + s.x[t][c];
      a.kpart[sidx * D + c] = part;
    }
    return;
  }
  if (tensor == 1) {
    for (int c = threadIdx.x; c < D; c += kThreads)
      if (blk_id == 0) a.k_mean[(size_t)bh * D + c] = 0.0f;
  }
  quant_token_major<D, BLK>(s, (tensor == 0 ? a.Qc : a.Kc) + tok0 * D, (tensor == 0 ? a.Qs : a.Ks) + sidx);
}

template <int DT, int D, int BLK>
__global__ __launch_bounds__(kThreads) void prologue_pass2(PrologueArgs a) {
  __shared__ ProLds<D, BLK> s;
  const int nb = a.N / BLK;
  const int blk_id = blockIdx.x % nb;
  const int bh = blockIdx.x / nb;
  const size_t tok0 = (size_t)bh * a.N + (size_t)blk_id * BLK;
  const size_t sidx = (size_t)bh * nb + blk_id;

  // Mean over all tokens of the head: block sums in ascending block order, then / N.
  for (int c = threadIdx.x; c < D; c += kThreads) {
    const float* part = a.kpart + (size_t)bh * nb * D + c;
    float tot = 0.0f;
    for (int b = 0; b < nb; ++b) tot = tot + part[(size_t)b * D];
    const float mu = tot / (float)a.N;
    s.mu[c] = mu;
    if (blk_id == 0) a.k_mean[(size_t)bh * D + c] = mu;
  }
  load_block<DT, D, BLK>(a.K + tok0 * D, s);
  if (threadIdx.x < BLK) s.rstd[threadIdx.x] = a.qk_norm ? a.k_rstd[tok0 + threadIdx.x] : 1.0f;
  __syncthreads();
  for (int e = threadIdx.x; e < BLK * D; e += kThreads) {
    const int t = e / D, c = e % D;
    const float kh = s.x[t][c] * s.rstd[t];
    s.x[t][c] = kh - s.mu[c];
  }
  __syncthreads();
  quant_token_major<D, BLK>(s, a.Kc + tok0 * D, a.Ks + sidx);
}

template <int DT, int D, int BLK>
static hipError_t launch_prologue_t(const PrologueArgs& a, hipStream_t st) {
  const int nb = a.N / BLK;
  const long long nblocks = (long long)a.BH * nb;
  const hipError_t e = launch_kernel(&prologue_pass1<DT, D, BLK>, dim3((unsigned)(nblocks * 3)), dim3(kThreads), st, a);
  if (e != hipSuccess || !a.k_smooth) return e;
  return launch_kernel(&prologue_pass2<DT, D, BLK>, dim3((unsigned)nblocks), dim3(kThreads), st, a);
}

hipError_t launch_prologue(const PrologueArgs& a, hipStream_t st) {
  return dispatch_dt_d_blk(a.dtype, a.D, a.BLK, [&](auto dt, auto d, auto blk) {
    return launch_prologue_t<decltype(dt)::value, decltype(d)::value, decltype(blk)::value>(a, st);
  });
}

}  // namespace sagebwd
