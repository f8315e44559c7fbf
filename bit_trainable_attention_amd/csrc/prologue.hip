// Quantisation prologue: QK-norm -> K-smoothing -> per-block INT8 codes.
// SageBwd article (aitrends.kr 8227): QK-norm paragraph (per-token RMSNorm, gain 1),
// K-smoothing paragraph (subtract the keys' per-channel mean right before quantising),
// per-block kernels paragraph (one scale per block of tokens).
//
// The results are specified bit for bit (include/sagebwd.h): every float32 operation
// below is one IEEE operation with round-to-nearest-even, no contraction into FMA,
// correctly rounded division and square root, and every sum runs in the stated order.
//
// Thread layout of a (head, block of BLK tokens) workgroup, 256 threads: thread (j, ch),
// j = tid / 16 (token slot), ch = tid % 16 (channel chunk), owns channels
// ch*CW .. ch*CW + CW - 1 (CW = D/16) of tokens t = 16p + j, p = 0 .. BLK/16 - 1, in
// registers. The 16 chunks of a token sit in one 16-lane row, so the token's sum of squares
// is each lane's chunk sum (ascending) followed by a pairwise tree across the row (DPP):
// xor 1, xor 2, then the half-row and row mirrors, which pair chunk blocks {0-3, 4-7} and
// {0-7, 8-15}. Float addition is commutative, so both lanes of a pair compute the same sum
// and every lane ends with the tree's result.
//
// pass1  one workgroup per (head, block, tensor):
//          Q: rstd, Q^ = Q*rstd; with Q-smoothing, the block's per-channel sums of Q^ (as
//             for K); without, block absmax and codes (token-major);
//          K: rstd; with K-smoothing, the block's per-channel sums of K^ (group t mod 16 in
//             ascending order, then the pairwise tree over the 16 groups); with neither
//             smoothing, codes;
//          V: block absmax, codes written channel-major (V^T): here thread (j, ch) holds
//             the BLK/16 consecutive tokens from (BLK/16)*j, transposes its code bytes in
//             registers (4 x 4 blocks, v_perm_b32) and stores each channel's run of token
//             codes into an LDS tile, whose rows leave in 16-byte chunks.
// pass2  (either smoothing) one workgroup per (head, block) for K, and with Q-smoothing one
//          more per (head, block) for Q: the head's mean (block sums in ascending block
//          order, / N; every workgroup of the head computes it, block 0's stores it),
//          x~ = x^ - mean, absmax, codes. With Q-smoothing the K workgroups also compute the
//          query mean and each key's bias b = Ks * (codes . q_mean) (SageBwd article,
//          Q-smoothing paragraph): per token, each lane's chunk in ascending channel order,
//          then the 16-lane tree.
#pragma clang fp contract(off)

#include "common.hpp"
#include "launch.hpp"

#include <mutex>

namespace sagebwd {

namespace {

constexpr int kThreads = 256;

// Per-thread slice of a block: P tokens x CW channels.
template <int D, int BLK>
struct Slice {
  static constexpr int CW = D / 16;
  static constexpr int P = BLK / 16;
  float x[P][CW];
};

template <int DT, int CW>
__device__ __forceinline__ void load_chunk(const unsigned short* __restrict__ src, float* x) {
  if constexpr (CW == 8) {
    const u16x8 v = *reinterpret_cast<const u16x8*>(src);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = to_f32<DT>(v[i]);
  } else {
    static_assert(CW == 4, "chunk width");
    const u16x4 v = *reinterpret_cast<const u16x4*>(src);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = to_f32<DT>(v[i]);
  }
}

// blk_src: the block's first token row; rows are sn elements apart; rows from nvalid on
// (a ragged last block) are zero tokens and are not read
template <int DT, int D, int BLK>
__device__ __forceinline__ void load_slice(const unsigned short* __restrict__ blk_src, int sn, int nvalid,
                                           Slice<D, BLK>& s, int j, int ch) {
  if (nvalid >= BLK) {   // a whole block (uniform branch): unguarded loads
#pragma unroll
    for (int p = 0; p < Slice<D, BLK>::P; ++p)
      load_chunk<DT, Slice<D, BLK>::CW>(blk_src + (size_t)(16 * p + j) * sn + ch * Slice<D, BLK>::CW, s.x[p]);
    return;
  }
#pragma unroll
  for (int p = 0; p < Slice<D, BLK>::P; ++p) {
    if (16 * p + j < nvalid) {
      load_chunk<DT, Slice<D, BLK>::CW>(blk_src + (size_t)(16 * p + j) * sn + ch * Slice<D, BLK>::CW, s.x[p]);
    } else {
#pragma unroll
      for (int i = 0; i < Slice<D, BLK>::CW; ++i) s.x[p][i] = 0.0f;
    }
  }
}

// As load_slice, but thread (j, ch) takes the P consecutive tokens P*j .. P*j + P - 1
// (slot p = token P*j + p): the V layout, whose codes leave channel-major.
template <int DT, int D, int BLK>
__device__ __forceinline__ void load_slice_consec(const unsigned short* __restrict__ blk_src, int sn, int nvalid,
                                                  Slice<D, BLK>& s, int j, int ch) {
  using S = Slice<D, BLK>;
  if (nvalid >= BLK) {
#pragma unroll
    for (int p = 0; p < S::P; ++p) load_chunk<DT, S::CW>(blk_src + (size_t)(S::P * j + p) * sn + ch * S::CW, s.x[p]);
    return;
  }
#pragma unroll
  for (int p = 0; p < S::P; ++p) {
    if (S::P * j + p < nvalid) {
      load_chunk<DT, S::CW>(blk_src + (size_t)(S::P * j + p) * sn + ch * S::CW, s.x[p]);
    } else {
#pragma unroll
      for (int i = 0; i < S::CW; ++i) s.x[p][i] = 0.0f;
    }
  }
}

// 4 x 4 byte transpose: r[t] holds bytes (b0 .. b3) of row t; out[c] gets byte c of rows
// 0 .. 3 (byte t of out[c] = byte c of r[t]). v_perm_b32 selects bytes 0-3 of its second
// operand and 4-7 of its first.
__device__ __forceinline__ void transpose4x4_bytes(const unsigned (&r)[4], unsigned (&out)[4]) {
  const unsigned e01 = __builtin_amdgcn_perm(r[1], r[0], 0x06020400u);   // r0.b0 r1.b0 r0.b2 r1.b2
  const unsigned o01 = __builtin_amdgcn_perm(r[1], r[0], 0x07030501u);   // r0.b1 r1.b1 r0.b3 r1.b3
  const unsigned e23 = __builtin_amdgcn_perm(r[3], r[2], 0x06020400u);
  const unsigned o23 = __builtin_amdgcn_perm(r[3], r[2], 0x07030501u);
  out[0] = __builtin_amdgcn_perm(e23, e01, 0x05040100u);
  out[2] = __builtin_amdgcn_perm(e23, e01, 0x07060302u);
  out[1] = __builtin_amdgcn_perm(o23, o01, 0x05040100u);
  out[3] = __builtin_amdgcn_perm(o23, o01, 0x07060302u);
}

// Sum of the 16 lanes of each row by the pairwise tree (xor 1, xor 2, half mirror, mirror).
template <int CTRL>
__device__ __forceinline__ float add_dpp(float v) {
  return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row_tree_sum(float v) {
  v = add_dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v = add_dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  v = add_dpp<0x141>(v);  // row_half_mirror: chunks 0-3 with 4-7 (and 8-11 with 12-15)
  v = add_dpp<0x140>(v);  // row_mirror: chunks 0-7 with 8-15
  return v;
}

// QK-norm of the thread's tokens in place; lane ch == 0 writes rstd of each token. Tokens
// from nvalid on (the padding of a ragged last block) are zeros and get rstd = 1, so they stay
// zero even with eps = 0 (where 1/sqrt(0) would make them 0 * inf = NaN).
template <int D, int BLK>
__device__ __forceinline__ void qk_norm_slice(Slice<D, BLK>& s, float eps, float* __restrict__ rstd_out, int j,
                                              int ch, int nvalid) {
  using S = Slice<D, BLK>;
#pragma unroll
  for (int p = 0; p < S::P; ++p) {
    float cs = 0.0f;
#pragma unroll
    for (int i = 0; i < S::CW; ++i) {
      const float sq = s.x[p][i] * s.x[p][i];
      cs = cs + sq;
    }
    const float ss = row_tree_sum(cs);
    const float ms = ss / (float)D;
    const float r = 16 * p + j < nvalid ? 1.0f / __builtin_sqrtf(ms + eps) : 1.0f;
#pragma unroll
    for (int i = 0; i < S::CW; ++i) s.x[p][i] = s.x[p][i] * r;
    if (ch == 0) rstd_out[16 * p + j] = r;
  }
}

// The learnable QK-norm gain of head h (NULL: gain 1): x^ = fl(x^ * g[h][c]) for the thread's
// channels (SageBwd article, QK-norm paragraph: RMSNorm per token, here with its weight).
template <int D, int BLK>
__device__ __forceinline__ void apply_gain_slice(Slice<D, BLK>& s, const float* __restrict__ gain, int h, int ch) {
  using S = Slice<D, BLK>;
  if (!gain) return;
  float g[S::CW];
#pragma unroll
  for (int i = 0; i < S::CW; ++i) g[i] = gain[(size_t)h * D + ch * S::CW + i];
#pragma unroll
  for (int p = 0; p < S::P; ++p)
#pragma unroll
    for (int i = 0; i < S::CW; ++i) s.x[p][i] = s.x[p][i] * g[i];
}

// Block absmax over the workgroup (exact: max is order independent).
template <int D, int BLK>
__device__ __forceinline__ float slice_absmax(const Slice<D, BLK>& s, float* red) {
  float m = 0.0f;
#pragma unroll
  for (int p = 0; p < Slice<D, BLK>::P; ++p)
#pragma unroll
    for (int i = 0; i < Slice<D, BLK>::CW; ++i) m = fmaxf(m, fabsf(s.x[p][i]));
  m = wave_max(m);
  if (lane_id() == 0) red[wave_id()] = m;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Codes of the thread's values under the block's absmax a, token-major; scale a/M with
// M = 127 (INT8) or 448 (FP8 e4m3).
template <int D, int BLK>
__device__ __forceinline__ void quant_slice_token_major(const Slice<D, BLK>& s, float a, bool fp8,
                                                        int8_t* __restrict__ blk_codes, float* __restrict__ scale_out,
                                                        int j, int ch) {
  using S = Slice<D, BLK>;
  const float M = fp8 ? 448.0f : 127.0f;
  const float inv = a > 0.0f ? M / a : 0.0f;
  if (threadIdx.x == 0) *scale_out = a > 0.0f ? a / M : 0.0f;
#pragma unroll
  for (int p = 0; p < S::P; ++p) {
    int8_t* dst = blk_codes + (size_t)(16 * p + j) * D + ch * S::CW;
    const unsigned w0 = code_word(fp8, s.x[p][0], s.x[p][1], s.x[p][2], s.x[p][3], inv);
    if constexpr (S::CW == 8) {
      const unsigned w1 = code_word(fp8, s.x[p][4], s.x[p][5], s.x[p][6], s.x[p][7], inv);
      *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
    } else {
      *reinterpret_cast<unsigned*>(dst) = w0;
    }
  }
}

template <int D, int BLK>
struct Pass1Lds {
  float red[kThreads / 64];
  union {
    float gs[16][D];                               // K: group sums per token slot
    int8_t vt[D][BLK];                             // V: codes, channel-major, chunk q of row c
                                                   // at chunk q ^ vt_swz(c)
  };
};

// The V tile's 16-byte chunk swizzle: the channel rows that one write instruction of the
// 16 channel groups touches start on the same bank, so each group's chunk is rotated.
template <int D, int BLK>
__device__ __forceinline__ int vt_swz(int c) {
  return (c / Slice<D, BLK>::CW) & (BLK / 16 - 1);
}

}  // namespace

template <int DT, int D, int BLK>
__global__ __launch_bounds__(kThreads) void prologue_pass1(PrologueArgs a) {
  using S = Slice<D, BLK>;
  __shared__ __attribute__((aligned(16))) Pass1Lds<D, BLK> lds;
  const int nb = a.N / BLK;
  const int tensor = blockIdx.x % 3;          // 0 = Q, 1 = K, 2 = V
  const int blk_id = (blockIdx.x / 3) % nb;
  const int bh = (blockIdx.x / 3) / nb;
  const size_t tok0 = (size_t)bh * a.N + (size_t)blk_id * BLK;   // first token row of the block
  const size_t sidx = (size_t)bh * nb + blk_id;                    // scale index
  const int j = threadIdx.x >> 4, ch = threadIdx.x & 15;

  S s;
  if (tensor == 2) {
    // V: quantise the raw values; codes stored channel-major: Vtc[bh][c][token]. Thread
    // (j, ch) holds the P consecutive tokens P*j .. of its CW channels, so after a 4 x 4
    // byte transpose of its code words each of its channels has P consecutive token codes,
    // which go to the LDS tile in one store.
    load_slice_consec<DT, D, BLK>(a.V + a.x16.row(bh, blk_id * BLK), a.x16.sn, a.Nv - blk_id * BLK, s, j, ch);
    const float amax = slice_absmax<D, BLK>(s, lds.red);
    const bool fp8 = a.fmt == FMT_FP8;
    const float M = fp8 ? 448.0f : 127.0f;
    const float inv = amax > 0.0f ? M / amax : 0.0f;
    if (threadIdx.x == 0) a.Vs[sidx] = amax > 0.0f ? amax / M : 0.0f;
    constexpr int TG = S::P / 4;    // groups of four tokens
    constexpr int CG = S::CW / 4;   // groups of four channels
    unsigned ct[S::CW][TG];         // ct[i][g]: tokens P*j + 4g .. + 3 of channel ch*CW + i
#pragma unroll
    for (int g = 0; g < TG; ++g)
#pragma unroll
      for (int q = 0; q < CG; ++q) {
        unsigned r[4], o[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float* x = s.x[4 * g + t] + 4 * q;
          r[t] = code_word(fp8, x[0], x[1], x[2], x[3], inv);
        }
        transpose4x4_bytes(r, o);
#pragma unroll
        for (int c = 0; c < 4; ++c) ct[4 * q + c][g] = o[c];
      }
    const int t0 = S::P * j;   // first token of the thread: chunk t0 / 16, byte t0 % 16
#pragma unroll
    for (int i = 0; i < S::CW; ++i) {
      const int c = ch * S::CW + i;
      int8_t* dst = &lds.vt[c][16 * ((t0 >> 4) ^ vt_swz<D, BLK>(c)) + (t0 & 15)];
      if constexpr (TG == 2) *reinterpret_cast<uint2*>(dst) = make_uint2(ct[i][0], ct[i][1]);
      else *reinterpret_cast<unsigned*>(dst) = ct[i][0];
    }
    __syncthreads();
    constexpr int kRowChunks = BLK / 16;
    for (int e = threadIdx.x; e < D * kRowChunks; e += kThreads) {
      const int c = e / kRowChunks, q = e % kRowChunks;
      *reinterpret_cast<i32x4*>(a.Vtc + ((size_t)bh * D + c) * a.N + (size_t)blk_id * BLK + 16 * q) =
          *reinterpret_cast<const i32x4*>(&lds.vt[c][16 * (q ^ vt_swz<D, BLK>(c))]);
    }
    return;
  }
  load_slice<DT, D, BLK>((tensor == 0 ? a.Q : a.K) + a.x16.row(bh, blk_id * BLK), a.x16.sn, a.Nv - blk_id * BLK, s,
                         j, ch);

  float* rstd_out = (tensor == 0 ? a.q_rstd : a.k_rstd) + tok0;
  if (a.qk_norm) {
    qk_norm_slice<D, BLK>(s, a.eps, rstd_out, j, ch, a.Nv - blk_id * BLK);
    apply_gain_slice<D, BLK>(s, tensor == 0 ? a.q_gain : a.k_gain, bh % a.x16.H, ch);
  } else if (ch == 0) {
#pragma unroll
    for (int p = 0; p < S::P; ++p) rstd_out[16 * p + j] = 1.0f;
  }

  if ((tensor == 1 && a.k_smooth) || (tensor == 0 && a.q_smooth)) {
    float* part_out = tensor == 1 ? a.kpart : a.qpart;
    // Per-channel block sums of K^ (or Q^): group j (tokens t = j mod 16) in ascending order ...
#pragma unroll
    for (int i = 0; i < S::CW; ++i) {
      float g = 0.0f;
#pragma unroll
      for (int p = 0; p < S::P; ++p) g = g + s.x[p][i];
      lds.gs[j][ch * S::CW + i] = g;
    }
    __syncthreads();
    // ... then the pairwise tree over the 16 groups.
    for (int c = threadIdx.x; c < D; c += kThreads) {
      float t8[8], t4[4], t2[2];
#pragma unroll
      for (int u = 0; u < 8; ++u) t8[u] = lds.gs[2 * u][c] + lds.gs[2 * u + 1][c];
#pragma unroll
      for (int u = 0; u < 4; ++u) t4[u] = t8[2 * u] + t8[2 * u + 1];
#pragma unroll
      for (int u = 0; u < 2; ++u) t2[u] = t4[2 * u] + t4[2 * u + 1];
      part_out[sidx * D + c] = t2[0] + t2[1];
    }
    return;
  }
  if (tensor == 1 && blk_id == 0) {
    for (int c = threadIdx.x; c < D; c += kThreads) a.k_mean[(size_t)bh * D + c] = 0.0f;
  }
  if (tensor == 1 && a.q_smooth) return;   // the keys' codes and biases come from pass2
  const float amax = slice_absmax<D, BLK>(s, lds.red);
  quant_slice_token_major<D, BLK>(s, amax, a.fmt == FMT_FP8, (tensor == 0 ? a.Qc : a.Kc) + tok0 * D,
                                  (tensor == 0 ? a.Qs : a.Ks) + sidx, j, ch);
}

// The head's per-channel mean from its blocks' channel sums (ascending block order, then one
// division by N) into mean[0..D); threads < D each own a channel.
template <int D>
__device__ __forceinline__ void head_mean(const float* __restrict__ part_head, int nb, int N, float* mean) {
  if (threadIdx.x < D) {
    const float* part = part_head + threadIdx.x;
    float tot = 0.0f;
    int b = 0;
    for (; b + 16 <= nb; b += 16) {   // 16 loads in flight, then the additions in block order
      float v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = part[(size_t)(b + i) * D];
#pragma unroll
      for (int i = 0; i < 16; ++i) tot = tot + v[i];
    }
    for (; b < nb; ++b) tot = tot + part[(size_t)b * D];
    mean[threadIdx.x] = tot / (float)N;
  }
}

template <int DT, int D, int BLK>
__global__ __launch_bounds__(kThreads) void prologue_pass2(PrologueArgs a) {
  using S = Slice<D, BLK>;
  __shared__ float red[kThreads / 64];
  __shared__ float mean[D];
  __shared__ float qmean[D];
  const int nb = a.N / BLK;
  const long long nblocks = (long long)a.BH * nb;
  const bool is_q = (long long)blockIdx.x >= nblocks;           // Q-smoothing workgroups follow
  const long long wg = is_q ? (long long)blockIdx.x - nblocks : (long long)blockIdx.x;
  const int blk_id = (int)(wg % nb);
  const int bh = (int)(wg / nb);
  const size_t tok0 = (size_t)bh * a.N + (size_t)blk_id * BLK;
  const size_t sidx = (size_t)bh * nb + blk_id;
  const int j = threadIdx.x >> 4, ch = threadIdx.x & 15;

  S s;
  load_slice<DT, D, BLK>((is_q ? a.Q : a.K) + a.x16.row(bh, blk_id * BLK), a.x16.sn, a.Nv - blk_id * BLK, s, j, ch);
  // mean of the head's keys (or queries) per channel; every workgroup of the head computes the
  // same value, the one of block 0 stores it
  const bool smooth = is_q || a.k_smooth;
  if (smooth) {
    head_mean<D>((is_q ? a.qpart : a.kpart) + (size_t)bh * nb * D, nb, a.Nv, mean);
    if (blk_id == 0 && threadIdx.x < D) (is_q ? a.q_mean : a.k_mean)[(size_t)bh * D + threadIdx.x] = mean[threadIdx.x];
  }
  if (!is_q && a.q_smooth) head_mean<D>(a.qpart + (size_t)bh * nb * D, nb, a.Nv, qmean);
  __syncthreads();
  float mu[S::CW], gn[S::CW];
  const float* gain = a.qk_norm ? (is_q ? a.q_gain : a.k_gain) : nullptr;
#pragma unroll
  for (int i = 0; i < S::CW; ++i) {
    mu[i] = smooth ? mean[ch * S::CW + i] : 0.0f;
    gn[i] = gain ? gain[(size_t)(bh % a.x16.H) * D + ch * S::CW + i] : 1.0f;
  }
  const float* rstd = is_q ? a.q_rstd : a.k_rstd;
#pragma unroll
  for (int p = 0; p < S::P; ++p) {
    const float r = a.qk_norm ? rstd[tok0 + 16 * p + j] : 1.0f;
    const bool valid = blk_id * BLK + 16 * p + j < a.Nv;   // padding tokens stay 0 (uniform but the last block)
#pragma unroll
    for (int i = 0; i < S::CW; ++i) {
      const float xh = (s.x[p][i] * r) * gn[i];   // gn = 1 without gains: exact
      s.x[p][i] = valid ? xh - mu[i] : 0.0f;
    }
  }
  const float amax = slice_absmax<D, BLK>(s, red);
  quant_slice_token_major<D, BLK>(s, amax, a.fmt == FMT_FP8, (is_q ? a.Qc : a.Kc) + tok0 * D, (is_q ? a.Qs : a.Ks) + sidx, j, ch);
  if (is_q || !a.q_smooth) return;
  // key bias b = Ks * (codes . q_mean): the codes as quant_slice_token_major made them
  const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
  const float scale = amax > 0.0f ? amax / 127.0f : 0.0f;
  float qm[S::CW];
#pragma unroll
  for (int i = 0; i < S::CW; ++i) qm[i] = qmean[ch * S::CW + i];
#pragma unroll
  for (int p = 0; p < S::P; ++p) {
    float dot = 0.0f;
#pragma unroll
    for (int i = 0; i < S::CW; ++i) {
      const float code = (float)(int8_t)quant_word(s.x[p][i], inv);
      dot = dot + code * qm[i];
    }
    dot = row_tree_sum(dot);
    if (ch == 0) a.kbias[tok0 + 16 * p + j] = scale * dot;
  }
}

template <int DT, int D, int BLK>
static hipError_t launch_prologue_t(const PrologueArgs& a, hipStream_t st) {
  const int nb = a.N / BLK;
  const long long nblocks = (long long)a.BH * nb;
  hipError_t e = launch_kernel(&prologue_pass1<DT, D, BLK>, dim3((unsigned)(nblocks * 3)), dim3(kThreads), st, a);
  if (e != hipSuccess || !(a.k_smooth || a.q_smooth)) return e;
  return launch_kernel(&prologue_pass2<DT, D, BLK>, dim3((unsigned)(nblocks * (a.q_smooth ? 2 : 1))),
                       dim3(kThreads), st, a);
}

// ---------------------------------------------------------------- allocation-free scratch
// The allocation-free prologue entry point takes its block-sum scratch from this array: each
// GPU the library runs on holds its own copy from the first call on it until the process
// ends. In host code `scratch` names a host-side stand-in, not device memory: the device
// address is looked up once per device (hipGetSymbolAddress, with that device current) and
// only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // per device ordinal; null until looked up
}  // namespace

hipError_t noalloc_scratch(hipStream_t st, void** out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (st) {
    // the work is enqueued on st, so the scratch must be the one of st's device, which must
    // be the current device (the symbol lookup below names the current device's copy)
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(st, &sdev);
    if (e != hipSuccess) return e;
    if ((int)sdev != dev) return hipErrorInvalidDevice;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_prologue(const PrologueArgs& a, hipStream_t st) {
  return dispatch_dt_d_blk(a.dtype, a.D, a.BLK, [&](auto dt, auto d, auto blk) {
    return launch_prologue_t<decltype(dt)::value, decltype(d)::value, decltype(blk)::value>(a, st);
  });
}

}  // namespace sagebwd
