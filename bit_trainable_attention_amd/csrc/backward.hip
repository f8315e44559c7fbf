// Fused INT8/FP16 attention backward.
// SageBwd article (aitrends.kr 8227): precision-split paragraph (recomputed QK^T, dV = P^T dO,
// dK = dS^T Q, dQ = dS K in INT8; dP = dO V^T alone in the 16-bit type), gradient
// paragraph (dQ = dS K and dK = dS^T Q), dS-magnitude paragraph (dS is what INT8 struggles
// with, so it is quantised on its own tile with its own absmax scale, in registers).
//
// Kernels:
//   bwd_pre      one workgroup per (head, block of BLK tokens): D = rowsum(dO o O),
//                block absmax and INT8 codes of dO written channel-major, Qc transposed
//                to channel-major, and the float32 dQ accumulator rows zeroed.
//   bwd_main     one workgroup per (head, key block of BLK keys); wave w owns 32 keys.
//                Streams query tiles of 64 rows (the P / dS quantisation tile height).
//                S = Q K~^T with v_mfma_i32_32x32x32_i8 in the layout lane = key,
//                registers = queries, which is directly the B operand of the two products
//                that contract over queries: dV^T = dO^T P and dK^T = Q^T dS. dP = dO V^T
//                uses v_mfma_f32_32x32x16_{f16,bf16} on the raw dO and V. dS codes go
//                through LDS once (transposed) for dQ = dS K, accumulated with float32
//                atomics into the workspace.
//   dq_finalize  RMSNorm backward of dQ and rounding to the dtype.
#include "common.hpp"
#include "launch.hpp"

namespace sagebwd {

namespace {

constexpr int kTq = 64;  // query rows per P / dS quantisation tile
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int perm_dword_pos(int kd) {
  // same permutation as the forward's V^T tile: within 32 positions, lane group g reads
  // positions {8j + 4g + i} as one 16-byte load at byte 16g.
  const int c32 = kd >> 3, k8 = kd & 7;
  return 32 * c32 + 16 * (k8 & 1) + 4 * (k8 >> 1);
}

}  // namespace

// ------------------------------------------------------------------------------ bwd_pre
template <int DT, int D, int BLK>
__global__ __launch_bounds__(256) void bwd_pre(BackwardArgs a) {
  __shared__ float xs[BLK][D + 1];
  __shared__ __attribute__((aligned(16))) int8_t qs[BLK][D + 4];
  __shared__ float red[4];
  const int nb = a.N / BLK;
  const int blk_id = blockIdx.x % nb;
  const int bh = blockIdx.x / nb;
  const size_t tok0 = (size_t)bh * a.N + (size_t)blk_id * BLK;
  const int tid = threadIdx.x;
  constexpr int CPR = D / 8;  // 16-byte chunks per row

  // dO, O: coalesced 8-element chunks; D via a segmented reduction over each row's chunks
  float amax = 0.0f;
  for (int ch = tid; ch < BLK * CPR; ch += 256) {
    const int t = ch / CPR, c = (ch % CPR) * 8;
    const u16x8 dv = *reinterpret_cast<const u16x8*>(a.dO + (tok0 + t) * D + c);
    const u16x8 ov = *reinterpret_cast<const u16x8*>(a.O + (tok0 + t) * D + c);
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = to_f32<DT>(dv[i]);
      xs[t][c + i] = x;
      amax = fmaxf(amax, fabsf(x));
      part = __builtin_fmaf(x, to_f32<DT>(ov[i]), part);
    }
    // CPR consecutive lanes share a row (CPR divides 64 and 256)
#pragma unroll
    for (int o = CPR / 2; o > 0; o >>= 1) part += __shfl_xor(part, o);
    if ((ch % CPR) == 0) a.Dvec[tok0 + t] = part;
  }
  // Qc block into LDS (bytes) for the transpose
  for (int ch = tid; ch < BLK * D / 16; ch += 256) {
    const int t = (ch * 16) / D, c = (ch * 16) % D;
    const i32x4 v = *reinterpret_cast<const i32x4*>(a.Qc + (tok0 + t) * D + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<int*>(&qs[t][c + 4 * i]) = v[i];
  }
  // zero the dQ accumulator rows of this block
  for (int e = tid; e < BLK * D / 4; e += 256)
    reinterpret_cast<float4*>(a.dq_acc + tok0 * D)[e] = make_float4(0.f, 0.f, 0.f, 0.f);

  amax = wave_max(amax);
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  const float am = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float inv = am > 0.0f ? 127.0f / am : 0.0f;
  if (tid == 0) a.dOs[(size_t)bh * nb + blk_id] = am > 0.0f ? am / 127.0f : 0.0f;
  // channel-major codes of dO and transposed Qc: word = 4 consecutive tokens of channel c
  for (int w = tid; w < BLK * D / 4; w += 256) {
    const int c = w / (BLK / 4), t = 4 * (w % (BLK / 4));
    const unsigned word = pack4_lo_bytes(quant_word(xs[t][c], inv), quant_word(xs[t + 1][c], inv),
                                         quant_word(xs[t + 2][c], inv), quant_word(xs[t + 3][c], inv));
    const size_t off = ((size_t)bh * D + c) * a.N + (size_t)blk_id * BLK + t;
    *reinterpret_cast<unsigned*>(a.dOtc + off) = word;
    const unsigned qw = (unsigned)(uint8_t)qs[t][c] | ((unsigned)(uint8_t)qs[t + 1][c] << 8) |
                        ((unsigned)(uint8_t)qs[t + 2][c] << 16) | ((unsigned)(uint8_t)qs[t + 3][c] << 24);
    *reinterpret_cast<unsigned*>(a.Qtc + off) = qw;
  }
}

// ------------------------------------------------------------------------------ bwd_main
template <int D, int BLK>
struct BwdLds {
  static constexpr int kRowQ = D + 16;        // Q codes, token-major
  static constexpr int kRowDO = 2 * D + 16;   // dO 16-bit, token-major
  static constexpr int kRowT = kTq + 16;      // dO^T / Q^T codes, channel-major, permuted
  static constexpr int kRowS = BLK + 16;      // dS codes [query][key]; K^T codes [channel][key]
  static constexpr int offQ = 0;
  static constexpr int offDO = offQ + kTq * kRowQ;
  static constexpr int offDOT = offDO + kTq * kRowDO;
  static constexpr int offQT = offDOT + D * kRowT;
  static constexpr int offLSE = offQT + D * kRowT;
  static constexpr int offDV = offLSE + kTq * 4;
  static constexpr int kTileBytes = offDV + kTq * 4;
  static constexpr int offDS = kTileBytes;
  static constexpr int offKT = offDS + kTq * kRowS;
  static constexpr int offRED = offKT + D * kRowS;
  static constexpr int kBytes = offRED + 64;
};

template <int DT, int D, int BLK>
__global__ __launch_bounds__(BLK * 2, 1) void bwd_main(BackwardArgs a) {
  using L = BwdLds<D, BLK>;
  constexpr int NW = BLK / 32;     // waves per workgroup
  constexpr int NT = NW * 64;      // threads
  constexpr int DC = D / 32;       // 32-channel chunks (int8 contraction / output tiles)
  constexpr int DH = D / 16;       // 16-channel chunks (16-bit contraction)
  constexpr int NU = kTq / 32;     // 32-query subtiles per query tile
  constexpr int KC = BLK / 32;     // 32-key chunks of the workgroup
  __shared__ __attribute__((aligned(16))) int8_t lds[L::kBytes];

  const int nb = a.N / BLK;
  const int bh = blockIdx.x % a.BH;
  const int kb = blockIdx.x / a.BH;            // key block; 0 first (most work when causal)
  const int w = wave_id(), l = lane_id(), g = l >> 5, lk = l & 31;
  const int tid = threadIdx.x;
  const int k0 = kb * BLK;
  const int key = k0 + 32 * w + lk;            // this lane's key
  const size_t hrow = (size_t)bh * a.N;

  // ---- per-wave constant operands: K codes (B of S) and V (B of dP) for this lane's key
  i32x4 kreg[DC];
  u16x8 vreg[DH];
#pragma unroll
  for (int kk = 0; kk < DC; ++kk) kreg[kk] = *reinterpret_cast<const i32x4*>(a.Kc + (hrow + key) * D + 32 * kk + 16 * g);
#pragma unroll
  for (int kk = 0; kk < DH; ++kk) vreg[kk] = *reinterpret_cast<const u16x8*>(a.V + (hrow + key) * D + 16 * kk + 8 * g);
  // ---- K^T codes of the whole key block in LDS (B operand of dQ = dS K)
  for (int ch = tid; ch < BLK * D / 16; ch += NT) {
    const int t = (ch * 16) / D, c = (ch * 16) % D;
    const i32x4 v = *reinterpret_cast<const i32x4*>(a.Kc + (hrow + k0 + t) * D + c);
#pragma unroll
    for (int i = 0; i < 16; ++i) lds[L::offKT + (c + i) * L::kRowS + t] = (int8_t)(v[i >> 2] >> (8 * (i & 3)));
  }
  const float sK = a.Ks[(size_t)bh * nb + kb];
  const float smc = a.sm_scale;

  f32x16 dk[DC], dv[DC];
#pragma unroll
  for (int ct = 0; ct < DC; ++ct) { dk[ct] = f32x16{}; dv[ct] = f32x16{}; }

  const int nqt = a.N / kTq;
  const int qt0 = a.causal ? k0 / kTq : 0;
  float* red = reinterpret_cast<float*>(lds + L::offRED);

  for (int qt = qt0; qt < nqt; ++qt) {
    const int q0 = qt * kTq;
    __syncthreads();  // previous tile's LDS reads are done
    // ---- stage the query tile
    for (int ch = tid; ch < kTq * D / 16; ch += NT) {
      const int t = (ch * 16) / D, c = (ch * 16) % D;
      *reinterpret_cast<i32x4*>(lds + L::offQ + t * L::kRowQ + c) =
          *reinterpret_cast<const i32x4*>(a.Qc + (hrow + q0 + t) * D + c);
    }
    for (int ch = tid; ch < kTq * D / 8; ch += NT) {
      const int t = (ch * 8) / D, c = (ch * 8) % D;
      *reinterpret_cast<u16x8*>(lds + L::offDO + t * L::kRowDO + 2 * c) =
          *reinterpret_cast<const u16x8*>(a.dO + (hrow + q0 + t) * D + c);
    }
    for (int ch = tid; ch < D * kTq / 16; ch += NT) {
      const int c = ch / (kTq / 16), cc = ch % (kTq / 16);
      const size_t goff = ((size_t)bh * D + c) * a.N + q0 + 16 * cc;
      const i32x4 vo = *reinterpret_cast<const i32x4*>(a.dOtc + goff);
      const i32x4 vq = *reinterpret_cast<const i32x4*>(a.Qtc + goff);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *reinterpret_cast<int*>(lds + L::offDOT + c * L::kRowT + perm_dword_pos(4 * cc + i)) = vo[i];
        *reinterpret_cast<int*>(lds + L::offQT + c * L::kRowT + perm_dword_pos(4 * cc + i)) = vq[i];
      }
    }
    if (tid < kTq) {
      reinterpret_cast<float*>(lds + L::offLSE)[tid] = a.lse[hrow + q0 + tid] * kLog2e;
      reinterpret_cast<float*>(lds + L::offDV)[tid] = a.Dvec[hrow + q0 + tid];
    }
    __syncthreads();

    const float sQ = a.Qs[(size_t)bh * nb + q0 / BLK];
    const float sdO = a.dOs[(size_t)bh * nb + q0 / BLK];
    const float c2 = (sQ * sK) * (smc * kLog2e);
    const bool diag = a.causal && (k0 + BLK - 1 > q0);

    // ---- S, P, dP, dS for the NU query subtiles of this wave's 32 keys
    float pf[NU][16], dsf[NU][16];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      i32x16 s = i32x16{};
#pragma unroll
      for (int kk = 0; kk < DC; ++kk) {
        const i32x4 aq = *reinterpret_cast<const i32x4*>(lds + L::offQ + (32 * u + lk) * L::kRowQ + 32 * kk + 16 * g);
        s = mfma_i8_32x32x32(aq, kreg[kk], s);
      }
      f32x16 dp = f32x16{};
#pragma unroll
      for (int kk = 0; kk < DH; ++kk) {
        const u16x8 ad = *reinterpret_cast<const u16x8*>(lds + L::offDO + (32 * u + lk) * L::kRowDO + 2 * (16 * kk + 8 * g));
        dp = mfma_16b_32x32x16<DT>(ad, vreg[kk], dp);
      }
      const float* lse2 = reinterpret_cast<const float*>(lds + L::offLSE) + 32 * u + 4 * g;
      const float* dvv = reinterpret_cast<const float*>(lds + L::offDV) + 32 * u + 4 * g;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = 8 * (r >> 2) + (r & 3);  // query offset inside the subtile, minus 4g
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf((float)s[r], c2, -lse2[qi]));
        if (diag && key > q0 + 32 * u + 4 * g + qi) p = 0.0f;
        pf[u][r] = p;
        dsf[u][r] = p * (dp[r] - dvv[qi]);
      }
    }
    // ---- P tile (kTq queries x this wave's 32 keys): absmax, codes
    float pm = 0.0f, dm = 0.0f;
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) { pm = fmaxf(pm, pf[u][r]); dm = fmaxf(dm, fabsf(dsf[u][r])); }
    pm = wave_max(pm);
    dm = wave_max(dm);
    if (l == 0) red[w] = dm;
    const float pinv = pm > 0.0f ? 127.0f / pm : 0.0f;
    const float sP = pm > 0.0f ? pm / 127.0f : 0.0f;
    i32x4 pcode[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        pcode[u][j] = (int)pack4_lo_bytes(quant_word(pf[u][4 * j], pinv), quant_word(pf[u][4 * j + 1], pinv),
                                          quant_word(pf[u][4 * j + 2], pinv), quant_word(pf[u][4 * j + 3], pinv));
    // ---- dV^T += dO^T P (int32 over the kTq queries)
    {
      const float sc = sP * sdO;
#pragma unroll
      for (int ct = 0; ct < DC; ++ct) {
        i32x16 acc = i32x16{};
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const i32x4 ao = *reinterpret_cast<const i32x4*>(lds + L::offDOT + (32 * ct + lk) * L::kRowT + 32 * u + 16 * g);
          acc = mfma_i8_32x32x32(ao, pcode[u], acc);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) dv[ct][r] += sc * (float)acc[r];
      }
    }
    // ---- dS tile (kTq queries x BLK keys) absmax across the waves
    __syncthreads();
    float da = red[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) da = fmaxf(da, red[i]);
    const float dinv = da > 0.0f ? 127.0f / da : 0.0f;
    const float sdS = da > 0.0f ? da / 127.0f : 0.0f;
    i32x4 dcode[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const unsigned w0 = quant_word(dsf[u][4 * j], dinv), w1 = quant_word(dsf[u][4 * j + 1], dinv);
        const unsigned w2 = quant_word(dsf[u][4 * j + 2], dinv), w3 = quant_word(dsf[u][4 * j + 3], dinv);
        dcode[u][j] = (int)pack4_lo_bytes(w0, w1, w2, w3);
        // dS codes, query-major, for dQ: query 32u + 8j + 4g + i, key 32w + lk
        int8_t* col = lds + L::offDS + (32 * w + lk);
        const int qb = 32 * u + 8 * j + 4 * g;
        col[(qb + 0) * L::kRowS] = (int8_t)w0;
        col[(qb + 1) * L::kRowS] = (int8_t)w1;
        col[(qb + 2) * L::kRowS] = (int8_t)w2;
        col[(qb + 3) * L::kRowS] = (int8_t)w3;
      }
    // ---- dK^T += Q^T dS (int32 over the kTq queries)
    {
      const float sc = smc * sdS * sQ;
#pragma unroll
      for (int ct = 0; ct < DC; ++ct) {
        i32x16 acc = i32x16{};
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const i32x4 aq = *reinterpret_cast<const i32x4*>(lds + L::offQT + (32 * ct + lk) * L::kRowT + 32 * u + 16 * g);
          acc = mfma_i8_32x32x32(aq, dcode[u], acc);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) dk[ct][r] += sc * (float)acc[r];
      }
    }
    __syncthreads();  // dS codes of every wave are in LDS
    // ---- dQ = dS K over the BLK keys: NU x DC output tiles of 32 x 32, split over the waves
    {
      const float sc = smc * sdS * sK;
      for (int tile = w; tile < NU * DC; tile += NW) {
        const int u = tile / DC, ct = tile % DC;
        i32x16 acc = i32x16{};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          const i32x4 as = *reinterpret_cast<const i32x4*>(lds + L::offDS + (32 * u + lk) * L::kRowS + 32 * kc + 16 * g);
          const i32x4 bk = *reinterpret_cast<const i32x4*>(lds + L::offKT + (32 * ct + lk) * L::kRowS + 32 * kc + 16 * g);
          acc = mfma_i8_32x32x32(as, bk, acc);
        }
        // result lane: channel 32ct + lk, query 32u + 8(r/4) + 4g + r%4
        float* dst = a.dq_acc + (hrow + q0 + 32 * u + 4 * g) * D + 32 * ct + lk;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          unsafeAtomicAdd(dst + (size_t)(8 * (r >> 2) + (r & 3)) * D, sc * (float)acc[r]);
      }
    }
  }

  // ---- epilogue: dV and dK (RMSNorm backward with K^ = K * rstd) for this lane's key
  unsigned short* dvrow = a.dV + (hrow + key) * D;
#pragma unroll
  for (int ct = 0; ct < DC; ++ct)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u16x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = from_f32<DT>(dv[ct][4 * j + i]);
      *reinterpret_cast<u16x4*>(dvrow + 32 * ct + 8 * j + 4 * g) = v;
    }
  unsigned short* dkrow = a.dK + (hrow + key) * D;
  if (a.qk_norm) {
    const float rs = a.k_rstd[hrow + key];
    const unsigned short* krow = a.K + (hrow + key) * D;
    float kh[DC][16];
    float dot = 0.0f;
#pragma unroll
    for (int ct = 0; ct < DC; ++ct)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u16x4 kv = *reinterpret_cast<const u16x4*>(krow + 32 * ct + 8 * j + 4 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          kh[ct][4 * j + i] = to_f32<DT>(kv[i]) * rs;
          dot = __builtin_fmaf(dk[ct][4 * j + i], kh[ct][4 * j + i], dot);
        }
      }
    dot += __shfl_xor(dot, 32);
    const float mean = dot / (float)D;
#pragma unroll
    for (int ct = 0; ct < DC; ++ct)
#pragma unroll
      for (int r = 0; r < 16; ++r) dk[ct][r] = rs * (dk[ct][r] - kh[ct][r] * mean);
  }
#pragma unroll
  for (int ct = 0; ct < DC; ++ct)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u16x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = from_f32<DT>(dk[ct][4 * j + i]);
      *reinterpret_cast<u16x4*>(dkrow + 32 * ct + 8 * j + 4 * g) = v;
    }
}

// ------------------------------------------------------------------------------ dq_finalize
// One group of D/8 lanes per token: dQ = rstd * (dQ^ - Q^ * mean_c(dQ^ o Q^)), Q^ = Q * rstd.
template <int DT, int D>
__global__ __launch_bounds__(256) void dq_finalize(BackwardArgs a) {
  constexpr int CPR = D / 8;
  const size_t tokens = (size_t)a.BH * a.N;
  const size_t gidx = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t tok = gidx / CPR;
  const int c = (int)(gidx % CPR) * 8;
  if (tok >= tokens) return;  // whole rows only: CPR divides 256, so a row never straddles this
  const float* src = a.dq_acc + tok * D + c;
  float dq[8];
  *reinterpret_cast<float4*>(dq) = *reinterpret_cast<const float4*>(src);
  *reinterpret_cast<float4*>(dq + 4) = *reinterpret_cast<const float4*>(src + 4);
  u16x8 out;
  if (a.qk_norm) {
    const float rs = a.q_rstd[tok];
    const u16x8 qv = *reinterpret_cast<const u16x8*>(a.Q + tok * D + c);
    float qh[8], dot = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      qh[i] = to_f32<DT>(qv[i]) * rs;
      dot = __builtin_fmaf(dq[i], qh[i], dot);
    }
#pragma unroll
    for (int o = CPR / 2; o > 0; o >>= 1) dot += __shfl_xor(dot, o);
    const float mean = dot / (float)D;
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = from_f32<DT>(rs * (dq[i] - qh[i] * mean));
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = from_f32<DT>(dq[i]);
  }
  *reinterpret_cast<u16x8*>(a.dQ + tok * D + c) = out;
}

template <int DT, int D, int BLK>
static hipError_t launch_backward_t(const BackwardArgs& a, hipStream_t st) {
  const long long nb = a.N / BLK;
  hipLaunchKernelGGL((bwd_pre<DT, D, BLK>), dim3((unsigned)(nb * a.BH)), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_main<DT, D, BLK>), dim3((unsigned)(nb * a.BH)), dim3(BLK * 2), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long threads = (long long)a.BH * a.N * (D / 8);
  hipLaunchKernelGGL((dq_finalize<DT, D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_backward(const BackwardArgs& a, hipStream_t st) {
  return dispatch_dt_d_blk(a.dtype, a.D, a.BLK, [&](auto dt, auto d, auto blk) {
    return launch_backward_t<decltype(dt)::value, decltype(d)::value, decltype(blk)::value>(a, st);
  });
}

}  // namespace sagebwd
