// Fused INT8 attention forward: O = softmax(sm * Q^ K~^T) V, O and row logsumexp.
// SageBwd article (aitrends.kr 8227), precision-split paragraph: QK^T and PV run in INT8;
// the TurboQuant blog's FlashAttention section: scores are processed tile by tile and
// never stored.
//
// Work decomposition (gfx950, 64-lane waves):
//   workgroup = 4 waves = 128 query rows of one head; wave w owns 32 rows.
//   Key tiles of BLK keys (one quantisation block of K and V) stream through LDS,
//   double-buffered: K codes token-major (rows padded to D+16 bytes) and V^T codes
//   channel-major (rows padded to BLK+16 bytes); the padding makes the 16-byte MFMA
//   operand reads of 8 consecutive rows fall on distinct banks.
//   S^T = K Q^T with v_mfma_i32_32x32x32_i8: lane l holds query l%32 and 16 keys per
//   32-key subtile, so the row max / row sum are lane-local plus one exchange with lane
//   l^32, and the quantised P~^T is already in the B-operand layout of O^T = V^T P~^T.
//   The V^T tile is permuted in LDS so that each A-operand read is one 16-byte load.
// Per key tile (the online-softmax step and the P~ quantisation tile, 32 rows x BLK keys):
//   m' = max(m, rowmax s); P~ = 2^(s*log2e - m'); alpha = 2^(m - m'); l = l*alpha + sum P~;
//   a = max P~ over the wave's tile; codes = rne(P~ * (127/a)); O = O*alpha + (a/127)*sV*int(PV).
// P~ * 127/a is produced by one exponential, 2^(s*log2e - m' + log2(127/a)), and rounded and
// packed by v_cvt_pk_u8_f32 (nearest even); only tiles on the diagonal carry masking work.
#include "common.hpp"
#include "launch.hpp"

#include <type_traits>

namespace sagebwd {

namespace {

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;
constexpr int kRowsPerBlock = kWaves * kRowsPerWave;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2_127 = 6.988684686772166f;  // log2(127)

template <int D, int BLK>
struct FwdLds {
  static constexpr int kRowK = D + 16;      // bytes per K row in LDS
  static constexpr int kRowV = BLK + 16;    // bytes per V^T row in LDS
  static constexpr int kBytesK = BLK * kRowK;
  static constexpr int kBytesV = D * kRowV;
  static constexpr int kBytes = kBytesK + kBytesV;
  // 16-byte chunks of one K tile and of one V^T tile, and per thread
  static constexpr int kChunks = BLK * D / 16;
  static constexpr int kPerThread = kChunks / (kWaves * 64);
};

// Byte offset, inside a V^T LDS row, of key-dword kd (keys 4kd..4kd+3): within each
// group of 32 keys, lane group g reads keys {8j + 4g + i} (j, i = 0..3) as one 16-byte load.
__device__ __forceinline__ int vt_dword_pos(int kd) {
  const int c32 = kd >> 3, k8 = kd & 7;
  return 32 * c32 + 16 * (k8 & 1) + 4 * (k8 >> 1);
}

template <int D, int BLK>
__device__ __forceinline__ void load_tile_regs(const ForwardArgs& a, size_t bh, int k0, i32x4* kreg, i32x4* vreg) {
  using L = FwdLds<D, BLK>;
  const int8_t* kbase = a.Kc + ((size_t)bh * a.N + k0) * D;
#pragma unroll
  for (int j = 0; j < L::kPerThread; ++j) {
    const int ci = threadIdx.x + j * kWaves * 64;
    kreg[j] = *reinterpret_cast<const i32x4*>(kbase + (size_t)ci * 16);
    const int c = ci / (BLK / 16), cc = ci % (BLK / 16);
    vreg[j] = *reinterpret_cast<const i32x4*>(a.Vtc + ((size_t)bh * D + c) * a.N + k0 + cc * 16);
  }
}

template <int D, int BLK>
__device__ __forceinline__ void store_tile_lds(int8_t* lds, const i32x4* kreg, const i32x4* vreg) {
  using L = FwdLds<D, BLK>;
#pragma unroll
  for (int j = 0; j < L::kPerThread; ++j) {
    const int ci = threadIdx.x + j * kWaves * 64;
    const int row = (ci * 16) / D, col = (ci * 16) % D;
    *reinterpret_cast<i32x4*>(lds + row * L::kRowK + col) = kreg[j];
    const int c = ci / (BLK / 16), cc = ci % (BLK / 16);
    int8_t* vrow = lds + L::kBytesK + c * L::kRowV;
#pragma unroll
    for (int w = 0; w < 4; ++w) *reinterpret_cast<int*>(vrow + vt_dword_pos(4 * cc + w)) = vreg[j][w];
  }
}

}  // namespace

template <int DT, int D, int BLK>
__global__ __launch_bounds__(kWaves * 64, 2) void fwd_kernel(ForwardArgs a) {
  using L = FwdLds<D, BLK>;
  constexpr int NSUB = BLK / 32;  // 32-key subtiles per key tile
  constexpr int DC = D / 32;      // 32-channel chunks
  __shared__ __attribute__((aligned(16))) int8_t lds[2][L::kBytes];

  const int nq = (a.N + kRowsPerBlock - 1) / kRowsPerBlock;
  const int bh = blockIdx.x % a.BH;
  const int qt = a.causal ? nq - 1 - (int)(blockIdx.x / a.BH) : (int)(blockIdx.x / a.BH);
  const int nb = a.N / BLK;
  const int w = wave_id(), l = lane_id(), g = l >> 5, lq = l & 31;
  const int q0 = qt * kRowsPerBlock;
  const int q0w = q0 + w * kRowsPerWave;
  const bool active = q0w < a.N;
  const int qrow = q0w + lq;  // this lane's query row

  // Q codes of this lane's query, as the B operand (contraction slots 16g..16g+15 of each
  // 32-channel chunk).
  i32x4 qreg[DC];
  float sQ = 0.0f;
  if (active) {
    const int8_t* qp = a.Qc + ((size_t)bh * a.N + qrow) * D + 16 * g;
#pragma unroll
    for (int kk = 0; kk < DC; ++kk) qreg[kk] = *reinterpret_cast<const i32x4*>(qp + 32 * kk);
    sQ = a.Qs[(size_t)bh * nb + q0w / BLK];
  }
  const int last_row = min(q0 + kRowsPerBlock, a.N) - 1;
  const int n_kt = a.causal ? last_row / BLK + 1 : nb;

  float m = -INFINITY, lsum_run = 0.0f;
  f32x16 o[DC];
#pragma unroll
  for (int ct = 0; ct < DC; ++ct) o[ct] = f32x16{};

  i32x4 kreg[L::kPerThread], vreg[L::kPerThread];
  load_tile_regs<D, BLK>(a, bh, 0, kreg, vreg);
  store_tile_lds<D, BLK>(lds[0], kreg, vreg);
  __syncthreads();

  for (int kt = 0; kt < n_kt; ++kt) {
    const bool has_next = kt + 1 < n_kt;
    if (has_next) load_tile_regs<D, BLK>(a, bh, (kt + 1) * BLK, kreg, vreg);
    const int k0 = kt * BLK;
    const int8_t* kl = lds[kt & 1];
    const int8_t* vl = lds[kt & 1] + L::kBytesK;
    // One key tile. DIAG: the tile crosses this wave's causal diagonal (keys above it are
    // masked); every other visited tile is wholly visible and carries no masking work.
    auto tile = [&](auto diag_c) {
      constexpr bool DIAG = decltype(diag_c)::value;
      // ---- S^T = K Q^T (exact int32)
      i32x16 s[NSUB];
#pragma unroll
      for (int t = 0; t < NSUB; ++t) {
        s[t] = i32x16{};
#pragma unroll
        for (int kk = 0; kk < DC; ++kk) {
          const i32x4 ak = *reinterpret_cast<const i32x4*>(kl + (32 * t + lq) * L::kRowK + 32 * kk + 16 * g);
          s[t] = mfma_i8_32x32x32(ak, qreg[kk], s[t]);
        }
      }
      if constexpr (DIAG) {
#pragma unroll
        for (int t = 0; t < NSUB; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * t + 8 * (r >> 2) + 4 * g + (r & 3);
            if (key > qrow) s[t][r] = INT32_MIN;
          }
      }
      int rmax = INT32_MIN;
#pragma unroll
      for (int t = 0; t < NSUB; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) rmax = max(rmax, s[t][r]);
      rmax = max(rmax, __shfl_xor(rmax, 32));

      const size_t sidx = (size_t)bh * nb + kt;
      const float sK = a.Ks[sidx], sV = a.Vs[sidx];
      const float c2 = (sQ * sK) * (a.sm_scale * kLog2e);
      // row max over the visible keys (a row with none in this tile keeps its old max)
      float rowmax = (float)rmax * c2;
      if constexpr (DIAG) rowmax = rmax == INT32_MIN ? -INFINITY : rowmax;
      const float m_new = fmaxf(m, rowmax);
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
      // P~ tile absmax a = max over rows of 2^(rowmax - m'); in log2 it is one wave max.
      // The quantisation factor 127/a is folded into the exponent, so the exponential
      // yields P~ * 127/a directly and its nearest-even integer is the code.
      const float pa_log = wave_max(rowmax - m_new);
      const float bias = kLog2_127 - pa_log - m_new;
      const float sP = __builtin_amdgcn_exp2f(pa_log) * (1.0f / 127.0f);

      float tsum = 0.0f;
      i32x4 pc[NSUB];
#pragma unroll
      for (int t = 0; t < NSUB; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float u[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float x = __builtin_fmaf((float)s[t][4 * j + i], c2, bias);
            if constexpr (DIAG) x = s[t][4 * j + i] == INT32_MIN ? -INFINITY : x;
            u[i] = __builtin_amdgcn_exp2f(x);
            tsum += u[i];
          }
          unsigned wd = __builtin_amdgcn_cvt_pk_u8_f32(u[0], 0, 0u);
          wd = __builtin_amdgcn_cvt_pk_u8_f32(u[1], 1, wd);
          wd = __builtin_amdgcn_cvt_pk_u8_f32(u[2], 2, wd);
          pc[t][j] = (int)__builtin_amdgcn_cvt_pk_u8_f32(u[3], 3, wd);
        }
      // l accumulates P~ before quantisation: sum(P~ * 127/a) * a/127
      lsum_run = lsum_run * alpha + tsum * sP;

      // ---- O^T = O^T * alpha + (a/127) sV (V^T P~^T), int32 over the BLK keys of one V block.
      // The rescale is skipped when no row of the wave moved its max (alpha == 1 exactly).
      const float spv = sP * sV;
      if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
        for (int ct = 0; ct < DC; ++ct)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[ct][r] *= alpha;
      }
#pragma unroll
      for (int ct = 0; ct < DC; ++ct) {
        i32x16 acc = i32x16{};
#pragma unroll
        for (int t = 0; t < NSUB; ++t) {
          const i32x4 av = *reinterpret_cast<const i32x4*>(vl + (32 * ct + lq) * L::kRowV + 32 * t + 16 * g);
          acc = mfma_i8_32x32x32(av, pc[t], acc);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) o[ct][r] = __builtin_fmaf(spv, (float)acc[r], o[ct][r]);
      }
      m = m_new;
    };
    if (active && (!a.causal || k0 <= q0w + kRowsPerWave - 1)) {
      if (a.causal && k0 + BLK - 1 > q0w) tile(std::true_type{});
      else tile(std::false_type{});
    }
    if (has_next) store_tile_lds<D, BLK>(lds[(kt + 1) & 1], kreg, vreg);
    __syncthreads();
  }

  if (!active) return;
  const float ltot = lsum_run + __shfl_xor(lsum_run, 32);
  const float linv = 1.0f / ltot;
  unsigned short* orow = a.O + ((size_t)bh * a.N + qrow) * D;
#pragma unroll
  for (int ct = 0; ct < DC; ++ct)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u16x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = from_f32<DT>(o[ct][4 * j + i] * linv);
      *reinterpret_cast<u16x4*>(orow + 32 * ct + 8 * j + 4 * g) = v;
    }
  if (g == 0) a.lse[(size_t)bh * a.N + qrow] = (m + __builtin_amdgcn_logf(ltot)) * kLn2;
}

template <int DT, int D, int BLK>
static hipError_t launch_forward_t(const ForwardArgs& a, hipStream_t st) {
  const long long nq = (a.N + kRowsPerBlock - 1) / kRowsPerBlock;
  return launch_kernel(&fwd_kernel<DT, D, BLK>, dim3((unsigned)(nq * a.BH)), dim3(kWaves * 64), st, a);
}

hipError_t launch_forward(const ForwardArgs& a, hipStream_t st) {
  return dispatch_dt_d_blk(a.dtype, a.D, a.BLK, [&](auto dt, auto d, auto blk) {
    return launch_forward_t<decltype(dt)::value, decltype(d)::value, decltype(blk)::value>(a, st);
  });
}

}  // namespace sagebwd
