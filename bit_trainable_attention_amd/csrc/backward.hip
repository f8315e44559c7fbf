// Fused INT8/FP16 attention backward.
// SageBwd article (aitrends.kr 8227): precision-split paragraph (recomputed QK^T, dV = P^T dO,
// dK = dS^T Q, dQ = dS K in INT8; dP = dO V^T alone in the 16-bit type), gradient
// paragraph (dQ = dS K and dK = dS^T Q), dS-magnitude paragraph (dS is what INT8 struggles
// with, so it is quantised on its own tile with its own absmax scale, in registers).
//
// Kernels:
//   bwd_pre      one workgroup per (head, block of BLK tokens): D = rowsum(dO o O),
//                lse * log2(e), block absmax and INT8 codes of dO written channel-major,
//                Qc transposed to channel-major, and the float32 dQ accumulator rows zeroed.
//   bwd_main     one workgroup per (head, key block of BLK keys); a pair of waves owns
//                each 32 keys. Streams query tiles of 64 rows (the P / dS quantisation
//                tile height), double-buffered in LDS with the next tile's global loads
//                in flight while the current one is computed.
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
  // Byte position of token-dword kd (tokens 4kd..4kd+3) in a channel-major row: inside each
  // group of 32 tokens, lane group g of an MFMA operand needs tokens {8j + 4g + i}
  // (j, i = 0..3), which this places at bytes 16g..16g+15 of the group.
  const int c32 = kd >> 3, k8 = kd & 7;
  return 32 * c32 + 16 * (k8 & 1) + 4 * (k8 >> 1);
}

// XOR swizzles of the 16-byte chunks of LDS rows: 8 consecutive rows read at the same
// logical chunk land in 8 different bank groups.
template <int ROWB>
__device__ __forceinline__ int swz(int row, int chunk) {
  if constexpr (ROWB >= 128) return chunk ^ (row & 7);
  else if constexpr (ROWB == 64) return chunk ^ ((row >> 1) & 3);
  else return chunk;
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations, not for its
// outstanding vector-memory operations (dQ atomics, direct-to-LDS copies in flight, whose
// completion is awaited explicitly where their data is published). The memory clobber keeps
// the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
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
    if ((ch % CPR) == 0) {
      a.Dvec[tok0 + t] = part;
      a.lse2[tok0 + t] = a.lse[tok0 + t] * kLog2e;
    }
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
  // channel-major codes of dO and transposed Qc: word = 4 consecutive tokens of channel c,
  // stored at its permuted position inside the 32-token group (see perm_dword_pos)
  for (int w = tid; w < BLK * D / 4; w += 256) {
    const int c = w / (BLK / 4), t = 4 * (w % (BLK / 4));
    const unsigned word = pack4_lo_bytes(quant_word(xs[t][c], inv), quant_word(xs[t + 1][c], inv),
                                         quant_word(xs[t + 2][c], inv), quant_word(xs[t + 3][c], inv));
    const size_t off = ((size_t)bh * D + c) * a.N + (size_t)blk_id * BLK + perm_dword_pos(t / 4);
    *reinterpret_cast<unsigned*>(a.dOtc + off) = word;
    const unsigned qw = (unsigned)(uint8_t)qs[t][c] | ((unsigned)(uint8_t)qs[t + 1][c] << 8) |
                        ((unsigned)(uint8_t)qs[t + 2][c] << 16) | ((unsigned)(uint8_t)qs[t + 3][c] << 24);
    *reinterpret_cast<unsigned*>(a.Qtc + off) = qw;
  }
}

// ------------------------------------------------------------------------------ bwd_main
// Workgroup = one key block of BLK keys, 2*BLK/32 waves (two per SIMD). The waves come in
// pairs: both waves of pair kg own the same 32 keys; wave half h = 0/1 computes S, P, dP and
// dS for query rows 32h..32h+31 of each 64-row query tile, and accumulates dK and dV for
// channel half h. The pair swaps its P and dS codes through LDS, so each wave holds the
// B operands of dV^T = dO^T P and dK^T = Q^T dS for all 64 queries.
template <int D, int BLK>
struct BwdLds {
  static constexpr int NKG = BLK / 32;        // 32-key groups
  static constexpr int NW = 2 * NKG;          // waves
  static constexpr int NT = NW * 64;
  static constexpr int kRowS = BLK + 16;      // dS codes [query][key]; K^T codes [channel][key]
  // one query-tile buffer (double-buffered), rows unpadded and chunk-swizzled:
  //   Q codes [kTq][D], dO [kTq][D] 16-bit, dO^T and Q^T codes [D][kTq], lse2 [kTq], D [kTq],
  //   and the tile's Q and dO block scales
  static constexpr int bQ = 0;
  static constexpr int bDO = bQ + kTq * D;
  static constexpr int bDOT = bDO + kTq * 2 * D;
  static constexpr int bQT = bDOT + D * kTq;
  static constexpr int bLSE = bQT + D * kTq;
  static constexpr int bDV = bLSE + kTq * 4;
  static constexpr int bSQ = bDV + kTq * 4;     // Q block scale of the tile (first word)
  static constexpr int bSDO = bSQ + 256;        // dO block scale of the tile (first word)
  static constexpr int kBuf = bSDO + 256;
  static constexpr int offDS = 2 * kBuf;
  static constexpr int offKT = offDS + kTq * kRowS;
  static constexpr int offK = offKT + D * kRowS;    // K codes [BLK][D], token-major, swizzled
  static constexpr int offXP = offK + BLK * D;      // P codes exchanged inside a pair [NW][64][16 B]
  static constexpr int offXD = offXP + NW * 1024;   // dS codes exchanged inside a pair
  static constexpr int offRED = offXD + NW * 1024;  // redP[NW], redD[NW]
  static constexpr int offDOT = offRED + 2 * NW * 4;  // epilogue: per-lane dK.K^ partial dots [NW][64]
  static constexpr int kBytes = offDOT + NW * 64 * 4;
  // 1 KB direct-to-LDS wave copies of the Q, dO, dO^T, Q^T parts of a tile
  static constexpr int kCopies = (bLSE - bQ) / 1024;
  static constexpr int kCopiesPerWave = (kCopies + NW - 1) / NW;
  static_assert((bLSE - bQ) % 1024 == 0, "tile parts are whole 1 KB copies");
};

// Direct buffer -> LDS copies (buffer_load ... lds): lane l reads 16 (or 4) bytes at byte
// offset voff + soff of the buffer [base, base + bytes) (reads past the end return zeros)
// and the hardware writes them to LDS at lds + 16*l (or 4*l). The bodies are compiled for
// the device only: this compiler's host pass cannot type-check the LDS-DMA builtin and,
// instead of reporting it, silently omits the host launch stubs of kernels that reach it.
__device__ __forceinline__ void buffer_to_lds16(const void* base, uint32_t bytes, int8_t* lds, uint32_t voff,
                                                uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                                                      0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
#endif
}
__device__ __forceinline__ void buffer_to_lds4(const void* base, uint32_t bytes, int8_t* lds, uint32_t voff,
                                               uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                                                      0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, voff, soff, 0, 0);
#endif
}

// Direct global -> LDS copies of one query tile. Each wave copy fills 1 KB of LDS, lane l
// the 16 bytes at 16*l; each lane's source is chosen so that the LDS image is the swizzled
// layout. Sources are addressed through buffer resources of the head's arrays: a per-lane
// 32-bit offset that does not depend on the query tile (computed once) plus a wave-uniform
// offset for the query tile and the copy.
template <int D, int BLK>
struct TileDma {
  using L = BwdLds<D, BLK>;
  static constexpr int nQc = kTq * D / 1024;       // copies of the Q codes part
  static constexpr int nDOc = kTq * 2 * D / 1024;  // copies of the dO part
  static constexpr int nTc = D * kTq / 1024;       // copies of each of dO^T, Q^T
  // head bases of the arrays (the buffer resources are built from these where they are used)
  const void *pQ, *pDO, *pDOT, *pQT, *pLSE, *pDV, *pQs, *pDOs;
  uint32_t loff[L::kCopiesPerWave];
  int N;

  __device__ __forceinline__ void init(const BackwardArgs& a, size_t hrow, int bh, int w, int l) {
    N = a.N;
    pQ = a.Qc + hrow * D;
    pDO = a.dO + hrow * D;
    pDOT = a.dOtc + (size_t)bh * D * a.N;
    pQT = a.Qtc + (size_t)bh * D * a.N;
    pLSE = a.lse2 + hrow;
    pDV = a.Dvec + hrow;
    pQs = a.Qs + (size_t)bh * (a.N / BLK);
    pDOs = a.dOs + (size_t)bh * (a.N / BLK);
#pragma unroll
    for (int j = 0; j < L::kCopiesPerWave; ++j) {
      const int cp = w + L::NW * j;
      uint32_t off = 0;
      if (cp < nQc) {
        const int q = (16 * l) / D, p = l % (D / 16);
        off = q * D + 16 * swz<D>(cp * (1024 / D) + q, p);
      } else if (cp < nQc + nDOc) {
        const int cd = cp - nQc, q = (16 * l) / (2 * D), p = l % (D / 8);
        off = 2 * (q * D + 8 * swz<2 * D>(cd * (512 / D) + q, p));
      } else if (cp < L::kCopies) {
        const int c3 = (cp - nQc - nDOc) % nTc, c = l / 4, p = l % 4;
        off = (uint32_t)c * (uint32_t)a.N + 16 * swz<kTq>(16 * c3 + c, p);
      }
      loff[j] = off;
    }
  }

  __device__ __forceinline__ void issue(int q0, int8_t* buf, int w) const {
    const uint32_t nd = (uint32_t)N * D;
#pragma unroll
    for (int j = 0; j < L::kCopiesPerWave; ++j) {
      const int cp = w + L::NW * j;
      int8_t* dst = buf + cp * 1024;
      if (cp < nQc) {
        buffer_to_lds16(pQ, nd, dst, loff[j], q0 * D + cp * 1024);
      } else if (cp < nQc + nDOc) {
        buffer_to_lds16(pDO, 2 * nd, dst, loff[j], 2 * q0 * D + (cp - nQc) * 1024);
      } else if (cp < nQc + nDOc + nTc) {
        buffer_to_lds16(pDOT, nd, dst, loff[j], 16 * (cp - nQc - nDOc) * N + q0);
      } else if (cp < L::kCopies) {
        buffer_to_lds16(pQT, nd, dst, loff[j], 16 * (cp - nQc - nDOc - nTc) * N + q0);
      }
    }
    if (w == L::NW - 1) {
      buffer_to_lds4(pLSE, 4 * (uint32_t)N, buf + L::bLSE, 4 * lane_id(), 4 * q0);
      buffer_to_lds4(pDV, 4 * (uint32_t)N, buf + L::bDV, 4 * lane_id(), 4 * q0);
    }
    if (w == L::NW - 2) {  // lane 0 carries the tile's block scale; lanes past the row read 0
      buffer_to_lds4(pQs, 4 * (uint32_t)(N / BLK), buf + L::bSQ, 4 * lane_id(), 4 * (q0 / BLK));
      buffer_to_lds4(pDOs, 4 * (uint32_t)(N / BLK), buf + L::bSDO, 4 * lane_id(), 4 * (q0 / BLK));
    }
  }
};

template <int DT, int D, int BLK>
__global__ __launch_bounds__(BLK * 4, 1) void bwd_main(BackwardArgs a) {
  using L = BwdLds<D, BLK>;
  constexpr int NKG = L::NKG;      // 32-key groups (wave pairs)
  constexpr int NW = L::NW;        // waves per workgroup
  constexpr int NT = L::NT;        // threads
  constexpr int DC = D / 32;       // 32-channel chunks (int8 contraction / output tiles)
  constexpr int DCH = DC / 2;      // 32-channel output tiles per channel half
  constexpr int DH = D / 16;       // 16-channel chunks (16-bit contraction)
  constexpr int KC = BLK / 32;     // 32-key chunks of the workgroup
  __shared__ __attribute__((aligned(16))) int8_t lds[L::kBytes];

  const int nb = a.N / BLK;
  const int bh = blockIdx.x % a.BH;
  const int kb = blockIdx.x / a.BH;            // key block; 0 first (most work when causal)
  const int w = __builtin_amdgcn_readfirstlane(wave_id()), l = lane_id(), g = l >> 5, lk = l & 31;
  const int kg = w % NKG, h = w / NKG;         // key group, query half / channel half
  const int partner = kg + NKG * (1 - h);
  const int tid = threadIdx.x;
  const int k0 = kb * BLK;
  const int key = k0 + 32 * kg + lk;           // this lane's key
  const size_t hrow = (size_t)bh * a.N;

  // ---- per-wave constant operand: V (B of dP) for this lane's key
  u16x8 vreg[DH];
#pragma unroll
  for (int kk = 0; kk < DH; ++kk) vreg[kk] = *reinterpret_cast<const u16x8*>(a.V + (hrow + key) * D + 16 * kk + 8 * g);
  // ---- K codes of the key block in LDS: token-major (B operand of S = Q K^T) and
  //      channel-major (B operand of dQ = dS K)
  for (int ch = tid; ch < BLK * D / 16; ch += NT) {
    const int t = (ch * 16) / D, c = (ch * 16) % D;
    const i32x4 v = *reinterpret_cast<const i32x4*>(a.Kc + (hrow + k0 + t) * D + c);
    *reinterpret_cast<i32x4*>(lds + L::offK + t * D + 16 * swz<D>(t, c / 16)) = v;
#pragma unroll
    for (int i = 0; i < 16; ++i) lds[L::offKT + (c + i) * L::kRowS + t] = (int8_t)(v[i >> 2] >> (8 * (i & 3)));
  }
  const float sK = a.Ks[(size_t)bh * nb + kb];
  const float smc = a.sm_scale;
  float* redP = reinterpret_cast<float*>(lds + L::offRED);
  float* redD = redP + NW;

  f32x16 dk[DCH], dv[DCH];
#pragma unroll
  for (int i = 0; i < DCH; ++i) { dk[i] = f32x16{}; dv[i] = f32x16{}; }

  const int nqt = a.N / kTq;
  const int qt0 = a.causal ? k0 / kTq : 0;
  TileDma<D, BLK> dma;
  dma.init(a, hrow, bh, w, l);
  dma.issue(qt0 * kTq, lds, w);
  wait_vmcnt<0>();
  lds_barrier();

  for (int qt = qt0; qt < nqt; ++qt) {
    const int q0 = qt * kTq;
    const bool has_next = qt + 1 < nqt;
    int8_t* buf = lds + ((qt - qt0) & 1) * L::kBuf;
    int8_t* nbuf = lds + (((qt - qt0) & 1) ^ 1) * L::kBuf;
    if (has_next) dma.issue(q0 + kTq, nbuf, w);

    const float sQ = *reinterpret_cast<const float*>(buf + L::bSQ);
    const float sdO = *reinterpret_cast<const float*>(buf + L::bSDO);
    const float c2 = (sQ * sK) * (smc * kLog2e);
    const bool diag = a.causal && (k0 + BLK - 1 > q0);

    // ---- S, P, dP, dS for query rows 32h..32h+31 of the tile and this pair's 32 keys
    i32x16 s = i32x16{};
#pragma unroll
    for (int kk = 0; kk < DC; ++kk) {
      const int q = 32 * h + lk, kl = 32 * kg + lk;
      const i32x4 aq = *reinterpret_cast<const i32x4*>(buf + L::bQ + q * D + 16 * swz<D>(q, 2 * kk + g));
      const i32x4 bk = *reinterpret_cast<const i32x4*>(lds + L::offK + kl * D + 16 * swz<D>(kl, 2 * kk + g));
      s = mfma_i8_32x32x32(aq, bk, s);
    }
    f32x16 dp = f32x16{};
#pragma unroll
    for (int kk = 0; kk < DH; ++kk) {
      const int q = 32 * h + lk;
      const u16x8 ad = *reinterpret_cast<const u16x8*>(buf + L::bDO + q * 2 * D + 16 * swz<2 * D>(q, 2 * kk + g));
      dp = mfma_16b_32x32x16<DT>(ad, vreg[kk], dp);
    }
    const float* lse2 = reinterpret_cast<const float*>(buf + L::bLSE) + 32 * h + 4 * g;
    const float* dvv = reinterpret_cast<const float*>(buf + L::bDV) + 32 * h + 4 * g;
    float pf[16], dsf[16];
    float pm = 0.0f, dm = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qi = 8 * (r >> 2) + (r & 3);  // query offset inside the 32 rows, minus 4g
      float p = __builtin_amdgcn_exp2f(__builtin_fmaf((float)s[r], c2, -lse2[qi]));
      if (diag && key > q0 + 32 * h + 4 * g + qi) p = 0.0f;
      pf[r] = p;
      dsf[r] = p * (dp[r] - dvv[qi]);
      pm = fmaxf(pm, p);
      dm = fmaxf(dm, fabsf(dsf[r]));
    }
    pm = wave_max(pm);
    dm = wave_max(dm);
    if (l == 0) { redP[w] = pm; redD[w] = dm; }
    lds_barrier();
    // P tile: 64 queries x this pair's 32 keys; dS tile: 64 queries x the block's BLK keys
    const float pa = fmaxf(redP[kg], redP[kg + NKG]);
    float da = redD[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) da = fmaxf(da, redD[i]);
    const float pinv = pa > 0.0f ? 127.0f / pa : 0.0f;
    const float sP = pa > 0.0f ? pa / 127.0f : 0.0f;
    const float dinv = da > 0.0f ? 127.0f / da : 0.0f;
    const float sdS = da > 0.0f ? da / 127.0f : 0.0f;
    i32x4 pcode[2], dcode[2];
    {
      i32x4 pc, dc;
      int8_t* col = lds + L::offDS + (32 * kg + lk);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pc[j] = (int)pack4_lo_bytes(quant_word(pf[4 * j], pinv), quant_word(pf[4 * j + 1], pinv),
                                    quant_word(pf[4 * j + 2], pinv), quant_word(pf[4 * j + 3], pinv));
        const unsigned w0 = quant_word(dsf[4 * j], dinv), w1 = quant_word(dsf[4 * j + 1], dinv);
        const unsigned w2 = quant_word(dsf[4 * j + 2], dinv), w3 = quant_word(dsf[4 * j + 3], dinv);
        dc[j] = (int)pack4_lo_bytes(w0, w1, w2, w3);
        // dS codes, query-major, for dQ: query 32h + 8j + 4g + i, key 32kg + lk
        const int qb = 32 * h + 8 * j + 4 * g;
        col[(qb + 0) * L::kRowS] = (int8_t)w0;
        col[(qb + 1) * L::kRowS] = (int8_t)w1;
        col[(qb + 2) * L::kRowS] = (int8_t)w2;
        col[(qb + 3) * L::kRowS] = (int8_t)w3;
      }
      *reinterpret_cast<i32x4*>(lds + L::offXP + w * 1024 + l * 16) = pc;
      *reinterpret_cast<i32x4*>(lds + L::offXD + w * 1024 + l * 16) = dc;
      pcode[h] = pc;
      dcode[h] = dc;
    }
    lds_barrier();
    pcode[1 - h] = *reinterpret_cast<const i32x4*>(lds + L::offXP + partner * 1024 + l * 16);
    dcode[1 - h] = *reinterpret_cast<const i32x4*>(lds + L::offXD + partner * 1024 + l * 16);

    // ---- dV^T += dO^T P and dK^T += Q^T dS for channel half h (int32 over the 64 queries)
    {
      const float sv = sP * sdO;
#pragma unroll
      for (int i = 0; i < DCH; ++i) {
        const int c = 32 * (DCH * h + i) + lk;
        i32x16 acc = i32x16{};
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const i32x4 ao = *reinterpret_cast<const i32x4*>(buf + L::bDOT + c * kTq + 16 * swz<kTq>(c, 2 * u + g));
          acc = mfma_i8_32x32x32(ao, pcode[u], acc);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) dv[i][r] += sv * (float)acc[r];
      }
      const float sk = smc * sdS * sQ;
#pragma unroll
      for (int i = 0; i < DCH; ++i) {
        const int c = 32 * (DCH * h + i) + lk;
        i32x16 acc = i32x16{};
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const i32x4 aq = *reinterpret_cast<const i32x4*>(buf + L::bQT + c * kTq + 16 * swz<kTq>(c, 2 * u + g));
          acc = mfma_i8_32x32x32(aq, dcode[u], acc);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) dk[i][r] += sk * (float)acc[r];
      }
    }

    // ---- dQ = dS K over the BLK keys: 2 x DC output tiles of 32 x 32, split over the waves
    {
      const float sc = smc * sdS * sK;
      for (int tile = w; tile < 2 * DC; tile += NW) {
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
    // The next tile's copies were issued before this iteration's dQ atomics; vector memory
    // operations complete in issue order, so allowing the atomics (16 per dQ tile) to stay
    // outstanding still waits for every copy.
    if constexpr (2 * DC <= NW) {
      if (w < 2 * DC) wait_vmcnt<16>();
      else wait_vmcnt<0>();
    } else {
      wait_vmcnt<16 * ((2 * DC) / NW)>();
    }
    lds_barrier();
  }

  // ---- epilogue: dV and dK (RMSNorm backward with K^ = K * rstd) for this lane's key, half h
  unsigned short* dvrow = a.dV + (hrow + key) * D;
#pragma unroll
  for (int i = 0; i < DCH; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = from_f32<DT>(dv[i][4 * j + e]);
      *reinterpret_cast<u16x4*>(dvrow + 32 * (DCH * h + i) + 8 * j + 4 * g) = v;
    }
  unsigned short* dkrow = a.dK + (hrow + key) * D;
  if (a.qk_norm) {
    const float rs = a.k_rstd[hrow + key];
    const unsigned short* krow = a.K + (hrow + key) * D;
    float kh[DCH][16];
    float dot = 0.0f;
#pragma unroll
    for (int i = 0; i < DCH; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u16x4 kv = *reinterpret_cast<const u16x4*>(krow + 32 * (DCH * h + i) + 8 * j + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kh[i][4 * j + e] = to_f32<DT>(kv[e]) * rs;
          dot = __builtin_fmaf(dk[i][4 * j + e], kh[i][4 * j + e], dot);
        }
      }
    float* dots = reinterpret_cast<float*>(lds + L::offDOT);
    dots[w * 64 + l] = dot;
    lds_barrier();
    dot += dots[partner * 64 + l];
    dot += __shfl_xor(dot, 32);
    const float mean = dot / (float)D;
#pragma unroll
    for (int i = 0; i < DCH; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) dk[i][r] = rs * (dk[i][r] - kh[i][r] * mean);
  }
#pragma unroll
  for (int i = 0; i < DCH; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = from_f32<DT>(dk[i][4 * j + e]);
      *reinterpret_cast<u16x4*>(dkrow + 32 * (DCH * h + i) + 8 * j + 4 * g) = v;
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
static hipError_t launch_backward_t(const BackwardArgs& a, int part, hipStream_t st) {
  const long long nb = a.N / BLK;
  if (part < 0 || part == 0) {
    hipLaunchKernelGGL((bwd_pre<DT, D, BLK>), dim3((unsigned)(nb * a.BH)), dim3(256), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (part < 0 || part == 1) {
    hipLaunchKernelGGL((bwd_main<DT, D, BLK>), dim3((unsigned)(nb * a.BH)), dim3(BLK * 4), 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (part < 0 || part == 2) {
    const long long threads = (long long)a.BH * a.N * (D / 8);
    hipLaunchKernelGGL((dq_finalize<DT, D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_backward(const BackwardArgs& a, int part, hipStream_t st) {
  return dispatch_dt_d_blk(a.dtype, a.D, a.BLK, [&](auto dt, auto d, auto blk) {
    return launch_backward_t<decltype(dt)::value, decltype(d)::value, decltype(blk)::value>(a, part, st);
  });
}

}  // namespace sagebwd
