// Fused INT8/FP16 attention backward.
// SageBwd article (aitrends.kr 8227): precision-split paragraph (recomputed QK^T, dV = P^T dO,
// dK = dS^T Q, dQ = dS K in INT8; dP = dO V^T alone in the 16-bit type), gradient
// paragraph (dQ = dS K and dK = dS^T Q), dS-magnitude paragraph (dS is what INT8 struggles
// with, so it is quantised on its own tile with its own absmax scale, in registers).
//
// Kernels:
//   bwd_pre      one workgroup per (head, block of BLK tokens). Computes D = rowsum(dO o O),
//                lse * log2(e), the block absmax and INT8 codes of dO, and writes, for every
//                64-query tile, a "packet": the exact LDS image the main kernel needs for that
//                tile (Q codes, dO, dO^T codes, Q^T codes, lse2, D, block scales), already
//                swizzled and permuted. Also zeroes the float32 dQ accumulator rows.
//   bwd_main     one workgroup per (head, key block of BLK keys); a pair of waves owns each
//                32 keys. Streams the query tiles' packets into double-buffered LDS with
//                buffer->LDS copies (the next tile is in flight while the current one is
//                computed). S = Q K~^T with v_mfma_i32_32x32x32_i8 in the layout lane = key,
//                registers = queries, which is directly the B operand of the two products that
//                contract over queries: dV^T = dO^T P and dK^T = Q^T dS. dP = dO V^T uses
//                v_mfma_f32_32x32x16_{f16,bf16} on the raw dO and V. dS codes go through LDS
//                once (query-major) for dQ = dS K, accumulated with float32 atomics.
//   bwd_dq       (dS spill mode) query-major dQ = dS K over the spilled dS tiles, fused with the
//                RMSNorm backward and the dtype rounding.
//   dq_finalize  (atomic mode) RMSNorm backward of the accumulated dQ and dtype rounding.
// dQ mode: in dS spill mode (the default while its O(N^2) scratch stays moderate) bwd_main
// writes each dS tile's INT8 codes once to the workspace (the split-reduction pass); in atomic
// mode it accumulates dQ with float32 atomics instead.
#include "common.hpp"
#include "launch.hpp"

#include <float.h>

#include <type_traits>

namespace sagebwd {

namespace {

constexpr int kTq = 64;  // query rows per P / dS quantisation tile
constexpr float kLog2e = 1.4426950408889634f;

// Byte position, inside a group of 32 tokens of a channel-major row, of token-dword kd
// (tokens 4kd..4kd+3, kd = 0..7): lane group g of an MFMA operand needs tokens {8j + 4g + i}
// (j, i = 0..3), which lands at bytes 16g..16g+15. Token t sits at 16*((t>>2)&1) + 4*(t>>3) + (t&3).
__device__ __forceinline__ int perm_dword_pos(int kd) { return 16 * (kd & 1) + 4 * (kd >> 1); }

// XOR swizzles of the 16-byte chunks of LDS rows: 8 consecutive rows read at the same
// logical chunk land in 8 different bank groups.
template <int ROWB>
__device__ __forceinline__ int swz(int row, int chunk) {
  if constexpr (ROWB >= 128) return chunk ^ (row & 7);
  else if constexpr (ROWB == 64) return chunk ^ ((row >> 1) & 3);
  else return chunk;
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations, not for its
// outstanding vector-memory operations (dQ atomics, buffer->LDS copies in flight, whose
// completion is awaited explicitly where their data is published). The memory clobber keeps
// the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Direct buffer -> LDS copy (buffer_load ... lds): lane l reads 16 bytes at byte offset
// voff + soff of the buffer [base, base + bytes) (reads past the end return zeros) and the
// hardware writes them to LDS at lds + 16*l (the 4-byte form: 4 bytes at lds + 4*l). The
// bodies are compiled for the device only:
// this compiler's host pass cannot type-check the LDS-DMA builtin and, instead of reporting
// it, silently omits the host launch stubs of kernels that reach it.
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

}  // namespace

// Layout of one 64-query tile packet (= of one LDS tile buffer), bytes.
template <int D>
struct Packet {
  static constexpr int bQ = 0;                // Q codes [64][D], chunk j of row r at slot swz<D>(r, j)
  static constexpr int bDO = 64 * D;          // dO [64][D] 16-bit, chunk j of row r at slot swz<2D>(r, j)
  static constexpr int bDOT = bDO + 128 * D;  // dO codes [D][64], tokens permuted, chunk swz<64>(c, j)
  static constexpr int bQT = bDOT + 64 * D;   // Q codes [D][64], same order as dO^T
  static constexpr int bLSE = bQT + 64 * D;   // lse * log2(e) [64] f32
  static constexpr int bDV = bLSE + 256;      // D = rowsum(dO o O) [64] f32
  static constexpr int bSQ = bDV + 256;       // Q block scale f32
  static constexpr int bSDO = bSQ + 4;        // dO block scale f32
  static constexpr int kBytes = (bSDO + 4 + 1023) / 1024 * 1024;
  static constexpr int kCopies = kBytes / 1024;  // 1 KB wave copies per packet
};

size_t packet_bytes(int d) { return d == 64 ? Packet<64>::kBytes : Packet<128>::kBytes; }

// dS spill: (query tile, key block) tiles of one head, causal ones packed key block by key
// block (key block kb holds query tiles kb*BLK/64 .. N/64-1).
long long spill_tiles_per_head(int N, int blk, int causal) {
  const long long nt = N / 64, nb = N / blk, r = blk / 64;
  return causal ? nb * nt - r * nb * (nb - 1) / 2 : nb * nt;
}
__device__ __forceinline__ long long spill_tile_index(int N, int blk, int causal, int kb, int qt) {
  const long long nt = N / 64, r = blk / 64;
  return causal ? (long long)kb * nt - r * (long long)kb * (kb - 1) / 2 + (qt - (long long)kb * r)
                : (long long)kb * nt + qt;
}

// ------------------------------------------------------------------------------ bwd_pre
template <int DT, int D, int BLK>
__global__ __launch_bounds__(256) void bwd_pre(BackwardArgs a) {
  using P = Packet<D>;
  __shared__ float xs[BLK][D + 1];
  __shared__ __attribute__((aligned(16))) int8_t qs[BLK][D + 4];
  __shared__ __attribute__((aligned(16))) int8_t ks[BLK][D + 4];
  __shared__ float red[4];
  const int nb = a.N / BLK;
  const int blk_id = blockIdx.x % nb;
  const int bh = blockIdx.x / nb;
  const size_t tok0 = (size_t)bh * a.N + (size_t)blk_id * BLK;
  const int tid = threadIdx.x;
  constexpr int CPR = D / 8;  // 16-byte dO chunks per row
  // packet of the block's first 64-token tile
  int8_t* pk0 = a.pk + ((size_t)bh * (a.N / kTq) + (size_t)blk_id * (BLK / kTq)) * P::kBytes;

  // dO, O: coalesced 8-element chunks; D via a segmented reduction over each row's chunks
  float amax = 0.0f;
  for (int ch = tid; ch < BLK * CPR; ch += 256) {
    const int t = ch / CPR, j = ch % CPR, c = j * 8;
    const u16x8 dv = *reinterpret_cast<const u16x8*>(a.dO + (tok0 + t) * D + c);
    const u16x8 ov = *reinterpret_cast<const u16x8*>(a.O + (tok0 + t) * D + c);
    int8_t* pk = pk0 + (t / kTq) * P::kBytes;
    const int r = t % kTq;
    *reinterpret_cast<u16x8*>(pk + P::bDO + r * 2 * D + 16 * swz<2 * D>(r, j)) = dv;
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
    if (j == 0) {
      reinterpret_cast<float*>(pk + P::bDV)[r] = part;
      reinterpret_cast<float*>(pk + P::bLSE)[r] = a.lse[tok0 + t] * kLog2e;
    }
  }
  // Q codes: token-major into the packets, and into LDS for the transpose
  for (int ch = tid; ch < BLK * D / 16; ch += 256) {
    const int t = (ch * 16) / D, j = ch % (D / 16), c = 16 * j;
    const i32x4 v = *reinterpret_cast<const i32x4*>(a.Qc + (tok0 + t) * D + c);
    const int r = t % kTq;
    *reinterpret_cast<i32x4*>(pk0 + (t / kTq) * P::kBytes + P::bQ + r * D + 16 * swz<D>(r, j)) = v;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<int*>(&qs[t][c + 4 * i]) = v[i];
  }
  if (a.spill) {
    // K codes of this key block, into LDS for the channel-major K^T packet
    for (int ch = tid; ch < BLK * D / 16; ch += 256) {
      const int t = (ch * 16) / D, c = (ch * 16) % D;
      const i32x4 v = *reinterpret_cast<const i32x4*>(a.Kc + (tok0 + t) * D + c);
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<int*>(&ks[t][c + 4 * i]) = v[i];
    }
  } else {
    // zero the dQ accumulator rows of this block
    for (int e = tid; e < BLK * D / 4; e += 256)
      reinterpret_cast<float4*>(a.dq_acc + tok0 * D)[e] = make_float4(0.f, 0.f, 0.f, 0.f);
  }

  amax = wave_max(amax);
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  const float am = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float inv = am > 0.0f ? 127.0f / am : 0.0f;
  if (tid < BLK / kTq) {
    int8_t* pk = pk0 + tid * P::kBytes;
    *reinterpret_cast<float*>(pk + P::bSDO) = am > 0.0f ? am / 127.0f : 0.0f;
    *reinterpret_cast<float*>(pk + P::bSQ) = a.Qs[(size_t)bh * nb + blk_id];
  }
  // channel-major codes of dO and of Q: word = 4 consecutive tokens of channel c, placed at
  // its permuted position inside the 32-token group and its swizzled 16-byte chunk
  for (int w = tid; w < BLK * D / 4; w += 256) {
    const int c = w / (BLK / 4), t = 4 * (w % (BLK / 4));
    const unsigned word = pack4_lo_bytes(quant_word(xs[t][c], inv), quant_word(xs[t + 1][c], inv),
                                         quant_word(xs[t + 2][c], inv), quant_word(xs[t + 3][c], inv));
    const unsigned qw = (unsigned)(uint8_t)qs[t][c] | ((unsigned)(uint8_t)qs[t + 1][c] << 8) |
                        ((unsigned)(uint8_t)qs[t + 2][c] << 16) | ((unsigned)(uint8_t)qs[t + 3][c] << 24);
    const int tl = t % kTq;
    const int p = 32 * (tl / 32) + perm_dword_pos((tl % 32) / 4);  // byte position in the 64-token row
    const int off = c * kTq + 16 * swz<kTq>(c, p / 16) + p % 16;
    int8_t* pk = pk0 + (t / kTq) * P::kBytes;
    *reinterpret_cast<unsigned*>(pk + P::bDOT + off) = word;
    *reinterpret_cast<unsigned*>(pk + P::bQT + off) = qw;
  }
  if (a.spill) {
    // K^T packet of this key block: [D][BLK] codes, chunk j of row c at slot swz<BLK>(c, j)
    int8_t* kt = a.ktp + ((size_t)bh * nb + blk_id) * (size_t)(D * BLK);
    for (int w = tid; w < BLK * D / 4; w += 256) {
      const int c = w / (BLK / 4), t = 4 * (w % (BLK / 4));
      const unsigned kw = (unsigned)(uint8_t)ks[t][c] | ((unsigned)(uint8_t)ks[t + 1][c] << 8) |
                          ((unsigned)(uint8_t)ks[t + 2][c] << 16) | ((unsigned)(uint8_t)ks[t + 3][c] << 24);
      *reinterpret_cast<unsigned*>(kt + c * BLK + 16 * swz<BLK>(c, t / 16) + t % 16) = kw;
    }
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
  using P = Packet<D>;
  static constexpr int NKG = BLK / 32;        // 32-key groups
  static constexpr int NW = 2 * NKG;          // waves
  static constexpr int kRowS = BLK + 16;      // dS codes [query][key]; K^T codes [channel][key]
  static constexpr int kBuf = P::kBytes;      // one tile buffer (double-buffered)
  static constexpr int offDS = 2 * kBuf;
  static constexpr int offKT = offDS + kTq * kRowS;
  static constexpr int offK = offKT + D * kRowS;    // K codes [BLK][D], token-major, swizzled
  static constexpr int offXP = offK + BLK * D;      // P codes exchanged inside a pair [NW][64][16 B]
  static constexpr int offXD = offXP + NW * 1024;   // dS codes exchanged inside a pair
  static constexpr int offRED = offXD + NW * 1024;  // redP[NW], redD[NW]
  static constexpr int offDOT = offRED + 2 * NW * 4;  // epilogue: per-lane dK.K^ partial dots [NW][64]
  static constexpr int kBytes = offDOT + NW * 64 * 4;
  static constexpr int kCopiesPerWave = (P::kCopies + NW - 1) / NW;
};

template <int DT, int D, int BLK, bool SPILL>
__global__ __launch_bounds__(BLK * 4, 1) void bwd_main(BackwardArgs a) {
  using L = BwdLds<D, BLK>;
  using P = Packet<D>;
  constexpr int NKG = L::NKG;      // 32-key groups (wave pairs)
  constexpr int NW = L::NW;        // waves per workgroup
  constexpr int NT = NW * 64;      // threads
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
  const int kl = 32 * kg + lk;                 // ... inside the block
  const size_t hrow = (size_t)bh * a.N;
  const int ntile = a.N / kTq;
  const int8_t* pkh = a.pk + (size_t)bh * ntile * P::kBytes;   // this head's packets
  const uint32_t pkh_bytes = (uint32_t)ntile * P::kBytes;

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
    if constexpr (!SPILL) {
#pragma unroll
      for (int i = 0; i < 16; ++i) lds[L::offKT + (c + i) * L::kRowS + t] = (int8_t)(v[i >> 2] >> (8 * (i & 3)));
    }
  }
  const float sK = a.Ks[(size_t)bh * nb + kb];
  const float smc = a.sm_scale;
  float* redP = reinterpret_cast<float*>(lds + L::offRED);
  float* redD = redP + NW;

  f32x16 dk[DCH], dv[DCH];
#pragma unroll
  for (int i = 0; i < DCH; ++i) { dk[i] = f32x16{}; dv[i] = f32x16{}; }

  // copies of packet qt into an LDS tile buffer: wave w moves KB cp = w, w + NW, ...
  auto issue = [&](int qt, int8_t* dst) {
#pragma unroll
    for (int j = 0; j < L::kCopiesPerWave; ++j) {
      const int cp = w + NW * j;
      if (cp < P::kCopies) buffer_to_lds16(pkh, pkh_bytes, dst + cp * 1024, 16 * l, qt * P::kBytes + cp * 1024);
    }
  };

  const int qt0 = a.causal ? k0 / kTq : 0;
  issue(qt0, lds);
  wait_vmcnt<0>();
  __syncthreads();

  for (int qt = qt0; qt < ntile; ++qt) {
    const int q0 = qt * kTq;
    const bool has_next = qt + 1 < ntile;
    int8_t* buf = lds + ((qt - qt0) & 1) * L::kBuf;
    int8_t* nbuf = lds + (((qt - qt0) & 1) ^ 1) * L::kBuf;
    if (has_next) issue(qt + 1, nbuf);

    const float sQ = *reinterpret_cast<const float*>(buf + P::bSQ);
    const float sdO = *reinterpret_cast<const float*>(buf + P::bSDO);
    const float c2 = (sQ * sK) * (smc * kLog2e);

    // ---- S, P, dP, dS for query rows 32h..32h+31 of the tile and this pair's 32 keys
    const int q = 32 * h + lk;
    i32x16 s = i32x16{};
#pragma unroll
    for (int kk = 0; kk < DC; ++kk) {
      const i32x4 aq = *reinterpret_cast<const i32x4*>(buf + P::bQ + q * D + 16 * swz<D>(q, 2 * kk + g));
      const i32x4 bk = *reinterpret_cast<const i32x4*>(lds + L::offK + kl * D + 16 * swz<D>(kl, 2 * kk + g));
      s = mfma_i8_32x32x32(aq, bk, s);
    }
    f32x16 dp = f32x16{};
#pragma unroll
    for (int kk = 0; kk < DH; ++kk) {
      const u16x8 ad = *reinterpret_cast<const u16x8*>(buf + P::bDO + q * 2 * D + 16 * swz<2 * D>(q, 2 * kk + g));
      dp = mfma_16b_32x32x16<DT>(ad, vreg[kk], dp);
    }
    const float* lse2 = reinterpret_cast<const float*>(buf + P::bLSE) + 32 * h + 4 * g;
    const float* dvv = reinterpret_cast<const float*>(buf + P::bDV) + 32 * h + 4 * g;
    float pf[16], dsf[16];
    float pm = 0.0f, dm = 0.0f;
    auto elems = [&](auto masked) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = 8 * (r >> 2) + (r & 3);  // query offset inside the 32 rows, minus 4g
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf((float)s[r], c2, -lse2[qi]));
        if constexpr (decltype(masked)::value) {
          if (key > q0 + 32 * h + 4 * g + qi) p = 0.0f;
        }
        pf[r] = p;
        dsf[r] = p * (dp[r] - dvv[qi]);
      }
      // tile maxima as three-input max trees (v_max3_f32, |x| as an operand modifier)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        pm = fmaxf(pm, fmaxf(pf[r], pf[r + 1]));
        dm = fmaxf(dm, fmaxf(fabsf(dsf[r]), fabsf(dsf[r + 1])));
      }
    };
    if (a.causal && k0 + BLK - 1 > q0) elems(std::true_type{});
    else elems(std::false_type{});
    pm = wave_max(pm);
    dm = wave_max(dm);
    if (l == 0) { redP[w] = pm; redD[w] = dm; }
    lds_barrier();
    // P tile: 64 queries x this pair's 32 keys; dS tile: 64 queries x the block's BLK keys
    const float pa = fmaxf(redP[kg], redP[kg + NKG]);
    float da = redD[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) da = fmaxf(da, redD[i]);
    // Tile scales a/127 and inverses 127/a (hardware reciprocal; a tile whose absmax is below
    // the smallest normal float is quantised against that bound so the reciprocal stays finite).
    const float pa_n = fmaxf(pa, FLT_MIN), da_n = fmaxf(da, FLT_MIN);
    const float pinv = 127.0f * __builtin_amdgcn_rcpf(pa_n), sP = pa_n * (1.0f / 127.0f);
    const float dinv = 127.0f * __builtin_amdgcn_rcpf(da_n), sdS = da_n * (1.0f / 127.0f);
    i32x4 pc, dc;  // this wave's codes (queries 32h..32h+31)
    {
      int8_t* col = lds + L::offDS + kl;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pc[j] = (int)pack4_lo_bytes(quant_word_fma(pf[4 * j], pinv), quant_word_fma(pf[4 * j + 1], pinv),
                                    quant_word_fma(pf[4 * j + 2], pinv), quant_word_fma(pf[4 * j + 3], pinv));
        const unsigned w0 = quant_word_fma(dsf[4 * j], dinv), w1 = quant_word_fma(dsf[4 * j + 1], dinv);
        const unsigned w2 = quant_word_fma(dsf[4 * j + 2], dinv), w3 = quant_word_fma(dsf[4 * j + 3], dinv);
        dc[j] = (int)pack4_lo_bytes(w0, w1, w2, w3);
        // dS codes, query-major, for dQ: query 32h + 8j + 4g + i, key kl
        const int qb = 32 * h + 8 * j + 4 * g;
        col[(qb + 0) * L::kRowS] = (int8_t)w0;
        col[(qb + 1) * L::kRowS] = (int8_t)w1;
        col[(qb + 2) * L::kRowS] = (int8_t)w2;
        col[(qb + 3) * L::kRowS] = (int8_t)w3;
      }
      *reinterpret_cast<i32x4*>(lds + L::offXP + w * 1024 + l * 16) = pc;
      *reinterpret_cast<i32x4*>(lds + L::offXD + w * 1024 + l * 16) = dc;
    }
    lds_barrier();
    // the partner's codes cover queries 32(1-h)..32(1-h)+31
    const i32x4 pco = *reinterpret_cast<const i32x4*>(lds + L::offXP + partner * 1024 + l * 16);
    const i32x4 dco = *reinterpret_cast<const i32x4*>(lds + L::offXD + partner * 1024 + l * 16);

    // ---- dV^T += dO^T P and dK^T += Q^T dS for channel half h (int32 over the 64 queries):
    //      own codes pair with the A-operand chunk of query half h, the partner's with 1-h
    {
      const float sv = sP * sdO;
#pragma unroll
      for (int i = 0; i < DCH; ++i) {
        const int c = 32 * (DCH * h + i) + lk;
        const i32x4 a0 = *reinterpret_cast<const i32x4*>(buf + P::bDOT + c * kTq + 16 * swz<kTq>(c, 2 * h + g));
        const i32x4 a1 = *reinterpret_cast<const i32x4*>(buf + P::bDOT + c * kTq + 16 * swz<kTq>(c, 2 * (1 - h) + g));
        i32x16 acc = mfma_i8_32x32x32(a0, pc, i32x16{});
        acc = mfma_i8_32x32x32(a1, pco, acc);
#pragma unroll
        for (int r = 0; r < 16; ++r) dv[i][r] += sv * (float)acc[r];
      }
      const float sk = smc * sdS * sQ;
#pragma unroll
      for (int i = 0; i < DCH; ++i) {
        const int c = 32 * (DCH * h + i) + lk;
        const i32x4 a0 = *reinterpret_cast<const i32x4*>(buf + P::bQT + c * kTq + 16 * swz<kTq>(c, 2 * h + g));
        const i32x4 a1 = *reinterpret_cast<const i32x4*>(buf + P::bQT + c * kTq + 16 * swz<kTq>(c, 2 * (1 - h) + g));
        i32x16 acc = mfma_i8_32x32x32(a0, dc, i32x16{});
        acc = mfma_i8_32x32x32(a1, dco, acc);
#pragma unroll
        for (int r = 0; r < 16; ++r) dk[i][r] += sk * (float)acc[r];
      }
    }

    if constexpr (SPILL) {
      // ---- spill the dS tile (query-major, rows swizzled) and its dQ multiplier; the
      //      query-major dQ pass contracts it with K
      const long long ti = (long long)bh * a.spill_tiles + spill_tile_index(a.N, BLK, a.causal, kb, qt);
      int8_t* dst = a.dsp + ti * (kTq * BLK);
      for (int ch = tid; ch < kTq * BLK / 16; ch += NT) {
        const int r = ch / (BLK / 16), j = ch % (BLK / 16);
        *reinterpret_cast<i32x4*>(dst + r * BLK + 16 * swz<BLK>(r, j)) =
            *reinterpret_cast<const i32x4*>(lds + L::offDS + r * L::kRowS + 16 * j);
      }
      if (tid == 0) a.dsm[ti] = smc * sdS * sK;
      // the next tile's copies were issued before these (at most 2) stores; in-order
      // completion makes this wait for every copy
      wait_vmcnt<2>();
    } else {
      // ---- dQ = dS K over the BLK keys: 2 x DC output tiles of 32 x 32, split over the
      //      waves, added to the float32 accumulator with atomics
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
      // The next tile's copies were issued before this iteration's dQ atomics; vector memory
      // operations complete in issue order, so allowing the atomics (16 per dQ tile) to stay
      // outstanding still waits for every copy.
      if constexpr (2 * DC <= NW) {
        if (w < 2 * DC) wait_vmcnt<16>();
        else wait_vmcnt<0>();
      } else {
        wait_vmcnt<16 * ((2 * DC) / NW)>();
      }
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

// ------------------------------------------------------------------------------ bwd_dq
// Query-major dQ pass over the spilled dS tiles: one workgroup (4 waves) per (head, 64-query
// tile). For every key block up to the diagonal, the tile's dS codes [64][BLK] and the block's
// K^T codes [D][BLK] stream through double-buffered LDS (buffer->LDS copies), and
// dQ^ += m(kb) * (dS_codes . K_codes) runs on v_mfma_i32_32x32x32_i8 with float32 accumulation
// in registers (m = sm_scale * s_dS * s_K of the tile). The epilogue applies the RMSNorm
// backward and writes dQ in the dtype; no float32 dQ buffer and no atomics.
template <int D, int BLK>
struct DqLds {
  static constexpr int bDS = 0;                     // dS codes [64][BLK], rows swizzled
  static constexpr int bKT = 64 * BLK;              // K^T codes [D][BLK], rows swizzled
  static constexpr int bM = bKT + D * BLK;          // tile multiplier (first word)
  static constexpr int kBuf = bM + 1024;
  static constexpr int kCopiesDS = 64 * BLK / 1024;
  static constexpr int kCopiesKT = D * BLK / 1024;
  // the epilogue reuses the buffers for the dQ^ tile [64][D] f32
  static constexpr int kBytes = 2 * kBuf > 64 * D * 4 ? 2 * kBuf : 64 * D * 4;
};

template <int DT, int D, int BLK>
__global__ __launch_bounds__(256) void bwd_dq(BackwardArgs a) {
  using L = DqLds<D, BLK>;
  constexpr int DC = D / 32, KC = BLK / 32;
  constexpr int TPW = (2 * DC) / 4;                 // 32 x 32 output tiles per wave
  __shared__ __attribute__((aligned(16))) int8_t lds[L::kBytes];
  const int ntile = a.N / kTq, nb = a.N / BLK;
  const int bh = blockIdx.x % a.BH;
  const int qt = a.causal ? ntile - 1 - (int)(blockIdx.x / a.BH) : (int)(blockIdx.x / a.BH);
  const int q0 = qt * kTq;
  const int w = __builtin_amdgcn_readfirstlane(wave_id()), l = lane_id(), g = l >> 5, lk = l & 31;
  const int kb_last = a.causal ? (q0 + kTq - 1) / BLK : nb - 1;
  const int8_t* dsh = a.dsp + (size_t)bh * a.spill_tiles * (kTq * BLK);
  const uint32_t dsh_bytes = (uint32_t)(a.spill_tiles * (kTq * BLK));
  const float* dmh = a.dsm + (size_t)bh * a.spill_tiles;
  const int8_t* kth = a.ktp + (size_t)bh * nb * (D * BLK);
  const uint32_t kth_bytes = (uint32_t)nb * (D * BLK);

  auto issue = [&](int kb, int8_t* buf) {
    const long long ti = spill_tile_index(a.N, BLK, a.causal, kb, qt);
    for (int cp = w; cp < L::kCopiesDS + L::kCopiesKT; cp += 4) {
      if (cp < L::kCopiesDS)
        buffer_to_lds16(dsh, dsh_bytes, buf + L::bDS + cp * 1024, 16 * l, (uint32_t)(ti * (kTq * BLK)) + cp * 1024);
      else
        buffer_to_lds16(kth, kth_bytes, buf + L::bKT + (cp - L::kCopiesDS) * 1024, 16 * l,
                        (uint32_t)kb * (D * BLK) + (cp - L::kCopiesDS) * 1024);
    }
    if (w == 3) buffer_to_lds4(dmh, (uint32_t)(a.spill_tiles * 4), buf + L::bM, 4 * l, (uint32_t)(ti * 4));
  };

  f32x16 dq[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) dq[i] = f32x16{};
  issue(0, lds);
  wait_vmcnt<0>();
  __syncthreads();
  for (int kb = 0; kb <= kb_last; ++kb) {
    int8_t* buf = lds + (kb & 1) * L::kBuf;
    if (kb < kb_last) issue(kb + 1, lds + ((kb & 1) ^ 1) * L::kBuf);
    const float m = *reinterpret_cast<const float*>(buf + L::bM);
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int tile = w + 4 * i, u = tile / DC, ct = tile % DC;
      const int qr = 32 * u + lk, cr = 32 * ct + lk;
      i32x16 acc = i32x16{};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const i32x4 as = *reinterpret_cast<const i32x4*>(buf + L::bDS + qr * BLK + 16 * swz<BLK>(qr, 2 * kc + g));
        const i32x4 bk = *reinterpret_cast<const i32x4*>(buf + L::bKT + cr * BLK + 16 * swz<BLK>(cr, 2 * kc + g));
        acc = mfma_i8_32x32x32(as, bk, acc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) dq[i][r] += m * (float)acc[r];
    }
    wait_vmcnt<0>();   // the next key block's copies (the only vector-memory operations here)
    lds_barrier();
  }
  // ---- epilogue: dQ^ tile to LDS [64][D] f32, then RMSNorm backward row by row
  float* t = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int tile = w + 4 * i, u = tile / DC, ct = tile % DC;
#pragma unroll
    for (int r = 0; r < 16; ++r) t[(32 * u + 8 * (r >> 2) + 4 * g + (r & 3)) * D + 32 * ct + lk] = dq[i][r];
  }
  __syncthreads();
  constexpr int CPR = D / 8;                        // lanes per row, 8 channels each
  const size_t hrow = (size_t)bh * a.N;
  for (int e = threadIdx.x; e < kTq * CPR; e += 256) {
    const int r = e / CPR, c = (e % CPR) * 8;
    const size_t tok = hrow + q0 + r;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = t[r * D + c + i];
    u16x8 out;
    if (a.qk_norm) {
      const float rs = a.q_rstd[tok];
      const u16x8 qv = *reinterpret_cast<const u16x8*>(a.Q + tok * D + c);
      float qh[8], dot = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        qh[i] = to_f32<DT>(qv[i]) * rs;
        dot = __builtin_fmaf(v[i], qh[i], dot);
      }
#pragma unroll
      for (int o = CPR / 2; o > 0; o >>= 1) dot += __shfl_xor(dot, o);
      const float mean = dot / (float)D;
#pragma unroll
      for (int i = 0; i < 8; ++i) out[i] = from_f32<DT>(rs * (v[i] - qh[i] * mean));
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) out[i] = from_f32<DT>(v[i]);
    }
    *reinterpret_cast<u16x8*>(a.dQ + tok * D + c) = out;
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
    const hipError_t e = launch_kernel(&bwd_pre<DT, D, BLK>, dim3((unsigned)(nb * a.BH)), dim3(256), st, a);
    if (e != hipSuccess) return e;
  }
  if (part < 0 || part == 1) {
    const hipError_t e =
        a.spill ? launch_kernel(&bwd_main<DT, D, BLK, true>, dim3((unsigned)(nb * a.BH)), dim3(BLK * 4), st, a)
                : launch_kernel(&bwd_main<DT, D, BLK, false>, dim3((unsigned)(nb * a.BH)), dim3(BLK * 4), st, a);
    if (e != hipSuccess) return e;
  }
  if (part < 0 || part == 2) {
    if (a.spill)
      return launch_kernel(&bwd_dq<DT, D, BLK>, dim3((unsigned)((long long)(a.N / kTq) * a.BH)), dim3(256), st, a);
    const long long threads = (long long)a.BH * a.N * (D / 8);
    return launch_kernel(&dq_finalize<DT, D>, dim3((unsigned)((threads + 255) / 256)), dim3(256), st, a);
  }
  return hipSuccess;
}

hipError_t launch_backward(const BackwardArgs& a, int part, hipStream_t st) {
  return dispatch_dt_d_blk(a.dtype, a.D, a.BLK, [&](auto dt, auto d, auto blk) {
    return launch_backward_t<decltype(dt)::value, decltype(d)::value, decltype(blk)::value>(a, part, st);
  });
}

}  // namespace sagebwd
