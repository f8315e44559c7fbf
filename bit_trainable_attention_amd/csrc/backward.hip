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
//                tile (Q codes, dO, dO^T codes, lse2, D, block scales), already swizzled and
//                permuted. Also writes the key blocks' K^T codes (spill mode) or zeroes the
//                float32 dQ accumulator rows (atomic mode).
//   bwd_main     one workgroup per (head, key block of BLK keys); each wave owns 16 keys.
//                Streams the query blocks' packets into double-buffered LDS with buffer->LDS
//                copies (issued two tiles ahead). S = Q K~^T on v_mfma_i32_16x16x64_i8 and
//                dP = dO V^T on v_mfma_f32_16x16x32_{f16,bf16}, in the layout lane = key,
//                registers = queries, which is directly the B operand of the two products
//                that contract over queries: dV^T = dO^T P and dK^T = Q^T dS. dS codes leave
//                key-major (spill mode) or go through LDS once for dQ = dS K with float32
//                atomics (atomic mode).
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

constexpr int kPq = 64;  // query rows of a tile packet and of a spilled dS^T tile
constexpr float kLog2e = 1.4426950408889634f;

// Byte position, inside a 64-token channel-major row of a tile packet, of token u: the
// backward's lane group g holds tokens {16t + 4g + r} (t, r = 0..3) as contraction slots
// 4t + r, so token 16t + 4g + r sits at byte 16g + 4t + r.
__device__ __forceinline__ int tile_token_pos(int u) { return 16 * ((u >> 2) & 3) + 4 * (u >> 4) + (u & 3); }

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations, not for its
// outstanding vector-memory operations (dQ atomics, buffer->LDS copies in flight, whose
// completion is awaited explicitly where their data is published). The memory clobber keeps
// the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// A wave-uniform float held in a scalar register.
__device__ __forceinline__ float uniform_f(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// Sum over each 16-lane row, returned to every lane of the row (DPP butterfly).
template <int CTRL>
__device__ __forceinline__ float add_dpp_row(float v) {
  return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row_sum16(float v) {
  v = add_dpp_row<0xB1>(v);
  v = add_dpp_row<0x4E>(v);
  v = add_dpp_row<0x141>(v);
  return add_dpp_row<0x140>(v);
}

}  // namespace

// Chunk swizzles of the packets' row-major regions (16-byte chunk j of row r is stored at
// chunk slot swz_q / swz_do). For d = 128 they follow measured LDS rates on gfx950: with
// j ^ (r & 7), the 256-byte dO rows read at ~117 B/clk per CU (j ^ (r & 15): ~204), and the
// transposing reads of the Q rows, which name rows r and r + 16 together, at ~116 B/clk
// (folding bit 4 of the row into the swizzle: ~175). d = 64 keeps the generic swizzle.
template <int D>
__device__ __forceinline__ int swz_q(int r, int j) {
  if constexpr (D == 128) return j ^ (((r >> 1) ^ ((r >> 4) << 2)) & 7);
  else return swz<D>(r, j);
}
template <int D>
__device__ __forceinline__ int swz_do(int r, int j) {
  if constexpr (D == 128) return j ^ (r & 15);
  else return swz<2 * D>(r, j);
}

// Chunk swizzle of the spilled dS^T tiles [BLK keys][64 query slots]: the dQ pass reads
// them with transposing reads that name key rows r .. r + 7 of four lane groups 16 rows apart
// together; folding bit 4 of the row in (measured on gfx950) raises that read rate from ~115
// to ~179 B/clk per CU over j ^ ((r >> 1) & 3).
__device__ __forceinline__ int swz_ds(int r, int j) { return j ^ (((r >> 1) ^ (r >> 4)) & 3); }

// Layout of one 64-query tile packet (= of one LDS tile buffer), bytes.
template <int D>
struct Packet {
  static constexpr int bQ = 0;                // Q codes [64][D], chunk j of row r at slot swz_q<D>(r, j)
  static constexpr int bDO = 64 * D;          // dO [64][D] 16-bit, chunk j of row r at slot swz_do<D>(r, j)
  static constexpr int bDOT = bDO + 128 * D;  // dO codes [D][64], token u at tile_token_pos(u), chunk swz<64>(c, j)
  static constexpr int bLSE = bDOT + 64 * D;  // lse * log2(e) [64] f32
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
// One workgroup per (head, block of BLK tokens), 256 threads: thread (j, ch), j = tid / 16,
// ch = tid % 16, owns channels ch*CW .. ch*CW + CW - 1 (CW = D/16) of the four consecutive
// tokens 64q + 4j + k (k = 0..3) of every 64-token tile q of the block, in registers. The
// 16 lanes of a row share their tokens, so D = rowsum(dO o O) is a DPP tree across the row,
// and a thread's four codes of one channel are one word at the packet's permuted token
// position. Channel-major rows (dO^T, K^T codes) are assembled in an LDS byte tile.
template <int DT, int D, int BLK>
__global__ __launch_bounds__(256) void bwd_pre(BackwardArgs a) {
  using P = Packet<D>;
  constexpr int CW = D / 16;                 // channels per thread
  constexpr int NQ = BLK / kPq;              // 64-token tiles of the block
  constexpr int TR = kPq + 4;                // LDS row stride of a transposed tile row (bytes)
  constexpr int KR = BLK + 4;                // ... of the block's K^T rows
  constexpr int kTile = NQ * D * TR > D * KR ? NQ * D * TR : D * KR;
  __shared__ __attribute__((aligned(16))) int8_t tt[kTile];
  __shared__ float red[4];
  const int nb = a.N / BLK;
  const int blk_id = blockIdx.x % nb;
  const int bh = blockIdx.x / nb;
  const size_t tok0 = (size_t)bh * a.N + (size_t)blk_id * BLK;
  const int tid = threadIdx.x, j = tid >> 4, ch = tid & 15;
  const int c0 = ch * CW;
  const int wpos = tile_token_pos(4 * j);    // packet position of tokens 4j..4j+3 (one word)
  // packet of the block's first 64-token tile
  int8_t* pk0 = a.pk + ((size_t)bh * (a.N / kPq) + (size_t)blk_id * NQ) * P::kBytes;

  // ---- dO (16-bit, straight into the packets), D = rowsum(dO o O), lse * log2(e)
  float x[NQ][4][CW];
  float amax = 0.0f;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    int8_t* pk = pk0 + q * P::kBytes;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = 4 * j + k;                       // token inside the tile
      const size_t tok = tok0 + kPq * q + r;
      const int n = blk_id * BLK + kPq * q + r;      // token of the head
      const bool valid = n < a.Nv;                   // (padding of a ragged last block: zeros)
      const size_t row16 = a.x16.row(bh, valid ? n : 0);
      const unsigned short* dsrc = a.dO + row16 + c0;
      const unsigned short* osrc = a.O + row16 + c0;
      float part = 0.0f;
      if constexpr (CW == 8) {
        u16x8 dv = u16x8{}, ov = u16x8{};
        if (valid) {
          dv = *reinterpret_cast<const u16x8*>(dsrc);
          ov = *reinterpret_cast<const u16x8*>(osrc);
        }
        *reinterpret_cast<u16x8*>(pk + P::bDO + r * 2 * D + 16 * swz_do<D>(r, ch)) = dv;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          x[q][k][i] = to_f32<DT>(dv[i]);
          part = __builtin_fmaf(x[q][k][i], to_f32<DT>(ov[i]), part);
        }
      } else {
        u16x4 dv = u16x4{}, ov = u16x4{};
        if (valid) {
          dv = *reinterpret_cast<const u16x4*>(dsrc);
          ov = *reinterpret_cast<const u16x4*>(osrc);
        }
        *reinterpret_cast<u16x4*>(pk + P::bDO + r * 2 * D + 16 * swz_do<D>(r, ch >> 1) + 8 * (ch & 1)) = dv;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[q][k][i] = to_f32<DT>(dv[i]);
          part = __builtin_fmaf(x[q][k][i], to_f32<DT>(ov[i]), part);
        }
      }
#pragma unroll
      for (int i = 0; i < CW; ++i) amax = fmaxf(amax, fabsf(x[q][k][i]));
      const float dsum = row_sum16(part);
      if (ch == 0) {
        reinterpret_cast<float*>(pk + P::bDV)[r] = dsum;
        // a padding query gets lse = +inf, so its P = 2^(s - lse) is 0 everywhere
        reinterpret_cast<float*>(pk + P::bLSE)[r] = valid ? a.lse[tok] * kLog2e : INFINITY;
      }
    }
  }
  amax = wave_max(amax);
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  const float am = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const bool fp8 = a.fmt == FMT_FP8;
  const float M = fp8 ? 448.0f : 127.0f;
  const float inv = am > 0.0f ? M / am : 0.0f;
  if (tid < NQ) {
    int8_t* pk = pk0 + tid * P::kBytes;
    *reinterpret_cast<float*>(pk + P::bSDO) = am > 0.0f ? am / M : 0.0f;
    *reinterpret_cast<float*>(pk + P::bSQ) = a.Qs[(size_t)bh * nb + blk_id];
  }

  // channel-major rows of a tile from the LDS tile [q][c][TR]: chunk g of row c (positions
  // 16g..16g+15) is stored at chunk swz<64>(c, g) of the packet region at offset `region`
  auto write_rows = [&](int region) {
    for (int e = tid; e < NQ * D * 4; e += 256) {
      const int q = e / (D * 4), c = (e / 4) % D, g = e % 4;
      const int8_t* src = tt + (q * D + c) * TR + 16 * g;
      i32x4 v;
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const int*>(src + 4 * u);
      *reinterpret_cast<i32x4*>(pk0 + q * P::kBytes + region + c * kPq + 16 * swz<kPq>(c, g)) = v;
    }
  };

  // ---- dO codes, channel-major (dO^T), tokens at their permuted positions
#pragma unroll
  for (int q = 0; q < NQ; ++q)
#pragma unroll
    for (int i = 0; i < CW; ++i)
      *reinterpret_cast<unsigned*>(tt + (q * D + c0 + i) * TR + wpos) =
          code_word(fp8, x[q][0][i], x[q][1][i], x[q][2][i], x[q][3][i], inv);
  __syncthreads();
  write_rows(P::bDOT);
  __syncthreads();

  // ---- Q codes, token-major into the packets (the key-block kernel reads its Q^T operands
  //      out of them with transposing reads)
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    int8_t* pk = pk0 + q * P::kBytes;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = 4 * j + k;
      const int8_t* src = a.Qc + (tok0 + kPq * q + r) * D + c0;
      if constexpr (CW == 8)
        *reinterpret_cast<uint2*>(pk + P::bQ + r * D + 16 * swz_q<D>(r, ch >> 1) + 8 * (ch & 1)) =
            *reinterpret_cast<const uint2*>(src);
      else
        *reinterpret_cast<unsigned*>(pk + P::bQ + r * D + 16 * swz_q<D>(r, ch >> 2) + 4 * (ch & 3)) =
            *reinterpret_cast<const unsigned*>(src);
    }
  }

  if (a.spill) {
    // ---- K^T packet of this key block: [D][BLK] codes, chunk j of row c at slot swz<BLK>(c, j)
    unsigned kbw[NQ][4][CW / 4];
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int8_t* src = a.Kc + (tok0 + kPq * q + 4 * j + k) * D + c0;
        if constexpr (CW == 8) {
          const uint2 v = *reinterpret_cast<const uint2*>(src);
          kbw[q][k][0] = v.x; kbw[q][k][1] = v.y;
        } else {
          kbw[q][k][0] = *reinterpret_cast<const unsigned*>(src);
        }
      }
    // byte i of the thread's four tokens -> one word per channel
    auto transpose4 = [&](const unsigned* w0, const unsigned* w1, const unsigned* w2, const unsigned* w3, int i) {
      const int wi = i >> 2, sh = 8 * (i & 3);
      return ((w0[wi] >> sh) & 0xFFu) | (((w1[wi] >> sh) & 0xFFu) << 8) | (((w2[wi] >> sh) & 0xFFu) << 16) |
             (((w3[wi] >> sh) & 0xFFu) << 24);
    };
    // (the LDS tile is free: the barrier after the dO^T rows)
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int i = 0; i < CW; ++i)
        *reinterpret_cast<unsigned*>(tt + (c0 + i) * KR + kPq * q + 4 * j) =
            transpose4(kbw[q][0], kbw[q][1], kbw[q][2], kbw[q][3], i);
    __syncthreads();
    int8_t* kt = a.ktp + ((size_t)bh * nb + blk_id) * (size_t)(D * BLK);
    for (int e = tid; e < D * (BLK / 16); e += 256) {
      const int c = e / (BLK / 16), g = e % (BLK / 16);
      const int8_t* src = tt + c * KR + 16 * g;
      i32x4 v;
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const int*>(src + 4 * u);
      *reinterpret_cast<i32x4*>(kt + c * BLK + 16 * swz<BLK>(c, g)) = v;
    }
  } else {
    // zero the dQ accumulator rows of this block
    for (int e = tid; e < BLK * D / 4; e += 256)
      reinterpret_cast<float4*>(a.dq_acc + tok0 * D)[e] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// ------------------------------------------------------------------------------ bwd_main
// Workgroup = one key block of BLK keys, NW = BLK/16 waves; wave w owns keys 16w..16w+15 of
// the block (lane l: key 16w + (l & 15), lane group g = l >> 4). The query tiles are whole
// query blocks of BLK rows (one or two 64-row packets, NH = BLK/64), so the block scales of
// Q and dO are constant over a tile and the int32 products below contract over all of its
// rows at once. The products run on gfx950's 16 x 16 MFMAs. S and dP of query sub-tile t
// (rows 16t..16t+15) leave row 16t + 4g + r and this lane's key in register r, so each lane
// holds P and dS of its key for 16 rows of every packet: the B operand (columns = keys,
// contraction = queries) of dV^T = dO^T P and dK^T = Q^T dS, contraction slot 4t + r of
// lane group g standing for row 16t + 4g + r of the packet. The packets store dO^T codes in
// that order; the Q^T operands come from the row-major Q codes through transposing reads.
//   P is quantised on the wave's own TQ x 16 tile (no cross-wave step), so dV runs before
//   the one workgroup barrier of the tile, which publishes the waves' |dS| maxima (dS is
//   quantised on TQ x 64 tiles: one query block by the 64 keys of four waves). Everything
//   the tile needs from LDS is in registers before that barrier, so right after it the tile
//   buffer takes the copies of the tile two steps ahead (two tile buffers); each wave waits
//   for its own copies just before the next barrier, which publishes them.
//   dS leaves as this lane's 16 codes per packet in 16-byte stores: the spilled tiles are
//   dS^T, key-major, one per 64-row packet, with one dQ multiplier per 64 keys.
//   With Q-smoothing (QS; SageBwd article, Q-smoothing paragraph) the lane's key bias enters
//   every P exponent, and the lane sums its dS codes (v_dot4 against ones) times the tile
//   scale; the epilogue adds sm_scale * (that sum over the four lane groups) * q_mean to dK^,
//   the pages' dK_bias = (dS^T 1) mu_Q^T.
template <int D, int BLK, bool SPILL>
struct BwdLds {
  using P = Packet<D>;
  static constexpr int NW = BLK / 16;             // waves
  static constexpr int NH = BLK / kPq;            // packets per query tile
  static constexpr int kBuf = NH * P::kBytes;     // one tile buffer (two of them)
  static constexpr int kTiles = 2 * kBuf;
  static constexpr int offKT = kTiles;            // atomic mode: K^T codes [D][BLK]
  static constexpr int kBytes = SPILL ? kTiles : kTiles + D * BLK;
  static constexpr int kCopies = NH * P::kCopies; // 1 KB copies of one tile
  static constexpr int kMinBlocks = BLK == 64 ? 2 : 1;   // workgroups per CU
};

template <int DT, int D, int BLK, bool SPILL, bool QS, int FMT, bool QA>
__global__ __launch_bounds__((BwdLds<D, BLK, SPILL>::NW * 64), (BwdLds<D, BLK, SPILL>::kMinBlocks))
void bwd_main(BackwardArgs a) {
  static_assert(!(QS && QA), "Q-smoothing is not combined with the Q-Attn split");
  using L = BwdLds<D, BLK, SPILL>;
  using P = Packet<D>;
  constexpr int NW = L::NW;        // waves per workgroup
  constexpr int NH = L::NH;        // packets per query tile
  constexpr int NT = NW * 64;      // threads
  constexpr int TQ = NH * kPq;     // query rows per tile (= BLK)
  constexpr int NS = TQ / 16;      // 16-row sub-tiles of a tile
  constexpr int KCH = D / 64;      // 64-channel chunks (INT8 contraction of S)
  constexpr int HCH = D / 32;      // 32-channel chunks (16-bit contraction of dP)
  constexpr int NCT = D / 16;      // 16-channel output tiles of dV^T, dK^T and dQ
  constexpr int KD = BLK / 64;     // 64-key dS tiles of a key block
  __shared__ __attribute__((aligned(1024))) int8_t lds[L::kBytes];
  // |dS| maxima of the waves [tile parity][wave], apart from the tile buffers so that reading
  // them never waits for copies in flight into the buffers
  __shared__ float redD[2 * NW];
  __shared__ float gred[NW][D];   // (gains) the waves' partial sums of dk_gain

  const int nb = a.N / BLK;
  const int bh = blockIdx.x % a.BH;
  const int kb = blockIdx.x / a.BH;            // key block; 0 first (most work when causal)
  const int w = __builtin_amdgcn_readfirstlane(wave_id()), l = lane_id(), g = l >> 4, lr = l & 15;
  const int tid = threadIdx.x;
  const int k0 = kb * BLK;                     // first key of the block
  const int kl = 16 * w + lr;                  // this lane's key inside the block
  const int key = k0 + kl;
  const int wg0 = 4 * (w / 4);                 // first wave of this wave's 64-key dS tile
  const int dg = kl >> 6;                      // that dS tile inside the key block
  const size_t hrow = (size_t)bh * a.N;
  const int ntq = a.N / TQ;                    // query tiles
  const int8_t* pkh = a.pk + (size_t)bh * ntq * L::kBuf;    // this head's packets
  const uint32_t pkh_bytes = (uint32_t)ntq * L::kBuf;

  // ---- per-lane constant operands: K codes (B of S) and V (B of dP) of this lane's key
  i32x4 kreg[KCH];
#pragma unroll
  for (int c = 0; c < KCH; ++c) kreg[c] = *reinterpret_cast<const i32x4*>(a.Kc + (hrow + key) * D + 64 * c + 16 * g);
  u16x8 vreg[HCH];
  const bool kvalid = key < a.Nv;              // (padding keys of a ragged last block: zeros)
  const size_t krow16 = a.x16.row(bh, kvalid ? key : 0);   // this lane's key row of the 16-bit tensors
#pragma unroll
  for (int c = 0; c < HCH; ++c)
    vreg[c] = kvalid ? *reinterpret_cast<const u16x8*>(a.V + krow16 + 32 * c + 8 * g) : u16x8{};
  if constexpr (!SPILL) {
    // K^T codes of the block for dQ = dS K: [D][BLK], chunk j of row c at slot swz<BLK>(c, j)
    for (int ch = tid; ch < BLK * D / 16; ch += NT) {
      const int t = (ch * 16) / D, c = (ch * 16) % D;
      const i32x4 v = *reinterpret_cast<const i32x4*>(a.Kc + (hrow + k0 + t) * D + c);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int cc = c + i;
        lds[L::offKT + cc * BLK + 16 * swz<BLK>(cc, t / 16) + t % 16] = (int8_t)(v[i >> 2] >> (8 * (i & 3)));
      }
    }
  }
  const float sK = a.Ks[(size_t)bh * nb + kb];
  const float smc = a.sm_scale;
  // (QS) this lane's key bias in log2 units, and its running sum of dequantised dS codes
  [[maybe_unused]] const float kb2 = QS ? a.kbias[hrow + key] * (smc * kLog2e) : 0.0f;
  [[maybe_unused]] float dsum = 0.0f;

  f32x4 dk[NCT], dv[NCT];
#pragma unroll
  for (int i = 0; i < NCT; ++i) { dk[i] = f32x4{}; dv[i] = f32x4{}; }

  // per-lane byte offsets of the operands inside a packet. Rows 16t + lr share their
  // swizzle for every t, except that at d = 128 the Q rows of odd t have bit 2 of the slot
  // flipped, i.e. their 64-channel chunks swapped (swz_q); so each operand address is
  // buffer + one of these offsets + a compile-time constant. Channel chunk c of a row (16
  // bytes at slot 4c + g, swizzled) sits at the chunk-0 offset XOR 64c: the swizzles XOR the
  // slot with a function of the row alone. Buffer offsets are multiples of 1 KB, so the XOR
  // may be applied after adding them; the kernels do so in the tile loop, which keeps one
  // register per operand stream instead of one per chunk.
  const int oQ0 = P::bQ + lr * D + 16 * swz_q<D>(lr, g);
  const int oDO0 = P::bDO + lr * 2 * D + 16 * swz_do<D>(lr, g);
  const int oT = P::bDOT + lr * kPq + 16 * swz<kPq>(lr, g);   // dO^T codes, channel 16n + lr
  // Q^T operands by transposing reads of the row-major Q codes: for channel tile n, lane
  // 16g + 2i + h names 8 bytes (channels 16n + 8h ..) of packet row 16(i/4) + 4g + i%4 (and
  // of that row + 32 for the second read), so lane 16g + m receives channel 16n + m of the
  // eight rows standing for contraction slots 16g .. 16g+7 (then 16g+8 .. 16g+15). Rows are
  // D >= 64 bytes with the 16-byte chunks XOR-swizzled, and buffers start on 1 KB
  // boundaries, so chunk n of the row is this offset XOR 16n.
  const int oQT = [&] {
    const int i = lr >> 1, row = 16 * (i >> 2) + 4 * g + (i & 3);
    return P::bQ + row * D + 16 * swz_q<D>(row, 0) + 8 * (l & 1);
  }();

  // copies of query tile qt into a tile buffer: wave w moves KB cp = w, w + NW, ...
  auto issue = [&](int qt, int8_t* dst) {
    constexpr int kFull = L::kCopies / NW, kRest = L::kCopies % NW;
#pragma unroll
    for (int j = 0; j < kFull; ++j) {
      const int cp = w + NW * j;
      buffer_to_lds16(pkh, pkh_bytes, dst + cp * 1024, 16 * l, qt * L::kBuf + cp * 1024);
    }
    if constexpr (kRest > 0) {
      const int cp = w + NW * kFull;
      if (w < kRest) buffer_to_lds16(pkh, pkh_bytes, dst + cp * 1024, 16 * l, qt * L::kBuf + cp * 1024);
    }
  };
  // vector-memory operations a wave issues per step after the step's copies: the dS^T
  // stores and dQ multipliers (spill), or the dQ atomics
  constexpr int kStores = SPILL ? 2 * NH : NCT * 4;

  const int qt0 = a.causal ? kb : 0;           // first query tile at or below the diagonal

  // ---- the phases of one query tile; state carried between them (registers)
  float sQ = 0.0f, sdO = 0.0f, c2 = 0.0f;
  using C = Codes<FMT>;
  typename C::acc4 s[NS];
  f32x4 dp[NS];
  float dsf[NS][4];
  i32x4 qtr[NH][NCT];
  i32x4 dc[NH];
  // FP8 with two 64-row halves: the Q^T operands and dS codes of both halves as one 32-byte
  // operand per lane, so dK takes one K = 128 product without operand copies. (dV keeps two
  // K = 32 products per half, and so does dK in the atomic dQ mode: 32-byte operands there
  // push the kernel past 256 registers.)
  constexpr bool P8 = FMT == FMT_FP8 && NH == 2 && SPILL;
  [[maybe_unused]] i32x8 qtr8[NCT];
  [[maybe_unused]] i32x8 dc8;
  auto dch = [&](int h) -> i32x4 {
    if constexpr (P8) return i32x4{dc8[4 * h], dc8[4 * h + 1], dc8[4 * h + 2], dc8[4 * h + 3]};
    else return dc[h];
  };

  // S = Q K~^T and dP = dO V^T for the 16-row sub-tiles of the tile at byte offset bofs
  // (LLVM's interleaving strategy 1 for this block: measured 1.7-2.6% faster than the
  // default schedule)
  auto phase_sdp = [&](int bofs) {
    // uniform values, kept in scalar registers
    sQ = uniform_f(*reinterpret_cast<const float*>(lds + bofs + P::bSQ));
    sdO = uniform_f(*reinterpret_cast<const float*>(lds + bofs + P::bSDO));
    c2 = uniform_f((sQ * sK) * (smc * kLog2e));
    const int qb = bofs + oQ0, db = bofs + oDO0;
    __builtin_amdgcn_iglp_opt(1);
#pragma unroll
    for (int t = 0; t < NS; ++t) {
      const int8_t* pb = lds + (t / 4) * P::kBytes;
      s[t] = typename C::acc4{};
      auto aq = [&](int c) {
        const int cq = D == 128 ? c ^ (t & 1) : c;   // (t % 4) & 1 == t & 1
        return *reinterpret_cast<const i32x4*>(pb + (qb ^ (64 * cq)) + 16 * (t % 4) * D);
      };
      if constexpr (FMT == FMT_FP8 && KCH == 2) {
        s[t] = C::mma16x2(aq(0), aq(1), kreg[0], kreg[1], s[t]);
      } else {
#pragma unroll
        for (int c = 0; c < KCH; ++c) s[t] = C::mma16(aq(c), kreg[c], s[t]);
      }
      dp[t] = f32x4{};
#pragma unroll
      for (int c = 0; c < HCH; ++c) {
        const u16x8 ad = *reinterpret_cast<const u16x8*>(pb + (db ^ (64 * c)) + 32 * (t % 4) * D);
        dp[t] = mfma_16b_16x16x32<DT>(ad, vreg[c], dp[t]);
      }
    }
  };

  // P = 2^(S c - lse2), dS = P (dP - D) of sub-tile t: register r is row 16t + 4g + r
  float pf[NS][4];
  auto elem_tile = [&](const int8_t* buf, int t, int q0, auto masked) {
    const int8_t* pb = buf + (t / 4) * P::kBytes;
    const f32x4 lse2 = *reinterpret_cast<const f32x4*>(pb + P::bLSE + 4 * (16 * (t % 4) + 4 * g));
    const f32x4 dvv = *reinterpret_cast<const f32x4*>(pb + P::bDV + 4 * (16 * (t % 4) + 4 * g));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float p = __builtin_amdgcn_exp2f(__builtin_fmaf((float)s[t][r], c2, QS ? kb2 - lse2[r] : -lse2[r]));
      if constexpr (decltype(masked)::value) {
        if ((a.causal && key > q0 + 16 * t + 4 * g + r) || !kvalid) p = 0.0f;
      }
      pf[t][r] = p;
      dsf[t][r] = p * (dp[t][r] - dvv[r]);
    }
  };

  // the tile maxima (|dS| maximum to the workgroup), P codes and dV, and the Q^T operands of
  // dK: every remaining read of the tile's buffer. With the Q-Attn split (QA) P is not
  // quantised: dV^T += dO^T P runs in 16 bits, P rounded to the dtype as the B operand
  // (slots 4t' + r of lane group g: rows 16t + 4g + r of sub-tiles t = 2u, 2u + 1) and dO^T
  // as the A operand by transposing reads of the packet's row-major dO (four rows 16t + 4g ..
  // + 3 per read, channels 16n .. 16n + 15).
  auto phase_post = [&](int bofs, int step) {
    const int8_t* buf = lds + bofs;
    if constexpr (QA) {
      float dm = fabsf(dsf[0][0]);
#pragma unroll
      for (int i = 1; i < 4 * NS; i += 2)
        dm = fmaxf(fmaxf(dm, fabsf(dsf[i / 4][i % 4])), i + 1 < 4 * NS ? fabsf(dsf[(i + 1) / 4][(i + 1) % 4]) : 0.0f);
      dm = wave_max_nonneg(dm);
      if (l == 0) redD[(step & 1) * NW + w] = dm;
      const int jl = l & 15, kr = jl >> 2, qq = jl & 3;
      // P as 16-bit B operands first (the float P registers are then free)
      u16x8 bp[NS / 2];
#pragma unroll
      for (int u = 0; u < NS / 2; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          bp[u][r] = from_f32<DT>(pf[2 * u][r]);
          bp[u][4 + r] = from_f32<DT>(pf[2 * u + 1][r]);
        }
#pragma unroll
      for (int n = 0; n < NCT; ++n) {
        const int ch = 2 * n + (qq >> 1);
        auto rd = [&](int t) {
          const int row = 16 * (t % 4) + 4 * g + kr;   // row of packet t / 4
          return lds_read_tr16(buf + (t / 4) * P::kBytes + P::bDO + row * 2 * D + 16 * swz_do<D>(row, ch) +
                               8 * (qq & 1));
        };
#pragma unroll
        for (int u = 0; u < NS / 2; ++u) {
          const u16x4 a0 = rd(2 * u), a1 = rd(2 * u + 1);
          const u16x8 ad = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
          dv[n] = mfma_16b_16x16x32<DT>(ad, bp[u], dv[n]);
        }
      }
    } else {
    // ---- tile maxima (chains of three-input maxima; the |dS| maximum goes to the workgroup)
    float pm = pf[0][0], dm = fabsf(dsf[0][0]);
#pragma unroll
    for (int i = 1; i < 4 * NS; i += 2) {
      const int t0 = i / 4, r0 = i % 4, t1 = (i + 1) / 4, r1 = (i + 1) % 4;
      pm = fmaxf(fmaxf(pm, pf[t0][r0]), i + 1 < 4 * NS ? pf[t1][r1] : 0.0f);
      dm = fmaxf(fmaxf(dm, fabsf(dsf[t0][r0])), i + 1 < 4 * NS ? fabsf(dsf[t1][r1]) : 0.0f);
    }
    wave_max2_nonneg(pm, dm);
    if (l == 0) redD[(step & 1) * NW + w] = dm;

    // ---- P codes on this wave's TQ x 16 tile, then dV^T += dO^T P (int32 over the TQ rows)
    {
      const float pa = fmaxf(pm, FLT_MIN);
      // (an all-zero tile, e.g. 16 padding keys: kMax / FLT_MIN overflows to +inf and 0 * inf
      // would make NaN codes, which FP8 products carry on; the clamp keeps 0 * pinv = 0 and
      // |x| * pinv <= kMax)
      const float pinv = fminf(C::kMax * __builtin_amdgcn_rcpf(pa), FLT_MAX);
      const float sv = pa * (1.0f / C::kMax) * sdO;
      i32x4 pc[NH];
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float* v = pf[4 * h + t];
          pc[h][t] = (int)tile_code_word<FMT>(v[0], v[1], v[2], v[3], pinv);
        }
#pragma unroll
      for (int n = 0; n < NCT; ++n) {
        typename C::acc4 acc{};
        auto ao = [&](int h) { return *reinterpret_cast<const i32x4*>(buf + h * P::kBytes + oT + 16 * n * kPq); };
#pragma unroll
        for (int h = 0; h < NH; ++h) acc = C::mma16(ao(h), pc[h], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) dv[n][r] = __builtin_fmaf(sv, (float)acc[r], dv[n][r]);
      }
    }
    }
    // ---- Q^T operands of dK (after the next barrier the buffer is refilled)
    const int qa = bofs + oQT;
#pragma unroll
    for (int n = 0; n < NCT; ++n) {
      const int8_t* pn = lds + (qa ^ (16 * n));
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const i32x2 x0 = lds_read_tr8(pn + h * P::kBytes);
        const i32x2 x1 = lds_read_tr8(pn + h * P::kBytes + 32 * D);
        if constexpr (P8) {
          qtr8[n][4 * h] = x0[0]; qtr8[n][4 * h + 1] = x0[1]; qtr8[n][4 * h + 2] = x1[0]; qtr8[n][4 * h + 3] = x1[1];
        } else {
          qtr[h][n] = i32x4{x0[0], x0[1], x1[0], x1[1]};
        }
      }
    }
  };

  // dS codes on the TQ x 64 tile of this wave's four-wave group (its |dS| maxima published
  // by the barrier after phase_post), dK^T += Q^T dS, and the spilled dS^T tile
  auto phase_dk = [&](int step, int qt) {
    float da = redD[(step & 1) * NW + wg0];
#pragma unroll
    for (int i = 1; i < 4; ++i) da = fmaxf(da, redD[(step & 1) * NW + wg0 + i]);
    da = fmaxf(da, FLT_MIN);
    // (clamped as pinv above: an all-zero dS tile, e.g. 64 padding keys of a ragged block,
    // must give codes 0, not 0 * inf = NaN)
    const float dinv = fminf(C::kMax * __builtin_amdgcn_rcpf(da), FLT_MAX);
    const float sdS = da * (1.0f / C::kMax);
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float* v = dsf[4 * h + t];
        const int wd = (int)tile_code_word<FMT>(v[0], v[1], v[2], v[3], dinv);
        if constexpr (P8) dc8[4 * h + t] = wd;
        else dc[h][t] = wd;
      }
    if constexpr (QS) {
      static_assert(FMT == FMT_INT8, "Q-smoothing sums INT8 codes");
      int isum = 0;
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int t = 0; t < 4; ++t) isum = __builtin_amdgcn_sdot4(dc[h][t], 0x01010101, isum, false);
      dsum = __builtin_fmaf(sdS, (float)isum, dsum);
    }
    {
      const float sk = smc * sdS * sQ;
#pragma unroll
      for (int n = 0; n < NCT; ++n) {
        typename C::acc4 acc{};
        if constexpr (P8) {
          acc = C::mma16w(qtr8[n], dc8, acc);
        } else {
#pragma unroll
          for (int h = 0; h < NH; ++h) acc = C::mma16(qtr[h][n], dc[h], acc);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) dk[n][r] = __builtin_fmaf(sk, (float)acc[r], dk[n][r]);
      }
    }
    if constexpr (SPILL) {
      // the dS^T tile of each packet [BLK][64] for the query-major dQ pass: key row kl,
      // chunk g (rows in the contraction order above) at slot swz_ds(kl, g); and the dQ
      // multiplier of its 64 keys (the same for the tile's packets)
      const long long ti = (long long)bh * a.spill_tiles + spill_tile_index(a.N, BLK, a.causal, kb, qt * NH);
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        // (non-temporal: the spill is read once, by the dQ pass, and must not push the packets,
        // which every key block reads again, out of L2)
        __builtin_nontemporal_store(dch(h), reinterpret_cast<i32x4*>(a.dsp + (ti + h) * (kPq * BLK) + kl * kPq +
                                                                      16 * swz_ds(kl, g)));
        if (l == 0) a.dsm[(ti + h) * KD + dg] = smc * sdS * sK;   // every wave of the group stores the same value
      }
    }
  };

  {
    issue(qt0, lds);
    if (qt0 + 1 < ntq) issue(qt0 + 1, lds + L::kBuf);
    wait_vmcnt<0>();
    __syncthreads();
    for (int qt = qt0; qt < ntq; ++qt) {
      const int q0 = qt * TQ;
      const int step = qt - qt0;
      const int bofs = (step & 1) * L::kBuf;   // byte offset of this tile's buffer
      // Issue priority: waves w and w + 4 share a SIMD, and without priorities the older one
      // leads every phase, then waits at the barrier while the younger one finishes alone.
      // The younger four lead S/dP, the elementwise work and dK; the older ones lead the
      // phase before the barrier (B2 H16 N8192 d128: 1.050/1.052 -> 1.036/1.035 ms).
      if (w >= 4) __builtin_amdgcn_s_setprio(2);
      phase_sdp(bofs);
      // diagonal tiles mask keys above the queries; the waves holding padding keys mask those
      if ((a.causal && k0 + 16 * w + 15 > q0) || k0 + 16 * w + 15 >= a.Nv) {
#pragma unroll
        for (int t = 0; t < NS; ++t) elem_tile(lds + bofs, t, q0, std::true_type{});
      } else {
#pragma unroll
        for (int t = 0; t < NS; ++t) elem_tile(lds + bofs, t, q0, std::false_type{});
      }
      if (w >= 4) __builtin_amdgcn_s_setprio(0);
      phase_post(bofs, step);
      // the copies of tile qt+1 (issued one step ago) must have landed before the barrier
      // that publishes them; issued after them: last step's stores or atomics
      wait_vmcnt<kStores>();
      lds_barrier();
      if (w >= 4) __builtin_amdgcn_s_setprio(2);
      if constexpr (SPILL) {
        if (qt + 2 < ntq) issue(qt + 2, lds + bofs);
      }
      phase_dk(step, qt);
      if constexpr (!SPILL) {
        // ---- dQ = dS K on the TQ x BLK tile, added to the float32 accumulator with atomics.
        //      The dS^T tile [BLK][TQ] goes through the released tile buffer once (chunk
        //      4h + g of key row kl at slot swz<TQ>(kl, 4h + g)) and is read back query by
        //      query (transposing reads); wave w computes query chunk w against all
        //      channels, one 64-key dS tile (one scale) at a time.
        int8_t* dst = lds + bofs;
#pragma unroll
        for (int h = 0; h < NH; ++h)
          *reinterpret_cast<i32x4*>(dst + kl * TQ + 16 * swz<TQ>(kl, 4 * h + g)) = dch(h);
        // the scale of every 64-key dS tile of the block
        float sc[KD];
#pragma unroll
        for (int kc = 0; kc < KD; ++kc) {
          float m = redD[(step & 1) * NW + 4 * kc];
#pragma unroll
          for (int i = 1; i < 4; ++i) m = fmaxf(m, redD[(step & 1) * NW + 4 * kc + i]);
          sc[kc] = smc * (fmaxf(m, FLT_MIN) * (1.0f / C::kMax)) * sK;
        }
        lds_barrier();
        f32x4 accf[NCT];
#pragma unroll
        for (int n = 0; n < NCT; ++n) accf[n] = f32x4{};
#pragma unroll
        for (int kc = 0; kc < KD; ++kc) {
          const int i = lr >> 1, hh = l & 1;
          const int r0 = 64 * kc + 16 * g + i, r1 = r0 + 8;
          const i32x2 x0 = lds_read_tr8(dst + r0 * TQ + 16 * swz<TQ>(r0, w) + 8 * hh);
          const i32x2 x1 = lds_read_tr8(dst + r1 * TQ + 16 * swz<TQ>(r1, w) + 8 * hh);
          const i32x4 as = {x0[0], x0[1], x1[0], x1[1]};
#pragma unroll
          for (int n = 0; n < NCT; ++n) {
            const int c = 16 * n + lr;
            const i32x4 bk = *reinterpret_cast<const i32x4*>(lds + L::offKT + c * BLK + 16 * swz<BLK>(c, 4 * kc + g));
            const auto acc = C::mma16(as, bk, typename C::acc4{});
#pragma unroll
            for (int r = 0; r < 4; ++r) accf[n][r] = __builtin_fmaf(sc[kc], (float)acc[r], accf[n][r]);
          }
        }
        // every wave has read the staged tile: the buffer takes the tile two steps ahead
        lds_barrier();
        if (qt + 2 < ntq) issue(qt + 2, lds + bofs);
        // result: query chunk w = 4h' + u of the tile, position 4g + r = row 16g + 4u + r of
        // packet h'
        const int qrow = q0 + kPq * (w / 4) + 16 * g + 4 * (w % 4);
#pragma unroll
        for (int n = 0; n < NCT; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            unsafeAtomicAdd(a.dq_acc + (hrow + qrow + r) * D + 16 * n + lr, accf[n][r]);
      }
    }
  }

  // ---- epilogue: dV and dK (RMSNorm backward with K^ = K * rstd) for this lane's key;
  //      lane group g holds channels 16n + 4g + r
  if constexpr (QS) {
    // dK_bias: the key's dS sum over all its query rows (the four lane groups hold the rows)
    dsum += __shfl_xor(dsum, 16);
    dsum += __shfl_xor(dsum, 32);
    const float* qm = a.q_mean + (size_t)bh * D;
#pragma unroll
    for (int n = 0; n < NCT; ++n) {
      const f32x4 mq = *reinterpret_cast<const f32x4*>(qm + 16 * n + 4 * g);
#pragma unroll
      for (int r = 0; r < 4; ++r) dk[n][r] = __builtin_fmaf(smc * dsum, mq[r], dk[n][r]);
    }
  }
  unsigned short* dvrow = a.dV + krow16;
  if (kvalid) {
#pragma unroll
    for (int n = 0; n < NCT; ++n) {
      u16x4 v;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = from_f32<DT>(dv[n][r]);
      *reinterpret_cast<u16x4*>(dvrow + 16 * n + 4 * g) = v;
    }
  }
  unsigned short* dkrow = a.dK + krow16;
  if (a.qk_norm) {
    // K^ = g o n with n = K * rstd: dn = g o dK^, dK = rstd * (dn - n * mean_c(dn o n)), and
    // the gain's gradient collects dK^ o n over the keys (g = 1 without gains)
    const float rs = a.k_rstd[hrow + key];
    const unsigned short* krow = a.K + krow16;
    const float* gain = a.k_gain ? a.k_gain + (size_t)(bh % a.x16.H) * D : nullptr;
    float kh[NCT][4];
    float dot = 0.0f;
#pragma unroll
    for (int n = 0; n < NCT; ++n) {
      const u16x4 kv = kvalid ? *reinterpret_cast<const u16x4*>(krow + 16 * n + 4 * g) : u16x4{};
      f32x4 gv = {1.0f, 1.0f, 1.0f, 1.0f};
      if (gain) gv = *reinterpret_cast<const f32x4*>(gain + 16 * n + 4 * g);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        kh[n][r] = to_f32<DT>(kv[r]) * rs;
        if (gain) {
          const float u = dk[n][r];
          dk[n][r] = u * gv[r];
          dv[n][r] = u * kh[n][r];   // dv is stored: its registers carry the gain products
        }
        dot = __builtin_fmaf(dk[n][r], kh[n][r], dot);
      }
    }
    dot += __shfl_xor(dot, 16);
    dot += __shfl_xor(dot, 32);
    const float mean = dot / (float)D;
#pragma unroll
    for (int n = 0; n < NCT; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) dk[n][r] = rs * (dk[n][r] - kh[n][r] * mean);
    if (gain) {
      // this key block's partial of dk_gain: over the wave's 16 keys (a DPP row sum), then over
      // the waves in order
#pragma unroll
      for (int n = 0; n < NCT; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float t = row_sum16(dv[n][r]);
          if (lr == 0) gred[w][16 * n + 4 * g + r] = t;
        }
      __syncthreads();
      if (tid < D) {
        float t = gred[0][tid];
#pragma unroll
        for (int i = 1; i < NW; ++i) t += gred[i][tid];
        a.gk_part[((size_t)bh * nb + kb) * D + tid] = t;
      }
    }
  }
  if (kvalid) {
#pragma unroll
    for (int n = 0; n < NCT; ++n) {
      u16x4 v;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = from_f32<DT>(dk[n][r]);
      *reinterpret_cast<u16x4*>(dkrow + 16 * n + 4 * g) = v;
    }
  }
}

// ------------------------------------------------------------------------------ dQ epilogue
// Rows [r0, r1) of one 64-query tile of dQ^ (query rows q0 + r, q0 = 64 qt, of head bh):
// RMSNorm backward with the gain (Q^ = g o n, n = Q * rstd: dn = g o dQ^, dQ = rstd * (dn -
// n * mean_c(dn o n)), g = 1 without gains), rounding to the dtype, and with gains each
// thread's share of the tile's dq_gain partial (dQ^ o n) added into gp[8]. 256 threads; D/8
// lanes per row, 8 channels each, so EPI_ROWS = 256 / (D/8) rows per round; row(r, c, v) fills
// v[0..7] with dQ^ of tile row r, channels c .. c + 7. r0 and r1 are multiples of EPI_ROWS.
template <int D>
constexpr int kEpiRows = 256 / (D / 8);

template <int DT, int D, typename RowF>
__device__ __forceinline__ void dq_epilogue_rows(const BackwardArgs& a, int bh, int qt, int r0, int r1, RowF&& row,
                                                 float* gp) {
  constexpr int CPR = D / 8;                        // lanes per row
  const size_t hrow = (size_t)bh * a.N;
  const int q0 = qt * kPq;
  const int c = (threadIdx.x % CPR) * 8;
  const float* gain = (a.qk_norm && a.q_gain) ? a.q_gain + (size_t)(bh % a.x16.H) * D + c : nullptr;
  float gv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) gv[i] = gain ? gain[i] : 1.0f;
  for (int r = r0 + (int)threadIdx.x / CPR; r < r1; r += kEpiRows<D>) {
    if (q0 + r >= a.Nv) break;   // padding rows of a ragged last block (and every later row)
    const size_t tok = hrow + q0 + r;
    const size_t row16 = a.x16.row(bh, q0 + r);
    float v[8];
    row(r, c, v);
    u16x8 out;
    if (a.qk_norm) {
      const float rs = a.q_rstd[tok];
      const u16x8 qv = *reinterpret_cast<const u16x8*>(a.Q + row16 + c);
      float qh[8], dot = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        qh[i] = to_f32<DT>(qv[i]) * rs;
        if (gain) {
          gp[i] = __builtin_fmaf(v[i], qh[i], gp[i]);
          v[i] = v[i] * gv[i];
        }
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
    *reinterpret_cast<u16x8*>(a.dQ + row16 + c) = out;
  }
}

// (gains) The tile's dq_gain partial from the threads' gp: summed over the threads of each
// channel in a fixed order through gred (kEpiRows * D floats of LDS the caller no longer
// needs), written to gq_part. Every thread of the workgroup calls it.
template <int D>
__device__ __forceinline__ void dq_gain_partial(const BackwardArgs& a, int bh, int qt, const float* gp, float* gred) {
  constexpr int CPR = D / 8;
  const int c = (threadIdx.x % CPR) * 8;
  __syncthreads();   // every row has been read: gred may overlap the rows' source
#pragma unroll
  for (int i = 0; i < 8; ++i) gred[(threadIdx.x / CPR) * D + c + i] = gp[i];
  __syncthreads();
  if (threadIdx.x < D) {
    float t = gred[threadIdx.x];
    for (int i = 1; i < kEpiRows<D>; ++i) t += gred[i * D + threadIdx.x];
    a.gq_part[((size_t)bh * (a.N / kPq) + qt) * D + threadIdx.x] = t;
  }
}

// ------------------------------------------------------------------------------ bwd_dq
// Query-major dQ pass over the spilled dS^T tiles: one workgroup (4 waves) per (head, 64-query
// tile). For every key block up to the diagonal and each of its 64-key dS tiles,
// dQ^ += m * (dS_codes . K_codes) runs on v_mfma_i32_16x16x64_i8 with float32 accumulation in
// registers (m = sm_scale * s_dS * s_K of that 64-key tile). The tile's dS^T codes [BLK][64]
// stream through a ring of three LDS buffers (buffer->LDS copies issued two key blocks ahead,
// non-temporal, so that the stream leaves the K^T codes in L2) and are read back query-major with
// transposing reads: the A operand (rows = queries, contraction = keys). Wave w computes all
// 64 queries against its own NPW 16-channel tiles, so it needs only those channels of the
// block's K^T codes (the B operand), which it loads straight into registers one key block
// ahead (they come from L2). Positions follow the spilled order (position 16g + 4t + r is
// query 16t + 4g + r). The epilogue applies the RMSNorm backward and writes dQ in the dtype;
// no float32 dQ buffer and no atomics.
template <int D, int BLK>
struct DqLds {
  static constexpr int kTile = kPq * BLK;           // one dS^T tile [BLK][64]
  static constexpr int bM = kTile;                  // then its dQ multipliers (one per 64 keys)
  static constexpr int kBuf = kTile + 1024;         // one ring slot
  static constexpr int kCopiesPerWave = kTile / 1024 / 4;
  // slot 0 also stages the epilogue's dQ^ rows, kEpiRows<D> at a time [kEpiRows][D] f32 (and
  // the gain partials' reduction of the same size)
  static constexpr int kEpi = kEpiRows<D> * D * 4;
  static constexpr int kBytes0 = kBuf > kEpi ? kBuf : kEpi;
};

template <int DT, int D, int BLK, int FMT>
__global__ __launch_bounds__(256) void bwd_dq(BackwardArgs a) {
  using C = Codes<FMT>;
  using L = DqLds<D, BLK>;
  constexpr int NCT = D / 16;                       // 16-channel tiles of dQ
  constexpr int NPW = NCT / 4;                      // ... per wave
  constexpr int KC = BLK / 64;                      // 64-key chunks of a block
  constexpr int CPW = L::kCopiesPerWave;
  // The three ring slots are distinct LDS objects, so the compiler sees that the reads of one
  // slot never alias the copies in flight into another (and inserts no wait for them).
  __shared__ __attribute__((aligned(1024))) int8_t slot0[L::kBytes0];
  __shared__ __attribute__((aligned(1024))) int8_t slot1[L::kBuf];
  __shared__ __attribute__((aligned(1024))) int8_t slot2[L::kBuf];
  const int ntile = a.N / kPq, nb = a.N / BLK;
  const int bh = blockIdx.x % a.BH;
  const int qt = a.causal ? ntile - 1 - (int)(blockIdx.x / a.BH) : (int)(blockIdx.x / a.BH);
  const int q0 = qt * kPq;
  const int w = __builtin_amdgcn_readfirstlane(wave_id()), l = lane_id(), g = l >> 4, lr = l & 15;
  const int kb_last = a.causal ? (q0 + kPq - 1) / BLK : nb - 1;
  const int8_t* dsh = a.dsp + (size_t)bh * a.spill_tiles * (kPq * BLK);
  const uint32_t dsh_bytes = (uint32_t)(a.spill_tiles * (kPq * BLK));
  const float* dmh = a.dsm + (size_t)bh * a.spill_tiles * KC;
  const int8_t* kth = a.ktp + (size_t)bh * nb * (D * BLK);
  auto slot = [&](auto s_c) -> int8_t* {
    constexpr int S = decltype(s_c)::value;
    if constexpr (S == 0) return slot0;
    else if constexpr (S == 1) return slot1;
    else return slot2;
  };

  // this wave's share of the copies of key block kb's dS^T tile (and, by wave 3, of its
  // multipliers) into ring slot S
  auto issue_ds = [&](int kb, auto s_c) {
    const long long ti = spill_tile_index(a.N, BLK, a.causal, kb, qt);
    int8_t* dst = slot(s_c);
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      const int cp = w + 4 * j;
      buffer_to_lds16<kCpolNT>(dsh, dsh_bytes, dst + cp * 1024, 16 * l, (uint32_t)(ti * (kPq * BLK)) + cp * 1024);
    }
    if (w == 3) buffer_to_lds4(dmh, (uint32_t)(a.spill_tiles * 4 * KC), dst + L::bM, 4 * l, (uint32_t)(ti * 4 * KC));
  };
  // K^T operands of key block kb: channel c = 16(NPW w + n) + lr, keys 64kc + 16g .. +15
  // (chunk 4kc + g of row c, at slot swz<BLK>(c, 4kc + g))
  i32x4 kt_next[NPW][KC];
  auto load_kt = [&](int kb) {
    const int8_t* kbp = kth + (size_t)kb * (D * BLK);
#pragma unroll
    for (int n = 0; n < NPW; ++n)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const int c = 16 * (NPW * w + n) + lr;
        kt_next[n][kc] = *reinterpret_cast<const i32x4*>(kbp + c * BLK + 16 * swz<BLK>(c, 4 * kc + g));
      }
  };

  f32x4 dq[4][NPW];
#pragma unroll
  for (int qs = 0; qs < 4; ++qs)
#pragma unroll
    for (int n = 0; n < NPW; ++n) dq[qs][n] = f32x4{};

  // One key block, in ring slot S. Issue order per block: K^T of the next block, then the
  // copies of the block two ahead, so when a block's operands are awaited only the next
  // block's copies were issued after them (vector-memory operations complete in order). Past
  // the last block the same operations are issued for the last block again (into the freed
  // slot, never read), which keeps that count fixed. The barrier publishes the block's tile
  // and frees the slot of the previous block for the block two ahead.
  auto step = [&](int kb, auto s_c) {
    constexpr int S = decltype(s_c)::value;
    if (w == 3) wait_vmcnt<CPW + 1>();
    else wait_vmcnt<CPW>();
    lds_barrier();
    i32x4 kt[NPW][KC];
#pragma unroll
    for (int n = 0; n < NPW; ++n)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) kt[n][kc] = kt_next[n][kc];
    load_kt(min(kb + 1, kb_last));
    issue_ds(min(kb + 2, kb_last), std::integral_constant<int, (S + 2) % 3>{});
    const int8_t* buf = slot(s_c);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const float m = reinterpret_cast<const float*>(buf + L::bM)[kc];
      // A: keys 64kc + 16g .. +15 of query position 16qs + lr, two transposing reads of 8 keys
      const int i = lr >> 1, hh = l & 1;
      const int r0 = 64 * kc + 16 * g + i, r1 = r0 + 8;
#pragma unroll
      for (int qs = 0; qs < 4; ++qs) {
        const i32x2 x0 = lds_read_tr8(buf + r0 * kPq + 16 * swz_ds(r0, qs) + 8 * hh);
        const i32x2 x1 = lds_read_tr8(buf + r1 * kPq + 16 * swz_ds(r1, qs) + 8 * hh);
        const i32x4 as = {x0[0], x0[1], x1[0], x1[1]};
#pragma unroll
        for (int n = 0; n < NPW; ++n) {
          const auto acc = C::mma16(as, kt[n][kc], typename C::acc4{});
#pragma unroll
          for (int r = 0; r < 4; ++r) dq[qs][n][r] = __builtin_fmaf(m, (float)acc[r], dq[qs][n][r]);
        }
      }
    }
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  issue_ds(0, S0{});
  load_kt(0);
  issue_ds(min(1, kb_last), S1{});
  for (int kb = 0; kb <= kb_last; kb += 3) {
    step(kb, S0{});
    if (kb + 1 <= kb_last) step(kb + 1, S1{});
    if (kb + 2 <= kb_last) step(kb + 2, S2{});
  }
  // every wave is done with the ring (and every copy has landed) before slot 0 takes the tile
  wait_vmcnt<0>();
  lds_barrier();

  // ---- epilogue: the dQ^ rows go through slot 0 kEpiRows at a time (lane group g holds rows
  //      16g + 4qs + r), then the RMSNorm backward row by row
  constexpr int ER = kEpiRows<D>;
  float* t = reinterpret_cast<float*>(slot0);
  float gp[8] = {};
#pragma unroll
  for (int p = 0; p < kPq / ER; ++p) {
    if (16 * g >= p * ER && 16 * g < (p + 1) * ER) {
#pragma unroll
      for (int qs = 0; qs < 4; ++qs)
#pragma unroll
        for (int n = 0; n < NPW; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r) t[(16 * g + 4 * qs + r - p * ER) * D + 16 * (NPW * w + n) + lr] = dq[qs][n][r];
    }
    __syncthreads();
    dq_epilogue_rows<DT, D>(a, bh, qt, p * ER, (p + 1) * ER, [&](int r, int c, float* v) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = t[(r - p * ER) * D + c + i];
    }, gp);
    __syncthreads();
  }
  if (a.qk_norm && a.q_gain) dq_gain_partial<D>(a, bh, qt, gp, t);
}

// ------------------------------------------------------------------------------ dq_finalize
// (atomic mode) One workgroup per (head, 64-query tile): the tile epilogue over the float32
// dQ^ accumulator rows.
template <int DT, int D>
__global__ __launch_bounds__(256) void dq_finalize(BackwardArgs a) {
  const int ntile = a.N / kPq;
  const int bh = blockIdx.x / ntile, qt = blockIdx.x % ntile;
  __shared__ float gred[kEpiRows<D> * D];
  const float* src = a.dq_acc + ((size_t)bh * a.N + (size_t)qt * kPq) * D;
  float gp[8] = {};
  dq_epilogue_rows<DT, D>(a, bh, qt, 0, kPq, [&](int r, int c, float* v) {
    *reinterpret_cast<float4*>(v) = *reinterpret_cast<const float4*>(src + (size_t)r * D + c);
    *reinterpret_cast<float4*>(v + 4) = *reinterpret_cast<const float4*>(src + (size_t)r * D + c + 4);
  }, gp);
  if (a.qk_norm && a.q_gain) dq_gain_partial<D>(a, bh, qt, gp, gred);
}

// ------------------------------------------------------------------------------ gain_reduce
// (gains) dq_gain[h] and dk_gain[h] (blockIdx.y = 0, 1): the per-tile partials of every batch
// entry of head h summed in a fixed order (batch, then tile).
template <int D>
__global__ __launch_bounds__(128) void gain_reduce(BackwardArgs a) {
  const int h = blockIdx.x, H = a.x16.H, B = a.BH / H;
  const bool is_q = blockIdx.y == 0;
  const int T = is_q ? a.N / kPq : a.N / a.BLK;
  const float* part = is_q ? a.gq_part : a.gk_part;
  float* out = is_q ? a.dq_gain : a.dk_gain;
  for (int c = threadIdx.x; c < D; c += 128) {
    float acc = 0.0f;
    for (int b = 0; b < B; ++b) {
      const float* pb = part + (size_t)(b * H + h) * T * D + c;
      for (int t = 0; t < T; ++t) acc += pb[(size_t)t * D];
    }
    out[(size_t)h * D + c] = acc;
  }
}

template <int DT, int D, int BLK>
static hipError_t launch_backward_t(const BackwardArgs& a, int part, hipStream_t st) {
  const long long nb = a.N / BLK;
  if (part < 0 || part == 0) {
    const hipError_t e = launch_kernel(&bwd_pre<DT, D, BLK>, dim3((unsigned)(nb * a.BH)), dim3(256), st, a);
    if (e != hipSuccess) return e;
  }
  if (part < 0 || part == 1) {
    auto go = [&](auto spill_c, auto qs_c, auto fmt_c, auto qa_c) {
      constexpr bool SP = decltype(spill_c)::value, QSV = decltype(qs_c)::value, QAV = decltype(qa_c)::value;
      constexpr int FM = decltype(fmt_c)::value;
      using L = BwdLds<D, BLK, SP>;
      return launch_kernel(&bwd_main<DT, D, BLK, SP, QSV, FM, QAV>, dim3((unsigned)(nb * a.BH)), dim3(L::NW * 64),
                           st, a);
    };
    using T = std::true_type;
    using F = std::false_type;
    using I8 = std::integral_constant<int, FMT_INT8>;
    using F8 = std::integral_constant<int, FMT_FP8>;
    hipError_t e;
    // (Q-smoothing takes INT8 codes and the SageBwd split only; the API refuses the others)
    if (a.q_smooth && (a.fmt != FMT_INT8 || a.qattn)) return hipErrorInvalidValue;
    if (a.qattn) {
      if (a.fmt == FMT_FP8) e = a.spill ? go(T{}, F{}, F8{}, T{}) : go(F{}, F{}, F8{}, T{});
      else e = a.spill ? go(T{}, F{}, I8{}, T{}) : go(F{}, F{}, I8{}, T{});
    } else if (a.fmt == FMT_FP8) {
      e = a.spill ? go(T{}, F{}, F8{}, F{}) : go(F{}, F{}, F8{}, F{});
    } else {
      e = a.spill ? (a.q_smooth ? go(T{}, T{}, I8{}, F{}) : go(T{}, F{}, I8{}, F{}))
                  : (a.q_smooth ? go(F{}, T{}, I8{}, F{}) : go(F{}, F{}, I8{}, F{}));
    }
    if (e != hipSuccess) return e;
  }
  if (part < 0 || part == 2) {
    const dim3 tiles((unsigned)((long long)(a.N / kPq) * a.BH));
    const hipError_t e = !a.spill            ? launch_kernel(&dq_finalize<DT, D>, tiles, dim3(256), st, a)
                         : a.fmt == FMT_FP8 ? launch_kernel(&bwd_dq<DT, D, BLK, FMT_FP8>, tiles, dim3(256), st, a)
                                            : launch_kernel(&bwd_dq<DT, D, BLK, FMT_INT8>, tiles, dim3(256), st, a);
    if (e != hipSuccess) return e;
    if (a.q_gain) return launch_kernel(&gain_reduce<D>, dim3((unsigned)a.x16.H, 2), dim3(128), st, a);
  }
  return hipSuccess;
}

hipError_t launch_backward(const BackwardArgs& a, int part, hipStream_t st) {
  return dispatch_dt_d_blk(a.dtype, a.D, a.BLK, [&](auto dt, auto d, auto blk) {
    return launch_backward_t<decltype(dt)::value, decltype(d)::value, decltype(blk)::value>(a, part, st);
  });
}

}  // namespace sagebwd
