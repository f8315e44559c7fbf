// Fused INT8 attention forward: O = softmax(sm * Q^ K~^T) V, O and row logsumexp.
// SageBwd article (aitrends.kr 8227), precision-split paragraph: QK^T and PV run in INT8;
// the TurboQuant blog's FlashAttention section: scores are processed tile by tile and
// never stored.
//
// Work decomposition (gfx950, 64-lane waves):
//   workgroup = 4 waves = 128 query rows of one head; wave w owns 32 rows.
//   Key tiles of BLK keys (one quantisation block of K and V) stream into double-buffered
//   LDS by buffer->LDS copies: K codes token-major and V^T codes channel-major, both with
//   their 16-byte chunks XOR-swizzled by row (swz_f) so the MFMA operand reads spread over
//   the banks (the copies take the permutation on their source addresses).
//   S^T = K Q^T with v_mfma_i32_32x32x32_i8 (FP8 codes: v_mfma_scale_f32_32x32x64_f8f6f4 on
//   two 32-channel chunks at once): lane l holds query l%32 and 16 keys per
//   32-key subtile, so the row max / row sum are lane-local plus one exchange with lane
//   l^32 (v_permlane32_swap). The quantised P~^T becomes the B operand of O^T = V^T P~^T
//   after two v_permlane32_swap per subtile, which put keys 16g..16g+15 in lane group g,
//   the order in which the V^T rows are stored.
// With Q-smoothing (QS) each score also gets its key's bias b_k (SageBwd article, Q-smoothing
// paragraph): t = S*sQ*sK + b_k in float per element, the row max is taken over t, and the
// exponent is t * sm*log2e + (row terms); the tile's BLK biases ride in LDS after K and V^T.
// Per key tile (the online-softmax step and the P~ quantisation tile, 32 rows x BLK keys):
//   m' = max(m, rowmax s); P~ = 2^(s*log2e - m'); a = max P~ over the wave's tile;
//   codes = rne(P~ * (M/a)); l = l*alpha + u*sum P~; O = O*alpha + u*(a/M)*sV*(PV of codes),
// with M = 127 for INT8 codes and 448 for FP8 (e4m3) codes,
// with O and l kept relative to a reference r that lags m: r' = m' when some row of the wave
// has m' > r + 8 (and on the first tile), else r' = r; alpha = 2^(r - r'), u = 2^(m' - r').
// Most tiles then leave r alone and skip the O rescale; the codes and the final O and LSE are
// the same as with r = m (only rounding differs).
// P~ * M/a is produced by one exponential, 2^(s*log2e - m' + log2(M/a)), and rounded and
// packed by v_cvt_pk_u8_f32 (INT8) or v_cvt_pk_fp8_f32 (FP8), both nearest even; only tiles
// on the diagonal carry masking work.
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
constexpr float kLazy = 8.0f;  // O and l may lag the running max by up to 2^kLazy

// Chunk swizzle of the K and V^T tiles, rows of RB bytes (an involution in j). The operand
// reads name rows 32t .. 32t+31 (lane l & 31), one chunk per lane half; on gfx950 they
// measured ~206 (RB = 128) and ~218 (RB = 64) B/clk per CU with these XORs, against ~117
// with j ^ (r & 7) and j ^ ((r >> 1) & 3). The XOR depends on the row only through r & 31,
// so a read of row block t sits 32 t RB bytes past the same per-lane offset (an immediate).
template <int RB>
__device__ __forceinline__ int swz_f(int r, int j) {
  if constexpr (RB == 128) return j ^ (((r >> 1) ^ ((r >> 4) & 1)) & 7);
  else return j ^ ((r >> 2) & 3);
}

// Chunk swizzle of the Q-Attn split's 16-bit V rows (2D bytes, 16-byte chunks). The PV
// operand reads (ds_read_b64_tr_b16) name 8 rows x 64 bytes at once (rows 4g + k, channel
// bytes 32cg .. 32cg + 31, two groups cg); XORing the chunk with bits of the row lets those 32
// chunks cover every bank group exactly twice (256-byte rows: row bits 0-1 into chunk bits
// 2-3; 128-byte rows, two per bank cycle: row bit 1 into chunk bit 2).
template <int D>
__device__ __forceinline__ int swz_v16(int r, int j) {
  if constexpr (D == 128) return j ^ ((r & 3) << 2);
  else return j ^ (((r >> 1) & 1) << 2);
}

// One key tile's LDS. SageBwd split: TK = BLK keys (one quantisation block of K and V), K
// codes and V^T codes. Q-Attn split (QA): TK = 64 keys, K codes and the tile's 16-bit V rows
// (the PV product runs in 16 bits; the online-softmax step is the 64-key tile).
template <int D, int BLK, bool QS = false, bool QA = false>
struct FwdLds {
  static constexpr int TK = QA ? 64 : BLK;
  static constexpr int kBytesK = TK * D;                 // K codes [TK][D], chunk j of row r at swz_f<D>(r, j)
  static constexpr int kBytesV = QA ? TK * 2 * D         // V [TK][D] 16-bit, chunk j of row r at swz_v16<D>(r, j)
                                    : D * BLK;           // V^T codes [D][BLK], chunk j of row c at swz_f<BLK>(c, j)
  static constexpr int kBytesKV = kBytesK + kBytesV;
  static constexpr int kBytes = kBytesKV + (QS ? 1024 : 0);   // (QS) key biases f32 [BLK], one 1 KB copy
  static constexpr int kCopies = kBytesKV / 1024;            // 1 KB copies of K and V per tile
  static constexpr int kCopiesPerWave = kCopies / kWaves;
  static_assert(kCopies % kWaves == 0, "copies per wave");
};

// Copies of key tile k0 into an LDS tile buffer: copy cp = w + kWaves*i moves LDS bytes
// [1024 cp, 1024 cp + 1024); lane l fills the chunk at 1024 cp + 16 l and reads the logical
// chunk that the swizzle puts there.
template <int D, int BLK, bool QS, bool QA>
__device__ __forceinline__ void issue_tile(const ForwardArgs& a, size_t bh, int k0, int8_t* dst, int w, int l) {
  using L = FwdLds<D, BLK, QS, QA>;
  const int8_t* kh = a.Kc + (size_t)bh * a.N * D;     // this head's K codes
  const uint32_t hbytes = (uint32_t)a.N * D;
  // (QA) the tile's 16-bit V rows, read through a descriptor based at row k0 whose range ends
  // after the last real token (the 16-bit tensors hold exactly Nv tokens): rows past it read
  // as zeros
  [[maybe_unused]] const unsigned short* vrow0 = nullptr;
  [[maybe_unused]] uint32_t vbytes = 0;
  if constexpr (QA) {
    vrow0 = a.V + a.x16.row((int)bh, k0);
    const int rows = min(L::TK, a.Nv - k0);
    vbytes = rows > 0 ? (uint32_t)((rows - 1) * a.x16.sn + D) * 2u : 0u;
  }
#pragma unroll
  for (int i = 0; i < L::kCopiesPerWave; ++i) {
    const int cp = w + kWaves * i;
    const int e = 64 * cp + l;                          // 16-byte chunk index inside the tile
    if (cp * 1024 < L::kBytesK) {
      const int r = e / (D / 16), pc = e % (D / 16);
      const int j = swz_f<D>(r, pc);                    // the swizzle is an involution
      buffer_to_lds16(kh, hbytes, dst + cp * 1024, (uint32_t)((k0 + r) * D + 16 * j), 0u);
    } else if constexpr (QA) {
      const int ev = e - L::kBytesK / 16;
      const int r = ev / (D / 8), pc = ev % (D / 8);
      const int j = swz_v16<D>(r, pc);
      buffer_to_lds16(vrow0, vbytes, dst + cp * 1024, (uint32_t)(r * a.x16.sn * 2 + 16 * j), 0u);
    } else {
      const int8_t* vh = a.Vtc + (size_t)bh * D * a.N;    // this head's V^T codes
      const int ev = e - L::kBytesK / 16;
      const int c = ev / (BLK / 16), pc = ev % (BLK / 16);
      const int j = swz_f<BLK>(c, pc);
      buffer_to_lds16(vh, hbytes, dst + cp * 1024, (uint32_t)(c * a.N + k0 + 16 * j), 0u);
    }
  }
  if constexpr (QS) {
    // the tile's key biases: 1 KB from key k0 on (lanes past the head's last key read zeros:
    // the copy's range ends with the head's biases)
    if (w == 0) buffer_to_lds16(a.kbias + bh * a.N, (uint32_t)a.N * 4, dst + L::kBytesKV, (uint32_t)(k0 * 4 + 16 * l), 0u);
  }
}

}  // namespace

template <int DT, int D, int BLK, bool QS, int FMT, bool QA>
__global__ __launch_bounds__(kWaves * 64, 2) void fwd_kernel(ForwardArgs a) {
  using L = FwdLds<D, BLK, QS, QA>;
  using C = Codes<FMT>;
  static_assert(FMT == FMT_INT8 || !QS, "Q-smoothing takes INT8 codes only");
  static_assert(!(QS && QA), "Q-smoothing is not combined with the Q-Attn split");
  constexpr int TK = L::TK;       // keys per tile (one online-softmax step)
  constexpr int NSUB = TK / 32;   // 32-key subtiles per key tile
  constexpr int DC = D / 32;      // 32-channel chunks
  __shared__ __attribute__((aligned(16))) int8_t lds[2][L::kBytes];

  const int nq = (a.N + kRowsPerBlock - 1) / kRowsPerBlock;
  const int bh = blockIdx.x % a.BH;
  const int qt = a.causal ? nq - 1 - (int)(blockIdx.x / a.BH) : (int)(blockIdx.x / a.BH);
  const int nb = a.N / BLK;
  const int w = wave_id(), l = lane_id(), g = l >> 5, lq = l & 31;
  const int q0 = qt * kRowsPerBlock;
  const int q0w = q0 + w * kRowsPerWave;
  const bool active = q0w < a.Nv;   // (rows from Nv on are the padding of a ragged last block)
  const int qrow = q0w + lq;  // this lane's query row
  // per-lane byte offsets of the K and V^T operand reads inside a 32-row block; row block t of
  // a tile adds 32 t RB bytes (swz_f depends on the row through r & 31 only)
  int koff[DC], voff[NSUB];
#pragma unroll
  for (int kk = 0; kk < DC; ++kk) koff[kk] = lq * D + 16 * swz_f<D>(lq, 2 * kk + g);
#pragma unroll
  for (int t = 0; t < NSUB; ++t) voff[t] = lq * BLK + 16 * swz_f<BLK>(lq, 2 * t + g);

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
  const int n_kt = a.causal ? last_row / TK + 1 : a.N / TK;

  // m: running row max (the reference of P~); mo: the reference of O and l, which follows m
  // only when some row of the wave has moved more than kLazy past it (and on the first tile)
  float m = -INFINITY, mo = -INFINITY, lsum_run = 0.0f;
  f32x16 o[DC];
#pragma unroll
  for (int ct = 0; ct < DC; ++ct) o[ct] = f32x16{};

  issue_tile<D, BLK, QS, QA>(a, bh, 0, lds[0], w, l);
  wait_vmcnt<0>();
  __syncthreads();
  // block scales of the current key tile, loaded one tile ahead (QA: V is not quantised)
  float sK_n = a.Ks[(size_t)bh * nb], sV_n = QA ? 1.0f : a.Vs[(size_t)bh * nb];

  for (int kt = 0; kt < n_kt; ++kt) {
    const bool has_next = kt + 1 < n_kt;
    if (has_next) issue_tile<D, BLK, QS, QA>(a, bh, (kt + 1) * TK, lds[(kt + 1) & 1], w, l);
    const float sK = sK_n, sV = sV_n;
    if (has_next) {
      sK_n = a.Ks[(size_t)bh * nb + (kt + 1) * TK / BLK];
      if constexpr (!QA) sV_n = a.Vs[(size_t)bh * nb + kt + 1];
    }
    const int k0 = kt * TK;
    const int8_t* kl = lds[kt & 1];
    const int8_t* vl = lds[kt & 1] + L::kBytesK;
    // One key tile. DIAG: the tile crosses this wave's causal diagonal (keys above it are
    // masked) or holds padding keys (from Nv on, a ragged last block); every other visited
    // tile is wholly visible and carries no masking work.
    auto tile = [&](auto diag_c) {
      constexpr bool DIAG = decltype(diag_c)::value;
      // (LLVM's interleaving strategy 1 on this block and on the PV block: measured 1-5%
      // faster than the default schedule)
      __builtin_amdgcn_iglp_opt(1);
      // ---- S^T = K Q^T (exact int32 for INT8 codes, float32 for FP8 codes)
      typename C::acc16 s[NSUB];
#pragma unroll
      for (int t = 0; t < NSUB; ++t) {
        s[t] = typename C::acc16{};
        auto ak = [&](int kk) { return *reinterpret_cast<const i32x4*>(kl + koff[kk] + 32 * t * D); };
#pragma unroll
        for (int kk = 0; kk < DC; kk += 2) s[t] = C::mma32x2(ak(kk), ak(kk + 1), qreg[kk], qreg[kk + 1], s[t]);
      }
      const float c2 = (sQ * sK) * (a.sm_scale * kLog2e);
      [[maybe_unused]] const float c3 = a.sm_scale * kLog2e;
      // row max over the visible keys (a row with none in this tile keeps its old max)
      float rowmax;
      [[maybe_unused]] float tf[QS ? NSUB : 1][16];   // (QS) S*sQ*sK + b_k per element
      if constexpr (QS) {
        const float* bl = reinterpret_cast<const float*>(lds[kt & 1] + L::kBytesKV);
        const float cq = sQ * sK;
        float fm = -INFINITY;
#pragma unroll
        for (int t = 0; t < NSUB; ++t)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x4 bq = *reinterpret_cast<const f32x4*>(bl + 32 * t + 8 * j + 4 * g);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float v = __builtin_fmaf((float)s[t][4 * j + i], cq, bq[i]);
              if constexpr (DIAG) {
                const int key = k0 + 32 * t + 8 * j + 4 * g + i;
                if ((a.causal && key > qrow) || key >= a.Nv) v = -INFINITY;
              }
              tf[t][4 * j + i] = v;
              fm = fmaxf(fm, v);
            }
          }
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(fm), __float_as_int(fm), false, false);
        rowmax = fmaxf(__int_as_float((int)sw[0]), __int_as_float((int)sw[1])) * c3;
      } else if constexpr (FMT == FMT_FP8) {
        if constexpr (DIAG) {
#pragma unroll
          for (int t = 0; t < NSUB; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = k0 + 32 * t + 8 * (r >> 2) + 4 * g + (r & 3);
              if ((a.causal && key > qrow) || key >= a.Nv) s[t][r] = -INFINITY;
            }
        }
        float rmax = -INFINITY;
#pragma unroll
        for (int t = 0; t < NSUB; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) rmax = fmaxf(rmax, s[t][r]);
        {
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_int(rmax), __float_as_int(rmax), false, false);
          rmax = fmaxf(__int_as_float((int)sw[0]), __int_as_float((int)sw[1]));
        }
        // (c2 is 0 for an all-zero block: a row with no visible key stays at -inf)
        rowmax = rmax == -INFINITY ? -INFINITY : rmax * c2;
      } else {
        if constexpr (DIAG) {
#pragma unroll
          for (int t = 0; t < NSUB; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = k0 + 32 * t + 8 * (r >> 2) + 4 * g + (r & 3);
              if ((a.causal && key > qrow) || key >= a.Nv) s[t][r] = INT32_MIN;
            }
        }
        int rmax = INT32_MIN;
#pragma unroll
        for (int t = 0; t < NSUB; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) rmax = max(rmax, s[t][r]);
        {
          const auto sw = __builtin_amdgcn_permlane32_swap(rmax, rmax, false, false);
          rmax = max((int)sw[0], (int)sw[1]);   // lanes l and l^32 hold the same query row (signed)
        }
        rowmax = (float)rmax * c2;
        if constexpr (DIAG) rowmax = rmax == INT32_MIN ? -INFINITY : rowmax;
      }
      const float m_new = fmaxf(m, rowmax);
      // (QA: the reference follows the running max exactly, so the 16-bit P~ are taken, and
      // rounded, against it as in the definition)
      const bool moved = __builtin_amdgcn_ballot_w64(m_new > mo + (QA ? 0.0f : kLazy)) != 0;
      const float mo_new = moved ? m_new : mo;
      const float alpha = __builtin_amdgcn_exp2f(mo - mo_new);   // 1 exactly when not moved
      const float up = __builtin_amdgcn_exp2f(m_new - mo_new);   // P~ in units of 2^mo_new
      if constexpr (QA) {
        // ---- P~ = 2^(s*c2 - m') rounded to the 16-bit type: the B operand of the 16-bit PV
        //      (register r of subtile t holds key 8*(r/4) + 4g + r%4: r = 0..7 feed the first
        //      16-key product, r = 8..15 the second, with the same key slots in V^T's reads)
        float tsum = 0.0f;
        u16x8 pb[NSUB][2];
#pragma unroll
        for (int t = 0; t < NSUB; ++t)
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float x = __builtin_fmaf((float)s[t][4 * j + i], c2, -m_new);
              if constexpr (DIAG && FMT == FMT_FP8) x = s[t][4 * j + i] == -INFINITY ? -INFINITY : x;
              if constexpr (DIAG && FMT == FMT_INT8) x = s[t][4 * j + i] == INT32_MIN ? -INFINITY : x;
              const float u = __builtin_amdgcn_exp2f(x);
              tsum += u;
              pb[t][j >> 1][4 * (j & 1) + i] = from_f32<DT>(u);
            }
        lsum_run = lsum_run * alpha + tsum;
        __builtin_amdgcn_iglp_opt(1);
        if (moved) {
#pragma unroll
          for (int ct = 0; ct < DC; ++ct)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[ct][r] *= alpha;
        }
        // ---- O^T += V^T P~^T in 16 bits, float32 accumulation. V^T's A operand (row =
        //      channel 32ct + 16cg + jl, key slots of lane group g) comes from the row-major V
        //      tile by two transposing reads of four key rows each.
        const int cg = (l >> 4) & 1, jl = l & 15, kr = jl >> 2, qq = jl & 3;
#pragma unroll
        for (int ct = 0; ct < DC; ++ct) {
          const int ch = 4 * ct + 2 * cg + (qq >> 1);
#pragma unroll
          for (int t = 0; t < NSUB; ++t)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int ra = 32 * t + 16 * h + 4 * g + kr, rb = ra + 8;
              const u16x4 a0 = lds_read_tr16(vl + ra * 2 * D + 16 * swz_v16<D>(ra, ch) + 8 * (qq & 1));
              const u16x4 a1 = lds_read_tr16(vl + rb * 2 * D + 16 * swz_v16<D>(rb, ch) + 8 * (qq & 1));
              const u16x8 av = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
              o[ct] = mfma_16b_32x32x16<DT>(av, pb[t][h], o[ct]);
            }
        }
        m = m_new;
        mo = mo_new;
        return;
      }
      // P~ tile absmax a = max over rows of 2^(rowmax - m'); in log2 it is one wave max.
      // The quantisation factor M/a is folded into the exponent, so the exponential
      // yields P~ * M/a directly and its nearest-even code is the code.
      // (padding rows of a ragged last block take no part in the tile's absmax)
      const float pa_log = wave_max(qrow < a.Nv ? rowmax - m_new : -INFINITY);
      const float bias = C::kLog2Max - pa_log - m_new;
      const float sP = __builtin_amdgcn_exp2f(pa_log) * (1.0f / C::kMax);

      float tsum = 0.0f;
      i32x4 pc[NSUB];
#pragma unroll
      for (int t = 0; t < NSUB; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float u[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float x;
            if constexpr (QS) {
              x = __builtin_fmaf(tf[t][4 * j + i], c3, bias);   // -inf stays -inf (masked)
            } else {
              x = __builtin_fmaf((float)s[t][4 * j + i], c2, bias);
              if constexpr (DIAG && FMT == FMT_FP8) x = s[t][4 * j + i] == -INFINITY ? -INFINITY : x;
              if constexpr (DIAG && FMT == FMT_INT8) x = s[t][4 * j + i] == INT32_MIN ? -INFINITY : x;
            }
            u[i] = __builtin_amdgcn_exp2f(x);
            tsum += u[i];
          }
          if constexpr (FMT == FMT_FP8) {
            pc[t][j] = (int)fp8_word(u[0], u[1], u[2], u[3]);
          } else {
            unsigned wd = __builtin_amdgcn_cvt_pk_u8_f32(u[0], 0, 0u);
            wd = __builtin_amdgcn_cvt_pk_u8_f32(u[1], 1, wd);
            wd = __builtin_amdgcn_cvt_pk_u8_f32(u[2], 2, wd);
            pc[t][j] = (int)__builtin_amdgcn_cvt_pk_u8_f32(u[3], 3, wd);
          }
        }
      // word j of lane group g holds keys 8j + 4g .. +3; group 0 needs keys 0..15 and group
      // 1 keys 16..31: swap words (0, 2) and (1, 3) across the lane halves
#pragma unroll
      for (int t = 0; t < NSUB; ++t) {
        const auto x02 = __builtin_amdgcn_permlane32_swap(pc[t][0], pc[t][2], false, false);
        const auto x13 = __builtin_amdgcn_permlane32_swap(pc[t][1], pc[t][3], false, false);
        pc[t] = i32x4{(int)x02[0], (int)x02[1], (int)x13[0], (int)x13[1]};
      }
      // l accumulates P~ before quantisation: sum(P~ * M/a) * a/M
      lsum_run = lsum_run * alpha + tsum * (sP * up);

      __builtin_amdgcn_iglp_opt(1);
      // ---- O^T = O^T * alpha + (a/M) sV (V^T P~^T) over the BLK keys of one V block.
      // O is rescaled only when its reference moved.
      const float spv = (sP * sV) * up;
      if (moved) {
#pragma unroll
        for (int ct = 0; ct < DC; ++ct)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[ct][r] *= alpha;
      }
#pragma unroll
      for (int ct = 0; ct < DC; ++ct) {
        typename C::acc16 acc{};
        auto av = [&](int t) { return *reinterpret_cast<const i32x4*>(vl + voff[t] + 32 * ct * BLK); };
#pragma unroll
        for (int t = 0; t < NSUB; t += 2) acc = C::mma32x2(av(t), av(t + 1), pc[t], pc[t + 1], acc);
#pragma unroll
        for (int r = 0; r < 16; ++r) o[ct][r] = __builtin_fmaf(spv, (float)acc[r], o[ct][r]);
      }
      m = m_new;
      mo = mo_new;
    };
    if (active && (!a.causal || k0 <= q0w + kRowsPerWave - 1)) {
      if ((a.causal && k0 + TK - 1 > q0w) || k0 + TK > a.Nv) tile(std::true_type{});
      else tile(std::false_type{});
    }
    wait_vmcnt<0>();   // the next tile's copies (the only vector-memory operations in the loop)
    __syncthreads();
  }

  // padding rows of a ragged last block (from Nv to the padded length N): lse = +inf, the
  // backward's convention for queries that see no key (their P is 0); no O row exists
  const bool pad_row = qrow >= a.Nv && qrow < a.N;
  if (!active) {
    if (g == 0 && pad_row) a.lse[(size_t)bh * a.N + qrow] = INFINITY;
    return;
  }
  const float ltot = lsum_run + __shfl_xor(lsum_run, 32);
  if (qrow >= a.Nv) {
    if (g == 0 && pad_row) a.lse[(size_t)bh * a.N + qrow] = INFINITY;
    return;
  }
  const float linv = 1.0f / ltot;
  unsigned short* orow = a.O + a.x16.row(bh, qrow);
#pragma unroll
  for (int ct = 0; ct < DC; ++ct)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u16x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = from_f32<DT>(o[ct][4 * j + i] * linv);
      *reinterpret_cast<u16x4*>(orow + 32 * ct + 8 * j + 4 * g) = v;
    }
  if (g == 0) a.lse[(size_t)bh * a.N + qrow] = (mo + __builtin_amdgcn_logf(ltot)) * kLn2;
}

template <int DT, int D, int BLK>
static hipError_t launch_forward_t(const ForwardArgs& a, hipStream_t st) {
  const long long nq = (a.N + kRowsPerBlock - 1) / kRowsPerBlock;
  const dim3 grid((unsigned)(nq * a.BH)), block(kWaves * 64);
  // (Q-smoothing takes INT8 codes and the SageBwd split only; the API refuses the others)
  if (a.q_smooth && (a.fmt != FMT_INT8 || a.qattn)) return hipErrorInvalidValue;
  if (a.qattn)
    return a.fmt == FMT_FP8 ? launch_kernel(&fwd_kernel<DT, D, BLK, false, FMT_FP8, true>, grid, block, st, a)
                            : launch_kernel(&fwd_kernel<DT, D, BLK, false, FMT_INT8, true>, grid, block, st, a);
  if (a.fmt == FMT_FP8) return launch_kernel(&fwd_kernel<DT, D, BLK, false, FMT_FP8, false>, grid, block, st, a);
  return a.q_smooth ? launch_kernel(&fwd_kernel<DT, D, BLK, true, FMT_INT8, false>, grid, block, st, a)
                    : launch_kernel(&fwd_kernel<DT, D, BLK, false, FMT_INT8, false>, grid, block, st, a);
}

hipError_t launch_forward(const ForwardArgs& a, hipStream_t st) {
  return dispatch_dt_d_blk(a.dtype, a.D, a.BLK, [&](auto dt, auto d, auto blk) {
    return launch_forward_t<decltype(dt)::value, decltype(d)::value, decltype(blk)::value>(a, st);
  });
}

}  // namespace sagebwd
