// Backward pass by recomputation, bf16 inputs, fp32 accumulation, gfx950.
//
// Pages cited (titles as published):
//   [TLDR]   "FlashAttention：メモリ効率的なアテンション計算" (tech-tldr.com)
//   [XYZ]    "FlashAttention: IOを意識した高速かつメモリ効率の高い厳密な
//            アテンション" (xyznot.com)
//   [REAPER] "3 · FlashAttention" (mkdocs.reaper.mx, chapter 3)
//   [Q67]    "FlashAttention：在线 softmax 与 IO-aware 注意力" (quant67.com)
//
// The forward saves only O and one logsumexp per row; the backward rebuilds
// each score/probability tile on chip from Q, K and that statistic instead
// of reading a stored N x N matrix ([TLDR] backward section; [XYZ] key
// ideas; [REAPER] 3.4; [Q67] section 5).  The gradient formulas are the
// chain rule applied to O = softmax(scale Q K^T) V:
//   P = exp(scale q_i.k_j - lse_i),  D_i = sum_c dO_ic O_ic,
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),
//   dK = scale dS^T Q,  dQ = scale dS K.
//
// Three kernels, no atomics (fp32 atomic adds run at about one 4-byte add
// per L2 channel per clock, too slow to fold dQ into the dK/dV pass):
//   preprocess : D_i and lse_i * log2(e) per row (a streaming pass).
//   dkdv       : a workgroup owns 128 keys (32 per wave and query half; K
//                and V held in LDS for the workgroup's life), or at d = 128
//                without mask or dropout 256 keys (32 per wave), and sweeps
//                the query tiles, accumulating dK^T and dV^T in registers;
//                each is written once.
//   dq         : a workgroup owns 128 or 256 queries (32 per wave, Q and dO
//                held in registers) and sweeps the key tiles, accumulating
//                dQ^T.
// Within a wave the vector work of one group of products is issued beside
// the next group's products (empty asm statements hold the order where the
// compiler would otherwise issue all products first).
// All contractions run on v_mfma_f32_32x32x16_bf16.  The dkdv pass computes
// S = Q K^T so that each lane owns one key (the N index of the D layout); P
// and dS then already have the B-operand layout for the contractions over
// queries.  The dq pass computes S^T = K Q^T (lane = query) for the same
// reason.  Every LDS tile is stored once, row-major; the transposed operands
// (Q^T and dO^T in dkdv, K^T in dq) come from ds_read_b64_tr_b16 reads of
// those same tiles, with one XOR swizzle that is conflict-free for both the
// row-wise and the transposed read pattern.  Causal key/query tiles that are
// fully masked are skipped ([REAPER], causal-mask question).
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

// ---------------------------------------------------------------------------
// preprocess: D_i = sum_c dO_ic * O_ic, lse2_i = lse_i * log2(e)
// (+inf for rows whose forward saw no key, so that every rebuilt
// probability of that row is exactly 0).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256)
void bwd_pre_kernel(const bf16* __restrict__ O, const bf16* __restrict__ dO,
                    const float* __restrict__ lse, float* __restrict__ ws_d,
                    float* __restrict__ ws_lse2, int64_t rows) {
  constexpr int TPR = D / 8;  // 16-byte chunks per row
  const int64_t row = (int64_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(O + row * D + part * 8);
    const u32x4 b = *reinterpret_cast<const u32x4*>(dO + row * D + part * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = fmaf(bf16_lo(a[i]), bf16_lo(b[i]), acc);
      acc = fmaf(bf16_hi(a[i]), bf16_hi(b[i]), acc);
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (part == 0 && row < rows) {
    ws_d[row] = acc;
    const float L = lse[row];
    ws_lse2[row] = (L == -INFINITY) ? INFINITY : L * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// dkdv pass
// ---------------------------------------------------------------------------
template <int D>
struct KVTile {
  static constexpr int NW = 8;                        // waves per workgroup
  static constexpr int BCK = 128;                     // keys per workgroup
  static constexpr int BRQ = (D == 128) ? 64 : 128;   // queries per LDS stage
  static constexpr int QB = BRQ / 32;                 // 32-query blocks per stage
  static constexpr int QBW = QB / 2;                  // blocks per wave
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int ROW = D * 2;
  static constexpr int KV_BYTES = BCK * ROW;          // K (or V) of the workgroup
  static constexpr int T_BYTES = BRQ * ROW;           // Q (or dO) of one stage
  // LDS: K | V | stage 0 | stage 1; stage = Q | dO | lse2[BRQ] | D[BRQ]
  static constexpr int OFF_V = KV_BYTES;
  static constexpr int OFF_ST = 2 * KV_BYTES;
  static constexpr int S_DO = T_BYTES;
  static constexpr int S_L = 2 * T_BYTES;
  static constexpr int S_D = S_L + BRQ * 4;
  static constexpr int STAGE = S_D + BRQ * 4;
  static constexpr int LDS = OFF_ST + 2 * STAGE;
  static constexpr int KV_BLK = KV_BYTES / 1024 / NW;  // 1-KB DMA blocks per wave
  static constexpr int T_BLK = T_BYTES / 1024 / NW;
  static constexpr int RED = 4 * 2 * DB * 16 * 64 * 4;  // partial dK, dV sums
  static_assert(RED <= LDS, "reduction buffer fits in the tile space");
  static_assert(KV_BLK * NW * 1024 == KV_BYTES && T_BLK * NW * 1024 == T_BYTES,
                "tiles split evenly into 1-KB blocks per wave");
};

// Per-lane offsets of the transposed operand of a 16-row k-step: source lane
// s = lane % 16 of group g = lane / 16 addresses row r2*8 + h*4 + s/4 at
// column db*32 + 16*(g & 1) + 4*(s % 4) (r2 = 0: slots 0-3, r2 = 1: slots
// 4-7).  The resulting slot order matches the register order of an MFMA
// D-layout block (rows {h*4 + 0..3} then {8 + h*4 + 0..3}).
template <int D, int DB>
__device__ __forceinline__ void tr_offsets(int lane, int toff[DB][2]) {
  const int s16 = lane & 15, g = lane >> 4, h = lane >> 5;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int col = db * 32 + 16 * (g & 1) + 4 * (s16 & 3);
#pragma unroll
    for (int r2 = 0; r2 < 2; ++r2) {
      toff[db][r2] = tile_off<D>(r2 * 8 + h * 4 + (s16 >> 2), col >> 3) +
                     (col & 7) * 2;
    }
  }
}

// Workgroup of 8 waves = 2 per SIMD.  Wave w owns keys k0 + 32*(w % 4) ..
// + 31 and the query half w / 4 of every staged query tile; the two waves
// owning the same keys add their partial dK, dV once at the end.  K and V of
// the workgroup's 128 keys stay in LDS for its whole life (read as B
// operands), which keeps the per-wave register footprint within the 256
// registers that two waves per SIMD allow.  Query tiles are double-buffered
// and filled by direct global-to-LDS loads.
template <int D, bool CAUSAL, bool SPARSE, bool DROP>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                     const bf16* __restrict__ V, const bf16* __restrict__ dO,
                     const float* __restrict__ ws_d,
                     const float* __restrict__ ws_lse2, float* __restrict__ dK,
                     float* __restrict__ dV, int n, int nk, int q_off,
                     int n_ktiles, int total, int bundle, float c_log2,
                     float scale,
                     const uint8_t* __restrict__ mask,
                     int mask_cols, int block_m, int block_n, Dropout drop,
                     int* __restrict__ visits) {
  using T = KVTile<D>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[T::LDS];

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int kw = w & 3;   // key block of this wave
  const int qh = w >> 2;  // query half of this wave

  const int lid = xcd_logical_id(blockIdx.x, total);
  // Under the causal rule early key tiles are the heavy ones.  Dense causal:
  // the workgroup takes key tiles u and n_ktiles-1-u of one head, whose
  // query counts add up to the same total for every u, so that all
  // workgroups carry equal work (the hardware hands workgroups to CUs in a
  // fixed rotation, which leaves CUs idle behind longer ones).
  constexpr bool PAIRS = CAUSAL && !SPARSE;
  int head, kt_a, kt_b = -1;
  if constexpr (PAIRS) {
    const int units = (n_ktiles + 1) / 2;
    const int u = lid % units;
    head = lid / units;
    kt_a = u;
    if (u != n_ktiles - 1 - u) kt_b = n_ktiles - 1 - u;
  } else {
    const CausalPlace pl = CAUSAL ? causal_place(lid, n_ktiles, total / n_ktiles, bundle)
                                  : CausalPlace{lid / n_ktiles, lid % n_ktiles};
    head = pl.head;
    kt_a = pl.rank;
  }
  const int64_t hoff = (int64_t)head * n * D;     // Q, dO: n rows per head
  const int64_t hoff_k = (int64_t)head * nk * D;  // K, V, dK, dV: nk rows
  const int64_t roff = (int64_t)head * n;
  drop.bh = (uint32_t)head;

  // One key tile of 128 keys.
  auto run_tile = [&](int kt) {
  const int k0 = kt * T::BCK;
  const int kw0 = k0 + 32 * kw;
  const int key = kw0 + l32;

  // K and V tiles of the workgroup (rows past the end read row nk - 1;
  // their dK, dV are never stored).
#pragma unroll
  for (int i = 0; i < T::KV_BLK; ++i) {
    dma_tile_block<D>(K + hoff_k, k0, nk, smem, w + T::NW * i, lane);
    dma_tile_block<D>(V + hoff_k, k0, nk, smem + T::OFF_V, w + T::NW * i, lane);
  }

  const int n_qt = (n + T::BRQ - 1) / T::BRQ;
  // Under the causal rule query row i sees key k0 from i = k0 - q_off on.
  const int qt_begin = CAUSAL ? max(0, k0 - q_off) / T::BRQ : 0;
  // DMA sources of the Q / dO tiles: lane `lane` fills bytes 16*lane of
  // 1-KB block w + NW*i, i.e. row o / ROW, physical chunk (o % ROW) / 16 =
  // logical chunk ^ swizzle; element offsets from the tile's first row.
  int goff[T::T_BLK];
#pragma unroll
  for (int i = 0; i < T::T_BLK; ++i) {
    const int o = (w + T::NW * i) * 1024 + lane * 16;
    const int row = o / T::ROW;
    goff[i] = row * D + ((((o % T::ROW) >> 4) ^ tile_swz<D>(row)) * 8);
  }
  // Stage fill: Q and dO tiles (1-KB blocks split over the waves) and the
  // per-row lse2 and D (one 256-B block per 64 rows, clamped rows; rows past
  // the end are masked in the math).
  auto issue_stage = [&](int qt, int stage) {
    unsigned char* st = smem + T::OFF_ST + stage * T::STAGE;
    const int q0 = qt * T::BRQ;
    if (q0 + T::BRQ <= n) {
      const bf16* qb = Q + hoff + (int64_t)q0 * D;
      const bf16* db = dO + hoff + (int64_t)q0 * D;
#pragma unroll
      for (int i = 0; i < T::T_BLK; ++i) {
        dma16(qb + (uint32_t)goff[i], st + (w + T::NW * i) * 1024);
        dma16(db + (uint32_t)goff[i], st + T::S_DO + (w + T::NW * i) * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < T::T_BLK; ++i) {
        dma_tile_block<D>(Q + hoff, q0, n, st, w + T::NW * i, lane);
        dma_tile_block<D>(dO + hoff, q0, n, st + T::S_DO, w + T::NW * i, lane);
      }
    }
    constexpr int RB = T::BRQ / 64;  // 256-B row blocks per statistic
    if (w < 2 * RB) {
      const int which = w / RB, rb = w % RB;
      const float* src = which ? ws_d : ws_lse2;
      const int row = min(q0 + rb * 64 + lane, n - 1);
      dma4(src + roff + row, st + (which ? T::S_D : T::S_L) + rb * 256);
    }
  };

  f32x16 adk[T::DB], adv[T::DB];
#pragma unroll
  for (int db = 0; db < T::DB; ++db) {
    adk[db] = zero16();
    adv[db] = zero16();
  }
  // Per-lane LDS offsets with this wave's fixed parts (its key block kw and
  // query half qh) folded in, so that every LDS read below is one register
  // plus an immediate offset under 64 KB (the stage parity, the block within
  // the stage and the Q / dO or K / V choice).
  //   aK: row-wise K (and, + OFF_V, V) operand: row kw*32 + l32, chunk ks*2 + h;
  //   aQ: row-wise Q (and, + S_DO, dO) operand of the wave's first query block
  //       in stage 0;
  //   aT: transposed reads of that block (slots 0-3 / 4-7, see tr_offsets);
  //   aL: this half-wave's lse2 entries of that block (+ S_D - S_L: D).
  //   (At d = 64 aQ is aK plus a wave-uniform difference, one add per
  //   read, which keeps the causal instance within its registers.)
  constexpr bool OWN_AQ = (D == 128);
  int aK[T::KS], aQ[OWN_AQ ? T::KS : 1];
  const int q_minus_k = T::OFF_ST + qh * T::QBW * 32 * T::ROW - kw * 32 * T::ROW;
#pragma unroll
  for (int ks = 0; ks < T::KS; ++ks) {
    const int o = tile_off<D>(l32, ks * 2 + h);
    aK[ks] = kw * 32 * T::ROW + o;
    if constexpr (OWN_AQ) aQ[ks] = aK[ks] + q_minus_k;
  }
  auto a_q = [&](int ks) { return OWN_AQ ? aQ[OWN_AQ ? ks : 0] : aK[ks] + q_minus_k; };
  int aT[T::DB][2];
  tr_offsets<D, T::DB>(lane, aT);
#pragma unroll
  for (int db = 0; db < T::DB; ++db) {
    aT[db][0] += T::OFF_ST + qh * T::QBW * 32 * T::ROW;
    aT[db][1] += T::OFF_ST + qh * T::QBW * 32 * T::ROW;
  }
  const int aL = T::OFF_ST + T::S_L + (qh * T::QBW * 32 + h * 4) * 4;

  // Block-sparse: the query tiles whose mask block in this workgroup's key
  // column is nonzero (a 64-row tile lies in one 128-multiple block row).
  MaskLine mline(SPARSE ? mask + k0 / block_n : mask, mask_cols,
                 SPARSE ? (n + block_m - 1) / block_m : 0, lane);
  auto next_on = [&](int qt) -> int {
    ++qt;
    if constexpr (SPARSE) {
      if (qt < n_qt) {
        const int row = (qt * T::BRQ) / block_m;
        const int nr = mline.next(row, lane);
        if (nr != row) qt = min(n_qt, (int)(((int64_t)nr * block_m) / T::BRQ));
      }
    }
    return __builtin_amdgcn_readfirstlane(qt);
  };
  // One query tile: wait for it (loaded one tile ahead) and let every wave
  // finish the previous one, load the next tile into the freed stage, then
  // accumulate this wave's query blocks.  MASK: the tile has queries before
  // some of this wave's keys (causal) or past the end; fully masked blocks
  // are skipped.  PAR is the stage parity when known at compile time (every
  // LDS address is then a register plus an immediate), else -1 (then
  // `stage`).  `qt_next` is the tile that follows.
  int nvis = 0;  // query tiles visited (diagnostic count)
  auto tile = [&](auto mask_tag, auto par_tag, int qt, int stage_rt, int qt_next) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr int PAR = decltype(par_tag)::value;
    const int stage = (PAR >= 0) ? PAR : stage_rt;
    ++nvis;
    wait_dma();
    __syncthreads();
    if (qt_next < n_qt) issue_stage(qt_next, stage ^ 1);
    const int so = stage * T::STAGE;  // immediate when the parity is static
#pragma unroll
    for (int qi = 0; qi < T::QBW; ++qi) {
      const int qb = qh * T::QBW + qi;
      const int qq0 = qt * T::BRQ + qb * 32;
      if (MASK && CAUSAL && qq0 + 31 + q_off < kw0) continue;  // every query before every key
      // Dropout: dV takes the kept probabilities (the 1/(1-p) factor is
      // applied at the end), dS the kept and rescaled dP.
      // (Dropout: the draw's ten rounds are spread between the products,
      // held there by empty asm statements; the compiler otherwise puts them
      // all in front.)
      uint32_t u[4], x[4];
      if constexpr (DROP) dropout_ctr_keylane(drop, key, qq0, lane, x);
      // S = Q K^T and dP = dO V^T (M = query, N = key), both operands from LDS.
      f32x16 s = zero16(), dp = zero16();
#pragma unroll
      for (int ks = 0; ks < T::KS; ++ks) {
        const unsigned char* pa = smem + a_q(ks) + so + qi * 32 * T::ROW;
        const bf16x8 kb = *reinterpret_cast<const bf16x8*>(smem + aK[ks]);
        const bf16x8 vb = *reinterpret_cast<const bf16x8*>(smem + T::OFF_V + aK[ks]);
        s = mfma32(*reinterpret_cast<const bf16x8*>(pa), kb, s);
        dp = mfma32(*reinterpret_cast<const bf16x8*>(pa + T::S_DO), vb, dp);
        if constexpr (DROP) {
          asm volatile("" : "+v"(s), "+v"(dp));
#pragma unroll
          for (int r = ks * 10 / T::KS; r < (ks + 1) * 10 / T::KS; ++r)
            philox_round(x, drop.k0 + r * kWeyl0, drop.k1 + r * kWeyl1);
          asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]));
        }
      }
      if constexpr (DROP) dropout_finish_keylane(x, lane, u);
      // Register i holds query qq0 + (i/4)*8 + h*4 + i%4.  With MASK, P is
      // zero for queries before this lane's key or past the end: qrel is the
      // first visible query relative to qq0 + h*4, qend the end.
      const int qlo = (CAUSAL ? key - q_off : 0) - qq0 - h * 4;
      const int qhi = n - qq0 - h * 4;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const unsigned char* pl = smem + aL + so + (qi * 32 + g * 8) * 4;
        const f32x4 L = *reinterpret_cast<const f32x4*>(pl);
        const f32x4 Dv = *reinterpret_cast<const f32x4*>(pl + (T::S_D - T::S_L));
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int i = 4 * g + t;
          float p = fast_exp2(fmaf(s[i], c_log2, -L[t]));
          if constexpr (MASK) {
            const int qr = g * 8 + t;
            if (qr < qlo || qr >= qhi) p = 0.f;
          }
          if constexpr (DROP) {
            const bool keep = dropout_keep(u[g], t, drop.t);
            s[i] = keep ? p : 0.f;
            dp[i] = p * ((keep ? dp[i] * drop.inv_keep : 0.f) - Dv[t]);
          } else {
            s[i] = p;
            dp[i] = p * (dp[i] - Dv[t]);
          }
        }
      }
      const bf16x8 pf[2] = {pack8(s, 0), pack8(s, 1)};
      const bf16x8 sf[2] = {pack8(dp, 0), pack8(dp, 1)};
      // dV^T += dO^T P and dK^T += Q^T dS (M = d, N = key, K = query); the
      // transposed operands come from transpose reads of the Q / dO tiles.
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int pk = so + (qi * 2 + s2) * 16 * T::ROW;
#pragma unroll
        for (int db = 0; db < T::DB; ++db) {
          const bf16x8 a_do = join_tr16(lds_read_tr16(smem + aT[db][0] + pk + T::S_DO),
                                        lds_read_tr16(smem + aT[db][1] + pk + T::S_DO));
          const bf16x8 a_q = join_tr16(lds_read_tr16(smem + aT[db][0] + pk),
                                       lds_read_tr16(smem + aT[db][1] + pk));
          adv[db] = mfma32(a_do, pf[s2], adv[db]);
          adk[db] = mfma32(a_q, sf[s2], adk[db]);
        }
      }
    }
  };

  using yes = std::true_type;
  using no = std::false_type;
  using par0 = std::integral_constant<int, 0>;
  using par1 = std::integral_constant<int, 1>;
  using par_rt = std::integral_constant<int, -1>;
  // Masked tiles: under the causal rule those holding a query that does not
  // see the workgroup's last key k0 + 127 (query + q_off < k0 + 127: they
  // meet the diagonal), and the tile reaching past the end.
  const int diag_last = k0 + T::BCK - 2 - q_off;  // last such query
  const int head_end =
      (CAUSAL && diag_last >= 0) ? min(n_qt, diag_last / T::BRQ + 1) : qt_begin;
  const int full_end = n / T::BRQ;  // tiles before this are fully in range
  if constexpr (SPARSE && D == 128) {
    // Visited tiles in order, each in the masked form, the stage parity
    // alternating at run time (a second, unmasked copy of the tile does not
    // fit the registers at d = 128).
    int qt = next_on(qt_begin - 1);
    if (qt < n_qt) issue_stage(qt, 0);
    int stage = 0;
#pragma unroll 1
    while (qt < n_qt) {
      const int qn = next_on(qt);
      tile(yes{}, par_rt{}, qt, stage, qn);
      qt = qn;
      stage ^= 1;
    }
  } else if constexpr (SPARSE) {
    // Visited tiles in order: those under the causal diagonal (masked),
    // then the unmasked ones in pairs with static stage parity (the parity
    // alternates over visited tiles), then the tile reaching past the end
    // (masked).  Separate loops keep each tile body one basic block.
    int qt = next_on(qt_begin - 1);
    if (qt < n_qt) issue_stage(qt, 0);
    int stage = 0;
#pragma unroll 1
    for (; qt < n_qt && qt < head_end; stage ^= 1) {
      const int qn = next_on(qt);
      tile(yes{}, par_rt{}, qt, stage, qn);
      qt = qn;
    }
    if (stage && qt < full_end) {
      const int qn = next_on(qt);
      tile(no{}, par1{}, qt, 1, qn);
      qt = qn;
      stage = 0;
    }
#pragma unroll 1
    while (qt < full_end) {
      int qn = next_on(qt);
      tile(no{}, par0{}, qt, 0, qn);
      qt = qn;
      stage = 1;
      if (qt >= full_end) break;
      qn = next_on(qt);
      tile(no{}, par1{}, qt, 1, qn);
      qt = qn;
      stage = 0;
    }
#pragma unroll 1
    for (; qt < n_qt; stage ^= 1) {
      const int qn = next_on(qt);
      tile(yes{}, par_rt{}, qt, stage, qn);
      qt = qn;
    }
  } else if (qt_begin < n_qt) {
    issue_stage(qt_begin, 0);
    // Unmasked tiles run in pairs with static stage parity (stage =
    // (qt - qt_begin) & 1).
    int qt = qt_begin;
#pragma unroll 1
    for (; qt < head_end; qt = __builtin_amdgcn_readfirstlane(qt + 1)) {
      tile(yes{}, par_rt{}, qt, (qt - qt_begin) & 1, qt + 1);
    }
    if (((qt - qt_begin) & 1) && qt < full_end) {
      tile(no{}, par1{}, qt, 1, qt + 1);
      qt = __builtin_amdgcn_readfirstlane(qt + 1);
    }
#pragma unroll 1
    while (qt + 1 < full_end) {
      tile(no{}, par0{}, qt, 0, qt + 1);
      tile(no{}, par1{}, qt + 1, 1, qt + 2);
      qt = __builtin_amdgcn_readfirstlane(qt + 2);
    }
#pragma unroll 1
    for (; qt < n_qt; qt = __builtin_amdgcn_readfirstlane(qt + 1)) {
      tile(yes{}, par_rt{}, qt, (qt - qt_begin) & 1, qt + 1);
    }
  }

  // Add the two query halves' partial sums through LDS, then store once.
  // The reduction buffer reuses the tile space: every fill issued by this
  // wave (K and V at the top, even when no query tile is visited) must have
  // landed before any wave writes there.
  wait_dma();
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
  auto slot = [&](int t, int db, int i) {
    return ((((kw * 2 + t) * T::DB + db) * 16 + i) * 64) + lane;
  };
  if (qh == 1) {
#pragma unroll
    for (int db = 0; db < T::DB; ++db) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        red[slot(0, db, i)] = adk[db][i];
        red[slot(1, db, i)] = adv[db][i];
      }
    }
  }
  __syncthreads();
  if (qh == 0 && key < nk) {
    float* dkr = dK + hoff_k + (int64_t)key * D;
    float* dvr = dV + hoff_k + (int64_t)key * D;
    // D layout of dK^T / dV^T: lane = key, register i -> d = db*32 + (i/4)*8 + h*4 + i%4.
#pragma unroll
    for (int db = 0; db < T::DB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = db * 32 + g * 8 + h * 4;
        f32x4 xk, xv;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          xk[t] = (adk[db][4 * g + t] + red[slot(0, db, 4 * g + t)]) * scale;
          xv[t] = adv[db][4 * g + t] + red[slot(1, db, 4 * g + t)];
          if constexpr (DROP) xv[t] *= drop.inv_keep;
        }
        *reinterpret_cast<f32x4*>(dkr + c) = xk;
        *reinterpret_cast<f32x4*>(dvr + c) = xv;
      }
    }
  }
  if (visits != nullptr && w == 0 && lane == 0) {
    visits[(int64_t)head * n_ktiles + kt] = nvis;
  }
  };

  run_tile(kt_a);
  if (PAIRS && kt_b >= 0) {
    __syncthreads();  // the partial sums are read before K/V are refilled
    run_tile(kt_b);
  }
}

// ---------------------------------------------------------------------------
// dkdv pass, d = 128 without mask or dropout: 256 keys per workgroup
// ---------------------------------------------------------------------------
// Each staged query tile serves 256 keys instead of 128, which halves the
// bytes moved into LDS per key.  K and V of the 256 keys fill 128 KB of LDS
// (each key's K row followed by its V row, so that the V operand is the K
// address plus an immediate), two 32-query stages of Q and dO the other
// 32 KB.  That leaves no LDS for the per-row statistics, and in the S = Q K^T
// layout a lane would need them for 16 query rows; instead they enter the
// products: one more k-step of 16 adds -lse2_i / c to S_ij (A operand: the
// value split into two bf16 parts in slots 0 and 1 of query i's lane, B:
// ones) and one adds -D_i to dP_ij, so that P = exp2(c S') and dS = P dP'.
// The two bf16 parts carry 16 significant bits (relative error ~2^-17,
// against the 2^-9 of the bf16 P and dS).  Wave w owns keys k0 + 32w .. +
// 31 and the whole 32-query block of every stage, so no cross-wave
// reduction is needed at the end.
struct KV256Tile {
  static constexpr int D = 128;
  static constexpr int NW = 8;                        // waves per workgroup
  static constexpr int BCK = 256;                     // keys per workgroup
  static constexpr int BRQ = 32;                      // queries per LDS stage
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int ROW = D * 2;                   // one row of K, V, Q or dO
  static constexpr int KV_ROW = 2 * ROW;              // K row, then V row, of a key
  static constexpr int KV_BYTES = BCK * KV_ROW;
  static constexpr int T_BYTES = BRQ * ROW;           // Q (or dO) of one stage
  // LDS: K/V rows | stage 0 | stage 1; stage = Q | dO
  static constexpr int OFF_ST = KV_BYTES;
  static constexpr int S_DO = T_BYTES;
  static constexpr int STAGE = 2 * T_BYTES;
  static constexpr int LDS = OFF_ST + 2 * STAGE;
  static constexpr int KV_BLK = KV_BYTES / 1024 / NW;  // 1-KB DMA blocks per wave
  static constexpr int T_BLK = T_BYTES / 1024 / NW;
  static_assert(LDS <= 160 * 1024, "fits the LDS of a CU");
  static_assert(KV_BLK * NW * 1024 == KV_BYTES && T_BLK * NW * 1024 == T_BYTES,
                "tiles split evenly into 1-KB blocks per wave");
};

// Element `off` of a buffer of `n` floats; past the end it reads as 0
// (hardware range check of the buffer resource).
__device__ __forceinline__ float load1_bounded(const float* base, int n, int off) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(base), (short)0, n * 4, 0x00020000);
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_raw_buffer_load_b32(r, off * 4, 0, 0));
}

// A operand of the extra k-step: x split into bf16 parts hi + lo in slots 0
// and 1 of the half-wave h = 0 (slots k = 0, 1 of row l32), zeros elsewhere.
// x = -inf gives hi = -inf, lo = 0.
__device__ __forceinline__ bf16x8 split_operand(float x, int h) {
  const float hi = __builtin_bit_cast(float, pack_bf16(x, 0.f) << 16);
  const float lo = (x == -INFINITY) ? 0.f : x - hi;
  u32x4 u = {h ? 0u : pack_bf16(hi, lo), 0u, 0u, 0u};
  return as_bf16x8(u);
}

template <bool CAUSAL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv256_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                        const bf16* __restrict__ V, const bf16* __restrict__ dO,
                        const float* __restrict__ ws_d,
                        const float* __restrict__ ws_lse2,
                        float* __restrict__ dK, float* __restrict__ dV, int n,
                        int nk, int q_off, int n_ktiles, int total,
                        float c_log2, float scale, int* __restrict__ visits) {
  using T = KV256Tile;
  constexpr int D = T::D;
  __shared__ __attribute__((aligned(16))) unsigned char smem[T::LDS];

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  const int lid = xcd_logical_id(blockIdx.x, total);
  // Causal: key tiles u and n_ktiles-1-u of one head per workgroup (equal
  // work for every workgroup, as in the 128-key kernel).
  int head, kt_a, kt_b = -1;
  if constexpr (CAUSAL) {
    const int units = (n_ktiles + 1) / 2;
    const int u = lid % units;
    head = lid / units;
    kt_a = u;
    if (u != n_ktiles - 1 - u) kt_b = n_ktiles - 1 - u;
  } else {
    head = lid / n_ktiles;
    kt_a = lid % n_ktiles;
  }
  const int64_t hoff = (int64_t)head * n * D;     // Q, dO: n rows per head
  const int64_t hoff_k = (int64_t)head * nk * D;  // K, V, dK, dV: nk rows
  const float* Lh = ws_lse2 + (int64_t)head * n;
  const float* Dh = ws_d + (int64_t)head * n;

  // One key tile; DOWN walks its query stages from the last one down
  // instead of up from the first.
  auto run_tile = [&](int kt, auto down_tag) {
  constexpr bool DOWN = decltype(down_tag)::value;
  const int k0 = kt * T::BCK;
  const int kw0 = k0 + 32 * w;
  const int key = kw0 + l32;

  // K and V rows of the workgroup's keys (rows past the end read row
  // nk - 1; their dK, dV are never stored).  Lane `lane` of 1-KB block b
  // fills bytes 16*lane of it: key 2b + lane/32, the K row for lanes
  // 0-15 and 32-47, the V row for the others, physical chunk = logical
  // chunk ^ swizzle of the key.
#pragma unroll
  for (int i = 0; i < T::KV_BLK; ++i) {
    const int b = w + T::NW * i;
    const int kr = 2 * b + (lane >> 5);
    const bf16* src = ((lane >> 4) & 1) ? V : K;
    const int c = (lane & 15) ^ tile_swz<D>(kr);
    dma16(src + hoff_k + (int64_t)min(k0 + kr, nk - 1) * D + c * 8,
          smem + b * 1024);
  }

  const int n_qt = (n + T::BRQ - 1) / T::BRQ;
  // Under the causal rule query row i sees key k0 from i = k0 - q_off on.
  const int qt_begin = CAUSAL ? max(0, k0 - q_off) / T::BRQ : 0;
  // Stage sources: lane `lane` fills bytes 16*lane of 1-KB block w of the
  // Q (dO) tile: row o / ROW, physical chunk = logical chunk ^ swizzle.
  const int o_st = w * 1024 + lane * 16;
  const int st_row = o_st / T::ROW;
  const int goff = st_row * D + ((((o_st % T::ROW) >> 4) ^ tile_swz<D>(st_row)) * 8);
  auto issue_stage = [&](int qt, int stage) {
    unsigned char* st = smem + T::OFF_ST + stage * T::STAGE + w * 1024;
    const int q0 = qt * T::BRQ;
    if (q0 + T::BRQ <= n) {
      dma16(Q + hoff + (int64_t)q0 * D + (uint32_t)goff, st);
      dma16(dO + hoff + (int64_t)q0 * D + (uint32_t)goff, st + T::S_DO);
    } else {
      dma_tile_block<D>(Q + hoff, q0, n, smem + T::OFF_ST + stage * T::STAGE, w, lane);
      dma_tile_block<D>(dO + hoff, q0, n, smem + T::OFF_ST + stage * T::STAGE + T::S_DO,
                        w, lane);
    }
  };

  f32x16 adk[T::DB], adv[T::DB];
#pragma unroll
  for (int db = 0; db < T::DB; ++db) {
    adk[db] = zero16();
    adv[db] = zero16();
  }
  // LDS offsets: aK the row-wise K operand (key w*32 + l32, chunk
  // ks*2 + h; + ROW: the V operand); aQ the row-wise Q (+ S_DO: dO) operand
  // of stage 0; aT the transposed reads of stage 0.
  // (The swizzle of key row w*32 + l32 equals that of Q row l32, so aQ is
  // aK plus one per-lane difference: one add per read, 7 registers fewer.)
  int aK[T::KS];
#pragma unroll
  for (int ks = 0; ks < T::KS; ++ks) {
    const int kr = w * 32 + l32;
    aK[ks] = kr * T::KV_ROW + (((ks * 2 + h) ^ tile_swz<D>(kr)) << 4);
  }
  const int q_minus_k = T::OFF_ST + l32 * T::ROW - (w * 32 + l32) * T::KV_ROW;
  // B operand of the extra k-steps: ones in slots k = 0, 1 (half-wave 0).
  const bf16x8 ones = as_bf16x8(u32x4{h ? 0u : 0x3f803f80u, 0u, 0u, 0u});
  const float neg_inv_c = -1.f / c_log2;
  int aT[T::DB][2];
  tr_offsets<D, T::DB>(lane, aT);
#pragma unroll
  for (int db = 0; db < T::DB; ++db) {
    aT[db][0] += T::OFF_ST;
    aT[db][1] += T::OFF_ST;
  }

  int nvis = 0;  // query tiles visited (diagnostic count)
  // Query row qq0 + l32's statistics, loaded one stage ahead (rows past the
  // end read 0 and are masked below).
  auto load_stats = [&](int qt, float& l, float& dd) {
    const int qq0 = qt * T::BRQ;
    l = load1_bounded(Lh + qq0, n - qq0, l32);
    dd = load1_bounded(Dh + qq0, n - qq0, l32);
  };
  float nl = 0.f, nd = 0.f;
  // One 32-query stage: wait for it (loaded one stage ahead) and let every
  // wave finish the previous one, load the next into the freed stage, then
  // the wave's 32 x 32 block.  MASK: some query of the stage does not see
  // some key of the workgroup, or the stage reaches past the end.
  auto tile = [&](auto mask_tag, auto par_tag, int qt, int stage_rt, int qt_next) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr int PAR = decltype(par_tag)::value;
    const int stage = (PAR >= 0) ? PAR : stage_rt;
    ++nvis;
    wait_dma();
    __syncthreads();
    const float cl = nl, cd = nd;
    if (qt_next < n_qt) {
      issue_stage(qt_next, stage ^ 1);
      load_stats(qt_next, nl, nd);
    }
    const int so = stage * T::STAGE;
    const int qq0 = qt * T::BRQ;
    if (MASK && CAUSAL && qq0 + 31 + q_off < kw0) return;  // every query before every key
    // S' = Q K^T - lse2 / c and dP' = dO V^T - D (M = query, N = key); the
    // statistics enter as the last k-step.  The block runs as four groups of
    // products, each next to the vector work that does not depend on it, so
    // that a wave's exponentials and products overlap: S'; dP' beside
    // P = exp2(c S') (two exponentials per product, held in place by empty
    // asm statements, which the compiler otherwise moves behind all the
    // products); dV beside dS = P dP'; dK.
    f32x16 s = zero16(), dp = zero16();
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) {
      const unsigned char* pa = smem + aK[ks] + q_minus_k + so;
      const bf16x8 kb = *reinterpret_cast<const bf16x8*>(smem + aK[ks]);
      s = mfma32(*reinterpret_cast<const bf16x8*>(pa), kb, s);
    }
    s = mfma32(split_operand(cl * neg_inv_c, h), ones, s);
    __builtin_amdgcn_sched_barrier(0);
    // Register i holds query qq0 + (i/4)*8 + h*4 + i%4.  With MASK, P is
    // zero for queries before this lane's key or past the end.
    const int qlo = (CAUSAL ? key - q_off : 0) - qq0 - h * 4;
    const int qhi = n - qq0 - h * 4;
    auto prob = [&](int i) {
      float p = fast_exp2(s[i] * c_log2);
      if constexpr (MASK) {
        const int qr = (i >> 2) * 8 + (i & 3);
        if (qr < qlo || qr >= qhi) p = 0.f;
      }
      return p;
    };
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) {
      const unsigned char* pa = smem + aK[ks] + q_minus_k + so;
      const bf16x8 vb = *reinterpret_cast<const bf16x8*>(smem + aK[ks] + T::ROW);
      dp = mfma32(*reinterpret_cast<const bf16x8*>(pa + T::S_DO), vb, dp);
      asm volatile("" : "+v"(dp));
      float p0 = prob(2 * ks), p1 = prob(2 * ks + 1);
      asm volatile("" : "+v"(p0), "+v"(p1));
      s[2 * ks] = p0;
      s[2 * ks + 1] = p1;
    }
    dp = mfma32(split_operand(-cd, h), ones, dp);
    const bf16x8 pf[2] = {pack8(s, 0), pack8(s, 1)};
    __builtin_amdgcn_sched_barrier(0);
    // dV^T += dO^T P (M = d, N = key, K = query), beside dS = P dP'.
#pragma unroll
    for (int i = 0; i < 16; ++i) dp[i] = s[i] * dp[i];
    const bf16x8 sf[2] = {pack8(dp, 0), pack8(dp, 1)};
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int pk = so + s2 * 16 * T::ROW;
#pragma unroll
      for (int db = 0; db < T::DB; ++db) {
        const bf16x8 a_do = join_tr16(lds_read_tr16(smem + aT[db][0] + pk + T::S_DO),
                                      lds_read_tr16(smem + aT[db][1] + pk + T::S_DO));
        adv[db] = mfma32(a_do, pf[s2], adv[db]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // dK^T += Q^T dS.
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int pk = so + s2 * 16 * T::ROW;
#pragma unroll
      for (int db = 0; db < T::DB; ++db) {
        const bf16x8 a_q = join_tr16(lds_read_tr16(smem + aT[db][0] + pk),
                                     lds_read_tr16(smem + aT[db][1] + pk));
        adk[db] = mfma32(a_q, sf[s2], adk[db]);
      }
    }
  };

  using yes = std::true_type;
  using no = std::false_type;
  using par0 = std::integral_constant<int, 0>;
  using par1 = std::integral_constant<int, 1>;
  using par_rt = std::integral_constant<int, -1>;
  const int diag_last = k0 + T::BCK - 2 - q_off;  // last query that misses a key
  const int head_end =
      (CAUSAL && diag_last >= 0) ? min(n_qt, diag_last / T::BRQ + 1) : qt_begin;
  const int full_end = n / T::BRQ;
  if (DOWN && qt_begin < n_qt) {
    // Highest stage first (stage = qt & 1): the stage reaching past the
    // end, then the unmasked stages [head_end, full_end) in pairs with
    // static parity (an odd stage first), then the masked stages down to
    // qt_begin.
    auto below = [&](int q) { return q - 1 >= qt_begin ? q - 1 : n_qt; };  // n_qt: none
    int qt = n_qt - 1;
    issue_stage(qt, qt & 1);
    load_stats(qt, nl, nd);
#pragma unroll 1
    for (; qt >= qt_begin && qt >= full_end; qt = __builtin_amdgcn_readfirstlane(qt - 1)) {
      tile(yes{}, par_rt{}, qt, qt & 1, below(qt));
    }
    if (qt >= head_end && qt >= qt_begin && !(qt & 1)) {
      tile(no{}, par0{}, qt, 0, below(qt));
      qt = __builtin_amdgcn_readfirstlane(qt - 1);
    }
#pragma unroll 1
    while (qt - 1 >= head_end && qt - 1 >= qt_begin) {
      tile(no{}, par1{}, qt, 1, qt - 1);
      tile(no{}, par0{}, qt - 1, 0, below(qt - 1));
      qt = __builtin_amdgcn_readfirstlane(qt - 2);
    }
#pragma unroll 1
    for (; qt >= qt_begin; qt = __builtin_amdgcn_readfirstlane(qt - 1)) {
      tile(yes{}, par_rt{}, qt, qt & 1, below(qt));
    }
  } else if (qt_begin < n_qt) {
    issue_stage(qt_begin, 0);
    load_stats(qt_begin, nl, nd);
    // Masked stages first (those holding a query that does not see the
    // workgroup's last key: query + q_off < k0 + 255), unmasked stages in
    // pairs with static stage parity (stage = (qt - qt_begin) & 1), the
    // stage reaching past the end masked.
    int qt = qt_begin;
#pragma unroll 1
    for (; qt < head_end; qt = __builtin_amdgcn_readfirstlane(qt + 1)) {
      tile(yes{}, par_rt{}, qt, (qt - qt_begin) & 1, qt + 1);
    }
    if (((qt - qt_begin) & 1) && qt < full_end) {
      tile(no{}, par1{}, qt, 1, qt + 1);
      qt = __builtin_amdgcn_readfirstlane(qt + 1);
    }
#pragma unroll 1
    while (qt + 1 < full_end) {
      tile(no{}, par0{}, qt, 0, qt + 1);
      tile(no{}, par1{}, qt + 1, 1, qt + 2);
      qt = __builtin_amdgcn_readfirstlane(qt + 2);
    }
#pragma unroll 1
    for (; qt < n_qt; qt = __builtin_amdgcn_readfirstlane(qt + 1)) {
      tile(yes{}, par_rt{}, qt, (qt - qt_begin) & 1, qt + 1);
    }
  }
  // Every fill issued by this wave has landed (the K/V fill included, even
  // when no query stage was visited) before the next tile's fills reuse LDS.
  wait_dma();

  if (key < nk) {
    float* dkr = dK + hoff_k + (int64_t)key * D;
    float* dvr = dV + hoff_k + (int64_t)key * D;
    // D layout of dK^T / dV^T: lane = key, register i -> d = db*32 + (i/4)*8 + h*4 + i%4.
#pragma unroll
    for (int db = 0; db < T::DB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = db * 32 + g * 8 + h * 4;
        f32x4 xk, xv;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          xk[t] = adk[db][4 * g + t] * scale;
          xv[t] = adv[db][4 * g + t];
        }
        *reinterpret_cast<f32x4*>(dkr + c) = xk;
        *reinterpret_cast<f32x4*>(dvr + c) = xv;
      }
    }
  }
  if (visits != nullptr && w == 0 && lane == 0) {
    visits[(int64_t)head * n_ktiles + kt] = nvis;
  }
  };

  // Causal pairs: the first (long) tile walks down from the last query
  // stage and the second walks up from its diagonal.  Tiles u and
  // n_ktiles-1-u hold the same total work for every u, so at any moment the
  // workgroups of a head read one of two query stages (the first tiles
  // going down from the end, the second tiles going up from a common
  // position), and their Q/dO reads share the XCD's L2 instead of spreading
  // over the whole head.
  run_tile(kt_a, std::integral_constant<bool, CAUSAL>{});
  if (CAUSAL && kt_b >= 0) {
    __syncthreads();  // every wave is done with K, V and the stages
    run_tile(kt_b, std::false_type{});
  }
}

// ---------------------------------------------------------------------------
// dq pass
// ---------------------------------------------------------------------------
template <int D, int NW_>
struct QTile {
  static constexpr int NW = NW_;
  static constexpr int BRQ = 32 * NW;                 // queries per workgroup
  static constexpr int BCK = (D == 128) ? 64 : 128;   // keys per LDS tile
  static constexpr int KS = D / 16;
  static constexpr int KB = BCK / 32;
  static constexpr int DB = D / 32;
  static constexpr int ROW = D * 2;
  static constexpr int T_BYTES = BCK * ROW;
  // stage layout: K | V, two stages
  static constexpr int OFF_V = T_BYTES;
  static constexpr int STAGE = 2 * T_BYTES;
  static constexpr int BLK = T_BYTES / 1024 / NW;     // 1-KB DMA blocks per wave
  static_assert(BLK * NW * 1024 == T_BYTES, "tile splits into 1-KB blocks");
};

// With d = 128 a workgroup has 8 waves (256 queries, one workgroup per CU),
// which halves the K/V tile traffic into LDS per query row; with d = 64 it
// has 4 waves and two run per CU.  Wave w owns queries q0 + 32w .. + 31; Q
// and dO stay in registers as B operands.  K/V tiles are double-buffered
// and filled by direct global-to-LDS loads one tile ahead.
template <int D, int NW, bool CAUSAL, bool SPARSE, bool DROP>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                   const bf16* __restrict__ V, const bf16* __restrict__ dO,
                   const bf16* __restrict__ O, const float* __restrict__ lse,
                   float* __restrict__ ws_d, float* __restrict__ ws_lse2,
                   float* __restrict__ dQ,
                   int n, int nk, int q_off, int n_qtiles, int total,
                   int bundle, float c_log2, float scale,
                   const uint8_t* __restrict__ mask, int mask_cols, int block_m,
                   int block_n, Dropout drop, int* __restrict__ visits) {
  using T = QTile<D, NW>;
  // (The dropout instances keep one block at a time: the pipeline does not
  // fit their registers next to the random bytes.)
  constexpr bool DQ_PIPE = !DROP;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * T::STAGE];

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  const int lid = xcd_logical_id(blockIdx.x, total);
  // Dense causal with 256-row tiles: the workgroup takes query tiles
  // n_qtiles-1-u and u of one head (equal work for every workgroup, see the
  // forward kernel).
  constexpr bool PAIRS = CAUSAL && !SPARSE && NW == 8;
  int head, qt_a, qt_b = -1;
  if constexpr (PAIRS) {
    const int units = (n_qtiles + 1) / 2;
    const int u = lid % units;
    head = lid / units;
    qt_a = n_qtiles - 1 - u;
    if (u != qt_a) qt_b = u;
  } else {
    const CausalPlace pl = CAUSAL ? causal_place(lid, n_qtiles, total / n_qtiles, bundle)
                                  : CausalPlace{lid / n_qtiles, lid % n_qtiles};
    head = pl.head;
    qt_a = CAUSAL ? (n_qtiles - 1 - pl.rank) : pl.rank;
  }
  const int64_t hoff = (int64_t)head * n * D;     // Q, dO, dQ: n rows per head
  const int64_t hoff_k = (int64_t)head * nk * D;  // K, V: nk rows
  const bf16* Kh = K + hoff_k;
  const bf16* Vh = V + hoff_k;
  drop.bh = (uint32_t)head;

  // One query tile of 32 * NW rows; REV walks its key tiles from the
  // diagonal down to key 0 instead of up.
  auto run_tile = [&](int qt, auto rev_tag) {
  constexpr bool REV = decltype(rev_tag)::value;
  const int q0 = qt * T::BRQ;
  const int qw0 = q0 + 32 * w;
  const int qrow = qw0 + l32;

  bf16x8 qf[T::KS], dof[T::KS];
#pragma unroll
  for (int ks = 0; ks < T::KS; ++ks) {
    qf[ks] = as_bf16x8(load_row16(Q + hoff, qrow, n, D, ks * 16 + h * 8));
    dof[ks] = as_bf16x8(load_row16(dO + hoff, qrow, n, D, ks * 16 + h * 8));
  }
  // The row statistics: with O given, computed here from O, dO and the
  // forward's logsumexp and written to the workspace for the dK/dV pass
  // (which then runs after this one), else read from the workspace.
  float lrow, drow;
  if (O != nullptr) {
    // D = sum_c dO_c O_c in fp32, summed in the order of the streaming
    // preprocess (one chain per 8 columns, then a pairwise tree over the
    // chunks), so that both routes give the same bits: this lane holds the
    // chunks 2ks + h, the tree's last level pairs the two half-waves.
    float part[T::KS];
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) {
      const u32x4 ov = load_row16(O + hoff, qrow, n, D, ks * 16 + h * 8);
      const u32x4 dv = __builtin_bit_cast(u32x4, dof[ks]);
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc = fmaf(bf16_lo(ov[i]), bf16_lo(dv[i]), acc);
        acc = fmaf(bf16_hi(ov[i]), bf16_hi(dv[i]), acc);
      }
      part[ks] = acc;
    }
#pragma unroll
    for (int st = T::KS / 2; st > 0; st >>= 1) {
#pragma unroll
      for (int ks = 0; ks < st; ++ks) part[ks] += part[ks + st];
    }
    const float dsum = sum_halves(part[0]);
    const float L = (qrow < n) ? lse[(int64_t)head * n + qrow] : -INFINITY;
    lrow = (L == -INFINITY) ? INFINITY : L * kLog2e;
    drow = (qrow < n) ? dsum : 0.f;
    if (h == 0 && qrow < n) {
      ws_d[(int64_t)head * n + qrow] = drow;
      ws_lse2[(int64_t)head * n + qrow] = lrow;
    }
  } else {
    lrow = (qrow < n) ? ws_lse2[(int64_t)head * n + qrow] : INFINITY;
    drow = (qrow < n) ? ws_d[(int64_t)head * n + qrow] : 0.f;
  }

  f32x16 adq[T::DB];
#pragma unroll
  for (int db = 0; db < T::DB; ++db) adq[db] = zero16();

  int aoff[T::KS];  // row-wise A operand: row l32 (+ kb*32), chunk ks*2 + h
#pragma unroll
  for (int ks = 0; ks < T::KS; ++ks) aoff[ks] = tile_off<D>(l32, ks * 2 + h);
  int toff[T::DB][2];
  tr_offsets<D, T::DB>(lane, toff);
  // DMA sources: lane `lane` fills bytes 16*lane of 1-KB block w + NW*i of a
  // tile, i.e. row o / ROW, physical chunk (o % ROW) / 16 = logical chunk ^
  // swizzle; element offsets from the tile's first row.
  int goff[T::BLK];
#pragma unroll
  for (int i = 0; i < T::BLK; ++i) {
    const int o = (w + NW * i) * 1024 + lane * 16;
    const int row = o / T::ROW;
    goff[i] = row * D + ((((o % T::ROW) >> 4) ^ tile_swz<D>(row)) * 8);
  }
  auto fill = [&](int kt, int stage) {
    unsigned char* st = smem + stage * T::STAGE;
    const int kb0 = kt * T::BCK;
    const bf16* kbase = Kh + (int64_t)kb0 * D;
    const bf16* vbase = Vh + (int64_t)kb0 * D;
    if (kb0 + T::BCK <= nk) {
#pragma unroll
      for (int i = 0; i < T::BLK; ++i) {
        dma16(kbase + (uint32_t)goff[i], st + (w + NW * i) * 1024);
        dma16(vbase + (uint32_t)goff[i], st + T::OFF_V + (w + NW * i) * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < T::BLK; ++i) {
        dma_tile_block<D>(Kh, kb0, nk, st, w + NW * i, lane);
        dma_tile_block<D>(Vh, kb0, nk, st + T::OFF_V, w + NW * i, lane);
      }
    }
  };

  const int n_kt = (nk + T::BCK - 1) / T::BCK;
  // (The tile's last row sees the keys up to q_off + that row, q_off >= 0.)
  const int kt_end =
      CAUSAL ? min(n_kt, (min(q0 + T::BRQ, n) - 1 + q_off) / T::BCK + 1) : n_kt;
  // Whether tile kt has keys after some query of this wave or past the end.
  auto needs_mask = [&](int kt) {
    const int kbase = kt * T::BCK;
    return (CAUSAL && kbase + T::BCK - 1 > qw0 + q_off) || (kbase + T::BCK > nk);
  };

  // One key tile: wait for it (loaded one tile ahead) and let every wave
  // finish the previous one, load the next tile into the freed stage, then
  // accumulate dQ^T.  PAR is the stage parity when known at compile time
  // (every LDS address is then a register plus an immediate), else -1.
  // Block-sparse: the key tiles whose mask block in this workgroup's row is
  // nonzero (a workgroup's 128 rows lie in one block row, a key tile in one
  // block column).
  MaskLine mline(SPARSE ? mask + (int64_t)(q0 / block_m) * mask_cols : mask, 1,
                 SPARSE ? mask_cols : 0, lane);
  auto next_on = [&](int kt) -> int {
    ++kt;
    if constexpr (SPARSE) {
      if (kt < kt_end) {
        const int col = (kt * T::BCK) / block_n;
        const int nc = mline.next(col, lane);
        if (nc != col) kt = min(kt_end, (int)(((int64_t)nc * block_n) / T::BCK));
      }
    }
    return __builtin_amdgcn_readfirstlane(kt);
  };
  int nvis = 0;  // key tiles visited (diagnostic count)
  auto tile = [&](auto mask_tag, auto par_tag, int kt, int stage_rt, int kt_next) {
    constexpr bool MASK = decltype(mask_tag)::value;
    constexpr int PAR = decltype(par_tag)::value;
    const int stage = (PAR >= 0) ? PAR : stage_rt;
    ++nvis;
    wait_dma();
    __syncthreads();
    if (kt_next >= 0 && kt_next < kt_end) fill(kt_next, stage ^ 1);
    const unsigned char* st = smem + stage * T::STAGE;
    const int kbase = kt * T::BCK;
    // Last visible key of this lane's row relative to the key in register 0
    // of block 0 (register i of block kb holds key kb*32 + (i/4)*8 + i%4
    // relative to it).
    const int lim = (CAUSAL ? min(qrow + q_off, nk - 1) : nk - 1) - kbase - h * 4;
    // S^T = K Q^T and dP^T = V dO^T of 32-key block kb (M = key, N = query).
    // Dropout: u receives the block's random bytes, the draw's ten rounds
    // spread between the products (held there by empty asm statements).
    auto scores = [&](int kb, f32x16& s, f32x16& dp, uint32_t (&u)[4]) {
      s = zero16();
      dp = zero16();
      if constexpr (DROP) dropout_ctr_rowlane(drop, qrow, kbase + kb * 32, lane, u);
#pragma unroll
      for (int ks = 0; ks < T::KS; ++ks) {
        const unsigned char* pa = st + kb * 32 * T::ROW + aoff[ks];
        s = mfma32(*reinterpret_cast<const bf16x8*>(pa), qf[ks], s);
        dp = mfma32(*reinterpret_cast<const bf16x8*>(pa + T::OFF_V), dof[ks], dp);
        if constexpr (DROP) {
          asm volatile("" : "+v"(s), "+v"(dp));
#pragma unroll
          for (int r = ks * 10 / T::KS; r < (ks + 1) * 10 / T::KS; ++r)
            philox_round(u, drop.k0 + r * kWeyl0, drop.k1 + r * kWeyl1);
          asm volatile("" : "+v"(u[0]), "+v"(u[1]), "+v"(u[2]), "+v"(u[3]));
        }
      }
      if constexpr (DROP) quad_transpose(u, lane);
    };
    // dS^T of block kb from its S^T and dP^T (bf16, the B operand of the dQ
    // product).
    auto dsv = [&](int kb, f32x16& s, f32x16& dp, bf16x8 (&sf)[2],
                   const uint32_t (&u)[4]) {
      // Dropout: dS takes the kept and rescaled dP.
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float p = fast_exp2(fmaf(s[i], c_log2, -lrow));
        if constexpr (MASK) {
          if (kb * 32 + (i >> 2) * 8 + (i & 3) > lim) p = 0.f;
        }
        float dpv = dp[i];
        if constexpr (DROP)
          dpv = dropout_keep(u[i >> 2], i & 3, drop.t) ? dpv * drop.inv_keep : 0.f;
        dp[i] = p * (dpv - drow);
      }
      sf[0] = pack8(dp, 0);
      sf[1] = pack8(dp, 1);
    };
    // dQ^T += K^T dS^T of block kb (M = d, N = query, K = key); K^T from
    // transpose reads of the K tile.
    auto dq = [&](int kb, const bf16x8 (&sf)[2]) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const unsigned char* pk = st + (kb * 2 + s2) * 16 * T::ROW;
#pragma unroll
        for (int db = 0; db < T::DB; ++db) {
          const bf16x8 a = join_tr16(lds_read_tr16(pk + toff[db][0]),
                                     lds_read_tr16(pk + toff[db][1]));
          adq[db] = mfma32(a, sf[s2], adq[db]);
        }
      }
    };
    if constexpr (DQ_PIPE) {
      // Software pipeline over the 32-key blocks: step kb issues the score
      // products of block kb + 1 and the dQ products of block kb - 1 next to
      // block kb's vector work.
      f32x16 s[2], dp[2];
      bf16x8 sf[2][2];
      uint32_t u[4];  // (no dropout here)
      scores(0, s[0], dp[0], u);
#pragma unroll
      for (int kb = 0; kb <= T::KB; ++kb) {
        if (kb + 1 < T::KB) scores(kb + 1, s[(kb + 1) & 1], dp[(kb + 1) & 1], u);
        if (kb >= 1) dq(kb - 1, sf[(kb - 1) & 1]);
        if (kb < T::KB) dsv(kb, s[kb & 1], dp[kb & 1], sf[kb & 1], u);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb) {
        f32x16 s, dp;
        bf16x8 sf[2];
        uint32_t u[4];
        scores(kb, s, dp, u);
        dsv(kb, s, dp, sf, u);
        dq(kb, sf);
        // One 32-key block at a time: its score registers are free before
        // the next block's products, room the scheduler uses to keep two LDS
        // operands in flight.
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  using yes = std::true_type;
  using no = std::false_type;
  using par0 = std::integral_constant<int, 0>;
  using par1 = std::integral_constant<int, 1>;
  using par_rt = std::integral_constant<int, -1>;
  if constexpr (SPARSE && D == 128) {
    // Visited tiles in order, each in the masked form, the stage parity
    // alternating at run time (a second, unmasked copy of the tile does not
    // fit the registers at d = 128).
    int kt = next_on(-1);
    if (kt < kt_end) fill(kt, 0);
    int stage = 0;
#pragma unroll 1
    while (kt < kt_end) {
      const int kn = next_on(kt);
      tile(yes{}, par_rt{}, kt, stage, kn);
      kt = kn;
      stage ^= 1;
    }
  } else if constexpr (SPARSE) {
    // Visited tiles in order: the unmasked ones in pairs with static stage
    // parity (the parity alternates over visited tiles), then those needing
    // this wave's element mask (they come last: keys increase along the
    // visit order).  Separate loops keep each tile body one basic block.
    int kt = next_on(-1);
    if (kt < kt_end) fill(kt, 0);
    int stage = 0;
#pragma unroll 1
    while (kt < kt_end && !needs_mask(kt)) {
      int kn = next_on(kt);
      tile(no{}, par0{}, kt, 0, kn);
      kt = kn;
      stage = 1;
      if (!(kt < kt_end && !needs_mask(kt))) break;
      kn = next_on(kt);
      tile(no{}, par1{}, kt, 1, kn);
      kt = kn;
      stage = 0;
    }
#pragma unroll 1
    for (; kt < kt_end; stage ^= 1) {
      const int kn = next_on(kt);
      tile(yes{}, par_rt{}, kt, stage, kn);
      kt = kn;
    }
  } else if constexpr (REV) {
    // Key tile kt sits in stage kt & 1 in either direction.  Downwards the
    // tiles needing the element mask come first, then (from an odd tile
    // on) unmasked pairs with static stage parity.
    int kt = kt_end - 1;
    if (kt >= 0) fill(kt, kt & 1);
#pragma unroll 1
    for (; kt >= 0 && (needs_mask(kt) || !(kt & 1));
         kt = __builtin_amdgcn_readfirstlane(kt - 1)) {
      tile(yes{}, par_rt{}, kt, kt & 1, kt - 1);
    }
#pragma unroll 1
    for (; kt > 0; kt = __builtin_amdgcn_readfirstlane(kt - 2)) {
      tile(no{}, par1{}, kt, 1, kt - 1);
      tile(no{}, par0{}, kt - 1, 0, kt - 2);
    }
  } else if (kt_end > 0) {
    fill(0, 0);
    // Tiles needing the element mask come last; unmasked tiles run in
    // pairs with static stage parity.
    int kt = 0;
#pragma unroll 1
    while (kt + 1 < kt_end && !needs_mask(kt + 1)) {
      tile(no{}, par0{}, kt, 0, kt + 1);
      tile(no{}, par1{}, kt + 1, 1, kt + 2);
      kt = __builtin_amdgcn_readfirstlane(kt + 2);
    }
    // (At most one unmasked tile remains here; it takes the masked form,
    // whose mask is then a no-op.)
#pragma unroll 1
    for (; kt < kt_end; kt = __builtin_amdgcn_readfirstlane(kt + 1)) {
      tile(yes{}, par_rt{}, kt, kt & 1, kt + 1);
    }
  }

  if (qrow < n) {
    float* dqr = dQ + hoff + (int64_t)qrow * D;
#pragma unroll
    for (int db = 0; db < T::DB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 x = {adq[db][4 * g] * scale, adq[db][4 * g + 1] * scale,
                   adq[db][4 * g + 2] * scale, adq[db][4 * g + 3] * scale};
        *reinterpret_cast<f32x4*>(dqr + db * 32 + g * 8 + h * 4) = x;
      }
    }
  }
  if (visits != nullptr && w == 0 && lane == 0) {
    visits[(int64_t)head * n_qtiles + qt] = nvis;
  }
  };

  // The second tile of a pair walks its keys downwards.  Tiles u and
  // n_qtiles-1-u together hold n_qtiles+1 tiles' worth of keys for every pair,
  // so at any time the workgroups of a head read one of two key tiles:
  // first tiles at position t going up, second tiles at the common position
  // (n_qtiles+1)*256 - t going down.  The re-reads of K and V then hit the
  // XCD's L2 instead of HBM.
  // (The dropout instance keeps the upward walk: the downward one would
  // not fit its registers.)
  run_tile(qt_a, std::false_type{});
  if constexpr (PAIRS) {
    if (qt_b >= 0) {
      __syncthreads();  // every wave is done with the K/V stages
      run_tile(qt_b, std::integral_constant<bool, !DROP>{});
    }
  }
}

template <int D>
hipError_t pre_t(const BwdArgs& a, hipStream_t s) {
  const int64_t rows = a.bh * a.n;
  const int per = 256 / (D / 8);
  const int64_t grid = (rows + per - 1) / per;
  return launch_kernel(bwd_pre_kernel<D>, dim3((unsigned)grid), dim3(256), s,
                       (const bf16*)a.o, (const bf16*)a.dout, a.lse, a.ws_d,
                       a.ws_lse2, rows);
}

template <int D, bool CAUSAL, bool SPARSE, bool DROP>
hipError_t dkdv_t(const BwdArgs& a, hipStream_t s) {
  using T = KVTile<D>;
  const int n_kt = (a.nk + T::BCK - 1) / T::BCK;
  // Dense causal workgroups take two key tiles each (see the kernel).
  const int units = (CAUSAL && !SPARSE) ? (n_kt + 1) / 2 : n_kt;
  const int total = (int)(a.bh * units);
  return launch_kernel(bwd_dkdv_kernel<D, CAUSAL, SPARSE, DROP>, dim3(total), dim3(512), s,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v,
                       (const bf16*)a.dout, (const float*)a.ws_d,
                       (const float*)a.ws_lse2, a.dk, a.dv, a.n, a.nk, a.q_off,
                       n_kt, total,
                       causal_bundle(n_kt, 1), a.scale * kLog2e, a.scale,
                       a.mask, a.mask_cols, a.block_m, a.block_n,
                       make_dropout(a.drop_t, a.seed_lo, a.seed_hi, a.q_off), a.visits_kv);
}

// d = 128 dense: 8-wave workgroups (256 query rows); block-sparse keeps 128
// rows so that a workgroup lies in one 128-multiple block row of the mask.
template <int D, bool CAUSAL, bool SPARSE, bool DROP>
hipError_t dq_t(const BwdArgs& a, hipStream_t s, bool stats) {
  constexpr int NW = (D == 128 && !SPARSE) ? 8 : 4;
  using T = QTile<D, NW>;
  const int n_qt = (a.n + T::BRQ - 1) / T::BRQ;
  // Dense causal 8-wave workgroups take two tiles each (see the kernel).
  const int units = (CAUSAL && !SPARSE && NW == 8) ? (n_qt + 1) / 2 : n_qt;
  const int total = (int)(a.bh * units);
  return launch_kernel(bwd_dq_kernel<D, NW, CAUSAL, SPARSE, DROP>, dim3(total),
                       dim3(NW * 64), s, (const bf16*)a.q, (const bf16*)a.k,
                       (const bf16*)a.v, (const bf16*)a.dout,
                       stats ? (const bf16*)a.o : nullptr, stats ? a.lse : nullptr,
                       a.ws_d, a.ws_lse2, a.dq, a.n, a.nk, a.q_off, n_qt,
                       total,
                       causal_bundle(n_qt, NW == 8 ? 1 : 2), a.scale * kLog2e,
                       a.scale, a.mask, a.mask_cols, a.block_m, a.block_n,
                       make_dropout(a.drop_t, a.seed_lo, a.seed_hi, a.q_off), a.visits_q);
}

template <bool CAUSAL>
hipError_t dkdv256_t(const BwdArgs& a, hipStream_t s) {
  using T = KV256Tile;
  const int n_kt = (a.nk + T::BCK - 1) / T::BCK;
  const int units = CAUSAL ? (n_kt + 1) / 2 : n_kt;
  const int total = (int)(a.bh * units);
  return launch_kernel(bwd_dkdv256_kernel<CAUSAL>, dim3(total), dim3(512), s,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v,
                       (const bf16*)a.dout, (const float*)a.ws_d,
                       (const float*)a.ws_lse2, a.dk, a.dv, a.n, a.nk, a.q_off,
                       n_kt, total, a.scale * kLog2e, a.scale, a.visits_kv);
}

// d = 128 without mask or dropout: the 256-key kernel; otherwise 128 keys
// per workgroup, with the block-sparse and/or dropout instances.
template <int D>
hipError_t dkdv_c(const BwdArgs& a, hipStream_t s) {
  if (D == 128 && !a.mask && a.drop_t == 0) {
    return a.causal ? dkdv256_t<true>(a, s) : dkdv256_t<false>(a, s);
  }
  if (a.mask) {
    if (a.drop_t > 0) {
      return a.causal ? dkdv_t<D, true, true, true>(a, s) : dkdv_t<D, false, true, true>(a, s);
    }
    return a.causal ? dkdv_t<D, true, true, false>(a, s) : dkdv_t<D, false, true, false>(a, s);
  }
  if (a.drop_t > 0) {
    return a.causal ? dkdv_t<D, true, false, true>(a, s) : dkdv_t<D, false, false, true>(a, s);
  }
  return a.causal ? dkdv_t<D, true, false, false>(a, s) : dkdv_t<D, false, false, false>(a, s);
}
template <int D>
hipError_t dq_c(const BwdArgs& a, hipStream_t s, bool stats) {
  if (a.mask) {
    if (a.drop_t > 0) {
      return a.causal ? dq_t<D, true, true, true>(a, s, stats) : dq_t<D, false, true, true>(a, s, stats);
    }
    return a.causal ? dq_t<D, true, true, false>(a, s, stats) : dq_t<D, false, true, false>(a, s, stats);
  }
  if (a.drop_t > 0) {
    return a.causal ? dq_t<D, true, false, true>(a, s, stats) : dq_t<D, false, false, true>(a, s, stats);
  }
  return a.causal ? dq_t<D, true, false, false>(a, s, stats) : dq_t<D, false, false, false>(a, s, stats);
}

}  // namespace

void bwd_dkdv_tile_grid(int d, bool sparse, int* rows, int* cols) {
  if (d == 128 && !sparse) {
    *rows = KV256Tile::BRQ;
    *cols = KV256Tile::BCK;
    return;
  }
  *rows = (d == 128) ? KVTile<128>::BRQ : KVTile<64>::BRQ;
  *cols = (d == 128) ? KVTile<128>::BCK : KVTile<64>::BCK;
}

void bwd_dq_tile_grid(int d, bool sparse, int* rows, int* cols) {
  *rows = (d == 128 && !sparse) ? QTile<128, 8>::BRQ : QTile<64, 4>::BRQ;
  *cols = (d == 128) ? QTile<128, 8>::BCK : QTile<64, 4>::BCK;
}

hipError_t launch_bwd_preprocess(const BwdArgs& a, hipStream_t s) {
  return a.d == 128 ? pre_t<128>(a, s) : pre_t<64>(a, s);
}

hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t s) {
  return a.d == 128 ? dkdv_c<128>(a, s) : dkdv_c<64>(a, s);
}

hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t s) {
  return a.d == 128 ? dq_c<128>(a, s, false) : dq_c<64>(a, s, false);
}

hipError_t launch_bwd_dq_stats(const BwdArgs& a, hipStream_t s) {
  return a.d == 128 ? dq_c<128>(a, s, true) : dq_c<64>(a, s, true);
}

}  // namespace fa
