// Forward pass, bf16 inputs, fp32 accumulation, gfx950 MFMA.
//
// Pages cited (titles as published):
//   [TLDR]   "FlashAttention：メモリ効率的なアテンション計算" (tech-tldr.com)
//   [XYZ]    "FlashAttention: IOを意識した高速かつメモリ効率の高い厳密な
//            アテンション" (xyznot.com)
//   [REAPER] "3 · FlashAttention" (mkdocs.reaper.mx, chapter 3)
//   [LLMSYS] "출력을 누적해 메모리 이동을 줄이는 FlashAttention"
//
// Algorithm: for a block of query rows, stream the key/value tiles
// through LDS; per tile compute the score tile on the matrix cores, update
// the running row max m, running exp-sum l and the unnormalised output
// accumulator, and divide by l once after the last tile ([TLDR] online
// softmax and tiling sections; [REAPER] sections 3.2-3.3; [LLMSYS] Fig. 3).
// The score and probability tiles live only in registers.  Under the causal
// rule key tiles entirely above the diagonal are never visited ([REAPER],
// causal-mask question); in the block-sparse variant key tiles whose mask
// block is 0 are never visited ([XYZ], block-sparse extension).
//
// MI355X mapping (wave w of a workgroup owns query rows q0 + 32w ..
// q0 + 32w + 31; two waves per SIMD: for d = 128 one workgroup of 8 waves
// per CU, otherwise two workgroups of 4 waves):
//   * S is computed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16:
//     K comes from LDS as the A operand, Q stays in registers as the B
//     operand for the whole key loop.  In the D layout each lane then owns a
//     single query row (lane % 32) and 16 keys per 32x32 block, so the row max
//     and row sum are in-register reductions plus one exchange between the
//     two halves of the wave, and the rescale factor is a per-lane scalar.
//   * The exponentials are exp2 with scale*log2(e) folded into one FMA.
//   * O^T = V^T P^T on the same MFMA: P leaves the exponentials already in
//     the B-operand layout (after bf16 rounding).  V stays row-major in LDS
//     and its transposed A operand is read with ds_read_b64_tr_b16; the key
//     order of those reads matches the key order of P's registers (the
//     contraction index is a dummy, so both sides only have to agree).
//   * Software pipeline inside each wave: while the matrix cores compute
//     the score tile of key tile j+1, the vector units turn tile j's scores
//     into probabilities (two after each product, an order held by empty
//     asm statements); while they compute tile j's PV product, the vector
//     units add tile j's row sum (d = 128) and mask and reduce tile j+1's
//     scores to its row max.  K therefore runs one tile ahead of V: both are
//     double-buffered in LDS and filled by direct global-to-LDS loads issued
//     one tile ahead.  With dropout the next tile's score products carry
//     this tile's random draws (the Philox rounds, spread between them)
//     instead, and the probabilities follow.
//   * The running max is only moved (and the accumulator rescaled) when a
//     row's tile max exceeds it by more than 8 in log2 units; any reference
//     value gives the same quotient, and probabilities stay below 2^8.
//   * 16-byte chunks are XOR-swizzled per row so that the tile fills and the
//     fragment reads are free of bank conflicts; LDS read addresses are
//     loop-invariant per-lane offsets.
//   * The workgroup order keeps each head on one XCD (shared L2) and, under
//     the causal rule, starts the longest query tiles first.
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

template <int D_, int NW_, int BC_ = (D_ == 128) ? 64 : 128>
struct FwdTile {
  static constexpr int D = D_;
  static constexpr int NW = NW_;                      // waves per workgroup
  static constexpr int BR = 32 * NW;                  // query rows per workgroup
  static constexpr int BC = BC_;                      // keys per tile
  static constexpr int KS = D / 16;                   // MFMA k-steps over d
  static constexpr int KB = BC / 32;                  // 32-key blocks per tile
  static constexpr int KK = BC / 16;                  // 16-key k-steps of PV
  static constexpr int DB = D / 32;                   // 32-wide blocks of d
  static constexpr int ROW = D * 2;                   // bytes per K / V row
  static constexpr int K_BYTES = BC * ROW;            // one K or V tile
  static constexpr int BLK = K_BYTES / 1024 / NW;     // 1-KB DMA blocks per wave
  static_assert(BLK * NW * 1024 == K_BYTES, "tile splits into 1-KB blocks");
  static constexpr float RESCALE_SLACK = 8.f;         // log2 units
};

// Chunk swizzle of the K tile.  Fragment reads take one chunk from 16
// consecutive rows per quarter-wave: with 256-B rows XOR by (row & 15), with
// 128-B rows (two rows per bank line) XOR by ((row >> 1) & 7).
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  return (D == 128) ? (row & 15) : ((row >> 1) & 7);
}
// Chunk swizzle of the V tile.  A transpose read takes a 64-B run (4 chunks)
// from 8 consecutive rows; XOR-ing bits 2-3 of the chunk index by
// (row & 3) (256-B rows) or by ((row >> 1) & 1) (128-B rows) puts rows 0-3
// on disjoint banks, so each read costs the minimum two LDS cycles.
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  return (D == 128) ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
}

// Source of lane `lane` in 1-KB block i (= w + NW*i) of a K or V tile with
// chunk swizzle SWZ: the lane fills bytes 16*lane of the block, i.e. row
// o / ROW, physical chunk (o % ROW) / 16, which holds logical chunk
// physical ^ SWZ(row).  Returns the element offset from the tile's first
// row; `row` receives the tile row.
template <class T, int (*SWZ)(int)>
__device__ __forceinline__ int tile_src(int w, int lane, int i, int& row) {
  const int o = (w + T::NW * i) * 1024 + lane * 16;
  row = o / T::ROW;
  return row * T::D + ((((o % T::ROW) >> 4) ^ SWZ(row)) * 8);
}

// Direct global-to-LDS fills of K and V tiles: each wave fills BLK of the
// tile's 1-KB blocks.  Full tiles use precomputed per-lane source offsets;
// rows of the last tile at or past n are clamped to n - 1.
template <class T>
struct TileFill {
  int koff[T::BLK], voff[T::BLK];
  int w, lane;

  __device__ __forceinline__ TileFill(int w_, int lane_) : w(w_), lane(lane_) {
#pragma unroll
    for (int i = 0; i < T::BLK; ++i) {
      int row;
      koff[i] = tile_src<T, swz_k<T::D>>(w, lane, i, row);
      voff[i] = tile_src<T, swz_v<T::D>>(w, lane, i, row);
    }
  }
  template <int (*SWZ)(int)>
  __device__ __forceinline__ void fill(const bf16* g, int kbase, int n,
                                       unsigned char* tile,
                                       const int (&off)[T::BLK]) const {
    const bf16* base = g + (int64_t)kbase * T::D;
    if (kbase + T::BC <= n) {
#pragma unroll
      for (int i = 0; i < T::BLK; ++i) {
        dma16(base + (uint32_t)off[i], tile + (w + T::NW * i) * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < T::BLK; ++i) {
        int row;
        const int o = tile_src<T, SWZ>(w, lane, i, row);
        const int over = max(kbase + row - (n - 1), 0);  // rows to pull back
        dma16(base + (o - over * T::D), tile + (w + T::NW * i) * 1024);
      }
    }
  }
  __device__ __forceinline__ void k(const bf16* g, int kbase, int n,
                                    unsigned char* tile) const {
    fill<swz_k<T::D>>(g, kbase, n, tile, koff);
  }
  __device__ __forceinline__ void v(const bf16* g, int kbase, int n,
                                    unsigned char* tile) const {
    fill<swz_v<T::D>>(g, kbase, n, tile, voff);
  }
};

// The per-wave part of the forward: 32 query rows, their Q fragments, the
// output accumulator and the online-softmax state ([TLDR] online softmax;
// [REAPER] 3.3), and the matrix-core and vector steps on one key tile.
template <class T, bool CAUSAL, bool DROP = false>
struct FwdWave {
  static constexpr int D = T::D;
  bf16x8 qf[T::KS];    // Q as the B operand of S^T = K Q^T
  f32x16 acc[T::DB];   // O^T, unnormalised
  // m is the reference max in log2 units of the scaled score; it only moves
  // when a tile max exceeds it by more than the slack, and any reference
  // gives the same quotient.  m_use is m with -inf replaced by 0, the value
  // subtracted inside the exponentials; l is the running exp-sum over this
  // half-wave's keys.
  float m, m_use, l;
  int koff[T::KS];     // K fragment LDS offsets
  int voff[T::DB];     // V^T fragment (transpose read) LDS offsets
  // n: query rows; nk: keys; q_off: the position of query row 0 in the key
  // sequence (the causal rule is key <= q_off + row).
  int qw0, qrow, h, n, nk, q_off;
  float c_log2;
  Dropout dr;          // used when DROP

  __device__ __forceinline__ FwdWave(const bf16* Qh, int qw0_, int lane, int n_,
                                     int nk_, int q_off_, float c_log2_)
      : m(-INFINITY), m_use(0.f), l(0.f), qw0(qw0_), qrow(qw0_ + (lane & 31)),
        h(lane >> 5), n(n_), nk(nk_), q_off(q_off_), c_log2(c_log2_) {
    const int l32 = lane & 31;
    // Slot j of k-step ks is Q[qrow][ks*16 + h*8 + j].
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) {
      qf[ks] = as_bf16x8(load_row16(Qh, qrow, n, D, ks * 16 + h * 8));
    }
#pragma unroll
    for (int db = 0; db < T::DB; ++db) acc[db] = zero16();
    // K fragment (A of S^T): row kb*32 + l32, chunk ks*2 + h.
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) {
      koff[ks] = l32 * T::ROW + (((ks * 2 + h) ^ swz_k<D>(l32)) << 4);
    }
    // V^T fragment (A of O^T) by transpose reads: source lane s = lane % 16
    // of group g = lane / 16 addresses key kk*16 + r2*8 + h*4 + s/4 at
    // column db*32 + 16*(g & 1) + 4*(s % 4); slots 0-3 (r2 = 0) and 4-7
    // (r2 = 1) then hold keys {h*4 + 0..3} and {8 + h*4 + 0..3} of the
    // 16-key group, the same keys P's registers hold.
    const int s16 = lane & 15, g = lane >> 4;
    const int krow = h * 4 + (s16 >> 2);
#pragma unroll
    for (int db = 0; db < T::DB; ++db) {
      const int col = db * 32 + 16 * (g & 1) + 4 * (s16 & 3);
      voff[db] = krow * T::ROW + (((col >> 3) ^ swz_v<D>(krow)) << 4) +
                 (col & 7) * 2;
    }
  }

  // S^T = K Q^T of the K tile at sk (KB blocks of 32 keys).
  __device__ __forceinline__ void scores(const unsigned char* sk,
                                         f32x16 (&s)[T::KB]) const {
#pragma unroll
    for (int kb = 0; kb < T::KB; ++kb) {
      s[kb] = zero16();
#pragma unroll
      for (int ks = 0; ks < T::KS; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
            sk + kb * 32 * T::ROW + koff[ks]);
        s[kb] = mfma32(a, qf[ks], s[kb]);
      }
    }
  }

  // Whether the tile starting at key kbase has keys past the diagonal or
  // past the sequence end for some row of this wave (wave-uniform).
  __device__ __forceinline__ bool needs_mask(int kbase) const {
    return (CAUSAL && kbase + T::BC - 1 > q_off + qw0) || (kbase + T::BC > nk);
  }
  // Set those keys to -inf.  lim is the last visible key of the lane's row
  // relative to the key in register 0 of block 0; register i of block kb
  // holds key kb*32 + (i/4)*8 + (i%4) relative to it.
  __device__ __forceinline__ void apply_mask(f32x16 (&s)[T::KB],
                                             int kbase) const {
    const int lim = (CAUSAL ? min(q_off + qrow, nk - 1) : nk - 1) - kbase - h * 4;
#pragma unroll
    for (int kb = 0; kb < T::KB; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (kb * 32 + (i >> 2) * 8 + (i & 3) > lim) s[kb][i] = -INFINITY;
      }
    }
  }
  // Row max of a score tile in log2 units.
  __device__ __forceinline__ float tile_max(const f32x16 (&s)[T::KB]) const {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < T::KB; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    }
    return max_halves(mx) * c_log2;
  }
  // Move the reference max to cover tile max mx; rescale l and the
  // accumulator when it moves (any lane of the wave).
  __device__ __forceinline__ void move_max(float mx) {
    const bool move = mx > m + T::RESCALE_SLACK;
    const float m_new = move ? mx : m;
    const float m_use_new = (m_new == -INFINITY) ? 0.f : m_new;
    if (__ballot(move)) {
      const float alpha = fast_exp2(m - m_use_new);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < T::DB; ++db) {
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
      }
    }
    m = m_new;
    m_use = m_use_new;
  }
  // Probabilities exp2(S*c - m) into the B-operand layout of the PV product
  // (bf16), and their fp32 row sum into l.  With dropout the row sum keeps
  // every probability (the softmax statistics are those of P) while the
  // PV operand has the dropped ones zeroed; the 1/(1-p) factor is applied
  // with the final division.  kbase: the tile's first key.
  template <bool DRAWN = false>
  __device__ __forceinline__ void probs(f32x16 (&s)[T::KB], bf16x8 (&pf)[T::KK],
                                        int kbase, const uint32_t (*drawn)[4] = nullptr) {
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < T::KB; ++kb) {
      uint32_t u[4];
      if constexpr (DROP && DRAWN) {
#pragma unroll
        for (int j = 0; j < 4; ++j) u[j] = drawn[kb][j];
      } else if constexpr (DROP) {
        dropout_bytes_rowlane(dr, qrow, kbase + kb * 32, __lane_id(), u);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(fmaf(s[kb][i], c_log2, -m_use));
        rs += p;
        if constexpr (DROP)
          s[kb][i] = dropout_keep(u[i >> 2], i & 3, dr.t) ? p : 0.f;
        else
          s[kb][i] = p;
      }
      pf[2 * kb] = pack8(s[kb], 0);
      pf[2 * kb + 1] = pack8(s[kb], 1);
    }
    l += rs;
  }
  // Whether the row sum of the probabilities is taken beside the PV
  // products (pv_rowsum) rather than beside the score products, which
  // carry the exponentials; at d = 64 that does not fit the registers.
  static constexpr bool kSumBesidePV = (D == 128);
  // The scores of the next tile (at sk, into s_next) and this tile's
  // probabilities (probs above, without dropout; the row sum here or in
  // pv_rowsum, see kSumBesidePV) in one sequence: 16 / KS probabilities
  // after each product, held in place by empty asm statements (the
  // compiler otherwise issues all the products first, and the exponentials
  // then wait behind them).  The fp32 probabilities stay in s.
  __device__ __forceinline__ void scores_probs(const unsigned char* sk,
                                               f32x16 (&s_next)[T::KB],
                                               f32x16 (&s)[T::KB],
                                               bf16x8 (&pf)[T::KK]) {
    constexpr int PER = 16 / T::KS;  // probabilities per product
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < T::KB; ++kb) {
      s_next[kb] = zero16();
#pragma unroll
      for (int ks = 0; ks < T::KS; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
            sk + kb * 32 * T::ROW + koff[ks]);
        s_next[kb] = mfma32(a, qf[ks], s_next[kb]);
        asm volatile("" : "+v"(s_next[kb]));
        const int e0 = PER * (kb * T::KS + ks);  // elements e0 .. e0 + PER - 1 of s
#pragma unroll
        for (int j = 0; j < PER; j += 2) {
          const int e = e0 + j;
          float p0 = fast_exp2(fmaf(s[e >> 4][e & 15], c_log2, -m_use));
          float p1 = fast_exp2(fmaf(s[e >> 4][(e & 15) + 1], c_log2, -m_use));
          asm volatile("" : "+v"(p0), "+v"(p1));
          if constexpr (!kSumBesidePV) {
            rs += p0;
            rs += p1;
          }
          s[e >> 4][e & 15] = p0;
          s[e >> 4][(e & 15) + 1] = p1;
        }
      }
    }
#pragma unroll
    for (int kb = 0; kb < T::KB; ++kb) {
      pf[2 * kb] = pack8(s[kb], 0);
      pf[2 * kb + 1] = pack8(s[kb], 1);
    }
    if constexpr (!kSumBesidePV) l += rs;
  }
  // Dropout: the scores of the next tile (at sk, into s_next) with the
  // random draws of the tile at kbase (this tile) spread between the
  // products: each block's ten Philox rounds in order, held in place by
  // empty asm statements.  u receives the tile's bytes for probs<true>.
  __device__ __forceinline__ void scores_draw(const unsigned char* sk,
                                              f32x16 (&s_next)[T::KB], int kbase,
                                              uint32_t (&u)[T::KB][4]) {
    constexpr int NM = T::KB * T::KS;  // products
    constexpr int NU = T::KB * 10;     // rounds
#pragma unroll
    for (int kb = 0; kb < T::KB; ++kb)
      dropout_ctr_rowlane(dr, qrow, kbase + kb * 32, __lane_id(), u[kb]);
#pragma unroll
    for (int kb = 0; kb < T::KB; ++kb) {
      s_next[kb] = zero16();
#pragma unroll
      for (int ks = 0; ks < T::KS; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
            sk + kb * 32 * T::ROW + koff[ks]);
        s_next[kb] = mfma32(a, qf[ks], s_next[kb]);
        asm volatile("" : "+v"(s_next[kb]));
        const int i = kb * T::KS + ks;
#pragma unroll
        for (int v = i * NU / NM; v < (i + 1) * NU / NM; ++v) {
          const int b = v / 10, r = v % 10;
          philox_round(u[b], dr.k0 + r * kWeyl0, dr.k1 + r * kWeyl1);
          asm volatile("" : "+v"(u[b][0]), "+v"(u[b][1]), "+v"(u[b][2]), "+v"(u[b][3]));
        }
      }
    }
#pragma unroll
    for (int kb = 0; kb < T::KB; ++kb) quad_transpose(u[kb], __lane_id());
  }
  // pv below, with the row sum of the probabilities in s (fp32, left there
  // by scores_probs) added into l beside the products, in the same order as
  // probs adds them: the score product phase carries the exponentials, this
  // one little vector work otherwise.
  __device__ __forceinline__ void pv_rowsum(const unsigned char* sv,
                                            const bf16x8 (&pf)[T::KK],
                                            const f32x16 (&s)[T::KB]) {
    constexpr int PER = (T::KB * 16) / (T::KK * T::DB);  // sums per product
    static_assert(PER * T::KK * T::DB == T::KB * 16, "even split");
    float rs = 0.f;
#pragma unroll
    for (int kk = 0; kk < T::KK; ++kk) {
#pragma unroll
      for (int db = 0; db < T::DB; ++db) {
        const unsigned char* p = sv + kk * 16 * T::ROW + voff[db];
        const bf16x8 a = join_tr16(lds_read_tr16(p), lds_read_tr16(p + 8 * T::ROW));
        acc[db] = mfma32(a, pf[kk], acc[db]);
        asm volatile("" : "+v"(acc[db]));
        const int e0 = PER * (kk * T::DB + db);
#pragma unroll
        for (int j = 0; j < PER; ++j) rs += s[(e0 + j) >> 4][(e0 + j) & 15];
        asm volatile("" : "+v"(rs));
      }
    }
    l += rs;
  }
  // O^T += V^T P^T for the V tile at sv.
  __device__ __forceinline__ void pv(const unsigned char* sv,
                                     const bf16x8 (&pf)[T::KK]) {
#pragma unroll
    for (int kk = 0; kk < T::KK; ++kk) {
#pragma unroll
      for (int db = 0; db < T::DB; ++db) {
        const unsigned char* p = sv + kk * 16 * T::ROW + voff[db];
        const bf16x8 a = join_tr16(lds_read_tr16(p), lds_read_tr16(p + 8 * T::ROW));
        acc[db] = mfma32(a, pf[kk], acc[db]);
      }
    }
  }
  // One division by l per row ([TLDR] online softmax; [LLMSYS] Fig. 1:
  // dividing once at the end equals dividing every probability), and
  // LSE = m + ln l in natural-log units.
  __device__ __forceinline__ void store(bf16* Oh, float* lse_h) const {
    const float l_tot = sum_halves(l);
    float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    if constexpr (DROP) inv *= dr.inv_keep;
    if (qrow >= n) return;
    bf16* orow = Oh + (int64_t)qrow * D;
#pragma unroll
    for (int db = 0; db < T::DB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 vv;
        vv[0] = pack_bf16(acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv);
        vv[1] = pack_bf16(acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + db * 32 + g * 8 + h * 4) = vv;
      }
    }
    if (h == 0) {
      lse_h[qrow] = (l_tot > 0.f) ? (m + fast_log2(l_tot)) * kLn2 : -INFINITY;
    }
  }
  // The same result over one chunk of the keys, kept in fp32 for the merge:
  // O_s = acc / l (0 if the chunk shows the row no key) and its logsumexp.
  __device__ __forceinline__ void store_partial(float* Os, float* lse_s) const {
    const float l_tot = sum_halves(l);
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    if (qrow >= n) return;
    float* orow = Os + (int64_t)qrow * D;
#pragma unroll
    for (int db = 0; db < T::DB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 v = {acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv,
                         acc[db][4 * g + 2] * inv, acc[db][4 * g + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + db * 32 + g * 8 + h * 4) = v;
      }
    }
    if (h == 0) {
      lse_s[qrow] = (l_tot > 0.f) ? (m + fast_log2(l_tot)) * kLn2 : -INFINITY;
    }
  }
};

// The key loop of one workgroup: key tiles first, next_on(first), ... up to
// kt_end (exclusive), K and V of the keys filled into kbuf / vbuf (two
// buffers each), each wave's online-softmax state in wv; `visited` receives
// the number of key tiles visited.  Every wave runs the same pipeline step
// per key tile:
//   block A: the scores of tile `nxt` on the matrix cores while the vector
//            units form tile `cur`'s probabilities;
//   block B: tile `cur`'s PV product on the matrix cores while the vector
//            units mask and reduce tile `nxt`'s scores.
template <class T, bool CAUSAL, bool DROP, class NextOn>
__device__ __forceinline__ void key_loop(FwdWave<T, CAUSAL, DROP>& wv,
                                         const TileFill<T>& fill,
                                         unsigned char* kbuf, unsigned char* vbuf,
                                         const bf16* Kh, const bf16* Vh,
                                         int n_keys, int first, int kt_end,
                                         NextOn next_on, int& visited) {
  int cur = first;
  visited = 0;
  if (cur < kt_end) {
    int nxt = next_on(cur);
    fill.k(Kh, cur * T::BC, n_keys, kbuf);
    fill.v(Vh, cur * T::BC, n_keys, vbuf);
    if (nxt < kt_end) fill.k(Kh, nxt * T::BC, n_keys, kbuf + T::K_BYTES);
    wait_dma();
    __syncthreads();
    // sa holds the current tile's scores; the next tile's scores go to sb
    // (and the roles swap) in the unrolled loop, so no copy is needed there.
    f32x16 sa[T::KB], sb[T::KB];
    wv.scores(kbuf, sa);
    if (wv.needs_mask(cur * T::BC)) wv.apply_mask(sa, cur * T::BC);
    wv.move_max(wv.tile_max(sa));

    // One step for tile `cur`, whose scores are in s and whose max is
    // already in m; the scores of tile `nxt` go to s_next.  MASK_NEXT
    // selects the masked form of block B, so that each block is one basic
    // block.  PAR is the LDS buffer parity of `cur` when it is known at
    // compile time (then every LDS address is a register plus an immediate),
    // or -1 to take it from the step count.
    auto step = [&](auto next_tag, auto mask_tag, auto par_tag, int it,
                    f32x16 (&s)[T::KB], f32x16 (&s_next)[T::KB]) {
      constexpr bool NEXT = decltype(next_tag)::value;
      constexpr bool MASK_NEXT = decltype(mask_tag)::value;
      constexpr int PAR = decltype(par_tag)::value;
      const int kb_cur = (PAR >= 0) ? PAR : (it & 1);
      // K of `cur` was in kbuf[kb_cur] (already consumed), K of `nxt` is in
      // kbuf[kb_cur ^ 1], V of `cur` is in vbuf[kb_cur].
      wait_dma();
      __syncthreads();
      int nxt2 = kt_end;
      if constexpr (NEXT) {
        nxt2 = next_on(nxt);
        if (nxt2 < kt_end) fill.k(Kh, nxt2 * T::BC, n_keys, kbuf + kb_cur * T::K_BYTES);
        fill.v(Vh, nxt * T::BC, n_keys, vbuf + (kb_cur ^ 1) * T::K_BYTES);
      }
      bf16x8 pf[T::KK];
      if constexpr (NEXT && !DROP) {
        wv.scores_probs(kbuf + (kb_cur ^ 1) * T::K_BYTES, s_next, s, pf);
      } else if constexpr (NEXT && DROP) {
        uint32_t u[T::KB][4];
        wv.scores_draw(kbuf + (kb_cur ^ 1) * T::K_BYTES, s_next, cur * T::BC, u);
        wv.template probs<true>(s, pf, cur * T::BC, u);
      } else {
        if constexpr (NEXT) wv.scores(kbuf + (kb_cur ^ 1) * T::K_BYTES, s_next);
        wv.probs(s, pf, cur * T::BC);
      }
      if constexpr (NEXT && !DROP && FwdWave<T, CAUSAL, DROP>::kSumBesidePV)
        wv.pv_rowsum(vbuf + kb_cur * T::K_BYTES, pf, s);
      else
        wv.pv(vbuf + kb_cur * T::K_BYTES, pf);
      if constexpr (NEXT) {
        if constexpr (MASK_NEXT) wv.apply_mask(s_next, nxt * T::BC);
        wv.move_max(wv.tile_max(s_next));
        cur = nxt;
        nxt = nxt2;
      }
    };
    using yes = std::true_type;
    using no = std::false_type;
    using par0 = std::integral_constant<int, 0>;
    using par1 = std::integral_constant<int, 1>;
    using par_rt = std::integral_constant<int, -1>;
    auto copy_b_to_a = [&]() {
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb) sa[kb] = sb[kb];
    };
    // Tiles needing the element mask come last (keys increase along the
    // visit order).  Unmasked steps run in pairs (parity 0 then 1, scores
    // in sa then sb); the rest take the parity from the step count.
    int it = 0;
#pragma unroll 1
    while (nxt < kt_end && !wv.needs_mask(nxt * T::BC)) {
      step(yes{}, no{}, par0{}, it, sa, sb);
      ++it;
      if (!(nxt < kt_end && !wv.needs_mask(nxt * T::BC))) {
        copy_b_to_a();
        break;
      }
      step(yes{}, no{}, par1{}, it, sb, sa);
      ++it;
    }
#pragma unroll 1
    for (; nxt < kt_end; ++it) {
      step(yes{}, yes{}, par_rt{}, it, sa, sb);
      copy_b_to_a();
    }
    step(no{}, no{}, par_rt{}, it, sa, sb);
    visited = it + 1;  // one step per visited key tile
  }
}

// Workgroup coordinates (head, first query row).
struct FwdPlace {
  int head, q0;
};
template <bool CAUSAL>
__device__ __forceinline__ FwdPlace fwd_place(int n_qtiles, int total, int br,
                                              int bundle) {
  const int lid = xcd_logical_id(blockIdx.x, total);
  if (CAUSAL) {
    const CausalPlace p = causal_place(lid, n_qtiles, total / n_qtiles, bundle);
    return {p.head, (n_qtiles - 1 - p.rank) * br};
  }
  return {lid / n_qtiles, (lid % n_qtiles) * br};
}

// With d = 128 (dense) a workgroup has 8 waves, one workgroup per CU: 256
// query rows share each K/V tile, halving the tile traffic into LDS per row.
// Otherwise a workgroup has 4 waves and two run per CU; the block-sparse
// kernel keeps 128 rows so that a workgroup's rows lie in one 128-row block
// row of the mask.  DROP instances apply dropout to P (Dropout, with the
// keep bits drawn per 4 x 4 score block from the seed, head, row and key).
template <int D, int NW, bool CAUSAL, bool SPARSE, bool DROP, bool COUNT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                     const bf16* __restrict__ V, bf16* __restrict__ O,
                     float* __restrict__ LSE, int n, int nk, int q_off,
                     int n_qtiles, int total,
                     int bundle, float c_log2, const uint8_t* __restrict__ mask,
                     int mask_cols, int block_m, int block_n, Dropout drop,
                     int* __restrict__ visits) {
  // (With dropout at d = 64 the key tile is 64 wide, as at d = 128: the
  // random bytes need registers that 128-key score tiles leave no room for.)
  using T = FwdTile<D, NW, (D == 128 || DROP) ? 64 : 128>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[4 * T::K_BYTES];
  unsigned char* const kbuf = smem;                  // K0 | K1
  unsigned char* const vbuf = smem + 2 * T::K_BYTES;  // V0 | V1

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  // Dense causal with 256-row tiles: the workgroup takes query tiles
  // n_qtiles-1-u and u of one head, whose key counts add up to the same
  // total for every u, so that all workgroups carry equal work (the
  // hardware hands workgroups to CUs in a fixed rotation, which leaves CUs
  // idle behind longer ones).
  constexpr bool PAIRS = CAUSAL && !SPARSE && NW == 8;
  FwdPlace pl;
  int q0_b = -1;  // the second tile's first row, -1 if none
  if constexpr (PAIRS) {
    const int units = (n_qtiles + 1) / 2;
    const int lid = xcd_logical_id(blockIdx.x, total);
    const int u = lid % units;
    pl = {lid / units, (n_qtiles - 1 - u) * T::BR};
    if (u != n_qtiles - 1 - u) q0_b = u * T::BR;
  } else {
    pl = fwd_place<CAUSAL>(n_qtiles, total, T::BR, bundle);
  }
  const int64_t hoff = (int64_t)pl.head * n * D;  // Q, O: n rows per head
  const int64_t hoff_k = (int64_t)pl.head * nk * D;  // K, V: nk rows
  const bf16* Kh = K + hoff_k;
  const bf16* Vh = V + hoff_k;
  const TileFill<T> fill(w, lane);
  const int n_ktiles = (nk + T::BC - 1) / T::BC;

  // One query tile of 32 * NW rows from row q0.
  auto run_tile = [&](int q0) {
    FwdWave<T, CAUSAL, DROP> wv(Q + hoff, q0 + 32 * w, lane, n, nk, q_off,
                                c_log2);
    if constexpr (DROP) {
      wv.dr = drop;
      wv.dr.bh = (uint32_t)pl.head;
    }
    // Key tiles to visit, in order.
    int kt_end = n_ktiles;
    // (Under the causal rule the tile's last row sees the keys up to
    // q_off + that row, q_off >= 0.)
    if (CAUSAL) kt_end = min(n_ktiles, (min(q0 + T::BR, n) - 1 + q_off) / T::BC + 1);
    // Block-sparse: the mask row of this workgroup's block row (a 64-entry
    // window at a time).  A key tile lies in one mask column.
    MaskLine mline(SPARSE ? mask + (int64_t)(q0 / block_m) * mask_cols : mask,
                   1, SPARSE ? mask_cols : 0, lane);
    // (readfirstlane keeps the index opaque to induction-variable rewriting,
    // which would otherwise turn every DMA source into a loop-carried 64-bit
    // pointer and exhaust the register file.)
    auto next_on = [&](int kt) -> int {
      ++kt;
      if constexpr (SPARSE) {
        if (kt < kt_end) {
          const int col = (kt * T::BC) / block_n;
          const int nc = mline.next(col, lane);
          if (nc != col) kt = min(kt_end, (int)(((int64_t)nc * block_n) / T::BC));
        }
      }
      return __builtin_amdgcn_readfirstlane(kt);
    };
    int nvis = 0;
    key_loop(wv, fill, kbuf, vbuf, Kh, Vh, nk, next_on(-1), kt_end, next_on,
             nvis);
    wv.store(O + hoff, LSE + (int64_t)pl.head * n);
    // Diagnostic count of the key tiles this query tile visited (COUNT
    // instances only).
    if (COUNT && w == 0 && lane == 0) {
      visits[(int64_t)pl.head * n_qtiles + q0 / T::BR] = nvis;
    }
  };

  run_tile(pl.q0);
  if (PAIRS && q0_b >= 0) {
    __syncthreads();  // every wave is done with the K/V buffers
    run_tile(q0_b);
  }
}

template <int D, bool CAUSAL, bool SPARSE, bool DROP, bool COUNT = false>
hipError_t launch_fwd(const FwdArgs& a, hipStream_t s) {
  constexpr int NW = (D == 128 && !SPARSE) ? 8 : 4;
  using T = FwdTile<D, NW>;
  const int n_qtiles = (a.n + T::BR - 1) / T::BR;
  // Dense causal 8-wave workgroups take two tiles each (see the kernel).
  const int units = (CAUSAL && !SPARSE && NW == 8) ? (n_qtiles + 1) / 2 : n_qtiles;
  const int total = (int)(a.bh * units);
  const int bundle = causal_bundle(n_qtiles, NW == 8 ? 1 : 2);
  return launch_kernel(fwd_bf16_kernel<D, NW, CAUSAL, SPARSE, DROP, COUNT>, dim3(total),
                       dim3(NW * 64), s, (const bf16*)a.q, (const bf16*)a.k,
                       (const bf16*)a.v, (bf16*)a.o, a.lse, a.n, a.nk, a.q_off,
                       n_qtiles, total, bundle, a.scale * kLog2e, a.mask, a.mask_cols,
                       a.block_m, a.block_n, make_dropout(a.drop_t, a.seed_lo, a.seed_hi, a.q_off),
                       a.visits);
}

template <int D>
hipError_t dispatch_mask(const FwdArgs& a, hipStream_t s) {
  if (a.visits) {  // diagnostic instances that also count visited tiles
    if (a.mask) {
      return a.causal ? launch_fwd<D, true, true, false, true>(a, s)
                      : launch_fwd<D, false, true, false, true>(a, s);
    }
    return a.causal ? launch_fwd<D, true, false, false, true>(a, s)
                    : launch_fwd<D, false, false, false, true>(a, s);
  }
  if (a.mask) {
    if (a.drop_t > 0) {
      return a.causal ? launch_fwd<D, true, true, true>(a, s)
                      : launch_fwd<D, false, true, true>(a, s);
    }
    return a.causal ? launch_fwd<D, true, true, false>(a, s)
                    : launch_fwd<D, false, true, false>(a, s);
  }
  if (a.drop_t > 0) {
    return a.causal ? launch_fwd<D, true, false, true>(a, s)
                    : launch_fwd<D, false, false, true>(a, s);
  }
  return a.causal ? launch_fwd<D, true, false, false>(a, s)
                  : launch_fwd<D, false, false, false>(a, s);
}

// Split-KV forward for a short block of queries against a long key
// sequence: with few query rows the query tiles alone leave most of the
// chip idle, so the keys are also cut into chunks handled by separate
// workgroups ([REAPER] section 3.6, decoding).  Each workgroup is one wave:
// 32 query rows against the key tiles of one chunk, 32 keys per tile so that
// five of them fit a CU's LDS and keep enough K/V bytes in flight.  It writes
// the chunk's normalised fp32 output and its logsumexp; splitkv_merge_kernel
// combines the chunks.  The queries are the last nq of the nk positions, so
// under the causal rule query i sees keys j <= nk - nq + i.  (A single query
// row takes splitkv_vec_kernel below instead.)
template <int D, bool CAUSAL>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 2)))
void splitkv_bf16_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                         const bf16* __restrict__ V, float* __restrict__ Opart,
                         float* __restrict__ LSEpart, int nq, int nk,
                         int n_qtiles, int n_splits, int tiles_per_split,
                         int total, int64_t bh, float c_log2) {
  using T = FwdTile<D, 1, kSplitKvTile>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[4 * T::K_BYTES];
  unsigned char* const kbuf = smem;
  unsigned char* const vbuf = smem + 2 * T::K_BYTES;

  const int lane = threadIdx.x;
  // Query tiles of one (head, chunk) are adjacent in the logical order and
  // so run on one XCD, sharing the chunk's K/V in its L2.
  const int lid = xcd_logical_id(blockIdx.x, total);
  const int qt = lid % n_qtiles;
  const int split = (lid / n_qtiles) % n_splits;
  const int head = lid / n_qtiles / n_splits;
  const int q_off = nk - nq;
  const bf16* Kh = K + (int64_t)head * nk * D;
  const bf16* Vh = V + (int64_t)head * nk * D;
  FwdWave<T, CAUSAL> wv(Q + (int64_t)head * nq * D, qt * 32, lane, nq, nk,
                        q_off, c_log2);
  const TileFill<T> fill(0, lane);

  const int n_ktiles = (nk + T::BC - 1) / T::BC;
  const int kt0 = split * tiles_per_split;
  int kt_end = min(kt0 + tiles_per_split, n_ktiles);
  if (CAUSAL) kt_end = min(kt_end, (q_off + min(qt * 32 + 32, nq) - 1) / T::BC + 1);
  auto next_on = [](int kt) -> int { return __builtin_amdgcn_readfirstlane(kt + 1); };
  int nvis = 0;
  key_loop(wv, fill, kbuf, vbuf, Kh, Vh, nk, kt0, kt_end, next_on, nvis);

  const int64_t prow = ((int64_t)split * bh + head) * nq;
  wv.store_partial(Opart + prow * D, LSEpart + prow);
}

// Decoding with a single query row: the chunk pass on the vector units.  A
// 32-row matrix product would discard 31 of its rows here, and the pass is
// bound by reading K and V once, so each wave streams one chunk with 16-byte
// loads (D/8 lanes per key row, 64/(D/8) key slots per load) and keeps an
// online-softmax state per key slot: reference max m (log2 units, moved only
// when a score exceeds it by more than 8), exp-sum l, and the lane's 8 output
// columns.  The slots are merged by the two-part rule at the end ([XYZ],
// incremental softmax tracking) and the chunk's O (divided by its exp-sum)
// and logsumexp are stored as the matrix-core chunk pass stores them.  One
// wave per chunk, four chunks per workgroup.  Chunk c of a head takes the
// key groups c, c + n_splits, c + 2 n_splits, ... (a group = the keys of one
// round of loads), so that the waves of a head read neighbouring addresses
// at the same time.
template <int D>
__global__ __launch_bounds__(256)
void splitkv_vec_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                        const bf16* __restrict__ V, float* __restrict__ Opart,
                        float* __restrict__ LSEpart, int nk, int n_splits,
                        int n_chunks, int64_t bh, float c_log2) {
  constexpr int LPK = D / 8;     // lanes per key row
  constexpr int KPS = 64 / LPK;  // key slots per wave
  constexpr int U = 4;           // loads of each of K and V in flight
  constexpr int G = KPS * U;     // keys of one round of loads
  constexpr float SLACK = 8.f;
  const int chunk = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * 4 + (threadIdx.x >> 6)));
  if (chunk >= n_chunks) return;
  const int lane = threadIdx.x & 63;
  const int head = chunk / n_splits;
  const int split = chunk % n_splits;
  const int slot = lane / LPK;
  const int c0 = (lane % LPK) * 8;

  // This lane's 8 query columns, scaled to log2 units.
  float qf[8];
  {
    const u32x4 qr = *reinterpret_cast<const u32x4*>(Q + (int64_t)head * D + c0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qf[2 * i] = bf16_lo(qr[i]) * c_log2;
      qf[2 * i + 1] = bf16_hi(qr[i]) * c_log2;
    }
  }
  const bf16* Kh = K + (int64_t)head * nk * D + c0;
  const bf16* Vh = V + (int64_t)head * nk * D + c0;

  float m = -INFINITY, l = 0.f;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int j0 = split * G; j0 < nk; j0 += n_splits * G) {
    u32x4 kr[U], vr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = j0 + u * KPS + slot;
      if (key < nk) {
        kr[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Kh + (int64_t)key * D));
        vr[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Vh + (int64_t)key * D));
      } else {
        kr[u] = u32x4{0u, 0u, 0u, 0u};
        vr[u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // Score of this slot's key: 8 products per lane, summed over the
      // LPK lanes of the key row.
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s = fmaf(qf[2 * i], bf16_lo(kr[u][i]), s);
        s = fmaf(qf[2 * i + 1], bf16_hi(kr[u][i]), s);
      }
#pragma unroll
      for (int off = LPK / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
      if (j0 + u * KPS + slot >= nk) s = -INFINITY;
      const bool move = s > m + SLACK;
      if (__ballot(move)) {
        const float m_new = move ? s : m;
        const float alpha = move ? fast_exp2(m - m_new) : 1.f;
        l *= alpha;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] *= alpha;
        m = m_new;
      }
      const float p = fast_exp2(s - ((m == -INFINITY) ? 0.f : m));
      l += p;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(p, bf16_lo(vr[u][i]), acc[2 * i]);
        acc[2 * i + 1] = fmaf(p, bf16_hi(vr[u][i]), acc[2 * i + 1]);
      }
    }
  }
  // Merge the key slots (lanes that differ in the slot bits of their index).
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(m, off);
    const float l2 = __shfl_xor(l, off);
    const float mx = fmaxf(m, m2);
    const float mu = (mx == -INFINITY) ? 0.f : mx;
    const float w1 = fast_exp2(m - mu), w2 = fast_exp2(m2 - mu);
    l = l * w1 + l2 * w2;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = acc[i] * w1 + __shfl_xor(acc[i], off) * w2;
    m = mx;
  }
  const int64_t prow = (int64_t)split * bh + head;  // the chunk's row (one query)
  const float inv = (l > 0.f) ? 1.f / l : 0.f;
  if (slot == 0) {
    float* orow = Opart + prow * D + c0;
    *reinterpret_cast<f32x4*>(orow) = f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    *reinterpret_cast<f32x4*>(orow + 4) = f32x4{acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
  }
  if (lane == 0) LSEpart[prow] = (l > 0.f) ? (m + fast_log2(l)) * kLn2 : -INFINITY;
}

// Merge of the chunk results of one query row by the two-part softmax rule
// ([XYZ], incremental softmax tracking), applied to all chunks at once: with
// M = max_s lse_s and w_s = exp(lse_s - M), O = sum_s w_s O_s / sum_s w_s and
// lse = M + ln sum_s w_s (each O_s is already divided by its own exp-sum, so
// the weights are the chunks' exp-sums relative to M).  A row no chunk shows
// any key gets O = 0 and lse = -inf.  D/4 lanes per row, four columns each.
template <int D>
__global__ __launch_bounds__(256)
void splitkv_merge_kernel(const float* __restrict__ Opart,
                          const float* __restrict__ LSEpart, bf16* __restrict__ O,
                          float* __restrict__ LSE, int64_t rows, int n_splits) {
  constexpr int LPR = D / 4;
  constexpr int RPW = 256 / LPR;
  const int64_t row = (int64_t)blockIdx.x * RPW + threadIdx.x / LPR;
  const int c = (threadIdx.x % LPR) * 4;
  if (row >= rows) return;
  float mx = -INFINITY;
  for (int s = 0; s < n_splits; ++s) mx = fmaxf(mx, LSEpart[s * rows + row]);
  float sum = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (mx != -INFINITY) {
    for (int s = 0; s < n_splits; ++s) {
      const float w = fast_exp2((LSEpart[s * rows + row] - mx) * kLog2e);
      const f32x4 o = *reinterpret_cast<const f32x4*>(
          Opart + (s * rows + row) * D + c);
      sum += w;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = fmaf(w, o[i], acc[i]);
    }
  }
  const float inv = (sum > 0.f) ? 1.f / sum : 0.f;
  u32x2 vv;
  vv[0] = pack_bf16(acc[0] * inv, acc[1] * inv);
  vv[1] = pack_bf16(acc[2] * inv, acc[3] * inv);
  *reinterpret_cast<u32x2*>(O + row * D + c) = vv;
  if (c == 0) LSE[row] = (sum > 0.f) ? mx + fast_log2(sum) * kLn2 : -INFINITY;
}

template <int D, bool CAUSAL>
hipError_t launch_splitkv_t(const SplitKvArgs& a, hipStream_t s) {
  hipError_t e;
  if (a.nq == 1) {
    // One query row (which sees every key, causal or not): the vector pass.
    const int chunks = (int)(a.bh * a.n_splits);
    e = launch_kernel(splitkv_vec_kernel<D>, dim3((unsigned)((chunks + 3) / 4)),
                      dim3(256), s, (const bf16*)a.q, (const bf16*)a.k,
                      (const bf16*)a.v, a.ws_o, a.ws_lse, a.nk, a.n_splits,
                      chunks, a.bh, a.scale * kLog2e);
  } else {
    const int n_qtiles = (a.nq + 31) / 32;
    const int total = (int)(a.bh * a.n_splits * n_qtiles);
    e = launch_kernel(
        splitkv_bf16_kernel<D, CAUSAL>, dim3(total), dim3(64), s,
        (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, a.ws_o, a.ws_lse,
        a.nq, a.nk, n_qtiles, a.n_splits, a.tiles_per_split, total, a.bh,
        a.scale * kLog2e);
  }
  if (e != hipSuccess) return e;
  const int64_t rows = a.bh * a.nq;
  constexpr int RPW = 256 / (D / 4);
  return launch_kernel(splitkv_merge_kernel<D>, dim3((unsigned)((rows + RPW - 1) / RPW)),
                       dim3(256), s, (const float*)a.ws_o,
                       (const float*)a.ws_lse, (bf16*)a.o, a.lse, rows,
                       a.n_splits);
}

}  // namespace

void fwd_bf16_tile_grid(int d, bool sparse, int* rows, int* cols) {
  const int nw = (d == 128 && !sparse) ? 8 : 4;
  *rows = 32 * nw;
  *cols = (d == 128) ? FwdTile<128, 8>::BC : FwdTile<64, 4>::BC;
}

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s) {
  return a.d == 128 ? dispatch_mask<128>(a, s) : dispatch_mask<64>(a, s);
}

hipError_t launch_splitkv_bf16(const SplitKvArgs& a, hipStream_t s) {
  if (a.d == 128) {
    return a.causal ? launch_splitkv_t<128, true>(a, s)
                    : launch_splitkv_t<128, false>(a, s);
  }
  return a.causal ? launch_splitkv_t<64, true>(a, s)
                  : launch_splitkv_t<64, false>(a, s);
}

}  // namespace fa
