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
//     into probabilities; while they compute tile j's PV product, the vector
//     units mask and reduce tile j+1's scores to its row max.  K therefore
//     runs one tile ahead of V: both are double-buffered in LDS and filled by
//     direct global-to-LDS loads issued one tile ahead.
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

template <int D, bool SPARSE>
struct FwdTile {
  // Waves per workgroup: with d = 128 one workgroup of 8 waves per CU
  // (256 query rows) halves the K/V tile traffic into LDS per query row.
  // The block-sparse kernel keeps 128 rows, so that a workgroup's rows lie
  // in one 128-row block row of the mask.
  static constexpr int NW = (D == 128 && !SPARSE) ? 8 : 4;
  static constexpr int BR = 32 * NW;                  // query rows per workgroup
  static constexpr int BC = (D == 128) ? 64 : 128;    // keys per tile
  static constexpr int KS = D / 16;                   // MFMA k-steps over d
  static constexpr int KB = BC / 32;                  // 32-key blocks per tile
  static constexpr int KK = BC / 16;                  // 16-key k-steps of PV
  static constexpr int DB = D / 32;                   // 32-wide blocks of d
  static constexpr int CPR = D / 8;                   // 16-B chunks per row
  static constexpr int ROW = D * 2;                   // bytes per K / V row
  static constexpr int K_BYTES = BC * ROW;            // one K or V tile
  static constexpr int LDS = 4 * K_BYTES;             // K0 | K1 | V0 | V1
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
  constexpr int D = T::ROW / 2;
  const int o = (w + T::NW * i) * 1024 + lane * 16;
  row = o / T::ROW;
  return row * D + ((((o % T::ROW) >> 4) ^ SWZ(row)) * 8);
}

// Issue the direct loads of one K or V tile starting at row kbase.  Full
// tiles use the precomputed per-lane offsets; rows of the last tile at or
// past n are clamped to n - 1.
template <class T, int (*SWZ)(int)>
__device__ __forceinline__ void fill_tile(const bf16* g, int kbase, int n,
                                          unsigned char* tile, int w, int lane,
                                          const int (&off)[T::BLK]) {
  constexpr int D = T::ROW / 2;
  const bf16* base = g + (int64_t)kbase * D;
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
      dma16(base + (o - over * D), tile + (w + T::NW * i) * 1024);
    }
  }
}

template <int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__((FwdTile<D, SPARSE>::NW * 64))
__attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                     const bf16* __restrict__ V, bf16* __restrict__ O,
                     float* __restrict__ LSE, int n, int n_qtiles, int total,
                     float c_log2, const uint8_t* __restrict__ mask,
                     int mask_cols, int block_m, int block_n) {
  using T = FwdTile<D, SPARSE>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[T::LDS];
  unsigned char* const kbuf = smem;
  unsigned char* const vbuf = smem + 2 * T::K_BYTES;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lane = tid & 63;
  const int h = lane >> 5;
  const int l32 = lane & 31;

  const int lid = xcd_logical_id(blockIdx.x, total);
  const int head = lid / n_qtiles;
  const int qt = CAUSAL ? (n_qtiles - 1 - lid % n_qtiles) : (lid % n_qtiles);
  const int q0 = qt * T::BR;
  const int64_t hoff = (int64_t)head * n * D;
  const bf16* Qh = Q + hoff;
  const bf16* Kh = K + hoff;
  const bf16* Vh = V + hoff;
  int koff_g[T::BLK], voff_g[T::BLK];  // per-lane DMA source offsets
#pragma unroll
  for (int i = 0; i < T::BLK; ++i) {
    int row;
    koff_g[i] = tile_src<T, swz_k<D>>(w, lane, i, row);
    voff_g[i] = tile_src<T, swz_v<D>>(w, lane, i, row);
  }

  const int qw0 = q0 + 32 * w;   // first query row of this wave
  const int qrow = qw0 + l32;    // query row of this lane

  // Q as the B operand of S^T = K Q^T: slot j of k-step ks is
  // Q[qrow][ks*16 + h*8 + j].
  bf16x8 qf[T::KS];
#pragma unroll
  for (int ks = 0; ks < T::KS; ++ks) {
    qf[ks] = as_bf16x8(load_row16(Qh, qrow, n, D, ks * 16 + h * 8));
  }

  // Key tiles to visit, in order.
  const int n_ktiles = (n + T::BC - 1) / T::BC;
  int kt_end = n_ktiles;
  if (CAUSAL) {
    const int last_q = min(q0 + T::BR, n) - 1;
    kt_end = min(n_ktiles, last_q / T::BC + 1);
  }
  const uint8_t* mrow =
      SPARSE ? mask + (int64_t)(q0 / block_m) * mask_cols : nullptr;
  // (readfirstlane keeps the index opaque to induction-variable rewriting,
  // which would otherwise turn every DMA source into a loop-carried 64-bit
  // pointer and exhaust the register file.)
  auto next_on = [&](int kt) -> int {
    ++kt;
    if constexpr (SPARSE) {
      while (kt < kt_end && mrow[(kt * T::BC) / block_n] == 0) ++kt;
    }
    return __builtin_amdgcn_readfirstlane(kt);
  };

  // Loop-invariant per-lane LDS read offsets.
  // K fragment (A of S^T): row kb*32 + l32, chunk ks*2 + h.
  int koff[T::KS];
#pragma unroll
  for (int ks = 0; ks < T::KS; ++ks) {
    koff[ks] = l32 * T::ROW + (((ks * 2 + h) ^ swz_k<D>(l32)) << 4);
  }
  // V^T fragment (A of O^T) by transpose reads: source lane s = lane % 16 of
  // group g = lane / 16 addresses key kk*16 + r2*8 + h*4 + s/4 at column
  // db*32 + 16*(g & 1) + 4*(s % 4); slots 0-3 (r2 = 0) and 4-7 (r2 = 1) then
  // hold keys {h*4 + 0..3} and {8 + h*4 + 0..3} of the 16-key group, the
  // same keys P's registers hold.
  int voff[T::DB];
  {
    const int s16 = lane & 15, g = lane >> 4;
    const int krow = h * 4 + (s16 >> 2);
#pragma unroll
    for (int db = 0; db < T::DB; ++db) {
      const int col = db * 32 + 16 * (g & 1) + 4 * (s16 & 3);
      voff[db] = krow * T::ROW + (((col >> 3) ^ swz_v<D>(krow)) << 4) +
                 (col & 7) * 2;
    }
  }

  // S^T = K Q^T of the tile in K buffer kb (KB blocks of 32 keys).
  auto scores = [&](const unsigned char* sk, f32x16 (&s)[T::KB]) {
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
  };

  // Element mask of a score tile starting at key kbase: keys past the
  // diagonal or past the sequence end get -inf.  Whether a tile needs it
  // is wave-uniform.
  auto needs_mask = [&](int kbase) {
    return (CAUSAL && kbase + T::BC - 1 > qw0) || (kbase + T::BC > n);
  };
  auto apply_mask = [&](f32x16 (&s)[T::KB], int kbase) {
    // Last visible key of this lane's row, relative to the key held in
    // register 0 of block 0; register i of block kb holds key
    // kb*32 + (i/4)*8 + (i%4) relative to it.
    const int lim = (CAUSAL ? min(qrow, n - 1) : n - 1) - kbase - h * 4;
#pragma unroll
    for (int kb = 0; kb < T::KB; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (kb * 32 + (i >> 2) * 8 + (i & 3) > lim) s[kb][i] = -INFINITY;
      }
    }
  };
  auto tile_max = [&](const f32x16 (&s)[T::KB]) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < T::KB; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    }
    return max_halves(mx) * c_log2;
  };

  f32x16 acc[T::DB];
#pragma unroll
  for (int db = 0; db < T::DB; ++db) acc[db] = zero16();
  // Online softmax state ([TLDR] online softmax; [REAPER] 3.3).  m is the
  // reference max in log2 units of the scaled score; it only moves when a
  // tile max exceeds it by more than the slack.  m_use is m with -inf
  // replaced by 0, the value subtracted inside the exponentials.
  float m = -INFINITY;
  float m_use = 0.f;
  float l = 0.f;  // running exp-sum over this half-wave's keys
  // Move the reference max to cover tile max mx; rescale l and the
  // accumulator when it moves (any lane of the wave).
  auto move_max = [&](float mx) {
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
  };

  int cur = next_on(-1);
  if (cur >= kt_end) goto epilogue;  // (block-sparse) nothing visible
  {
    int nxt = next_on(cur);
    fill_tile<T, swz_k<D>>(Kh, cur * T::BC, n, kbuf, w, lane, koff_g);
    fill_tile<T, swz_v<D>>(Vh, cur * T::BC, n, vbuf, w, lane, voff_g);
    if (nxt < kt_end) {
      fill_tile<T, swz_k<D>>(Kh, nxt * T::BC, n, kbuf + T::K_BYTES, w, lane, koff_g);
    }
    wait_dma();
    __syncthreads();
    f32x16 s[T::KB];
    scores(kbuf, s);
    if (needs_mask(cur * T::BC)) apply_mask(s, cur * T::BC);
    move_max(tile_max(s));

    // One pipeline step for tile `cur`, whose scores are in s and whose max
    // is already folded into m.  Block A: the scores of tile `nxt` on the
    // matrix cores while the vector units form tile `cur`'s probabilities.
    // Block B: tile `cur`'s PV product on the matrix cores while the vector
    // units mask and reduce tile `nxt`'s scores.  MASK_NEXT selects the
    // masked form of block B, so that each block is one basic block.
    auto step = [&](auto next_tag, auto mask_tag, int it) {
      constexpr bool NEXT = decltype(next_tag)::value;
      constexpr bool MASK_NEXT = decltype(mask_tag)::value;
      const int kb_cur = it & 1;
      // Buffers: K of `cur` was in kbuf[kb_cur] (already consumed), K of
      // `nxt` is in kbuf[kb_cur ^ 1], V of `cur` is in vbuf[kb_cur].
      wait_dma();
      __syncthreads();
      int nxt2 = kt_end;
      if constexpr (NEXT) {
        nxt2 = next_on(nxt);
        if (nxt2 < kt_end) {
          fill_tile<T, swz_k<D>>(Kh, nxt2 * T::BC, n,
                                 kbuf + kb_cur * T::K_BYTES, w, lane, koff_g);
        }
        fill_tile<T, swz_v<D>>(Vh, nxt * T::BC, n,
                               vbuf + (kb_cur ^ 1) * T::K_BYTES, w, lane, voff_g);
      }

      // Block A.
      f32x16 s_next[T::KB];
      if constexpr (NEXT) scores(kbuf + (kb_cur ^ 1) * T::K_BYTES, s_next);
      bf16x8 pf[T::KK];
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          s[kb][i] = fast_exp2(fmaf(s[kb][i], c_log2, -m_use));
          rs += s[kb][i];
        }
        pf[2 * kb] = pack8(s[kb], 0);
        pf[2 * kb + 1] = pack8(s[kb], 1);
      }
      l += rs;

      // Block B: O^T += V^T P^T for tile `cur`.
      const unsigned char* sv = vbuf + kb_cur * T::K_BYTES;
#pragma unroll
      for (int kk = 0; kk < T::KK; ++kk) {
#pragma unroll
        for (int db = 0; db < T::DB; ++db) {
          const unsigned char* pv = sv + kk * 16 * T::ROW + voff[db];
          const bf16x8 a =
              join_tr16(lds_read_tr16(pv), lds_read_tr16(pv + 8 * T::ROW));
          acc[db] = mfma32(a, pf[kk], acc[db]);
        }
      }
      if constexpr (NEXT) {
        if constexpr (MASK_NEXT) apply_mask(s_next, nxt * T::BC);
        move_max(tile_max(s_next));
#pragma unroll
        for (int kb = 0; kb < T::KB; ++kb) s[kb] = s_next[kb];
        cur = nxt;
        nxt = nxt2;
      }
    };
    // Tiles needing the element mask come last (keys increase along the
    // visit order), so the unmasked and masked steps run as two loops.
    int it = 0;
#pragma unroll 1
    for (; nxt < kt_end && !needs_mask(nxt * T::BC); ++it) {
      step(std::true_type{}, std::false_type{}, it);
    }
#pragma unroll 1
    for (; nxt < kt_end; ++it) step(std::true_type{}, std::true_type{}, it);
    step(std::false_type{}, std::false_type{}, it);
  }

epilogue:
  // One division by l per row ([TLDR] online softmax; [LLMSYS] Fig. 1:
  // dividing once at the end equals dividing every probability).
  const float l_tot = sum_halves(l);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  if (qrow < n) {
    bf16* orow = O + hoff + (int64_t)qrow * D;
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
      LSE[(int64_t)head * n + qrow] =
          (l_tot > 0.f) ? (m + fast_log2(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

template <int D, bool CAUSAL, bool SPARSE>
hipError_t launch_fwd_bf16_t(const FwdArgs& a, hipStream_t s) {
  using T = FwdTile<D, SPARSE>;
  const int n_qtiles = (a.n + T::BR - 1) / T::BR;
  const int total = (int)(a.bh * n_qtiles);
  return launch_kernel(fwd_bf16_kernel<D, CAUSAL, SPARSE>, dim3(total),
                       dim3(T::NW * 64), s, (const bf16*)a.q, (const bf16*)a.k,
                       (const bf16*)a.v, (bf16*)a.o, a.lse, a.n, n_qtiles,
                       total, a.scale * kLog2e, a.mask, a.mask_cols, a.block_m,
                       a.block_n);
}

template <int D>
hipError_t dispatch_mask(const FwdArgs& a, hipStream_t s) {
  if (a.mask) {
    return a.causal ? launch_fwd_bf16_t<D, true, true>(a, s)
                    : launch_fwd_bf16_t<D, false, true>(a, s);
  }
  return a.causal ? launch_fwd_bf16_t<D, true, false>(a, s)
                  : launch_fwd_bf16_t<D, false, false>(a, s);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s) {
  return a.d == 128 ? dispatch_mask<128>(a, s) : dispatch_mask<64>(a, s);
}

}  // namespace fa
