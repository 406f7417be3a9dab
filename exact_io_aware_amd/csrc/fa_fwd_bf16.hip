// Forward pass, bf16 inputs, fp32 accumulation, gfx950 MFMA.
//
// Pages cited (titles as published):
//   [TLDR]   "FlashAttention：メモリ効率的なアテンション計算" (tech-tldr.com)
//   [XYZ]    "FlashAttention: IOを意識した高速かつメモリ効率の高い厳密な
//            アテンション" (xyznot.com)
//   [REAPER] "3 · FlashAttention" (mkdocs.reaper.mx, chapter 3)
//   [LLMSYS] "출력을 누적해 메모리 이동을 줄이는 FlashAttention"
//
// Algorithm: for a block of 128 query rows, stream the key/value tiles
// through LDS; per tile compute the score tile on the matrix cores, update
// the running row max m, running exp-sum l and the unnormalised output
// accumulator, and divide by l once after the last tile ([TLDR] online
// softmax and tiling sections; [REAPER] sections 3.2-3.3; [LLMSYS] Fig. 3).
// The score and probability tiles live only in registers.  Under the causal
// rule key tiles entirely above the diagonal are never visited ([REAPER],
// causal-mask question); in the block-sparse variant key tiles whose mask
// block is 0 are never visited ([XYZ], block-sparse extension).
//
// MI355X mapping (one workgroup = 4 waves, wave w owns query rows
// q0 + 32w .. q0 + 32w + 31):
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
//   * K and V tiles are double-buffered in LDS (one barrier per tile); the
//     next tile's global loads are issued before the current tile's math.
//   * 16-byte chunks are XOR-swizzled per row so that both the row-wise
//     stores and the fragment reads are free of bank conflicts; every LDS
//     read address is a loop-invariant per-lane base plus a constant.
//   * The workgroup order keeps each head on one XCD (shared L2) and, under
//     the causal rule, starts the longest query tiles first.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

template <int D>
struct FwdTile {
  static constexpr int NW = 4;                        // waves per workgroup
  static constexpr int BR = 32 * NW;                  // query rows per workgroup
  static constexpr int BC = (D == 128) ? 64 : 128;    // keys per tile
  static constexpr int KS = D / 16;                   // MFMA k-steps over d
  static constexpr int KB = BC / 32;                  // 32-key blocks per tile
  static constexpr int KK = BC / 16;                  // 16-key k-steps of PV
  static constexpr int DB = D / 32;                   // 32-wide blocks of d
  static constexpr int CPR = D / 8;                   // 16-B chunks per row
  static constexpr int ROW = D * 2;                   // bytes per K / V row
  static constexpr int K_BYTES = BC * ROW;
  static constexpr int STAGE = 2 * K_BYTES;           // K tile then V tile
  static constexpr int LPT = BC * CPR / 256;          // chunks per thread
  static_assert(LPT == 4, "four 16-B chunks of K and of V per thread");
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

template <int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                     const bf16* __restrict__ V, bf16* __restrict__ O,
                     float* __restrict__ LSE, int n, int n_qtiles, int total,
                     float c_log2, const uint8_t* __restrict__ mask,
                     int mask_cols, int block_m, int block_n) {
  using T = FwdTile<D>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * T::STAGE];

  const int tid = threadIdx.x;
  const int w = tid >> 6;
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

  const int qw0 = q0 + 32 * w;   // first query row of this wave
  const int qrow = qw0 + l32;    // query row of this lane

  // Q as the B operand of S^T = K Q^T: slot j of k-step ks is
  // Q[qrow][ks*16 + h*8 + j].
  bf16x8 qf[T::KS];
#pragma unroll
  for (int ks = 0; ks < T::KS; ++ks) {
    qf[ks] = as_bf16x8(load_row16(Qh, qrow, n, D, ks * 16 + h * 8));
  }

  // Key tiles to visit.
  const int n_ktiles = (n + T::BC - 1) / T::BC;
  int kt_end = n_ktiles;
  if (CAUSAL) {
    const int last_q = min(q0 + T::BR, n) - 1;
    kt_end = min(n_ktiles, last_q / T::BC + 1);
  }
  const uint8_t* mrow =
      SPARSE ? mask + (int64_t)(q0 / block_m) * mask_cols : nullptr;
  auto tile_on = [&](int kt) -> bool {
    return !SPARSE || mrow[(kt * T::BC) / block_n] != 0;
  };
  auto next_on = [&](int kt) -> int {
    ++kt;
    if constexpr (SPARSE) {
      while (kt < kt_end && !tile_on(kt)) ++kt;
    }
    return kt;
  };

  // Global -> register staging of one K/V tile: thread tid owns chunks
  // e = tid + 256 i (row e / CPR, chunk e % CPR) of both tiles, so each
  // quarter-wave stores whole rows (conflict-free under the row swizzles).
  u32x4 kpre[T::LPT], vpre[T::LPT];
  auto load_tile = [&](int kt) {
    const int kbase = kt * T::BC;
#pragma unroll
    for (int i = 0; i < T::LPT; ++i) {
      const int e = tid + 256 * i;
      kpre[i] = load_row16(Kh, kbase + e / T::CPR, n, D, (e % T::CPR) * 8);
      vpre[i] = load_row16(Vh, kbase + e / T::CPR, n, D, (e % T::CPR) * 8);
    }
  };
  auto store_tile = [&](int stage) {
    unsigned char* sk = smem + stage * T::STAGE;
    unsigned char* sv = sk + T::K_BYTES;
#pragma unroll
    for (int i = 0; i < T::LPT; ++i) {
      const int e = tid + 256 * i;
      const int row = e / T::CPR, c = e % T::CPR;
      *reinterpret_cast<u32x4*>(sk + row * T::ROW + ((c ^ swz_k<D>(row)) << 4)) =
          kpre[i];
      *reinterpret_cast<u32x4*>(sv + row * T::ROW + ((c ^ swz_v<D>(row)) << 4)) =
          vpre[i];
    }
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

  f32x16 acc[T::DB];
#pragma unroll
  for (int db = 0; db < T::DB; ++db) acc[db] = zero16();
  float m = -INFINITY;  // running max, log2 units of the scaled score
  float l = 0.f;        // running exp-sum over this half-wave's keys

  int kt = tile_on(0) ? 0 : next_on(0);
  if (kt < kt_end) load_tile(kt);
  int stage = 0;
  while (kt < kt_end) {
    store_tile(stage);
    __syncthreads();
    const int kt_next = next_on(kt);
    if (kt_next < kt_end) load_tile(kt_next);

    const unsigned char* sk = smem + stage * T::STAGE;
    const unsigned char* sv = sk + T::K_BYTES;
    const int kbase = kt * T::BC;
    const bool wave_on = !CAUSAL || kbase <= qw0 + 31;
    if (wave_on) {
      // S^T = K Q^T for KB blocks of 32 keys.
      f32x16 s[T::KB];
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
      // Element mask: keys past the diagonal or past the sequence end.
      const bool need_mask =
          (CAUSAL && kbase + T::BC - 1 > qw0) || (kbase + T::BC > n);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < T::KB; ++kb) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kbase + kb * 32 + (i >> 2) * 8 + h * 4 + (i & 3);
            if ((CAUSAL && key > qrow) || key >= n) s[kb][i] = -INFINITY;
          }
        }
      }
      // Online softmax update ([TLDR] online softmax; [REAPER] 3.3).
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
      }
      mx = fmaxf(mx, xor32(mx));
      const float m_new = fmaxf(m, mx * c_log2);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m - m_use);
      float rs = 0.f;
      bf16x8 pf[T::KK];
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(fmaf(s[kb][i], c_log2, -m_use));
          s[kb][i] = p;
          rs += p;
        }
        pf[2 * kb] = pack8(s[kb], 0);
        pf[2 * kb + 1] = pack8(s[kb], 1);
      }
      l = l * alpha + rs;
      m = m_new;
      // alpha == 1 exactly when the row max did not move; skip the multiply
      // when that holds for the whole wave (an exact shortcut).
      if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < T::DB; ++db) {
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
        }
      }
      // O^T += V^T P^T.
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
    }
    stage ^= 1;
    kt = kt_next;
  }

  // Epilogue: one division by l per row ([TLDR] online softmax; [LLMSYS]
  // Fig. 1: dividing once at the end equals dividing every probability).
  const float l_tot = l + xor32(l);
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
  using T = FwdTile<D>;
  const int n_qtiles = (a.n + T::BR - 1) / T::BR;
  const int total = (int)(a.bh * n_qtiles);
  return launch_kernel(fwd_bf16_kernel<D, CAUSAL, SPARSE>, dim3(total),
                       dim3(256), s, (const bf16*)a.q, (const bf16*)a.k,
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
