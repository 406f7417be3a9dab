// Forward pass in float32 throughout (plain FMA on the vector units).
//
// Pages cited (titles as published):
//   [TLDR]   "FlashAttention：メモリ効率的なアテンション計算" (tech-tldr.com)
//   [XYZ]    "FlashAttention: IOを意識した高速かつメモリ効率の高い厳密な
//            アテンション" (xyznot.com)
//   [REAPER] "3 · FlashAttention" (mkdocs.reaper.mx, chapter 3)
//   [Q67]    "FlashAttention：在线 softmax 与 IO-aware 注意力" (quant67.com)
//
// The same tiled online-softmax recurrence as the bf16 kernel ([TLDR] online
// softmax and tiling sections; [REAPER] 3.2-3.3), with every product and sum
// in fp32 for callers who need fp32 accuracy.  [Q67] section 3 shows a
// one-row-per-block version with one block reduction per key; here a group
// of D/32 lanes owns one query row (each lane 32 of its d coordinates), the
// dot products are finished with one or two lane exchanges, key/value tiles
// of 64 rows are staged in LDS and shared by the 64 or 128 rows of a
// workgroup, and the softmax state is updated once per 16 keys rather than
// once per key.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kNumCus = 256;  // compute units of an MI355X

// KSPLIT groups of lanes share the workgroup's rows and split every key
// tile between them (group g takes keys 16g .. 16g + 15 of each 64-key
// tile); their partial states are merged at the end by the two-part rule
// ([XYZ], incremental softmax tracking).  KSPLIT = 4 is used when the
// problem has too few rows to fill the chip, so that each lane walks a
// quarter of the keys.
template <int D, int KSPLIT = 1>
struct F32Tile {
  static constexpr int TPR = D / 32;                // lanes per query row
  static constexpr int GROUP = 256 / KSPLIT;        // lanes per key group
  static constexpr int ROWS = GROUP / TPR;          // query rows per workgroup
  static constexpr int BC = 64;                     // keys per LDS tile
  static constexpr int CH = 16;                     // keys per softmax update
  static_assert(KSPLIT == 1 || KSPLIT * CH == BC, "one chunk per group");
};

template <int D, bool CAUSAL, bool SPARSE, int KSPLIT>
__global__ __launch_bounds__(256)
void fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                    const float* __restrict__ V, float* __restrict__ O,
                    float* __restrict__ LSE, int n, int nk, int q_off,
                    int n_qtiles, float c_log2, const uint8_t* __restrict__ mask,
                    int mask_cols, int block_m, int block_n) {
  using T = F32Tile<D, KSPLIT>;
  __shared__ __attribute__((aligned(16))) float smem[2 * T::BC * D];
  float* const sK = smem;
  float* const sV = smem + T::BC * D;

  const int tid = threadIdx.x;
  const int grp = tid / T::GROUP;       // key group (0 when KSPLIT = 1)
  const int gtid = tid % T::GROUP;
  const int part = gtid % T::TPR;
  const int head = blockIdx.x / n_qtiles;
  const int qt = CAUSAL ? (n_qtiles - 1 - blockIdx.x % n_qtiles)
                        : (blockIdx.x % n_qtiles);
  const int q0 = qt * T::ROWS;
  const int qrow = q0 + gtid / T::TPR;
  const int64_t hoff = (int64_t)head * n * D;     // Q, O: n rows per head
  const int64_t hoff_k = (int64_t)head * nk * D;  // K, V: nk rows
  const int c0 = part * 32;  // first d coordinate owned by this lane

  float q[32], acc[32];
#pragma unroll
  for (int c = 0; c < 32; c += 4) {
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (qrow < n) {
      x = *reinterpret_cast<const f32x4*>(Q + hoff + (int64_t)qrow * D + c0 + c);
    }
    q[c] = x[0];
    q[c + 1] = x[1];
    q[c + 2] = x[2];
    q[c + 3] = x[3];
  }
#pragma unroll
  for (int c = 0; c < 32; ++c) acc[c] = 0.f;
  float m = -INFINITY, l = 0.f;

  const int n_ktiles = (nk + T::BC - 1) / T::BC;
  int kt_end = n_ktiles;
  // (Row i sees the keys up to q_off + i under the causal rule, q_off >= 0.)
  if (CAUSAL) kt_end = min(n_ktiles, (min(q0 + T::ROWS, n) - 1 + q_off) / T::BC + 1);
  const uint8_t* mrow =
      SPARSE ? mask + (int64_t)(q0 / block_m) * mask_cols : nullptr;

  for (int kt = 0; kt < kt_end; ++kt) {
    const int kbase = kt * T::BC;
    if (SPARSE && mrow[kbase / block_n] == 0) continue;  // uniform
    __syncthreads();
    for (int e = tid * 4; e < T::BC * D; e += 256 * 4) {
      const int row = e / D;
      f32x4 kx = {0.f, 0.f, 0.f, 0.f}, vx = {0.f, 0.f, 0.f, 0.f};
      if (kbase + row < nk) {
        const int64_t off = hoff_k + (int64_t)(kbase + row) * D + (e % D);
        kx = *reinterpret_cast<const f32x4*>(K + off);
        vx = *reinterpret_cast<const f32x4*>(V + off);
      }
      *reinterpret_cast<f32x4*>(sK + e) = kx;
      *reinterpret_cast<f32x4*>(sV + e) = vx;
    }
    __syncthreads();
    const int kend = min(T::BC, nk - kbase);
    for (int k0 = grp * T::CH; k0 < kend; k0 += T::CH * KSPLIT) {
      float s[T::CH];
#pragma unroll
      for (int j = 0; j < T::CH; ++j) {
        const float* kr = sK + (k0 + j) * D + c0;
        float dot = 0.f;
#pragma unroll
        for (int c = 0; c < 32; c += 4) {
          const f32x4 kx = *reinterpret_cast<const f32x4*>(kr + c);
          dot = fmaf(q[c], kx[0], dot);
          dot = fmaf(q[c + 1], kx[1], dot);
          dot = fmaf(q[c + 2], kx[2], dot);
          dot = fmaf(q[c + 3], kx[3], dot);
        }
        if constexpr (T::TPR >= 2) dot += __shfl_xor(dot, 1);
        if constexpr (T::TPR >= 4) dot += __shfl_xor(dot, 2);
        const int key = kbase + k0 + j;
        s[j] = ((CAUSAL && key > q_off + qrow) || key >= nk) ? -INFINITY : dot;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < T::CH; ++j) mx = fmaxf(mx, s[j]);
      const float m_new = fmaxf(m, mx * c_log2);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m - m_use);
      float rs = 0.f;
#pragma unroll
      for (int j = 0; j < T::CH; ++j) {
        s[j] = fast_exp2(fmaf(s[j], c_log2, -m_use));
        rs += s[j];
      }
      l = l * alpha + rs;
      m = m_new;
#pragma unroll
      for (int c = 0; c < 32; ++c) acc[c] *= alpha;
#pragma unroll
      for (int j = 0; j < T::CH; ++j) {
        const float* vr = sV + (k0 + j) * D + c0;
#pragma unroll
        for (int c = 0; c < 32; c += 4) {
          const f32x4 vx = *reinterpret_cast<const f32x4*>(vr + c);
          acc[c] = fmaf(s[j], vx[0], acc[c]);
          acc[c + 1] = fmaf(s[j], vx[1], acc[c + 1]);
          acc[c + 2] = fmaf(s[j], vx[2], acc[c + 2]);
          acc[c + 3] = fmaf(s[j], vx[3], acc[c + 3]);
        }
      }
    }
  }

  if constexpr (KSPLIT > 1) {
    // Groups 1.. leave (m, l, acc) in LDS; group 0 merges them: with
    // M = max m_g, l = sum_g 2^(m_g - M) l_g and acc = sum_g 2^(m_g - M) acc_g.
    __syncthreads();
    float* st = smem;  // (KSPLIT - 1) x GROUP x (32 + 2) floats
    constexpr int STR = 34;
    static_assert((KSPLIT - 1) * T::GROUP * STR <= 2 * T::BC * D,
                  "merge state fits in the tile space");
    if (grp > 0) {
      float* my = st + ((grp - 1) * T::GROUP + gtid) * STR;
#pragma unroll
      for (int c = 0; c < 32; ++c) my[c] = acc[c];
      my[32] = m;
      my[33] = l;
    }
    __syncthreads();
    if (grp > 0) return;
    float mg[KSPLIT];
    mg[0] = m;
#pragma unroll
    for (int g = 1; g < KSPLIT; ++g) mg[g] = st[((g - 1) * T::GROUP + gtid) * STR + 32];
    float M = mg[0];
#pragma unroll
    for (int g = 1; g < KSPLIT; ++g) M = fmaxf(M, mg[g]);
    const float M_use = (M == -INFINITY) ? 0.f : M;
    const float a0 = fast_exp2(m - M_use);
    l *= a0;
#pragma unroll
    for (int c = 0; c < 32; ++c) acc[c] *= a0;
#pragma unroll
    for (int g = 1; g < KSPLIT; ++g) {
      const float* o = st + ((g - 1) * T::GROUP + gtid) * STR;
      const float a = fast_exp2(mg[g] - M_use);
      l = fmaf(a, o[33], l);
#pragma unroll
      for (int c = 0; c < 32; ++c) acc[c] = fmaf(a, o[c], acc[c]);
    }
    m = M;
  }
  if (qrow < n) {
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
    float* orow = O + hoff + (int64_t)qrow * D + c0;
#pragma unroll
    for (int c = 0; c < 32; c += 4) {
      f32x4 x = {acc[c] * inv, acc[c + 1] * inv, acc[c + 2] * inv,
                 acc[c + 3] * inv};
      *reinterpret_cast<f32x4*>(orow + c) = x;
    }
    if (part == 0) {
      LSE[(int64_t)head * n + qrow] =
          (l > 0.f) ? (m + fast_log2(l)) * kLn2 : -INFINITY;
    }
  }
}

template <int D, bool CAUSAL, bool SPARSE, int KSPLIT>
hipError_t launch_k(const FwdArgs& a, hipStream_t s) {
  using T = F32Tile<D, KSPLIT>;
  const int n_qtiles = (a.n + T::ROWS - 1) / T::ROWS;
  const int total = (int)(a.bh * n_qtiles);
  return launch_kernel(fwd_f32_kernel<D, CAUSAL, SPARSE, KSPLIT>, dim3(total),
                       dim3(256), s, (const float*)a.q, (const float*)a.k,
                       (const float*)a.v, (float*)a.o, a.lse, a.n, a.nk, a.q_off,
                       n_qtiles,
                       a.scale * kLog2e, a.mask, a.mask_cols, a.block_m,
                       a.block_n);
}

// Problems with fewer than two workgroups per CU in the plain layout take
// the key-split layout (four times the workgroups, a quarter of the keys
// per lane).
template <int D, bool CAUSAL, bool SPARSE>
hipError_t launch_t(const FwdArgs& a, hipStream_t s) {
  using T = F32Tile<D, 1>;
  const int64_t wgs = a.bh * ((a.n + T::ROWS - 1) / T::ROWS);
  if (wgs < 2 * kNumCus) return launch_k<D, CAUSAL, SPARSE, 4>(a, s);
  return launch_k<D, CAUSAL, SPARSE, 1>(a, s);
}

template <int D>
hipError_t dispatch(const FwdArgs& a, hipStream_t s) {
  if (a.mask) {
    return a.causal ? launch_t<D, true, true>(a, s)
                    : launch_t<D, false, true>(a, s);
  }
  return a.causal ? launch_t<D, true, false>(a, s)
                  : launch_t<D, false, false>(a, s);
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s) {
  return a.d == 128 ? dispatch<128>(a, s) : dispatch<64>(a, s);
}

}  // namespace fa
