// Backward pass in float32 throughout (plain FMA on the vector units).
//
// Pages cited (titles as published):
//   [TLDR]   "FlashAttention：メモリ効率的なアテンション計算" (tech-tldr.com)
//   [XYZ]    "FlashAttention: IOを意識した高速かつメモリ効率の高い厳密な
//            アテンション" (xyznot.com)
//   [REAPER] "3 · FlashAttention" (mkdocs.reaper.mx, chapter 3)
//   [Q67]    "FlashAttention：在线 softmax 与 IO-aware 注意力" (quant67.com)
//
// The same recomputation scheme as the bf16 backward ([TLDR] backward
// section; [REAPER] 3.4; [Q67] section 5): nothing of size N x N is stored;
// every probability is rebuilt from q, k and the saved logsumexp,
// P = exp(S - LSE), and the gradients of L = sum(O * dO) follow by the chain
// rule: D_i = sum_c dO_ic O_ic, dV = P^T dO, dP = dO V^T, dS = P * (dP - D),
// dQ = scale dS K, dK = scale dS^T Q.  Three kernels: the row pass (D and
// LSE in base-2 units), a key pass (dK, dV) and a query pass (dQ); no
// atomics, every output element is written once.
//
// Mapping: a group of D/32 lanes owns one key row (key pass) or one query
// row (query pass), each lane 32 of its d coordinates in registers; the
// other side's rows are staged through LDS in tiles shared by the whole
// workgroup, and each dot product is finished with one or two lane
// exchanges.  Every product and sum is fp32, for callers who need fp32
// accuracy; the bf16 kernels are the fast path.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

template <int D>
struct F32BwdTile {
  static constexpr int TPR = D / 32;       // lanes per row
  static constexpr int ROWS = 256 / TPR;   // rows owned by a workgroup
  static constexpr int BT = 32;            // rows per LDS tile of the other side
};

// Row pass: D_i = sum_c dO_ic O_ic and LSE_i * log2(e) (+inf for a row that
// saw no key, so that every rebuilt probability of that row is exactly 0).
template <int D>
__global__ __launch_bounds__(256)
void bwd_pre_f32_kernel(const float* __restrict__ O, const float* __restrict__ dO,
                        const float* __restrict__ lse, float* __restrict__ ws_d,
                        float* __restrict__ ws_lse2, int64_t rows) {
  constexpr int TPR = D / 4;  // 16-byte chunks per row
  const int64_t row = (int64_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(O + row * D + part * 4);
    const f32x4 b = *reinterpret_cast<const f32x4*>(dO + row * D + part * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = fmaf(a[i], b[i], acc);
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (part == 0 && row < rows) {
    ws_d[row] = acc;
    const float L = lse[row];
    ws_lse2[row] = (L == -INFINITY) ? INFINITY : L * kLog2e;
  }
}

// The 32 coordinates of row `row` owned by this lane (zeros past n).
__device__ __forceinline__ void load32(const float* base, int row, int n, int d,
                                       int c0, float (&x)[32]) {
#pragma unroll
  for (int c = 0; c < 32; c += 4) {
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (row < n) v = *reinterpret_cast<const f32x4*>(base + (int64_t)row * d + c0 + c);
    x[c] = v[0];
    x[c + 1] = v[1];
    x[c + 2] = v[2];
    x[c + 3] = v[3];
  }
}

__device__ __forceinline__ void store32(float* base, int row, int d, int c0,
                                        const float (&x)[32], float mul) {
#pragma unroll
  for (int c = 0; c < 32; c += 4) {
    const f32x4 v = {x[c] * mul, x[c + 1] * mul, x[c + 2] * mul, x[c + 3] * mul};
    *reinterpret_cast<f32x4*>(base + (int64_t)row * d + c0 + c) = v;
  }
}

// Partial dot product of this lane's 32 coordinates with an LDS row, then
// summed over the D/32 lanes of the row.
template <int TPR>
__device__ __forceinline__ float dot32(const float (&x)[32], const float* s) {
  float dot = 0.f;
#pragma unroll
  for (int c = 0; c < 32; c += 4) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(s + c);
    dot = fmaf(x[c], v[0], dot);
    dot = fmaf(x[c + 1], v[1], dot);
    dot = fmaf(x[c + 2], v[2], dot);
    dot = fmaf(x[c + 3], v[3], dot);
  }
  if constexpr (TPR >= 2) dot += __shfl_xor(dot, 1);
  if constexpr (TPR >= 4) dot += __shfl_xor(dot, 2);
  return dot;
}

// Key pass: the workgroup owns ROWS keys and sweeps the query rows in tiles
// of BT (Q, dO, LSE*log2e, D staged in LDS); under the causal rule query
// tiles entirely before the first key are skipped, in the block-sparse form
// query tiles whose mask block is 0.
template <int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(256)
void bwd_dkdv_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                         const float* __restrict__ V, const float* __restrict__ dO,
                         const float* __restrict__ ws_d,
                         const float* __restrict__ ws_lse2, float* __restrict__ dK,
                         float* __restrict__ dV, int n, int nk, int q_off,
                         int n_ktiles, float c_log2,
                         float scale, const uint8_t* __restrict__ mask,
                         int mask_cols, int block_m, int block_n) {
  using T = F32BwdTile<D>;
  __shared__ __attribute__((aligned(16))) float sQ[T::BT * D];
  __shared__ __attribute__((aligned(16))) float sdO[T::BT * D];
  __shared__ float sL[T::BT], sD[T::BT];

  const int tid = threadIdx.x;
  const int part = tid % T::TPR;
  const int head = blockIdx.x / n_ktiles;
  const int k0 = (blockIdx.x % n_ktiles) * T::ROWS;
  const int key = k0 + tid / T::TPR;
  const int c0 = part * 32;
  const int64_t hoff = (int64_t)head * n * D;     // Q, dO: n rows per head
  const int64_t hoff_k = (int64_t)head * nk * D;  // K, V, dK, dV: nk rows
  const float* Lh = ws_lse2 + (int64_t)head * n;
  const float* Dh = ws_d + (int64_t)head * n;

  float k[32], v[32], dk[32], dv[32];
  load32(K + hoff_k, key, nk, D, c0, k);
  load32(V + hoff_k, key, nk, D, c0, v);
#pragma unroll
  for (int c = 0; c < 32; ++c) {
    dk[c] = 0.f;
    dv[c] = 0.f;
  }

  const int n_qt = (n + T::BT - 1) / T::BT;
  // Under the causal rule query row i sees key k0 from i = k0 - q_off on.
  const int qt0 = CAUSAL ? max(0, k0 - q_off) / T::BT : 0;
  for (int qt = qt0; qt < n_qt; ++qt) {
    const int q0 = qt * T::BT;
    if (SPARSE && mask[(int64_t)(q0 / block_m) * mask_cols + k0 / block_n] == 0) {
      continue;  // uniform: the tile lies in one block row, the keys in one block column
    }
    __syncthreads();
    for (int e = tid * 4; e < T::BT * D; e += 256 * 4) {
      const int row = q0 + e / D;
      f32x4 qx = {0.f, 0.f, 0.f, 0.f}, dx = {0.f, 0.f, 0.f, 0.f};
      if (row < n) {
        const int64_t off = hoff + (int64_t)row * D + (e % D);
        qx = *reinterpret_cast<const f32x4*>(Q + off);
        dx = *reinterpret_cast<const f32x4*>(dO + off);
      }
      *reinterpret_cast<f32x4*>(sQ + e) = qx;
      *reinterpret_cast<f32x4*>(sdO + e) = dx;
    }
    if (tid < T::BT) {
      const int row = q0 + tid;
      sL[tid] = (row < n) ? Lh[row] : INFINITY;  // rows past n: P = 0
      sD[tid] = (row < n) ? Dh[row] : 0.f;
    }
    __syncthreads();
    for (int i = 0; i < T::BT; ++i) {
      const float s = dot32<T::TPR>(k, sQ + i * D + c0);
      const float dp = dot32<T::TPR>(v, sdO + i * D + c0);
      const int q = q0 + i;
      const bool vis = (key < nk) && (!CAUSAL || key <= q_off + q);
      const float p = vis ? fast_exp2(fmaf(s, c_log2, -sL[i])) : 0.f;
      const float ds = p * (dp - sD[i]);
      const float* qr = sQ + i * D + c0;
      const float* dr = sdO + i * D + c0;
#pragma unroll
      for (int c = 0; c < 32; c += 4) {
        const f32x4 qx = *reinterpret_cast<const f32x4*>(qr + c);
        const f32x4 dx = *reinterpret_cast<const f32x4*>(dr + c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dv[c + e] = fmaf(p, dx[e], dv[c + e]);
          dk[c + e] = fmaf(ds, qx[e], dk[c + e]);
        }
      }
    }
  }
  if (key < nk) {
    store32(dK + hoff_k, key, D, c0, dk, scale);
    store32(dV + hoff_k, key, D, c0, dv, 1.f);
  }
}

// Query pass: the workgroup owns ROWS query rows and sweeps the keys in
// tiles of BT (K and V staged in LDS), up to the diagonal under the causal
// rule, skipping key tiles whose mask block is 0 in the block-sparse form.
template <int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(256)
void bwd_dq_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                       const float* __restrict__ V, const float* __restrict__ dO,
                       const float* __restrict__ ws_d,
                       const float* __restrict__ ws_lse2, float* __restrict__ dQ,
                       int n, int nk, int q_off, int n_qtiles, float c_log2,
                       float scale, const uint8_t* __restrict__ mask, int mask_cols,
                       int block_m, int block_n) {
  using T = F32BwdTile<D>;
  __shared__ __attribute__((aligned(16))) float sK[T::BT * D];
  __shared__ __attribute__((aligned(16))) float sV[T::BT * D];

  const int tid = threadIdx.x;
  const int part = tid % T::TPR;
  const int head = blockIdx.x / n_qtiles;
  const int qt = CAUSAL ? (n_qtiles - 1 - blockIdx.x % n_qtiles)
                        : (blockIdx.x % n_qtiles);
  const int q0 = qt * T::ROWS;
  const int qrow = q0 + tid / T::TPR;
  const int c0 = part * 32;
  const int64_t hoff = (int64_t)head * n * D;     // Q, dO, dQ: n rows per head
  const int64_t hoff_k = (int64_t)head * nk * D;  // K, V: nk rows

  float q[32], dout[32], dq[32];
  load32(Q + hoff, qrow, n, D, c0, q);
  load32(dO + hoff, qrow, n, D, c0, dout);
#pragma unroll
  for (int c = 0; c < 32; ++c) dq[c] = 0.f;
  const float lse2 = (qrow < n) ? ws_lse2[(int64_t)head * n + qrow] : INFINITY;
  const float drow = (qrow < n) ? ws_d[(int64_t)head * n + qrow] : 0.f;

  const int n_kt = (nk + T::BT - 1) / T::BT;
  int kt_end = n_kt;
  // (Row i sees the keys up to q_off + i under the causal rule, q_off >= 0.)
  if (CAUSAL) kt_end = min(n_kt, (min(q0 + T::ROWS, n) - 1 + q_off) / T::BT + 1);
  const uint8_t* mrow =
      SPARSE ? mask + (int64_t)(q0 / block_m) * mask_cols : nullptr;
  for (int kt = 0; kt < kt_end; ++kt) {
    const int kbase = kt * T::BT;
    if (SPARSE && mrow[kbase / block_n] == 0) continue;  // uniform
    __syncthreads();
    for (int e = tid * 4; e < T::BT * D; e += 256 * 4) {
      const int row = kbase + e / D;
      f32x4 kx = {0.f, 0.f, 0.f, 0.f}, vx = {0.f, 0.f, 0.f, 0.f};
      if (row < nk) {
        const int64_t off = hoff_k + (int64_t)row * D + (e % D);
        kx = *reinterpret_cast<const f32x4*>(K + off);
        vx = *reinterpret_cast<const f32x4*>(V + off);
      }
      *reinterpret_cast<f32x4*>(sK + e) = kx;
      *reinterpret_cast<f32x4*>(sV + e) = vx;
    }
    __syncthreads();
    for (int j = 0; j < T::BT; ++j) {
      const float s = dot32<T::TPR>(q, sK + j * D + c0);
      const float dp = dot32<T::TPR>(dout, sV + j * D + c0);
      const int key = kbase + j;
      const bool vis = (key < nk) && (!CAUSAL || key <= q_off + qrow);
      const float p = vis ? fast_exp2(fmaf(s, c_log2, -lse2)) : 0.f;
      const float ds = p * (dp - drow);
      const float* kr = sK + j * D + c0;
#pragma unroll
      for (int c = 0; c < 32; c += 4) {
        const f32x4 kx = *reinterpret_cast<const f32x4*>(kr + c);
#pragma unroll
        for (int e = 0; e < 4; ++e) dq[c + e] = fmaf(ds, kx[e], dq[c + e]);
      }
    }
  }
  if (qrow < n) store32(dQ + hoff, qrow, D, c0, dq, scale);
}

template <int D>
hipError_t pre_t(const BwdArgs& a, hipStream_t s) {
  const int64_t rows = a.bh * a.n;
  const int64_t grid = (rows + 256 / (D / 4) - 1) / (256 / (D / 4));
  return launch_kernel(bwd_pre_f32_kernel<D>, dim3((unsigned)grid), dim3(256), s,
                       (const float*)a.o, (const float*)a.dout, a.lse, a.ws_d,
                       a.ws_lse2, rows);
}

template <int D, bool CAUSAL, bool SPARSE>
hipError_t dkdv_t(const BwdArgs& a, hipStream_t s) {
  using T = F32BwdTile<D>;
  const int n_kt = (a.nk + T::ROWS - 1) / T::ROWS;
  return launch_kernel(bwd_dkdv_f32_kernel<D, CAUSAL, SPARSE>,
                       dim3((unsigned)(a.bh * n_kt)), dim3(256), s,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v,
                       (const float*)a.dout, (const float*)a.ws_d,
                       (const float*)a.ws_lse2, a.dk, a.dv, a.n, a.nk, a.q_off,
                       n_kt,
                       a.scale * kLog2e, a.scale, a.mask, a.mask_cols,
                       a.block_m, a.block_n);
}

template <int D, bool CAUSAL, bool SPARSE>
hipError_t dq_t(const BwdArgs& a, hipStream_t s) {
  using T = F32BwdTile<D>;
  const int n_qt = (a.n + T::ROWS - 1) / T::ROWS;
  return launch_kernel(bwd_dq_f32_kernel<D, CAUSAL, SPARSE>,
                       dim3((unsigned)(a.bh * n_qt)), dim3(256), s,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v,
                       (const float*)a.dout, (const float*)a.ws_d,
                       (const float*)a.ws_lse2, a.dq, a.n, a.nk, a.q_off, n_qt,
                       a.scale * kLog2e, a.scale, a.mask, a.mask_cols,
                       a.block_m, a.block_n);
}

template <int D>
hipError_t dkdv_d(const BwdArgs& a, hipStream_t s) {
  if (a.mask) {
    return a.causal ? dkdv_t<D, true, true>(a, s) : dkdv_t<D, false, true>(a, s);
  }
  return a.causal ? dkdv_t<D, true, false>(a, s) : dkdv_t<D, false, false>(a, s);
}

template <int D>
hipError_t dq_d(const BwdArgs& a, hipStream_t s) {
  if (a.mask) {
    return a.causal ? dq_t<D, true, true>(a, s) : dq_t<D, false, true>(a, s);
  }
  return a.causal ? dq_t<D, true, false>(a, s) : dq_t<D, false, false>(a, s);
}

}  // namespace

hipError_t launch_bwd_preprocess_f32(const BwdArgs& a, hipStream_t s) {
  return a.d == 128 ? pre_t<128>(a, s) : pre_t<64>(a, s);
}
hipError_t launch_bwd_dkdv_f32(const BwdArgs& a, hipStream_t s) {
  return a.d == 128 ? dkdv_d<128>(a, s) : dkdv_d<64>(a, s);
}
hipError_t launch_bwd_dq_f32(const BwdArgs& a, hipStream_t s) {
  return a.d == 128 ? dq_d<128>(a, s) : dq_d<64>(a, s);
}

}  // namespace fa
