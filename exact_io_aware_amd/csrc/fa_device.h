// Device-side building blocks for the gfx950 (CDNA4) attention kernels:
// vector types, the bf16 MFMA wrapper, swizzled LDS addressing, cross-half
// wave exchange and the XCD-aware workgroup order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// MFMA: D(32x32, f32) += A(32x16, bf16) * B(16x32, bf16), one wave64.
// Operand layouts (lane l, half h = l / 32):
//   A: lane holds A[m = l % 32][k = h*8 + 0..7]
//   B: lane holds B[k = h*8 + 0..7][n = l % 32]
//   D: register i of lane l holds D[m = (i/4)*8 + h*4 + i%4][n = l % 32]
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) {
  return __builtin_bit_cast(bf16x8, u);
}

// Round two floats to bf16 (nearest-even) and pack: lo in bits 0..15.
// A two-lane vector conversion maps to a single v_cvt_pk_bf16_f32.
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// Pack 8 consecutive registers of a D-layout accumulator into a bf16x8
// operand (register 8s + j becomes operand slot j).
__device__ __forceinline__ bf16x8 pack8(const f32x16& x, int s) {
  u32x4 u;
  u[0] = pack_bf16(x[8 * s + 0], x[8 * s + 1]);
  u[1] = pack_bf16(x[8 * s + 2], x[8 * s + 3]);
  u[2] = pack_bf16(x[8 * s + 4], x[8 * s + 5]);
  u[3] = pack_bf16(x[8 * s + 6], x[8 * s + 7]);
  return as_bf16x8(u);
}

// Value held by lane l ^ 32 (the other half of the wave).
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}
__device__ __forceinline__ float fast_log2(float x) {
  return __builtin_amdgcn_logf(x);
}

// ---------------------------------------------------------------------------
// Swizzled LDS tiles.  A tile is a stack of rows of ROW_BYTES bytes, each
// split into 16-byte chunks.  Chunk c of row r is stored at chunk slot
// c ^ swz(r), so that the 16 rows read together by one quarter-wave's
// 16-byte loads (same logical chunk, consecutive rows) land on distinct
// banks.
// ---------------------------------------------------------------------------
template <int ROW_BYTES>
__device__ __forceinline__ int swz(int r) {
  static_assert(ROW_BYTES == 128 || ROW_BYTES == 256, "row size");
  if constexpr (ROW_BYTES == 256) {
    return r & 15;
  } else {
    return (r >> 1) & 7;
  }
}

template <int ROW_BYTES>
__device__ __forceinline__ int lds_off(int r, int c) {
  return r * ROW_BYTES + ((c ^ swz<ROW_BYTES>(r)) << 4);
}

// Position of key offset o (0..15) inside a 16-key group of a transposed
// tile.  The D layout of an MFMA result gives half h of the wave the keys
// {h*4 + 0..3, 8 + h*4 + 0..3} of each 16-key group, while an operand slot
// j of half h reads position h*8 + j; storing runs of 4 keys in the order
// 0, 2, 1, 3 makes the two agree.  (The contraction index is a dummy, so any
// order works as long as both operands use the same one.)
__device__ __forceinline__ int perm_run(int run) {
  return ((run & 1) << 1) | (run >> 1);  // 0->0, 1->2, 2->1, 3->3
}

// Transpose 4 rows x 8 columns of bf16 (in[r] = 16 bytes of row r) into
// 8 columns x 4 rows: out[e] = {row0, row1, row2, row3} of column e packed in
// two dwords.
__device__ __forceinline__ void transpose4x8(const u32x4 in[4], u32x2 out[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
    out[e][0] = __builtin_amdgcn_perm(in[1][e >> 1], in[0][e >> 1], sel);
    out[e][1] = __builtin_amdgcn_perm(in[3][e >> 1], in[2][e >> 1], sel);
  }
}

// 16-byte global load of row `row` (zero when row >= n).
__device__ __forceinline__ u32x4 load_row16(const bf16* base, int row, int n,
                                            int ld, int col) {
  u32x4 z = {0u, 0u, 0u, 0u};
  if (row < n) {
    z = *reinterpret_cast<const u32x4*>(base + (int64_t)row * ld + col);
  }
  return z;
}

// ---------------------------------------------------------------------------
// Workgroup order.  Consecutive workgroup ids are dealt round-robin over the
// 8 XCDs, each with its own L2.  Renumbering so that each XCD receives a
// contiguous range of logical ids keeps all tiles of a head on one XCD, so
// the K/V re-reads of that head hit the same L2.
// ---------------------------------------------------------------------------
constexpr int kNumXcd = 8;

// ---------------------------------------------------------------------------
// Host-side launch returning the launch's own status (hipLaunchKernel does
// not report errors left over from earlier, unrelated calls).
// ---------------------------------------------------------------------------
template <typename T>
struct ident {
  using type = T;
};

template <typename... P>
inline hipError_t launch_kernel(void (*kern)(P...), dim3 grid, dim3 block,
                                hipStream_t s,
                                typename ident<P>::type... args) {
  void* argv[] = {(void*)&args..., nullptr};
  return hipLaunchKernel((const void*)kern, grid, block, argv, 0, s);
}

__device__ __forceinline__ int xcd_logical_id(int g, int total) {
  if (total % kNumXcd != 0) return g;
  const int per = total / kNumXcd;
  return (g % kNumXcd) * per + g / kNumXcd;
}

}  // namespace fa
