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
// Reductions over the two 32-lane halves of a wave.  v_permlane32_swap
// exchanges the upper half of its first operand with the lower half of its
// second; with both operands equal to x, the two results hold x's lower half
// twice and its upper half twice, so one max or add gives every lane the
// combined value (identically in both halves).  A VALU op, unlike a
// ds_bpermute it needs no LDS round trip.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                                  __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                                  __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}
__device__ __forceinline__ float fast_log2(float x) {
  return __builtin_amdgcn_logf(x);
}
// The two bf16 values of a 32-bit word (element 2i in the low half, 2i + 1
// in the high half) as floats (exact).
__device__ __forceinline__ float bf16_lo(uint32_t u) {
  return __uint_as_float(u << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t u) {
  return __uint_as_float(u & 0xffff0000u);
}

// Chunk swizzle for a row-major bf16 tile with D columns that is read both
// row-wise (16 consecutive rows, one 16-B chunk each, as an MFMA A operand)
// and by transpose reads (8 consecutive rows, one 64-B run each).  The
// row-wise pattern needs the swizzle to be a bijection over 16 consecutive
// rows; the transpose pattern needs rows 0-3 of each group of 8 to land on
// disjoint 64-B bank groups.  A bit rotation of the row index gives both:
//   D = 128 (256-B rows): bits (r1 r0 | r3 r2) of r;
//   D = 64 (128-B rows, two rows per bank line): t = (r >> 1) & 7 rotated.
template <int D>
__device__ __forceinline__ int tile_swz(int r) {
  if constexpr (D == 128) {
    return ((r & 3) << 2) | ((r >> 2) & 3);
  } else {
    const int t = (r >> 1) & 7;
    return ((t & 1) << 2) | (t >> 1);
  }
}

template <int D>
__device__ __forceinline__ int tile_off(int r, int c) {
  return r * (D * 2) + ((c ^ tile_swz<D>(r)) << 4);
}

// ---------------------------------------------------------------------------
// LDS transpose read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane i receives element (i % 4) of the 8-byte rows addressed by
// lanes i/4, 4 + i/4, 8 + i/4 and 12 + i/4, in that order.  If source lane s
// addresses row R(s / 4) at column C + 4 * (s % 4) of a row-major bf16 tile,
// lane i therefore receives column C + i of rows R(0..3): four consecutive
// contraction-index values at a fixed output column, which is the MFMA
// operand layout of the transposed tile.
// ---------------------------------------------------------------------------
typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i16x4 lds_read_tr16(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
}

// Two transpose reads (slots 0-3 and 4-7) joined into one MFMA operand.
__device__ __forceinline__ bf16x8 join_tr16(i16x4 lo, i16x4 hi) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// 16-byte global load of row `row`, clamped to the last row n - 1 (n >= 1).
// Rows past the end therefore read valid memory with arbitrary finite
// contents; every caller masks or discards what they contribute.
__device__ __forceinline__ u32x4 load_row16(const bf16* base, int row, int n,
                                            int ld, int col) {
  const int r = min(row, n - 1);
  return *reinterpret_cast<const u32x4*>(base + (int64_t)r * ld + col);
}

// ---------------------------------------------------------------------------
// Global -> LDS direct loads (gfx950 global_load_lds_dwordx4 / _dword).  Lane
// l of a wave writes its 16 (or 4) bytes at lds + 16*l (4*l): a wave fills
// one contiguous 1-KB (256-B) block per instruction, and the swizzle of the
// destination tile is obtained by choosing each lane's source address.  The
// data lands asynchronously; "s_waitcnt vmcnt(0)" followed by a workgroup
// barrier makes it visible to every wave.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

__device__ __forceinline__ void dma16(const void* src, unsigned char* lds) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, unsigned char* lds) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)src, (lds_void_t*)lds, 4, 0, 0);
}
__device__ __forceinline__ void wait_dma() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Fill 1-KB block `blk` of a swizzled row-major tile (rows of D bf16) from
// global rows row0, row0 + 1, ... of `g` (rows clamped to n - 1).
template <int D>
__device__ __forceinline__ void dma_tile_block(const bf16* g, int row0, int n,
                                               unsigned char* tile, int blk,
                                               int lane) {
  const int o = blk * 1024 + lane * 16;
  const int row = o / (D * 2);
  const int c = ((o % (D * 2)) >> 4) ^ tile_swz<D>(row);
  dma16(g + (int64_t)min(row0 + row, n - 1) * D + c * 8, tile + blk * 1024);
}

// ---------------------------------------------------------------------------
// Workgroup order.  Consecutive workgroup ids are dealt round-robin over the
// 8 XCDs, each with its own L2.  Renumbering so that each XCD receives a
// contiguous range of logical ids keeps all tiles of a head on one XCD, so
// the K/V re-reads of that head hit the same L2.
// ---------------------------------------------------------------------------
constexpr int kNumXcd = 8;

__device__ __forceinline__ int xcd_logical_id(int g, int total) {
  if (total % kNumXcd != 0) return g;
  const int per = total / kNumXcd;
  return (g % kNumXcd) * per + g / kNumXcd;
}

// Order of the workgroups of a causal problem, whose tiles of one head
// carry different amounts of work.  Logical ids (XCD-contiguous, above) run
// over bundles of `bundle` consecutive heads; inside a bundle they go
// heaviest tile first across the bundle's heads.  With bundle = 1 this is
// head by head, heaviest tile first, which keeps one head's K/V hot in an
// XCD's L2 when its tiles fill the XCD; when a head has fewer tiles than an
// XCD has workgroup slots, bundle = slots / tiles (rounded up) keeps the
// longest-first order across the XCD.  Returns the head and the tile's rank
// (0 = heaviest).  Used where a workgroup takes one tile (4-wave forward and
// dQ instances, block-sparse instances); the dense one-workgroup-per-CU
// kernels instead pair tiles u and n-1-u so that all workgroups carry equal
// work.
struct CausalPlace {
  int head, rank;
};
__device__ __forceinline__ CausalPlace causal_place(int lid, int n_tiles,
                                                    int n_heads, int bundle) {
  const int per = bundle * n_tiles;
  const int b = lid / per;
  const int h0 = b * bundle;
  const int nb = min(bundle, n_heads - h0);
  const int idx = lid - b * per;
  return {h0 + idx % nb, idx / nb};
}

// Bundle size for causal_place: enough heads to fill the workgroup slots of
// one XCD (32 CUs times the workgroups that fit on a CU).
inline int causal_bundle(int n_tiles, int wgs_per_cu) {
  const int slots = 32 * wgs_per_cu;
  return n_tiles >= slots ? 1 : (slots + n_tiles - 1) / n_tiles;
}

// ---------------------------------------------------------------------------
// Dropout on the attention probabilities ([XYZ] key ideas: dropout is one of
// the steps fused into the attention kernel).  The random numbers come from
// the counter-based generator Philox4x32-10 (Salmon, Moraes, Dror, Shaw,
// "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011).  Element (bh, i,
// j) of head bh, query row i and key j takes byte (j & 3) of word (i & 3) of
// the call with counter (i >> 2, j >> 2, bh, off) and key (seed low, seed
// high), off being the position of query row 0 among the keys (0 when
// queries and keys are the same tokens); it is kept iff that byte is >= t
// (drop probability t / 256).  One call covers a 4 x 4 block of scores, so
// the mask does not depend on the tiling.
// ---------------------------------------------------------------------------
struct Dropout {
  uint32_t k0, k1;  // seed words
  uint32_t bh;      // head index b * H + h
  uint32_t t;       // keep iff byte >= t
  float inv_keep;   // 256 / (256 - t)
  uint32_t off;     // counter word 3: position of query row 0
};

inline Dropout make_dropout(int t, uint32_t seed_lo, uint32_t seed_hi,
                            int q_off) {
  return Dropout{seed_lo, seed_hi, 0u, (uint32_t)t, 256.f / (float)(256 - t),
                 (uint32_t)q_off};
}

// a ^ b ^ c in one instruction (gfx950's three-input bitwise operation
// with truth table 0x96); the compiler emits two v_xor_b32 for the
// expression.
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

// One round of Philox4x32: two 32 x 32 -> 64-bit products with the
// published multipliers and a word permutation, with the round's keys
// (the seed words advanced by the published Weyl increments, kWeyl0/1 per
// round).
constexpr uint32_t kWeyl0 = 0x9E3779B9u, kWeyl1 = 0xBB67AE85u;
__device__ __forceinline__ void philox_round(uint32_t (&x)[4], uint32_t k0,
                                             uint32_t k1) {
  const uint64_t p0 = (uint64_t)x[0] * 0xD2511F53u;
  const uint64_t p1 = (uint64_t)x[2] * 0xCD9E8D57u;
  const uint32_t y0 = xor3((uint32_t)(p1 >> 32), x[1], k0);
  const uint32_t y2 = xor3((uint32_t)(p0 >> 32), x[3], k1);
  x[0] = y0;
  x[1] = (uint32_t)p1;
  x[2] = y2;
  x[3] = (uint32_t)p0;
}

// One Philox4x32-10 call: ten rounds.
__device__ __forceinline__ void philox4x32_10(uint32_t (&x)[4], uint32_t k0,
                                              uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) philox_round(x, k0 + r * kWeyl0, k1 + r * kWeyl1);
}

// Transpose of a 4 x 4 matrix of words held by a quad of lanes (lanes 4m ..
// 4m+3, word index w): afterwards lane q holds in w[g] what lane g held in
// w[q].  Two stages of lane exchanges within the quad (DPP quad
// permutations): transpose each 2 x 2 block, then swap the off-diagonal
// blocks.
__device__ __forceinline__ void quad_transpose(uint32_t (&w)[4], int lane) {
  const bool odd = lane & 1, upper = lane & 2;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const uint32_t send = odd ? w[2 * b] : w[2 * b + 1];
    const uint32_t r = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0xB1, 0xF, 0xF, false);
    if (odd) w[2 * b] = r; else w[2 * b + 1] = r;
  }
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const uint32_t send = upper ? w[b] : w[2 + b];
    const uint32_t r = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0x4E, 0xF, 0xF, false);
    if (upper) w[b] = r; else w[2 + b] = r;
  }
}

// Random bytes for the score registers of one 32 x 32 MFMA block in the
// layout with lane = query row (register r of the block holds key
// 8 (r / 4) + 4 h + r % 4 relative to key0, h = lane / 32): word g of the
// result holds, in byte t, the byte of key key0 + 8 g + 4 h + t.  row is this
// lane's query; key0 is a multiple of 32, rows 4m .. 4m + 3 sit in the lanes
// of one quad.  The counter alone (dropout_ctr_rowlane) lets a caller spread
// the ten rounds (philox_round) between products and finish with
// quad_transpose.
__device__ __forceinline__ void dropout_ctr_rowlane(const Dropout& dr, int row,
                                                    int key0, int lane,
                                                    uint32_t (&x)[4]) {
  const int h = (lane >> 5) & 1, q = lane & 3;
  // this lane draws the 4 x 4 block of keys key0 + 8 q + 4 h ...
  x[0] = (uint32_t)row >> 2;
  x[1] = (uint32_t)(key0 + 8 * q + 4 * h) >> 2;
  x[2] = dr.bh;
  x[3] = dr.off;
}
__device__ __forceinline__ void dropout_bytes_rowlane(const Dropout& dr, int row,
                                                      int key0, int lane,
                                                      uint32_t (&out)[4]) {
  dropout_ctr_rowlane(dr, row, key0, lane, out);
  philox4x32_10(out, dr.k0, dr.k1);
  // ... whose word q' belongs to row 4 (row >> 2) + q', the lane q' of the quad
  quad_transpose(out, lane);
}

// The same in the layout with lane = key (register r of the block holds
// query 8 (r / 4) + 4 h + r % 4 relative to row0): word g of the result
// holds, in byte t, the byte of query row0 + 8 g + 4 h + t and this lane's
// key.  key is this lane's key; keys 4m .. 4m + 3 sit in one quad.  Split
// into the counter (dropout_ctr_keylane), the ten rounds (philox_round,
// which a caller may spread between products) and the regrouping
// (dropout_finish_keylane).
__device__ __forceinline__ void dropout_ctr_keylane(const Dropout& dr, int key,
                                                    int row0, int lane,
                                                    uint32_t (&x)[4]) {
  const int h = (lane >> 5) & 1, q = lane & 3;
  x[0] = (uint32_t)(row0 + 8 * q + 4 * h) >> 2;
  x[1] = (uint32_t)key >> 2;
  x[2] = dr.bh;
  x[3] = dr.off;
}
__device__ __forceinline__ void dropout_finish_keylane(const uint32_t (&x)[4],
                                                       int lane,
                                                       uint32_t (&out)[4]) {
  // Word u of x belongs to query row0 + 8 q + 4 h + u and holds the four
  // keys of the quad in its bytes; regroup so that word c holds key c's
  // bytes of the four queries (byte u = query u): a 4 x 4 byte transpose,
  // two byte permutations per word ...
  const uint32_t lo01 = __builtin_amdgcn_perm(x[1], x[0], 0x05010400u);
  const uint32_t hi01 = __builtin_amdgcn_perm(x[1], x[0], 0x07030602u);
  const uint32_t lo23 = __builtin_amdgcn_perm(x[3], x[2], 0x05010400u);
  const uint32_t hi23 = __builtin_amdgcn_perm(x[3], x[2], 0x07030602u);
  out[0] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
  out[1] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
  out[2] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
  out[3] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
  // ... and hand word c to the lane of key c
  quad_transpose(out, lane);
}
__device__ __forceinline__ void dropout_bytes_keylane(const Dropout& dr, int key,
                                                      int row0, int lane,
                                                      uint32_t (&out)[4]) {
  uint32_t x[4];
  dropout_ctr_keylane(dr, key, row0, lane, x);
  philox4x32_10(x, dr.k0, dr.k1);
  dropout_finish_keylane(x, lane, out);
}

// Keep test of byte t of a word.
__device__ __forceinline__ bool dropout_keep(uint32_t word, int t, uint32_t thr) {
  return ((word >> (8 * t)) & 0xFFu) >= thr;
}


// One row (or column) of a block mask, read 64 entries at a time: each
// lane loads one byte and a ballot turns the window into a 64-bit set held
// in scalar registers, so finding the next visible block is a bit scan
// rather than one scalar load per probe (scalar loads share their wait
// counter with LDS reads, and each probe would wait for those too).
struct MaskLine {
  const uint8_t* p;   // entry c is p[c * stride]
  int64_t stride;
  int cols, win0;
  uint64_t bits;      // entries win0 .. win0 + 63 that are nonzero

  __device__ __forceinline__ MaskLine(const uint8_t* p_, int64_t stride_,
                                      int cols_, int lane)
      : p(p_), stride(stride_), cols(cols_) {
    load(0, lane);
  }
  __device__ __forceinline__ void load(int w0, int lane) {
    win0 = w0;
    const int c = w0 + lane;
    const bool on = (c < cols) && p[(int64_t)c * stride] != 0;
    bits = __ballot(on);
  }
  // The first nonzero entry at or after c (cols if there is none).
  __device__ __forceinline__ int next(int c, int lane) {
    while (c < cols) {
      if (c >= win0 + 64) load(c & ~63, lane);
      const uint64_t b = bits >> (c - win0);
      if (b) return c + __builtin_ctzll(b);
      c = win0 + 64;
    }
    return cols;
  }
};

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

}  // namespace fa
