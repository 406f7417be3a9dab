// Internal declarations shared by the C-ABI layer and the HIP kernel files.
// Not installed; the public interface is include/fa.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// Forward problem, already validated by the C-ABI layer.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t bh;              // B * H
  int n;                   // query rows
  int nk;                  // keys
  int q_off;               // position of query row 0 among the keys (causal
                           // rule: key j visible to row i iff j <= q_off + i)
  int d;                   // head dim (64 or 128)
  float scale;             // > 0
  int causal;
  const uint8_t* mask;     // nullptr = dense
  int mask_cols;           // ceil(nk / block_n)
  int block_m;             // multiple of 128
  int block_n;             // multiple of 128
  int drop_t = 0;          // dropout threshold t (0 = no dropout; bf16 only)
  uint32_t seed_lo = 0;    // dropout seed words
  uint32_t seed_hi = 0;
  int* visits = nullptr;   // diagnostic: key tiles visited per query tile
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  float* dq;
  float* dk;
  float* dv;
  float* ws_d;             // B*H*n: rowsum(dO * O)
  float* ws_lse2;          // B*H*n: lse * log2(e), +inf for empty rows
  int64_t bh;
  int n;                   // query rows
  int nk;                  // keys
  int q_off;               // as FwdArgs::q_off
  int d;
  float scale;
  int causal;
  const uint8_t* mask;     // nullptr = dense
  int mask_cols;           // ceil(nk / block_n)
  int block_m;             // multiple of 128
  int block_n;             // multiple of 128
  int drop_t = 0;          // dropout threshold t (0 = no dropout; bf16 only)
  uint32_t seed_lo = 0;    // dropout seed words
  uint32_t seed_hi = 0;
  int* visits_kv = nullptr;  // diagnostic: query tiles visited per key tile
  int* visits_q = nullptr;   // diagnostic: key tiles visited per query tile
};

// Split-KV forward: nq queries (the last nq of the nk positions) against nk
// keys, the keys cut into n_splits chunks of tiles_per_split tiles of
// kSplitKvTile keys, every chunk non-empty.
constexpr int kSplitKvTile = 32;
// Waves of the one-query split-KV pass: two per SIMD of a 256-CU MI355X,
// all resident at once.  Measured on B=16 H=32 Nk=16384 d=128: 1536-2048
// waves read K and V fastest (6.8 TB/s); 1024 are too few (5.2 TB/s), and
// 3072-8192 run 2-4% slower than 2048.
constexpr int kSplitKvWaves = 2048;
struct SplitKvArgs {
  const void* q;           // bh x nq x d
  const void* k;           // bh x nk x d
  const void* v;           // bh x nk x d
  void* o;                 // bh x nq x d
  float* lse;              // bh x nq
  float* ws_o;             // n_splits x bh x nq x d: chunk outputs
  float* ws_lse;           // n_splits x bh x nq: chunk logsumexps
  int64_t bh;
  int nq;
  int nk;
  int d;
  float scale;
  int causal;
  int n_splits;
  int tiles_per_split;
};

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s);
hipError_t launch_splitkv_bf16(const SplitKvArgs& a, hipStream_t s);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s);
hipError_t launch_bwd_preprocess(const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_dkdv(const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t s);
// The dQ pass that also computes the row statistics from o, dout and lse and
// stores them in the workspace, in place of the preprocess (the dK/dV pass
// then follows it).
hipError_t launch_bwd_dq_stats(const BwdArgs& a, hipStream_t s);
// float32 inputs (q, k, v, o, dout are float*).
hipError_t launch_bwd_preprocess_f32(const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_dkdv_f32(const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_dq_f32(const BwdArgs& a, hipStream_t s);

// Tile geometry of the bf16 kernels (rows x cols of one work tile and of
// the tiles it visits): forward query tile x key tile, dK/dV query stage x
// key tile, dQ query tile x key tile.
void fwd_bf16_tile_grid(int d, bool sparse, int* rows, int* cols);
void bwd_dkdv_tile_grid(int d, bool sparse, int* rows, int* cols);
void bwd_dq_tile_grid(int d, bool sparse, int* rows, int* cols);

// Library-owned scratch of the entry points that allocate nothing
// (fa_noalloc.hip): its size, and its device address on the current device
// (looked up once per device).
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void** out);

}  // namespace fa
