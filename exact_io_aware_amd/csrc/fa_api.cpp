// C-ABI entry points (declared in include/fa.h): argument validation and
// dispatch to the HIP kernels.  Every check runs before any HIP call, so a
// rejected call enqueues nothing and touches no device state.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <limits>

#include "../../include/fa.h"
#include "fa_internal.h"

namespace {

constexpr int64_t kMaxN = (int64_t)1 << 30;

bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// Checks shared by every entry point that takes a problem shape.  Sets
// *empty when there is nothing to compute.
fa_status check_shape(int64_t B, int64_t H, int64_t N, int64_t d, fa_dtype dt,
                      bool* empty, int64_t* bh) {
  if (B < 0 || H < 0 || N < 0 || d < 0) return FA_ERR_SHAPE;
  if (dt != FA_F32 && dt != FA_BF16) return FA_ERR_DTYPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  *empty = (B == 0 || H == 0 || N == 0);
  if (*empty) {
    *bh = 0;
    return FA_OK;
  }
  if (N > kMaxN) return FA_ERR_SHAPE;
  if (B > std::numeric_limits<int64_t>::max() / H) return FA_ERR_SHAPE;
  const int64_t bh_ = B * H;
  // Every element offset must fit in int64 and every grid in int32:
  // at most 2^31 - 1 workgroups of >= 64 rows.
  if (bh_ > ((int64_t)1 << 62) / (N * d)) return FA_ERR_SHAPE;
  if (bh_ * ((N + 63) / 64) > (int64_t)0x7fffffff) return FA_ERR_SHAPE;
  // The row passes launch one workgroup per 8-16 rows.
  if (bh_ * N > ((int64_t)1 << 34)) return FA_ERR_SHAPE;
  *bh = bh_;
  return FA_OK;
}

// The key length of a call whose keys may differ from its queries (Nq =
// the N checked above): 1 <= Nk <= 2^30 when there are queries, the same
// offset and grid limits on the key side, and Nq <= Nk under the causal rule
// (the queries are the last Nq of the Nk tokens).
fa_status check_keys(int64_t bh, int64_t Nq, int64_t Nk, int64_t d,
                     int causal) {
  if (Nk < 0) return FA_ERR_SHAPE;
  if (bh == 0) return FA_OK;  // nothing to compute (B, H or Nq is 0)
  if (Nk == 0 || Nk > kMaxN) return FA_ERR_SHAPE;
  if (causal && Nq > Nk) return FA_ERR_SHAPE;
  if (bh > ((int64_t)1 << 62) / (Nk * d)) return FA_ERR_SHAPE;
  if (bh * ((Nk + 63) / 64) > (int64_t)0x7fffffff) return FA_ERR_SHAPE;
  return FA_OK;
}

bool scale_ok(float scale) { return isfinite(scale) && scale > 0.f; }

size_t ws_rows(int64_t bh, int64_t n) {
  // Two float arrays of bh*n rows, the second starting 256-byte aligned.
  return (size_t)(((bh * n) + 63) / 64 * 64);
}

size_t ws_bytes(int64_t bh, int64_t n) { return 2 * ws_rows(bh, n) * 4; }

fa_status from_hip(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

// Dropout threshold t = round(256 p) (drop probability t / 256); valid for a
// finite p >= 0 with t <= 255.
bool dropout_t(float p, int* t) {
  if (!isfinite(p) || p < 0.f || p > 1.f) return false;
  const long r = lrintf(p * 256.f);
  if (r > 255) return false;
  *t = (int)r;
  return true;
}

fa_status fwd_common(const void* q, const void* k, const void* v, void* o,
                     float* lse, int64_t B, int64_t H, int64_t N, int64_t d,
                     fa_dtype dt, float scale, int causal, const uint8_t* mask,
                     int64_t block_m, int64_t block_n, bool sparse_call,
                     void* stream, int drop_t = 0, uint64_t seed = 0,
                     bool count_call = false, int32_t* visits = nullptr,
                     size_t visits_len = 0, int64_t Nk = -1) {
  bool empty = false;
  int64_t bh = 0;
  fa_status st = check_shape(B, H, N, d, dt, &empty, &bh);
  if (st != FA_OK) return st;
  if (Nk < 0) Nk = N;  // keys and queries are the same tokens
  st = check_keys(bh, N, Nk, d, causal);
  if (st != FA_OK) return st;
  if (!scale_ok(scale)) return FA_ERR_ARG;
  if (sparse_call) {
    if (block_m <= 0 || block_n <= 0 || block_m % 128 != 0 ||
        block_n % 128 != 0 || block_m > kMaxN || block_n > kMaxN) {
      return FA_ERR_MASK;
    }
  }
  if (count_call && dt != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (empty) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) ||
      !aligned(o, 16) || !aligned(lse, 4)) {
    return FA_ERR_ALIGN;
  }
  if (count_call) {
    if (!visits) return FA_ERR_NULL;
    if (!aligned(visits, 4)) return FA_ERR_ALIGN;
    int rows = 0, cols = 0;
    fa::fwd_bf16_tile_grid((int)d, mask != nullptr, &rows, &cols);
    if (visits_len < (size_t)(bh * ((N + rows - 1) / rows))) return FA_ERR_ARG;
  }
  fa::FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.bh = bh;
  a.n = (int)N;
  a.nk = (int)Nk;
  a.q_off = (int)(Nk - N);
  a.d = (int)d;
  a.scale = scale;
  a.causal = causal ? 1 : 0;
  a.mask = sparse_call ? mask : nullptr;
  a.block_m = (int)(sparse_call ? block_m : 128);
  a.block_n = (int)(sparse_call ? block_n : 128);
  a.mask_cols = (int)((Nk + a.block_n - 1) / a.block_n);
  a.drop_t = drop_t;
  a.seed_lo = (uint32_t)seed;
  a.seed_hi = (uint32_t)(seed >> 32);
  a.visits = count_call ? visits : nullptr;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return from_hip(dt == FA_BF16 ? fa::launch_fwd_bf16(a, s)
                                : fa::launch_fwd_f32(a, s));
}

// Validation shared by fa_bwd and its passes.  `need` lists which pointers
// the caller must supply.
enum : unsigned {
  NEED_Q = 1u, NEED_K = 2u, NEED_V = 4u, NEED_O = 8u, NEED_DO = 16u,
  NEED_LSE = 32u, NEED_DQ = 64u, NEED_DK = 128u, NEED_DV = 256u,
};

fa_status bwd_common(unsigned need, const void* q, const void* k,
                     const void* v, const void* o, const void* dout,
                     const float* lse, float* dq, float* dk, float* dv,
                     const void* workspace, size_t workspace_bytes, int64_t B,
                     int64_t H, int64_t N, int64_t d, fa_dtype dt, float scale,
                     bool check_scale, int causal, fa::BwdArgs* out,
                     bool* empty, const uint8_t* mask = nullptr,
                     int64_t block_m = 128, int64_t block_n = 128,
                     bool sparse_call = false, int64_t Nk = -1) {
  int64_t bh = 0;
  fa_status st = check_shape(B, H, N, d, dt, empty, &bh);
  if (st != FA_OK) return st;
  if (Nk < 0) Nk = N;  // keys and queries are the same tokens
  st = check_keys(bh, N, Nk, d, causal);
  if (st != FA_OK) return st;
  if (check_scale && !scale_ok(scale)) return FA_ERR_ARG;
  if (sparse_call) {
    if (block_m <= 0 || block_n <= 0 || block_m % 128 != 0 ||
        block_n % 128 != 0 || block_m > kMaxN || block_n > kMaxN) {
      return FA_ERR_MASK;
    }
  }
  if (*empty) return FA_OK;
  const void* ptrs[] = {q, k, v, o, dout, lse, dq, dk, dv};
  for (int i = 0; i < 9; ++i) {
    if ((need >> i) & 1u) {
      if (!ptrs[i]) return FA_ERR_NULL;
      if (!aligned(ptrs[i], i == 5 ? 4 : 16)) return FA_ERR_ALIGN;  // lse: 4
    }
  }
  if (!workspace) return FA_ERR_NULL;
  if (!aligned(workspace, 16)) return FA_ERR_ALIGN;
  if (workspace_bytes < ws_bytes(bh, N)) return FA_ERR_ARG;
  fa::BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  float* ws = const_cast<float*>(static_cast<const float*>(workspace));
  a.ws_d = ws;
  a.ws_lse2 = ws + ws_rows(bh, N);
  a.bh = bh;
  a.n = (int)N;
  a.nk = (int)Nk;
  a.q_off = (int)(Nk - N);
  a.d = (int)d;
  a.scale = scale;
  a.causal = causal ? 1 : 0;
  a.mask = sparse_call ? mask : nullptr;
  a.block_m = (int)(sparse_call ? block_m : 128);
  a.block_n = (int)(sparse_call ? block_n : 128);
  a.mask_cols = (int)((Nk + a.block_n - 1) / a.block_n);
  *out = a;
  return FA_OK;
}

// Chunk plan of the split-KV forward.  requested > 0 caps the chunk count;
// 0 picks enough chunks for about 2048 workgroups (eight per CU) with at
// least 8 key tiles (256 keys) per chunk.  The tiles are then spread evenly
// and the count lowered until no chunk is empty.
struct SplitPlan {
  int64_t bh = 0;
  int splits = 0;
  int tiles_per_split = 0;
  bool empty = true;
};

fa_status splitkv_plan(int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                       int64_t d, int64_t requested, SplitPlan* p) {
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0 || d < 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (requested < 0) return FA_ERR_ARG;
  p->empty = (B == 0 || H == 0 || Nq == 0);
  if (p->empty) return FA_OK;
  if (Nq > Nk || Nk > kMaxN) return FA_ERR_SHAPE;
  if (B > std::numeric_limits<int64_t>::max() / H) return FA_ERR_SHAPE;
  const int64_t bh = B * H;
  if (bh > ((int64_t)1 << 62) / (Nk * d)) return FA_ERR_SHAPE;
  const int64_t tile = fa::kSplitKvTile;
  const int64_t n_kt = (Nk + tile - 1) / tile;
  const int64_t base = bh * ((Nq + 31) / 32);
  int64_t sp;
  if (requested > 0) {
    sp = std::min(requested, n_kt);
  } else if (Nq == 1) {
    // One query row: one wave per chunk (the vector pass), about
    // kSplitKvWaves waves in all, at least 8 tiles per chunk.
    sp = std::max<int64_t>(1, fa::kSplitKvWaves / bh);
    sp = std::min(sp, std::max<int64_t>(1, n_kt / 8));
  } else {
    sp = std::max<int64_t>(1, (2048 + base - 1) / base);
    sp = std::min(sp, std::max<int64_t>(1, n_kt / 8));
  }
  const int64_t tps = (n_kt + sp - 1) / sp;
  sp = (n_kt + tps - 1) / tps;
  if (base > (int64_t)0x7fffffff / sp) return FA_ERR_SHAPE;
  // The merge launches one workgroup per 8 (d = 128) or 16 rows.
  if (bh * Nq > ((int64_t)1 << 34)) return FA_ERR_SHAPE;
  // The chunk outputs must be addressable in int64 as well.
  if (sp * bh > ((int64_t)1 << 62) / (Nq * (d + 1))) return FA_ERR_SHAPE;
  p->bh = bh;
  p->splits = (int)sp;
  p->tiles_per_split = (int)tps;
  return FA_OK;
}

// Workspace of the split-KV forward: the chunk outputs (float, d per row)
// then the chunk logsumexps.
size_t splitkv_ws_bytes(const SplitPlan& p, int64_t Nq, int64_t d) {
  const size_t rows = (size_t)p.splits * (size_t)p.bh * (size_t)Nq;
  return rows * (size_t)d * 4 + (rows * 4 + 15) / 16 * 16;
}

// The three backward passes for the input dtype.
hipError_t run_pre(const fa::BwdArgs& a, fa_dtype dt, hipStream_t s) {
  return dt == FA_F32 ? fa::launch_bwd_preprocess_f32(a, s)
                      : fa::launch_bwd_preprocess(a, s);
}
hipError_t run_dkdv(const fa::BwdArgs& a, fa_dtype dt, hipStream_t s) {
  return dt == FA_F32 ? fa::launch_bwd_dkdv_f32(a, s) : fa::launch_bwd_dkdv(a, s);
}
hipError_t run_dq(const fa::BwdArgs& a, fa_dtype dt, hipStream_t s) {
  return dt == FA_F32 ? fa::launch_bwd_dq_f32(a, s) : fa::launch_bwd_dq(a, s);
}
// The whole backward.  bf16: the dQ pass computes the row statistics itself
// and leaves them in the workspace for the dK/dV pass (one streaming read of
// O and one launch fewer than the preprocess); float32: the three passes.
// Both orders give the same bits as the three separate calls.
hipError_t run_bwd(const fa::BwdArgs& a, fa_dtype dt, hipStream_t s) {
  hipError_t e;
  if (dt == FA_F32) {
    e = run_pre(a, dt, s);
    if (e != hipSuccess) return e;
    e = run_dkdv(a, dt, s);
    if (e != hipSuccess) return e;
    return run_dq(a, dt, s);
  }
  e = fa::launch_bwd_dq_stats(a, s);
  if (e != hipSuccess) return e;
  return run_dkdv(a, dt, s);
}

}  // namespace

extern "C" {

int64_t fa_fwd_splitkv_chunks(int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                              int64_t d, int64_t n_splits) {
  SplitPlan p;
  if (splitkv_plan(B, H, Nq, Nk, d, n_splits, &p) != FA_OK || p.empty) return 0;
  return p.splits;
}

size_t fa_fwd_splitkv_workspace_bytes(int64_t B, int64_t H, int64_t Nq,
                                      int64_t Nk, int64_t d, int64_t n_splits) {
  SplitPlan p;
  if (splitkv_plan(B, H, Nq, Nk, d, n_splits, &p) != FA_OK || p.empty) return 0;
  return splitkv_ws_bytes(p, Nq, d);
}

fa_status fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o,
                         float* lse, void* workspace, size_t workspace_bytes,
                         int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                         int64_t d, fa_dtype dt, float scale, int causal,
                         int64_t n_splits, void* stream) {
  if (dt != FA_F32 && dt != FA_BF16) return FA_ERR_DTYPE;
  SplitPlan p;
  fa_status st = splitkv_plan(B, H, Nq, Nk, d, n_splits, &p);
  if (st != FA_OK) return st;
  if (!scale_ok(scale)) return FA_ERR_ARG;
  if (dt != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (p.empty) return FA_OK;
  if (!q || !k || !v || !o || !lse || !workspace) return FA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) ||
      !aligned(o, 16) || !aligned(lse, 4) || !aligned(workspace, 16)) {
    return FA_ERR_ALIGN;
  }
  if (workspace_bytes < splitkv_ws_bytes(p, Nq, d)) return FA_ERR_ARG;
  fa::SplitKvArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.ws_o = static_cast<float*>(workspace);
  a.ws_lse = a.ws_o + (size_t)p.splits * (size_t)p.bh * (size_t)Nq * (size_t)d;
  a.bh = p.bh;
  a.nq = (int)Nq;
  a.nk = (int)Nk;
  a.d = (int)d;
  a.scale = scale;
  a.causal = causal ? 1 : 0;
  a.n_splits = p.splits;
  a.tiles_per_split = p.tiles_per_split;
  return from_hip(fa::launch_splitkv_bf16(a, reinterpret_cast<hipStream_t>(stream)));
}

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o,
                 float* lse, int64_t B, int64_t H, int64_t N, int64_t d,
                 fa_dtype dt, float scale, int causal, void* stream) {
  return fwd_common(q, k, v, o, lse, B, H, N, d, dt, scale, causal, nullptr,
                    128, 128, false, stream);
}

fa_status fa_fwd_blocksparse(const void* q, const void* k, const void* v,
                             void* o, float* lse, int64_t B, int64_t H,
                             int64_t N, int64_t d, fa_dtype dt, float scale,
                             int causal, const uint8_t* mask, int64_t block_m,
                             int64_t block_n, void* stream) {
  return fwd_common(q, k, v, o, lse, B, H, N, d, dt, scale, causal, mask,
                    block_m, block_n, true, stream);
}

fa_status fa_fwd_dropout(const void* q, const void* k, const void* v, void* o,
                         float* lse, int64_t B, int64_t H, int64_t N,
                         int64_t d, fa_dtype dt, float scale, int causal,
                         float p_drop, uint64_t seed, void* stream) {
  bool empty = false;
  int64_t bh = 0;
  fa_status st = check_shape(B, H, N, d, dt, &empty, &bh);
  if (st != FA_OK) return st;
  int t = 0;
  if (!scale_ok(scale) || !dropout_t(p_drop, &t)) return FA_ERR_ARG;
  if (dt != FA_BF16) return FA_ERR_UNSUPPORTED;
  return fwd_common(q, k, v, o, lse, B, H, N, d, dt, scale, causal, nullptr,
                    128, 128, false, stream, t, seed);
}

size_t fa_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d) {
  bool empty = false;
  int64_t bh = 0;
  if (check_shape(B, H, N, d, FA_BF16, &empty, &bh) != FA_OK || empty) return 0;
  return ws_bytes(bh, N);
}

fa_status fa_bwd_preprocess(const void* o, const void* dout, const float* lse,
                            void* workspace, size_t workspace_bytes,
                            int64_t B, int64_t H, int64_t N, int64_t d,
                            fa_dtype dt, void* stream) {
  fa::BwdArgs a{};
  bool empty = false;
  fa_status st = bwd_common(NEED_O | NEED_DO | NEED_LSE, nullptr, nullptr,
                            nullptr, o, dout, lse, nullptr, nullptr, nullptr,
                            workspace, workspace_bytes, B, H, N, d, dt, 1.f,
                            false, 0, &a, &empty);
  if (st != FA_OK || empty) return st;
  return from_hip(run_pre(a, dt, reinterpret_cast<hipStream_t>(stream)));
}

fa_status fa_bwd_dkdv(const void* q, const void* k, const void* v,
                      const void* dout, float* dk, float* dv,
                      const void* workspace, size_t workspace_bytes,
                      int64_t B, int64_t H, int64_t N, int64_t d, fa_dtype dt,
                      float scale, int causal, void* stream) {
  fa::BwdArgs a{};
  bool empty = false;
  fa_status st = bwd_common(NEED_Q | NEED_K | NEED_V | NEED_DO | NEED_DK | NEED_DV,
                            q, k, v, nullptr, dout, nullptr, nullptr, dk, dv,
                            workspace, workspace_bytes, B, H, N, d, dt, scale,
                            true, causal, &a, &empty);
  if (st != FA_OK || empty) return st;
  return from_hip(run_dkdv(a, dt, reinterpret_cast<hipStream_t>(stream)));
}

fa_status fa_bwd_dq(const void* q, const void* k, const void* v,
                    const void* dout, float* dq, const void* workspace,
                    size_t workspace_bytes, int64_t B, int64_t H, int64_t N,
                    int64_t d, fa_dtype dt, float scale, int causal,
                    void* stream) {
  fa::BwdArgs a{};
  bool empty = false;
  fa_status st = bwd_common(NEED_Q | NEED_K | NEED_V | NEED_DO | NEED_DQ, q, k,
                            v, nullptr, dout, nullptr, dq, nullptr, nullptr,
                            workspace, workspace_bytes, B, H, N, d, dt, scale,
                            true, causal, &a, &empty);
  if (st != FA_OK || empty) return st;
  return from_hip(run_dq(a, dt, reinterpret_cast<hipStream_t>(stream)));
}

fa_status fa_bwd_dq_stats(const void* q, const void* k, const void* v,
                          const void* o, const void* dout, const float* lse,
                          float* dq, void* workspace, size_t workspace_bytes,
                          int64_t B, int64_t H, int64_t N, int64_t d,
                          fa_dtype dt, float scale, int causal, void* stream) {
  fa::BwdArgs a{};
  bool empty = false;
  fa_status st = bwd_common(NEED_Q | NEED_K | NEED_V | NEED_O | NEED_DO |
                                NEED_LSE | NEED_DQ,
                            q, k, v, o, dout, lse, dq, nullptr, nullptr,
                            workspace, workspace_bytes, B, H, N, d, dt, scale,
                            true, causal, &a, &empty);
  if (st != FA_OK || empty) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dt == FA_F32) {
    st = from_hip(run_pre(a, dt, s));
    if (st != FA_OK) return st;
    return from_hip(run_dq(a, dt, s));
  }
  return from_hip(fa::launch_bwd_dq_stats(a, s));
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o,
                 const void* dout, const float* lse, float* dq, float* dk,
                 float* dv, void* workspace, size_t workspace_bytes,
                 int64_t B, int64_t H, int64_t N, int64_t d, fa_dtype dt,
                 float scale, int causal, void* stream) {
  fa::BwdArgs a{};
  bool empty = false;
  fa_status st = bwd_common(0x1ffu, q, k, v, o, dout, lse, dq, dk, dv,
                            workspace, workspace_bytes, B, H, N, d, dt, scale,
                            true, causal, &a, &empty);
  if (st != FA_OK || empty) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return from_hip(run_bwd(a, dt, s));
}

fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v,
                         const void* o, const void* dout, const float* lse,
                         float* dq, float* dk, float* dv, int64_t B,
                         int64_t H, int64_t N, int64_t d, fa_dtype dt,
                         float scale, int causal, void* stream) {
  {
    bool empty = false;
    int64_t bh = 0;
    fa_status st = check_shape(B, H, N, d, dt, &empty, &bh);
    if (st != FA_OK) return st;
    if (!empty && ws_bytes(bh, N) > fa::noalloc_scratch_bytes()) {
      return FA_ERR_SCRATCH;
    }
  }
  // Validate every argument as fa_bwd does, with an aligned stand-in for the
  // workspace pointer (never dereferenced); the real address comes after.
  void* const stand_in = reinterpret_cast<void*>((uintptr_t)256);
  fa::BwdArgs a{};
  bool empty = false;
  fa_status st = bwd_common(0x1ffu, q, k, v, o, dout, lse, dq, dk, dv,
                            stand_in, fa::noalloc_scratch_bytes(), B, H, N,
                            d, dt, scale, true, causal, &a, &empty);
  if (st != FA_OK || empty) return st;
  void* ws = nullptr;
  if (fa::noalloc_scratch(&ws) != hipSuccess) return FA_ERR_HIP;
  a.ws_d = static_cast<float*>(ws);
  a.ws_lse2 = a.ws_d + ws_rows(a.bh, N);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return from_hip(run_bwd(a, dt, s));
}

fa_status fa_bwd_dropout(const void* q, const void* k, const void* v,
                         const void* o, const void* dout, const float* lse,
                         float* dq, float* dk, float* dv, void* workspace,
                         size_t workspace_bytes, int64_t B, int64_t H,
                         int64_t N, int64_t d, fa_dtype dt, float scale,
                         int causal, float p_drop, uint64_t seed,
                         void* stream) {
  fa::BwdArgs a{};
  bool empty = false;
  fa_status st = bwd_common(0x1ffu, q, k, v, o, dout, lse, dq, dk, dv,
                            workspace, workspace_bytes, B, H, N, d, dt, scale,
                            true, causal, &a, &empty);
  if (st != FA_OK) return st;
  int t = 0;
  if (!dropout_t(p_drop, &t)) return FA_ERR_ARG;
  if (dt != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (empty) return FA_OK;
  a.drop_t = t;
  a.seed_lo = (uint32_t)seed;
  a.seed_hi = (uint32_t)(seed >> 32);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return from_hip(run_bwd(a, dt, s));
}

fa_status fa_bwd_blocksparse(const void* q, const void* k, const void* v,
                             const void* o, const void* dout, const float* lse,
                             float* dq, float* dk, float* dv, void* workspace,
                             size_t workspace_bytes, int64_t B, int64_t H,
                             int64_t N, int64_t d, fa_dtype dt, float scale,
                             int causal, const uint8_t* mask, int64_t block_m,
                             int64_t block_n, void* stream) {
  fa::BwdArgs a{};
  bool empty = false;
  fa_status st = bwd_common(0x1ffu, q, k, v, o, dout, lse, dq, dk, dv,
                            workspace, workspace_bytes, B, H, N, d, dt, scale,
                            true, causal, &a, &empty, mask, block_m, block_n,
                            true);
  if (st != FA_OK || empty) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return from_hip(run_bwd(a, dt, s));
}

fa_status fa_fwd_general(const void* q, const void* k, const void* v, void* o,
                         float* lse, int64_t B, int64_t H, int64_t Nq,
                         int64_t Nk, int64_t d, fa_dtype dt, float scale,
                         int causal, const uint8_t* mask, int64_t block_m,
                         int64_t block_n, float p_drop, uint64_t seed,
                         void* stream) {
  if (Nk < 0) return FA_ERR_SHAPE;  // (fwd_common reads Nk < 0 as Nk = Nq)
  bool empty = false;
  int64_t bh = 0;
  fa_status st = check_shape(B, H, Nq, d, dt, &empty, &bh);
  if (st != FA_OK) return st;
  st = check_keys(bh, Nq, Nk, d, causal);
  if (st != FA_OK) return st;
  int t = 0;
  if (!scale_ok(scale) || !dropout_t(p_drop, &t)) return FA_ERR_ARG;
  if (t > 0 && dt != FA_BF16) return FA_ERR_UNSUPPORTED;
  return fwd_common(q, k, v, o, lse, B, H, Nq, d, dt, scale, causal, mask,
                    block_m, block_n, mask != nullptr, stream, t, seed, false,
                    nullptr, 0, Nk);
}

fa_status fa_bwd_general(const void* q, const void* k, const void* v,
                         const void* o, const void* dout, const float* lse,
                         float* dq, float* dk, float* dv, void* workspace,
                         size_t workspace_bytes, int64_t B, int64_t H,
                         int64_t Nq, int64_t Nk, int64_t d, fa_dtype dt,
                         float scale, int causal, const uint8_t* mask,
                         int64_t block_m, int64_t block_n, float p_drop,
                         uint64_t seed, void* stream) {
  if (Nk < 0) return FA_ERR_SHAPE;  // (bwd_common reads Nk < 0 as Nk = Nq)
  fa::BwdArgs a{};
  bool empty = false;
  fa_status st = bwd_common(0x1ffu, q, k, v, o, dout, lse, dq, dk, dv,
                            workspace, workspace_bytes, B, H, Nq, d, dt, scale,
                            true, causal, &a, &empty, mask, block_m, block_n,
                            mask != nullptr, Nk);
  if (st != FA_OK) return st;
  int t = 0;
  if (!dropout_t(p_drop, &t)) return FA_ERR_ARG;
  if (t > 0 && dt != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (empty) return FA_OK;
  a.drop_t = t;
  a.seed_lo = (uint32_t)seed;
  a.seed_hi = (uint32_t)(seed >> 32);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return from_hip(run_bwd(a, dt, s));
}

fa_status fa_tile_grid(int pass, int64_t d, int sparse, int64_t* rows,
                       int64_t* cols) {
  if (!rows || !cols) return FA_ERR_NULL;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  int r = 0, c = 0;
  switch (pass) {
    case 0: fa::fwd_bf16_tile_grid((int)d, sparse != 0, &r, &c); break;
    case 1: fa::bwd_dkdv_tile_grid((int)d, sparse != 0, &r, &c); break;
    case 2: fa::bwd_dq_tile_grid((int)d, sparse != 0, &r, &c); break;
    default: return FA_ERR_ARG;
  }
  *rows = r;
  *cols = c;
  return FA_OK;
}

fa_status fa_fwd_tile_visits(const void* q, const void* k, const void* v,
                             void* o, float* lse, int64_t B, int64_t H,
                             int64_t N, int64_t d, fa_dtype dt, float scale,
                             int causal, const uint8_t* mask, int64_t block_m,
                             int64_t block_n, int32_t* visits,
                             size_t visits_len, void* stream) {
  return fwd_common(q, k, v, o, lse, B, H, N, d, dt, scale, causal, mask,
                    block_m, block_n, true, stream, 0, 0, true, visits,
                    visits_len);
}

fa_status fa_bwd_tile_visits(const void* q, const void* k, const void* v,
                             const void* o, const void* dout, const float* lse,
                             float* dq, float* dk, float* dv, void* workspace,
                             size_t workspace_bytes, int64_t B, int64_t H,
                             int64_t N, int64_t d, fa_dtype dt, float scale,
                             int causal, const uint8_t* mask, int64_t block_m,
                             int64_t block_n, int32_t* visits_kv,
                             size_t kv_len, int32_t* visits_q, size_t q_len,
                             void* stream) {
  fa::BwdArgs a{};
  bool empty = false;
  fa_status st = bwd_common(0x1ffu, q, k, v, o, dout, lse, dq, dk, dv,
                            workspace, workspace_bytes, B, H, N, d, dt, scale,
                            true, causal, &a, &empty, mask, block_m, block_n,
                            true);
  if (st != FA_OK) return st;
  if (dt != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (empty) return FA_OK;
  if (!visits_kv || !visits_q) return FA_ERR_NULL;
  if (!aligned(visits_kv, 4) || !aligned(visits_q, 4)) return FA_ERR_ALIGN;
  int rows = 0, cols = 0;
  fa::bwd_dkdv_tile_grid((int)d, mask != nullptr, &rows, &cols);
  if (kv_len < (size_t)(a.bh * ((N + cols - 1) / cols))) return FA_ERR_ARG;
  fa::bwd_dq_tile_grid((int)d, mask != nullptr, &rows, &cols);
  if (q_len < (size_t)(a.bh * ((N + rows - 1) / rows))) return FA_ERR_ARG;
  a.visits_kv = visits_kv;
  a.visits_q = visits_q;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return from_hip(run_bwd(a, dt, s));
}

const char* fa_status_str(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: negative or overflowing size";
    case FA_ERR_DTYPE: return "FA_ERR_DTYPE: unknown dtype";
    case FA_ERR_UNSUPPORTED:
      return "FA_ERR_UNSUPPORTED: head dim must be 64 or 128, or dtype not provided by this call";
    case FA_ERR_MASK:
      return "FA_ERR_MASK: block sizes must be positive multiples of 128";
    case FA_ERR_HIP: return "FA_ERR_HIP: a HIP kernel launch failed";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: tensor pointer not 16-byte aligned";
    case FA_ERR_ARG:
      return "FA_ERR_ARG: scale must be finite and > 0, workspace large enough, "
             "drop probability in [0, 255/256]";
    case FA_ERR_SCRATCH:
      return "FA_ERR_SCRATCH: problem exceeds the library's fixed scratch "
             "(fa_bwd_noalloc needs B*H*N <= 2^20 rows)";
  }
  return "unknown fa_status";
}

const char* fa_version(void) { return "exact_io_aware_amd 0.1.0 gfx950"; }

}  // extern "C"
