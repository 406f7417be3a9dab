/*
 * fa.h — C ABI of the exact IO-aware attention library for AMD Instinct
 * MI355X (gfx950).
 *
 * Computes exact scaled-dot-product attention O = softmax(scale * Q K^T) V
 * with tiled online softmax: the N x N score and probability matrices are
 * never written to device memory; the backward recomputes them tile by tile
 * from a saved per-row logsumexp.
 *
 * Pages cited (titles as published):
 *   [TLDR]   "FlashAttention：メモリ効率的なアテンション計算" (tech-tldr.com)
 *   [XYZ]    "FlashAttention: IOを意識した高速かつメモリ効率の高い厳密な
 *            アテンション" (xyznot.com, summary of arXiv 2205.14135)
 *   [REAPER] "3 · FlashAttention" (mkdocs.reaper.mx, chapter 3)
 *   [LLMSYS] "출력을 누적해 메모리 이동을 줄이는 FlashAttention"
 *            (llm-systems-engineering.pages.dev)
 *   [Q67]    "FlashAttention：在线 softmax 与 IO-aware 注意力" (quant67.com)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout.  Q, K, V, O, dO, dQ, dK, dV are dense row-major tensors of shape
 *   B x H x N x d (d fastest, no padding): element (b, h, i, c) sits at
 *   offset ((b*H + h)*N + i)*d + c.  LSE and the backward workspace rows are
 *   B x H x N float32 arrays in the same (b, h, i) order.  Queries and keys
 *   have the same length N, except in fa_fwd_splitkv, fa_fwd_general and
 *   fa_bwd_general (Nq query rows, Nk key rows).
 * Pointers.  Every tensor pointer is a device pointer owned by the caller,
 *   aligned to 16 bytes.  The library allocates no device memory; its only
 *   global state is the per-device address of the scratch array of
 *   fa_bwd_noalloc.  Concurrent calls on different streams are safe as long
 *   as their output buffers do not overlap (fa_bwd_noalloc: see there).
 * Stream.  `stream` is a hipStream_t passed as void* (NULL = the null
 *   stream).  Work is enqueued and the call returns without synchronising;
 *   outputs are valid once the stream has reached that point.
 * Sizes.  B, H, N >= 0; when any of them is 0 the call does nothing and
 *   returns FA_OK (pointers are not inspected).  d must be 64 or 128.
 * dtype.  FA_BF16: Q, K, V, O, dO are bfloat16 (round-to-nearest-even
 *   storage), arithmetic is bf16 x bf16 products accumulated in float32.
 *   FA_F32: Q, K, V, O, dO are float32 throughout (fa_fwd_splitkv is bf16
 *   only).
 *   LSE, dQ, dK, dV and the workspace are always float32.
 * scale.  Finite and > 0 (the usual value is 1/sqrt(d), [Q67] section 1).
 * Causal.  causal != 0 makes key j visible to query i iff j <= i.
 * Errors.  Arguments are checked first, before any HIP call; a failed check
 *   returns its FA_ERR_* code with nothing enqueued.  A failed kernel launch
 *   returns FA_ERR_HIP.  Nothing is printed and nothing aborts.
 */
#ifndef EXACT_IO_AWARE_FA_H
#define EXACT_IO_AWARE_FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,        /* a required pointer is NULL                     */
  FA_ERR_SHAPE = 2,       /* negative size, or sizes whose product overflows */
  FA_ERR_DTYPE = 3,       /* dtype not FA_F32 / FA_BF16                     */
  FA_ERR_UNSUPPORTED = 4, /* valid request this build does not provide      */
  FA_ERR_MASK = 5,        /* block-mask geometry invalid                    */
  FA_ERR_HIP = 6,         /* a HIP launch failed                            */
  FA_ERR_ALIGN = 7,       /* a tensor pointer is not 16-byte aligned        */
  FA_ERR_ARG = 8,         /* scale not finite and > 0, workspace too small,
                             drop probability out of range                 */
  FA_ERR_SCRATCH = 9,     /* problem larger than the library's fixed scratch
                             (fa_bwd_noalloc)                              */
} fa_status;

typedef enum { FA_F32 = 0, FA_BF16 = 1 } fa_dtype;

/*
 * fa_fwd — forward pass.
 *
 * For each (b, h) and query row i:
 *   S_ij = scale * q_i . k_j (masked entries -inf),
 *   O_i  = sum_j softmax(S_i)_j v_j,
 *   lse_i = ln sum_j exp(S_ij)   (natural log, scaled-score units).
 * Defined by the three steps of standard attention ([Q67] section 1;
 * [REAPER] section 3.1) and computed by the tiled online-softmax recurrence
 * with an unnormalised accumulator divided once at the end ([TLDR] online
 * softmax and tiling sections; [REAPER] sections 3.2-3.3; [LLMSYS] Fig. 2-3).
 * A row that sees no key gets O_i = 0 and lse_i = -inf.
 *
 * q, k, v : inputs, B x H x N x d, dtype `dt`.
 * o       : output, B x H x N x d, dtype `dt`.
 * lse     : output, B x H x N float32.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o,
                 float* lse, int64_t B, int64_t H, int64_t N, int64_t d,
                 fa_dtype dt, float scale, int causal, void* stream);

/*
 * fa_fwd_blocksparse — forward pass restricted to the nonzero blocks of a
 * block mask ([XYZ] section "Block-Sparse FlashAttention").
 *
 * mask : device uint8 array, row-major, shape
 *        ceil(N / block_m) x ceil(N / block_n), shared by every (b, h).
 *        Key j is visible to query i iff mask[i / block_m][j / block_n] != 0
 *        (AND the causal rule when causal != 0).  Tiles whose mask block is 0
 *        are skipped entirely.  mask == NULL means every block is on (the
 *        call is then identical to fa_fwd).
 * block_m, block_n : positive multiples of 128.
 * Other arguments and outputs as fa_fwd.  FA_ERR_MASK for invalid block
 * sizes.
 */
fa_status fa_fwd_blocksparse(const void* q, const void* k, const void* v,
                             void* o, float* lse, int64_t B, int64_t H,
                             int64_t N, int64_t d, fa_dtype dt, float scale,
                             int causal, const uint8_t* mask, int64_t block_m,
                             int64_t block_n, void* stream);

/*
 * fa_fwd_splitkv — forward pass of a short block of queries against a long
 * key sequence (decoding: one or a few new tokens against the whole
 * context), with the keys cut into chunks processed in parallel ([REAPER]
 * section 3.6) and the chunk results combined by the two-part softmax rule
 * m = max(m1, m2), l = e^(m1 - m) l1 + e^(m2 - m) l2 ([XYZ], incremental
 * softmax tracking).  Result as fa_fwd on the same rows:
 *   O_i = sum_j softmax(S_i)_j v_j,  lse_i = ln sum_j exp(S_ij),
 * S_ij = scale * q_i . k_j, up to rounding order.
 *
 * q          : input, B x H x Nq x d bfloat16.
 * k, v       : inputs, B x H x Nk x d bfloat16, 1 <= Nq <= Nk (when B, H
 *              and Nq are nonzero; Nq > Nk is FA_ERR_SHAPE).
 * o          : output, B x H x Nq x d bfloat16.
 * lse        : output, B x H x Nq float32.
 * causal     : the queries are the last Nq positions of the sequence: query
 *              i sees key j iff j <= Nk - Nq + i.  With Nq = Nk this is the
 *              causal rule of fa_fwd.
 * n_splits   : >= 0.  0 picks the chunk count from the shape; a positive
 *              value caps it.  The count actually used is
 *              fa_fwd_splitkv_chunks(), at most the number of 32-key tiles;
 *              every chunk holds keys (whole 32-key tiles; with Nq = 1
 *              interleaved groups of 16 (d = 128) or 32 (d = 64) keys).
 * workspace  : caller-owned device scratch of at least
 *              fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, n_splits)
 *              bytes, 16-byte aligned; contents on entry ignored.  Holds the
 *              chunk outputs (float32) and chunk logsumexps.
 * Two kernels run in order on `stream`: the chunk pass and the merge.  With
 * Nq = 1 the chunk pass runs on the vector units, one wave per chunk (a
 * matrix product would waste 31 of its 32 rows; the pass is bound by reading
 * K and V), and the automatic chunk count keeps every wave resident at once.
 * FA_BF16 only (FA_F32 returns FA_ERR_UNSUPPORTED); FA_ERR_ARG for negative
 * n_splits, a bad scale or a short workspace.
 */
fa_status fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o,
                         float* lse, void* workspace, size_t workspace_bytes,
                         int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                         int64_t d, fa_dtype dt, float scale, int causal,
                         int64_t n_splits, void* stream);

/* Key chunks fa_fwd_splitkv uses for this shape and n_splits, and the bytes
 * of workspace it needs (both 0 for empty or invalid shapes). */
int64_t fa_fwd_splitkv_chunks(int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                              int64_t d, int64_t n_splits);
size_t fa_fwd_splitkv_workspace_bytes(int64_t B, int64_t H, int64_t Nq,
                                      int64_t Nk, int64_t d, int64_t n_splits);

/*
 * fa_bwd — backward pass by recomputation ([TLDR] backward section; [XYZ]
 * key ideas, recomputation; [REAPER] section 3.4; [Q67] section 5).
 *
 * Gradients of L = sum(O * dO) with respect to Q, K, V (exact gradient of
 * fa_fwd; no gradient flows into lse).  With P the attention probabilities
 * rebuilt from q, k and the saved lse:
 *   D_i = sum_c dO_ic O_ic,  dV = P^T dO,  dP = dO V^T,
 *   dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
 * Kernels run in order on `stream`.  FA_BF16: a query-tile pass producing dQ
 * that also computes D and the base-2 logsumexp per row and leaves them in
 * the workspace, then a key-tile pass producing dK and dV.  FA_F32: a row
 * pass computing D, the key-tile pass, then the query-tile pass.  No
 * atomics; results are bitwise reproducible and equal those of the three
 * separate calls below.
 *
 * q, k, v, o, dout : inputs, B x H x N x d, dtype `dt` (o and lse from
 *                    fa_fwd on the same q, k, v, scale, causal).
 * lse              : input, B x H x N float32.
 * dq, dk, dv       : outputs, B x H x N x d float32 (overwritten).
 * workspace        : caller-owned device scratch of at least
 *                    fa_bwd_workspace_bytes(B, H, N, d) bytes, 16-byte
 *                    aligned; its contents on entry are ignored.
 * FA_BF16: bf16 inputs on the matrix cores (bf16 products, fp32
 * accumulation; P and dS rounded to bf16 before their products).  FA_F32:
 * float32 inputs, every product and sum in fp32 on the vector units (for
 * accuracy, not speed).
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o,
                 const void* dout, const float* lse, float* dq, float* dk,
                 float* dv, void* workspace, size_t workspace_bytes,
                 int64_t B, int64_t H, int64_t N, int64_t d, fa_dtype dt,
                 float scale, int causal, void* stream);

/*
 * fa_bwd_blocksparse — backward pass of fa_fwd_blocksparse: the exact
 * gradient of that forward ([XYZ] section "Block-Sparse FlashAttention": the
 * backward visits the same nonzero blocks as the forward), by recomputation
 * as fa_bwd.  Query/key tiles whose mask block is 0 are skipped in both
 * gradient passes; a query that sees no key gets dQ = 0 and a key no query
 * sees gets dK = dV = 0.
 *
 * mask, block_m, block_n : as fa_fwd_blocksparse (mask == NULL means every
 *                          block is on: identical to fa_bwd).
 * o, lse                 : from fa_fwd_blocksparse with the same mask.
 * Other arguments, workspace and outputs as fa_bwd.  FA_ERR_MASK for invalid
 * block sizes.
 */
fa_status fa_bwd_blocksparse(const void* q, const void* k, const void* v,
                             const void* o, const void* dout, const float* lse,
                             float* dq, float* dk, float* dv, void* workspace,
                             size_t workspace_bytes, int64_t B, int64_t H,
                             int64_t N, int64_t d, fa_dtype dt, float scale,
                             int causal, const uint8_t* mask, int64_t block_m,
                             int64_t block_n, void* stream);

/*
 * fa_fwd_dropout — forward pass with dropout on the attention probabilities
 * ([XYZ] key ideas: dropout is among the steps fused into the one attention
 * kernel, with the matrix products, the mask and the softmax).
 *
 *   P = softmax(S) as in fa_fwd,  O = (Z * P / (1 - p)) V,
 *   lse_i = ln sum_j exp(S_ij)   (of P itself: dropout does not change it),
 * where Z_ij is 0 (dropped) or 1 (kept).  The pages define neither the
 * dropout nor its random numbers; this library fixes them as follows.
 *   p      : p_drop quantised to t / 256 with t = round(256 p_drop); t must
 *            be <= 255 (0 <= p_drop <= 255/256, else FA_ERR_ARG).  t = 0
 *            gives exactly fa_fwd.
 *   Z_ij   : kept iff u >= t, u the random byte of element (bh, i, j),
 *            bh = b*H + h: byte (j & 3) (bits 8(j&3) .. 8(j&3)+7) of word
 *            (i & 3) of Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel
 *            Random Numbers: As Easy as 1, 2, 3", SC 2011) applied to the
 *            counter (i >> 2, j >> 2, bh, 0) with the key (seed & 0xffffffff,
 *            seed >> 32).  The mask depends only on (seed, bh, i, j), not on
 *            the launch configuration; call fa_bwd_dropout with the same
 *            seed and p_drop.
 * Other arguments, outputs and errors as fa_fwd.  FA_BF16 only (FA_F32
 * returns FA_ERR_UNSUPPORTED); for dropout with a block mask or with Nq !=
 * Nk see fa_fwd_general.  (The shape limits shared by every call keep B*H
 * below 2^31, so bh always fits its counter word.)
 */
fa_status fa_fwd_dropout(const void* q, const void* k, const void* v, void* o,
                         float* lse, int64_t B, int64_t H, int64_t N,
                         int64_t d, fa_dtype dt, float scale, int causal,
                         float p_drop, uint64_t seed, void* stream);

/*
 * fa_bwd_dropout — backward pass of fa_fwd_dropout (same q, k, v, scale,
 * causal, p_drop, seed; o and lse from that call): the exact gradient of
 * L = sum(O * dO) with the mask Z fixed,
 *   dV = (Z * P / (1 - p))^T dO,   dP = Z * (dO V^T) / (1 - p),
 *   D_i = sum_c dO_ic O_ic (= sum_j P_ij dP_ij),   dS = P * (dP - D),
 *   dQ = scale dS K,   dK = scale dS^T Q,
 * by recomputation as fa_bwd (the mask is regenerated, never stored).
 * Arguments, workspace, outputs and errors as fa_bwd and fa_fwd_dropout.
 */
fa_status fa_bwd_dropout(const void* q, const void* k, const void* v,
                         const void* o, const void* dout, const float* lse,
                         float* dq, float* dk, float* dv, void* workspace,
                         size_t workspace_bytes, int64_t B, int64_t H,
                         int64_t N, int64_t d, fa_dtype dt, float scale,
                         int causal, float p_drop, uint64_t seed,
                         void* stream);

/*
 * fa_bwd_noalloc — fa_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same three kernels and results (bitwise equal to fa_bwd),
 * with the per-row workspace taken from a scratch array that the library
 * holds in device memory instead of from the caller.  The caller still
 * passes every input and output.  The call allocates nothing and frees
 * nothing (its first call on a device looks up that device's copy of the
 * array, which lives until the process ends).
 *
 * Limit: B*H*N <= 2^20 rows (the scratch holds two float arrays of 2^20
 * rows, 8 MiB); larger problems return FA_ERR_SCRATCH before any HIP call.
 * Nothing in the scratch needs to start at zero: the row pass writes every
 * row the gradient passes read.  All calls on one GPU share that GPU's
 * scratch and it keeps the last call's contents, so calls that overlap in
 * time on one GPU (different streams, or different host threads) race;
 * serialise them.  The stream must belong to the current device.
 * Arguments, outputs and other errors as fa_bwd.
 */
fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v,
                         const void* o, const void* dout, const float* lse,
                         float* dq, float* dk, float* dv, int64_t B,
                         int64_t H, int64_t N, int64_t d, fa_dtype dt,
                         float scale, int causal, void* stream);

/*
 * fa_fwd_general / fa_bwd_general — the forward and backward with every
 * option of the other calls available together:
 *   * Nq queries against Nk keys.  Under the causal rule the queries are
 *     the last Nq of the Nk tokens: query row i sits at position
 *     Nk - Nq + i and sees key j iff j <= Nk - Nq + i (a prompt fed in
 *     chunks against the keys of the chunks before it, or a decoding step;
 *     [REAPER] section 3.6).  With Nq = Nk this is fa_fwd's causal rule.
 *   * an optional block mask (mask != NULL), as fa_fwd_blocksparse but of
 *     shape ceil(Nq / block_m) x ceil(Nk / block_n); key j is visible to
 *     query i iff mask[i / block_m][j / block_n] != 0 AND the causal rule;
 *     block_m and block_n are ignored when mask == NULL.
 *   * optional dropout (p_drop > 0), as fa_fwd_dropout, with the counter
 *     of element (bh, i, j) set to (i >> 2, j >> 2, bh, (Nk - Nq) mod 2^32),
 *     i the row of Q: chunks at different offsets draw disjoint random
 *     numbers, and Nq = Nk gives fa_fwd_dropout's mask.  bf16 only
 *     (FA_F32 with p_drop > 0 returns FA_ERR_UNSUPPORTED).
 * A row that sees no key gets O = 0, lse = -inf and dQ = 0; a key that no
 * query sees gets dK = dV = 0.
 *
 * q, o, dout : B x H x Nq x d, dtype `dt`;  k, v : B x H x Nk x d, dtype dt.
 * lse        : B x H x Nq float32.
 * dq         : B x H x Nq x d float32;  dk, dv : B x H x Nk x d float32.
 * workspace  : at least fa_bwd_workspace_bytes(B, H, Nq, d) bytes (the
 *              per-row workspace is per query row).
 * Sizes: B, H, Nq >= 0 (any of them 0: nothing to do, FA_OK); otherwise
 * 1 <= Nk <= 2^30, and Nq <= Nk when causal != 0 (else FA_ERR_SHAPE).
 * fa_bwd_general takes o and lse from fa_fwd_general with the same
 * arguments.  Other arguments and errors as fa_fwd / fa_bwd (FA_ERR_MASK
 * for invalid block sizes with a mask, FA_ERR_ARG for p_drop outside
 * [0, 255/256]).  With Nq = Nk, mask == NULL and p_drop = 0 the results
 * equal fa_fwd / fa_bwd bitwise.
 */
fa_status fa_fwd_general(const void* q, const void* k, const void* v, void* o,
                         float* lse, int64_t B, int64_t H, int64_t Nq,
                         int64_t Nk, int64_t d, fa_dtype dt, float scale,
                         int causal, const uint8_t* mask, int64_t block_m,
                         int64_t block_n, float p_drop, uint64_t seed,
                         void* stream);
fa_status fa_bwd_general(const void* q, const void* k, const void* v,
                         const void* o, const void* dout, const float* lse,
                         float* dq, float* dk, float* dv, void* workspace,
                         size_t workspace_bytes, int64_t B, int64_t H,
                         int64_t Nq, int64_t Nk, int64_t d, fa_dtype dt,
                         float scale, int causal, const uint8_t* mask,
                         int64_t block_m, int64_t block_n, float p_drop,
                         uint64_t seed, void* stream);

/* Bytes of workspace fa_bwd and fa_bwd_blocksparse need (0 for empty
 * problems); fa_bwd_general needs fa_bwd_workspace_bytes(B, H, Nq, d). */
size_t fa_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d);

/*
 * The passes of fa_bwd as separate calls, for callers that time or schedule
 * them individually.  Calling preprocess, then dkdv and dq (in either order,
 * after preprocess) on the same workspace equals fa_bwd bitwise; so does
 * calling dq_stats, then dkdv.
 *
 * fa_bwd_preprocess : reads o, dout, lse; writes the per-row D and the
 *                     base-2 logsumexp into `workspace`.
 * fa_bwd_dkdv       : reads q, k, v, dout and `workspace`; writes dk, dv.
 * fa_bwd_dq         : reads q, k, v, dout and `workspace`; writes dq.
 * fa_bwd_dq_stats   : preprocess and dq in one: reads q, k, v, o, dout, lse;
 *                     writes dq and the workspace rows preprocess writes
 *                     (FA_BF16: one kernel, D_i formed from the O and dO rows
 *                     the dQ pass holds; FA_F32: the two kernels).
 * Arguments they do not use may be NULL.  Validation as fa_bwd.
 */
fa_status fa_bwd_preprocess(const void* o, const void* dout, const float* lse,
                            void* workspace, size_t workspace_bytes,
                            int64_t B, int64_t H, int64_t N, int64_t d,
                            fa_dtype dt, void* stream);
fa_status fa_bwd_dkdv(const void* q, const void* k, const void* v,
                      const void* dout, float* dk, float* dv,
                      const void* workspace, size_t workspace_bytes,
                      int64_t B, int64_t H, int64_t N, int64_t d, fa_dtype dt,
                      float scale, int causal, void* stream);
fa_status fa_bwd_dq(const void* q, const void* k, const void* v,
                    const void* dout, float* dq, const void* workspace,
                    size_t workspace_bytes, int64_t B, int64_t H, int64_t N,
                    int64_t d, fa_dtype dt, float scale, int causal,
                    void* stream);
fa_status fa_bwd_dq_stats(const void* q, const void* k, const void* v,
                          const void* o, const void* dout, const float* lse,
                          float* dq, void* workspace, size_t workspace_bytes,
                          int64_t B, int64_t H, int64_t N, int64_t d,
                          fa_dtype dt, float scale, int causal, void* stream);

/*
 * Diagnostics: the tile schedule of the bf16 kernels.  The causal rule
 * visits, for a block of queries, only the key blocks at or before its last
 * query ([REAPER], causal-mask question: with T square blocks per side,
 * T(T+1)/2 of the T^2 blocks), and the block-sparse forms only the blocks
 * whose mask entry is nonzero ([XYZ], section "Block-Sparse
 * FlashAttention").  These calls report what the kernels actually visited.
 *
 * fa_tile_grid — rows x cols of one pass's tiles, for head dim d (64 or 128)
 *   and the dense (sparse = 0) or block-sparse (sparse != 0) instances:
 *     pass 0, forward:     query tile rows x key tile keys;
 *     pass 1, dK/dV pass:  query stage rows x key tile keys (a workgroup owns
 *                          one key tile and visits query stages);
 *     pass 2, dQ pass:     query tile rows x key tile keys.
 *   FA_ERR_ARG for another pass, FA_ERR_UNSUPPORTED for another d,
 *   FA_ERR_NULL for a NULL output.
 *
 * fa_fwd_tile_visits — exactly fa_fwd_blocksparse (mask == NULL: fa_fwd),
 *   same kernel and results, and in addition, for head bh = b*H + h and
 *   query tile i (pass 0 grid, Tq = ceil(N / rows) tiles per head),
 *   visits[bh * Tq + i] = the number of key tiles the kernel visited.
 *   visits: device int32 buffer of visits_len >= B*H*Tq elements (else
 *   FA_ERR_ARG), 4-byte aligned.  FA_BF16 only (else FA_ERR_UNSUPPORTED).
 *
 * fa_bwd_tile_visits — exactly fa_bwd_blocksparse (mask == NULL: fa_bwd),
 *   and in addition visits_kv[bh * Tk + j] = query stages visited by key
 *   tile j in the dK/dV pass (pass 1 grid, Tk = ceil(N / cols)) and
 *   visits_q[bh * Tq + i] = key tiles visited by query tile i in the dQ
 *   pass (pass 2 grid, Tq = ceil(N / rows)).  Lengths, alignment and dtype
 *   as fa_fwd_tile_visits.
 */
fa_status fa_tile_grid(int pass, int64_t d, int sparse, int64_t* rows,
                       int64_t* cols);
fa_status fa_fwd_tile_visits(const void* q, const void* k, const void* v,
                             void* o, float* lse, int64_t B, int64_t H,
                             int64_t N, int64_t d, fa_dtype dt, float scale,
                             int causal, const uint8_t* mask, int64_t block_m,
                             int64_t block_n, int32_t* visits,
                             size_t visits_len, void* stream);
fa_status fa_bwd_tile_visits(const void* q, const void* k, const void* v,
                             const void* o, const void* dout, const float* lse,
                             float* dq, float* dk, float* dv, void* workspace,
                             size_t workspace_bytes, int64_t B, int64_t H,
                             int64_t N, int64_t d, fa_dtype dt, float scale,
                             int causal, const uint8_t* mask, int64_t block_m,
                             int64_t block_n, int32_t* visits_kv,
                             size_t kv_len, int32_t* visits_q, size_t q_len,
                             void* stream);

/* Static description of a status code (never NULL). */
const char* fa_status_str(fa_status s);

/* Library version string, e.g. "exact_io_aware_amd 0.1.0 gfx950". */
const char* fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_IO_AWARE_FA_H */
