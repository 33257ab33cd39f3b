/*
 * mala.h - C ABI of the MassAlloc Attention (MALA) library for AMD gfx950.
 *
 * MALA ("MassAlloc Attention: Let Attention Allocate Its Own Compute") is
 * causal tiled softmax attention in which every legal (query block, key
 * block) tile gets score discovery S = Q_i K_j^T, and the post-score work of
 * the tile (forward: softmax update, V load, PV; backward: P reconstruction,
 * dP, dS, dQ, dK, dV) runs only when a log-domain contribution test retains
 * the tile. The test compares the tile's row maxima with the running (or,
 * in backward, the finalized) softmax normalizer against the length-aware
 * threshold tau / L_q.
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 * - Layout: every q/k/v/o/dO/dQ/dK/dV tensor is BSHD, i.e. [batch, seq,
 *   heads, head_dim], fully contiguous (head_dim fastest). z (the
 *   log-normalizer) is [batch, heads_q, seqlen_q] float32, contiguous.
 * - The softmax scale 1/sqrt(head_dim) is already folded into q (MALA page,
 *   problem setup); natural exp/log throughout.
 * - Grouped-query attention: query head h reads KV head
 *   h / (heads_q / heads_kv); KV tensors are never expanded.
 * - Causality: query row q (0-based) sees key k iff k <= q + causal_offset,
 *   and L_q = q + causal_offset + 1 (equal-length training: offset 0, so
 *   L_q = q + 1; decode of N_q tokens: offset seqlen_k - N_q, so a single
 *   token has L_0 = seqlen_k) - MALA page, section 2.
 * - tau >= 0. tau = 0 disables skipping (the FullAttn limit of the page).
 *   tau may exceed 1.
 * - Pointers are device pointers (hipMalloc / torch CUDA tensors) unless a
 *   comment says otherwise, 16-byte aligned. The library never allocates,
 *   frees or keeps them: the caller owns every buffer, including workspaces.
 * - stream: a hipStream_t passed as void* (NULL = the null stream). Every
 *   call validates its arguments synchronously on the host, then enqueues
 *   kernels on the stream and returns without synchronizing. Kernel faults
 *   surface at the caller's next synchronization.
 * - The library keeps no global state and calls are thread-safe, except
 *   for mala_decode_noalloc, whose per-device scratch array is shared by
 *   every call on that device (see there).
 * - Optional outputs (NULL = off):
 *   stats     int64[4] device buffer; the call ADDS to it (caller zeroes):
 *             [0] legal tiles tested, [1] tiles retained,
 *             [2] post-score key slots (B_k per retained tile per valid
 *                 query row; the page's allocation metric),
 *             [3] tiles whose post-decision operand was loaded: V tiles
 *                 copied (forward: once per 128-row workgroup and key
 *                 tile, so two 64-row blocks that share a workgroup share
 *                 one copy; decode: once per KV head, split and tile) or
 *                 dO tiles loaded (backward, key-major pass).
 *   tile_mask uint8 device buffer; the call writes 1 (retained) or 0
 *             (skipped) for every legal tile it tests and leaves entries of
 *             non-legal tiles untouched (prefill the buffer, e.g. with 255).
 *   Production callers pass NULL for both: the operator itself
 *   materializes no mask (MALA page, fused operators).
 */
#ifndef MALA_H
#define MALA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define MALA_OK 0
#define MALA_EINVAL (-1)      /* bad argument: null pointer, misaligned pointer,
                                 non-positive size, a size above 2^30, a row
                                 (heads_q x head_dim elements) above 2^24,
                                 tau < 0 or NaN, heads_q not a multiple of
                                 heads_kv, causal_offset outside
                                 [0, seqlen_k - seqlen_q], bad split count */
#define MALA_EUNSUPPORTED (-2) /* head_dim / block_q / block_k / dtype combination
                                  not compiled (see below) */
#define MALA_EWORKSPACE (-3)  /* workspace NULL or smaller than the size query */
#define MALA_EHIP (-4)        /* a HIP launch or runtime call failed */
#define MALA_ETOOLARGE (-5)   /* the problem needs more scratch than
                                 mala_decode_noalloc holds */

/* Bytes of the device scratch array behind mala_decode_noalloc (per GPU). */
#define MALA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

typedef enum mala_dtype {
  MALA_BF16 = 0, /* bf16 tensors, fp32 accumulation, bf16 MFMA */
  MALA_FP32 = 1  /* fp32 tensors, fp32 arithmetic throughout */
} mala_dtype;

/* Problem description (MALA page, problem setup: Q in R^{N_q x d_h},
 * K, V in R^{N_k x d_h}, query blocks I_i of B_q rows, key blocks J_j of
 * B_k rows; tau and L_q as above). Compiled variants:
 *   forward  : head_dim in {64, 128}; block_q in {64, 128}; block_k in {64, 128}
 *   backward : bf16; head_dim in {64, 128}; block_q = block_k = 64
 *   decode   : head_dim 128, bf16; block_k in {64, 128, 256};
 *              heads_q / heads_kv <= 16 */
typedef struct mala_problem {
  int64_t batch;
  int64_t heads_q;
  int64_t heads_kv;
  int64_t seqlen_q;
  int64_t seqlen_k;
  int64_t head_dim;
  int32_t block_q;
  int32_t block_k;
  float tau;
  int32_t dtype;          /* mala_dtype */
  int64_t causal_offset;  /* query row q sees keys k <= q + causal_offset */
} mala_problem;

#define MALA_STAT_LEGAL_TILES 0
#define MALA_STAT_RETAINED_TILES 1
#define MALA_STAT_POST_SCORE_SLOTS 2
#define MALA_STAT_LOADED_TILES 3
#define MALA_NUM_STATS 4

/* Forward pass / inference prefill (MALA page, "Online Sparse Softmax" and
 * "Fused forward execution"). For every query block (independent work
 * items), key blocks are visited from the diagonal (the highest legal key
 * block) downward; each gets QK score discovery and the block test
 *   retain  <=>  exists a valid row q with a legal key in the tile such that
 *                rowmax_q - (m_q + log l_q) >= log tau - log L_q
 * (l_q = 0 counts as +inf, so every row's first legal tile is retained).
 * Retained tiles load V and apply the online-softmax update; skipped tiles
 * leave (m, l, O) unchanged.
 *   q [B, Nq, Hq, d], k, v [B, Nk, Hkv, d]   inputs (dtype of the problem)
 *   o [B, Nq, Hq, d]                          output, softmax over retained keys
 *   z [B, Hq, Nq] float32                     output, z_q = m_q + log l_q
 *   tile_mask [B, Hq, ceil(Nq/Bq), ceil(Nk/Bk)]  optional, see above */
int mala_fwd(const mala_problem* prob, const void* q, const void* k, const void* v,
             void* o, float* z, int64_t* stats, uint8_t* tile_mask, void* stream);

/* Forward / prefill on latent (MLA-shaped) attention: every query head
 * scores one shared cached row per position, and the value is the cached
 * latent itself, the first d_v columns of that row (the absorbed form of
 * multi-head latent attention on the attention tutorial page, section "MLA:
 * compress the cached representation"; the MALA page's per-slot accounting
 * counts 2 h d_v post-score FLOPs, d_v != d_qk). The rule, tiles, test,
 * traversal and outputs are those of mala_fwd with k = kv and
 * v = kv[..., :d_v]; V_j comes from the K tile already read, so a skipped
 * tile saves the exponentials and the P V contraction, not HBM bytes.
 *   prob       heads_kv must be 1; head_dim = d_qk; compiled: bf16,
 *              d_qk = 576, d_v = 512, block_q = block_k = 64
 *   q [B, Nq, Hq, d_qk]; kv [B, Nk, 1, d_qk] (contiguous rows)
 *   d_v        value width: 8 <= d_v <= d_qk, a multiple of 8
 *   o [B, Nq, Hq, d_v]; z [B, Hq, Nq] float32
 *   stats      as mala_fwd; MALA_STAT_LOADED_TILES counts retained tiles
 *              (the tiles whose value rows enter P V)
 *   tile_mask  [B, Hq, ceil(Nq/Bq), ceil(Nk/Bk)] optional
 * Errors: MALA_EINVAL also for heads_kv != 1 or a bad d_v. */
int mala_fwd_latent(const mala_problem* prob, const void* q, const void* kv, int64_t d_v,
                    void* o, float* z, int64_t* stats, uint8_t* tile_mask, void* stream);

/* Forward / prefill over packed variable-length sequences (the forward rule
 * of mala_fwd, applied per sequence; the tutorial page's implementation
 * checklist names packed sequences, cache offsets and empty rows among the
 * visibility contracts). Sequence b owns q/o rows [cu_seqlens_q[b],
 * cu_seqlens_q[b+1]) and k/v rows [cu_seqlens_k[b], cu_seqlens_k[b+1]) of
 * the packed tensors; its causal alignment is bottom-right, offset
 * N_k(b) - N_q(b) (chunked prefill: a chunk of N_q new tokens attends to the
 * N_k - N_q cached ones and causally to itself), L_q = q + offset + 1. When
 * N_k(b) < N_q(b) the first N_q - N_k rows see no key: their o is 0 and z is
 * -inf. Query blocks, tiles and the test are those of mala_fwd, per sequence.
 *   prob       batch = number of sequences; seqlen_q / seqlen_k = the longest
 *              N_q(b) / N_k(b) (they size the grid and tile_mask; longer
 *              sequences are cut at these lengths); causal_offset must be 0;
 *              bf16 only; head_dim, block_q, block_k as mala_fwd
 *   q [total_q, Hq, d], k, v [total_k, Hkv, d]  packed (THD), contiguous
 *   cu_seqlens_q int32 [B + 1], cu_seqlens_k int32 [B + 1]  device,
 *              non-decreasing prefix offsets (clamped to [0, total])
 *   o [total_q, Hq, d]; z [Hq, total_q] float32
 *   tile_mask [B, Hq, ceil(seqlen_q/Bq), ceil(seqlen_k/Bk)] optional */
int mala_fwd_varlen(const mala_problem* prob, const void* q, const void* k, const void* v,
                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int64_t total_q,
                    int64_t total_k, void* o, float* z, int64_t* stats, uint8_t* tile_mask,
                    void* stream);

/* Workspace bytes mala_bwd needs: three fp32 values per query row (-z_q
 * log2 e, the test offset z_q + log tau - log L_q, and D_q; B Hq 3 Nq'
 * floats with Nq' = Nq rounded up to a multiple of 128), 4 KB of partial
 * maxima of |dO|, and a 16-bit copy of dO (B Nq Hq d 2 bytes). */
size_t mala_bwd_workspace_size(const mala_problem* prob);

/* Backward pass (MALA page, "Offline Sparse Probability" and "Fused
 * backward execution"). Key-major: for every key block j and, per query
 * head of its KV group, every query block i from the diagonal upward,
 * S = Q_i K_j^T is recomputed and the tile is retained iff some legal
 * (q, k) has S_qk - z_q >= log tau - log L_q. Retained tiles rebuild
 * P = exp(S - z) and run dV += P^T dO, dP = dO V^T, dS = P (dP - D),
 * dQ += dS K, dK += dS^T Q, with D_q = sum_d dO_qd O_qd. dQ is formed by a
 * query-major pass that repeats the same test with identical arithmetic, so
 * all three gradients use one set of decisions and the result is
 * deterministic (no atomics).
 *   q, k, v, o, dout as in mala_fwd (o: the forward output)
 *   z [B, Hq, Nq] float32        the forward's finalized log-normalizer
 *   dq [B, Nq, Hq, d]            output
 *   dk, dv [B, Nk, Hkv, d]       outputs, summed over each KV group's heads
 *   workspace / ws_bytes         >= mala_bwd_workspace_size(prob) bytes of
 *                                device memory; contents on entry ignored
 * Precision: S, dP, dS and the products run on the matrix cores with fp32
 * accumulation. dP and dV take dO (and V) as fp16 values scaled by powers
 * of two (exact for every value within 2^28 of its tensor's, or V tile's,
 * largest magnitude) and P rounded to fp16; dK and dQ take dS as a bf16
 * pair (rounded value plus its rounding residual). A non-finite value in
 * dout leaves the gradients unspecified.
 *   tile_mask [B, Hq, ceil(Nq/Bq), ceil(Nk/Bk)]  optional: the decisions of
 *                                the key-major pass (the one dK, dV use)
 *   tile_mask_dq                 optional, same shape and conventions: the
 *                                decisions the query-major pass takes for
 *                                dQ on its own (equal to tile_mask tile for
 *                                tile: one decision per tile, "Offline
 *                                Sparse Probability"); a debug check */
int mala_bwd(const mala_problem* prob, const void* q, const void* k, const void* v,
             const void* o, const void* dout, const float* z, void* dq, void* dk,
             void* dv, void* workspace, size_t ws_bytes, int64_t* stats,
             uint8_t* tile_mask, uint8_t* tile_mask_dq, void* stream);

/* Workspace bytes mala_bwd_latent needs: the per-row term D_q and the fp32
 * partial row gradients of the key-major pass (0 for an invalid problem or
 * heads_kv != 1). */
size_t mala_bwd_latent_workspace_size(const mala_problem* prob);

/* Backward pass on latent (MLA-shaped) attention: mala_bwd's rule (MALA
 * page, "Offline Sparse Probability" and "Fused backward execution") on the
 * cache form of mala_fwd_latent, where the cached row kv_s is the key and
 * its first d_v columns the value (the absorbed form of the tutorial page's
 * MLA section). The row's gradient is the sum of both uses,
 * dkv = dK + [dV, 0], summed over every query head. Decisions, D_q and P are
 * mala_bwd's; the result is deterministic (no atomics on gradients).
 *   prob       heads_kv = 1; head_dim = d_qk; the other fields as mala_bwd
 *   q [B, Nq, Hq, d_qk]; kv [B, Nk, 1, d_qk]
 *   o, dout [B, Nq, Hq, d_v]; z [B, Hq, Nq] float32 (mala_fwd_latent's)
 *   dq [B, Nq, Hq, d_qk]; dkv [B, Nk, 1, d_qk]   outputs
 *   d_v        value width, a multiple of 8 in (0, d_qk]
 *   workspace / ws_bytes  >= mala_bwd_latent_workspace_size(prob) bytes of
 *              device memory; contents on entry ignored
 *   tile_mask [B, Hq, ceil(Nq/Bq), ceil(Nk/Bk)] optional (key-major pass)
 *   tile_mask_dq  optional, the query-major pass's own decisions (as mala_bwd)
 * Compiled: bf16, d_qk 576, d_v 512, block_q = block_k = 64 (other shapes
 * return MALA_EUNSUPPORTED).
 * Errors: MALA_EINVAL also for heads_kv != 1 or a bad d_v. */
int mala_bwd_latent(const mala_problem* prob, const void* q, const void* kv, int64_t d_v,
                    const void* o, const void* dout, const float* z, void* dq, void* dkv,
                    void* workspace, size_t ws_bytes, int64_t* stats, uint8_t* tile_mask,
                    uint8_t* tile_mask_dq, void* stream);

/* Workspace bytes mala_decode needs for num_splits split partials. */
size_t mala_decode_workspace_size(const mala_problem* prob, int num_splits);

/* Decode of a short query with optional split-KV (MALA page, split-KV
 * paragraph and "Fused decoding execution": the forward rule with a short
 * query against a longer KV sequence). The query holds the N_q = seqlen_q
 * newest tokens of each sequence (1 <= N_q <= 16, N_q <= seqlen_k,
 * causal_offset = seqlen_k - N_q): token t sits at position
 * seqlen_k - N_q + t, sees the keys up to it and uses L = position + 1 in
 * its threshold (a single token: L_0 = seqlen_k). The N_q rows of a query
 * head form one query block - one decision per (head, tile), a tile retained
 * iff one of the rows passes its own test, each row with its own running
 * state. The T = ceil(Nk/Bk) key tiles are cut into num_splits contiguous
 * ranges [floor(s T / S), floor((s + 1) T / S)); each split starts from an
 * empty state, visits its tiles from the most recent one downward and tests
 * them against its own partial normalizer; a KV tile's V is loaded iff some
 * head of the group retains it. Each row's split partials are merged by the
 * normalizer-aware combine z = log sum_s exp(z_s), o = sum_s exp(z_s - z) o_s
 * (a split where the row has no key takes no part).
 *   q [B, N_q, Hq, d]; k_cache, v_cache [B, Nk, Hkv, d]
 *   o [B, N_q, Hq, d]; z [B, Hq, N_q] float32
 *   num_splits in [1, T]
 *   tile_mask [B, Hq, T] optional per-(head, tile) decisions
 * The kernels score a KV group's (query head, token) pairs together as the
 * 16 columns of the matrix-core op: (Hq / Hkv) * N_q > 16 returns
 * MALA_EUNSUPPORTED. */
int mala_decode(const mala_problem* prob, const void* q, const void* k_cache,
                const void* v_cache, void* o, float* z, int num_splits, void* workspace,
                size_t ws_bytes, int64_t* stats, uint8_t* tile_mask, void* stream);

/* mala_decode for callers that cannot allocate device memory - code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same rule, arguments, outputs, validation and kernels as mala_decode, but
 * no workspace argument: the split partials live in a file-scope device
 * array of MALA_NOALLOC_SCRATCH_BYTES bytes inside the library, one copy on
 * each GPU the library runs on, held until the process ends. Its device
 * address is looked up once per device, on the first call with that device
 * current; the call itself allocates and frees nothing.
 *   Limit: mala_decode_workspace_size(prob, num_splits) must not exceed
 *   MALA_NOALLOC_SCRATCH_BYTES (64 MiB: e.g. batch 64 x 32 query heads x
 *   head_dim 128 at up to 63 splits); larger problems return MALA_ETOOLARGE
 *   before anything is launched.
 *   Sharing: every call on one GPU uses that GPU's one array, and each call
 *   overwrites the partials it reads back (nothing needs to start at zero).
 *   Calls that overlap in time on one GPU - on different streams, or from
 *   different host threads without ordering - race on the array and give
 *   undefined results; calls on one stream are ordered and safe. */
int mala_decode_noalloc(const mala_problem* prob, const void* q, const void* k_cache,
                        const void* v_cache, void* o, float* z, int num_splits, int64_t* stats,
                        uint8_t* tile_mask, void* stream);

/* Short-query decode over a paged KV cache with per-sequence lengths
 * (MALA page, "Fused decoding execution" and split-KV paragraph; the
 * tutorial page's implementation checklist names cache offsets, packed
 * sequences, cache updates and empty rows among the contracts a kernel must
 * honour; the block-table layout that maps each sequence's key positions to
 * fixed-size pages is the common serving form, adopted here as a reading,
 * not taken from the pages). Sequence b has N_k(b) = seq_lens[b] keys; its key k is row
 * k % page_size of page block_table[b * max_pages_per_seq + k / page_size].
 * Everything else is mala_decode's rule, per sequence: token t at position
 * N_k(b) - N_q + t, T_b = ceil(N_k(b) / block_k) tiles, split s of
 * num_splits covers tiles [floor(s T_b / S), floor((s + 1) T_b / S)); a split
 * whose range is empty (T_b < S) holds no keys and drops out of the combine;
 * a row at a negative position (N_k(b) < N_q), and every row of a sequence
 * with no keys, yields o = 0, z = -inf.
 *   prob       batch, heads_q, heads_kv, head_dim, block_k, tau, dtype as in
 *              mala_decode; seqlen_q = N_q; seqlen_k = max_pages_per_seq *
 *              page_size (the table's capacity); causal_offset =
 *              seqlen_k - N_q
 *   q [B, N_q, Hq, d]; o [B, N_q, Hq, d]; z [B, Hq, N_q] float32
 *   k_pages, v_pages [num_pages, page_size, Hkv, d]
 *   block_table int32 [B, max_pages_per_seq] (device, 4-byte aligned); page
 *              ids outside [0, num_pages) are clamped (no fault; results for
 *              such a table are undefined)
 *   seq_lens   int32 [B] (device); values are clamped to [0, capacity]
 *   page_size  a power of two in [16, 4096]
 *   num_splits in [1, ceil(capacity / block_k)]; workspace as
 *              mala_decode_workspace_size(prob, num_splits)
 *   tile_mask [B, Hq, ceil(capacity / block_k)] optional; entries of tiles
 *              past a sequence's end are left untouched
 * Compiled variants as mala_decode. */
int mala_decode_paged(const mala_problem* prob, const void* q, const void* k_pages,
                      const void* v_pages, const int32_t* block_table, const int32_t* seq_lens,
                      int64_t num_pages, int32_t page_size, int32_t max_pages_per_seq, void* o,
                      float* z, int num_splits, void* workspace, size_t ws_bytes, int64_t* stats,
                      uint8_t* tile_mask, void* stream);

/* Single-token decode on latent (MLA-shaped) attention: mala_decode's rule
 * (MALA page, split-KV paragraph and "Fused decoding execution") on the
 * cache form of mala_fwd_latent (one cached row kv_s per position; the
 * value is its first d_v columns, the absorbed form of the tutorial page's
 * MLA section). Each split starts from an empty state, visits its tiles
 * from the most recent one down and tests every query head against its own
 * partial normalizer with L_0 = seqlen_k; a head that does not retain a
 * tile leaves its state unchanged; split partials are merged as in
 * mala_decode. The value shares the cached row, so a skipped tile saves the
 * exponentials and the P V contraction but no memory traffic.
 *   prob       heads_kv = 1; head_dim = d_qk; seqlen_q = 1;
 *              causal_offset = seqlen_k - 1; num_splits in [1, T],
 *              T = ceil(seqlen_k / block_k)
 *   q [B, 1, Hq, d_qk]; kv_cache [B, Nk, 1, d_qk]; o [B, 1, Hq, d_v];
 *   z [B, Hq] float32
 *   d_v        value width, a multiple of 8 in (0, d_qk]
 *   workspace  >= mala_decode_workspace_size(prob, num_splits) bytes
 *   tile_mask [B, Hq, T] optional per-head decisions
 * Compiled: bf16, d_qk 576, d_v 512, block_k 64, heads_q a multiple of 16
 * (other shapes return MALA_EUNSUPPORTED).
 * Errors: MALA_EINVAL also for heads_kv != 1 or a bad d_v. */
int mala_decode_latent(const mala_problem* prob, const void* q, const void* kv_cache, int64_t d_v,
                       void* o, float* z, int num_splits, void* workspace, size_t ws_bytes,
                       int64_t* stats, uint8_t* tile_mask, void* stream);

/* ---------------------------------------------------------------------------
 * Operator-fidelity instrumentation (MALA page, experiments: the omitted-mass
 * definition and the operator-fidelity protocol, which compares the screened
 * operator with a screening-disabled run, tau = 0, on the same inputs).
 * Same conventions as above: device pointers, 16-byte aligned, synchronous
 * validation, asynchronous launch on `stream`, nothing allocated.
 * ------------------------------------------------------------------------- */

/* Omitted mass of n query rows: omitted[r] = 1 - exp(z_screened[r] -
 * z_reference[r]), the dense softmax mass on the positions the screened
 * operator left out, where z_screened is mala_fwd's z at tau and z_reference
 * its z at tau = 0 (FullAttn). Computed as -expm1 of the fp32 difference; not
 * clamped, so rounding can give values of order -1e-7 when nothing was
 * omitted. z_*, omitted: float32 [n] (e.g. [B, Hq, Nq] flattened). */
int mala_omitted_mass(const float* z_screened, const float* z_reference, float* omitted, int64_t n,
                      void* stream);

/* Per-head squared errors for relative L2 (the page reports, per head,
 * ||x - ref||_2 / ||ref||_2 for O, dQ, dK and dV): for BSHD tensors x, ref
 * [batch, seqlen, heads, head_dim] of `dtype` (mala_dtype),
 *   sq_diff[b * heads + h] = sum over (n, d) of (x - ref)^2,
 *   sq_ref [b * heads + h] = sum over (n, d) of ref^2,
 * accumulated in float64 with a fixed reduction order (deterministic).
 * sq_diff, sq_ref: float64 [batch * heads] device buffers (overwritten). */
int mala_sq_err_heads(const void* x, const void* ref, int64_t batch, int64_t seqlen, int64_t heads,
                      int64_t head_dim, int32_t dtype, double* sq_diff, double* sq_ref, void* stream);

/* Histogram of realized post-score key slots per query (the page's
 * allocation metric, recorded per query in its fidelity study) from a tile
 * mask written by mala_fwd or mala_bwd for problem `prob` (1 = retained; any
 * other value, e.g. the 255 prefill of non-legal tiles, is not counted).
 * For every query block the count c of retained tiles in its mask row is
 * taken, and each valid query row of the block adds 1 to hist[c]; the row's
 * post-score slots are c * block_k. hist: int64 [ceil(Nk/Bk) + 1] device
 * buffer, ADDED to (caller zeroes), summed over batch and query heads. */
int mala_slot_histogram(const mala_problem* prob, const uint8_t* tile_mask, int64_t* hist,
                        void* stream);

/* Deterministic Rademacher probe (the page drives its backward comparison
 * with one) from the SplitMix64 generator of Steele, Lea and Flood (2014) in
 * counter form: x_i = mix(seed + (i + 1) * 0x9E3779B97F4A7C15) with the
 * published 64-bit mixing function, i.e. output i of SplitMix64 seeded with
 * `seed`; out[i] = -1 if bit 63 of x_i is set, else +1. out: n elements of
 * `dtype` (bf16 or float32). */
int mala_rademacher(void* out, int64_t n, int32_t dtype, uint64_t seed, void* stream);

/* Static description of a status code. */
const char* mala_error_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MALA_H */
