/*
 * dsa.h -- C ABI of the DeepSeek Sparse Attention (DSA) hot path on MI355X (gfx950).
 *
 * The path has three steps, each a call below:
 *   1. dsa_index_scores   lightning-indexer scores per (query, key)
 *   2. dsa_topk           per-query top-k selection, emitted as index lists and
 *                         as the attention mask (selection bits + tile classes)
 *   3. dsa_sparse_attn_fwd / dsa_sparse_attn_bwd
 *                         flash attention restricted to the selected keys
 *                         (forward; dQ/dK/dV backward)
 * dsa_build_mask turns index lists that come from elsewhere into the same mask.
 *
 * Sources (page title, section):
 *   "DeepSeek3.2: Onboard sparse attention", Background: an indexer computes a
 *     parametric index score as a query-key product, and a non-parametric top-k
 *     picks the keys and values each query attends to. Section "What this PR
 *     does", item 1: the top-k indices become an index mask that is added to
 *     the ordinary attention mask. Training only. Item 2: the 671B config uses
 *     64 index heads of dim 128 and top-k 2048.
 *   "Support Ring Attention with DeepSeek DSA Sparse Indexer", Forward Flow:
 *     the index mask is [batch, S, S] and shared by all heads. It is combined
 *     with the causal condition (diagonal included), and logits are scaled
 *     query-key products on kept entries. Backward Flow: dQ = dP K,
 *     dK = dP^T Q, dV = P^T dO on the same mask. Tests: the mask is threaded
 *     with and without segment IDs.
 *   "Integrate DeepSeek Sparse Attention with Tokamax Flash Attention",
 *     Description: flash attention takes a 3-D dynamic index mask in place of
 *     additive masking.
 *
 * Definitions used by every call:
 *   valid(t) = { s : s <= t and (seg == NULL or seg[b,s] == seg[b,t]) }
 *   I[b,t,s] = sum_j w[b,t,j] * max(0, sum_d q_idx[b,t,j,d] * k_idx[b,s,d])
 *   T(b,t)   = the n = min(K, |valid(t)|) keys of valid(t) with the largest
 *              scores; equal scores go to the smaller s; -0 == +0
 *   attention of query t, head h, over T(t):
 *              P = softmax_s(scale * q[b,t,h] . k[b,s,h]),  O = sum_s P v[b,s,h]
 *              LSE = log(sum_s exp(scale * q . k))   (natural log, float32)
 *   A row with T(t) empty gives O = 0, LSE = -inf and zero gradients.
 *
 * Conventions:
 *   - Every tensor is caller-owned DEVICE memory, contiguous row-major in the
 *     layout given next to it, and at least 16-byte aligned. The library never
 *     allocates and keeps no state besides a per-thread error string.
 *   - `stream` is a hipStream_t (NULL = the null stream). Every call only
 *     enqueues work on it and returns; nothing waits. A kernel fault shows up
 *     at the caller's next synchronisation.
 *   - Return value: DSA_OK, or an error code with no work enqueued. Arguments
 *     are checked on the host before any launch: NULL pointers, sizes < 1,
 *     misaligned pointers, unsupported dtype or dims, row ranges outside [0,S),
 *     ld < S, workspace too small. A failed launch returns DSA_ERR_HIP.
 *     dsa_last_error() then gives the detail.
 *   - Outputs are overwritten, never accumulated into.
 *   - bf16 tensors hold bfloat16 bit patterns. Every product is accumulated in
 *     float32, and stores round to nearest even.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1, /* NULL pointer, size < 1, bad range, misalignment */
  DSA_ERR_UNSUPPORTED = 2, /* valid but not implemented (dtype/dim combination) */
  DSA_ERR_WORKSPACE = 3,   /* workspace smaller than dsa_bwd_workspace_min_bytes() */
  DSA_ERR_HIP = 4          /* a HIP launch failed */
} dsa_status;

typedef enum { DSA_BF16 = 0, DSA_FP32 = 1 } dsa_dtype;

/* Tile of the attention kernels. The tile-class map of the mask is laid out on
 * this grid: one class per (128 queries) x (64 keys). */
#define DSA_TILE_Q 128
#define DSA_TILE_K 64

/* Tile classes stored in the mask. */
#define DSA_TILE_EMPTY 0 /* no selected (t, s) in the tile */
#define DSA_TILE_PARTIAL 1
#define DSA_TILE_FULL 2 /* every (t, s) with t < S selected; keys all < S */

/* ---------------------------------------------------------------------------
 * Size of the attention mask buffer for B x S, in bytes. Layout:
 *   sel_bits  uint64 [B][S][W], W = ceil(S/64). Bit (s % 64) of word s/64 of
 *             row (b,t) is 1 iff s is in T(b,t). Bits beyond S are 0.
 *   tile_cls  uint8  [B][ceil(S/DSA_TILE_Q)][ceil(S/DSA_TILE_K)], starting at
 *             byte B*S*W*8. Class of each tile of the selection matrix.
 * Produced only by dsa_topk or dsa_build_mask. Every set bit lies in valid(t),
 * so the mask already combines index, causal and segment conditions: the
 * attention calls take no segment IDs and apply the mask as given. A caller
 * who builds index sets elsewhere passes them, with the segment IDs, through
 * dsa_build_mask, which drops every entry outside valid(t). Writing mask bits
 * by hand is outside the contract (a bit outside valid(t) would be attended).
 * ------------------------------------------------------------------------- */
size_t dsa_mask_bytes(int B, int S);

/* ---------------------------------------------------------------------------
 * dsa_index_scores -- indexer scores I[b,t,s] for the query rows
 * t in [row0, row0 + nrows).
 * Source: "DeepSeek3.2: Onboard sparse attention", Background (the index score
 * is a query-key product of the indexer) and item 2 (64 x 128 index heads).
 *   q_idx   [B,S,Hi,Di]  in_dtype   index queries (after any RoPE)
 *   k_idx   [B,S,Di]     in_dtype   index keys, one per token, shared by heads
 *   w       [B,S,Hi]     in_dtype   per-token, per-index-head weights
 *   seg     [B,S] int32 or NULL     segment IDs (NULL = one segment)
 *   scores  [B,nrows,ld] score_dtype   out: row r holds query t = row0 + r.
 *           Entry s is written with I[b,t,s] for every s in valid(t); entries
 *           outside valid(t) are left unspecified.
 * in_dtype DSA_BF16 or DSA_FP32; score_dtype DSA_FP32 or DSA_BF16 (bf16 is
 * the float32 score rounded to nearest even). Any Hi, Di >= 1 are accepted.
 * bf16 inputs with Hi in {32, 64} and Di in {64, 128} take the MFMA kernel;
 * the rest take a plain kernel.
 * ------------------------------------------------------------------------- */
dsa_status dsa_index_scores(const void* q_idx, const void* k_idx, const void* w,
                            const int32_t* seg, int B, int S, int Hi, int Di,
                            dsa_dtype in_dtype, int row0, int nrows, void* scores,
                            dsa_dtype score_dtype, int64_t ld, void* stream);

/* ---------------------------------------------------------------------------
 * dsa_quant_fp8_rows -- quantize rows to OCP FP8 E4M3 with one scale per row.
 * Source: "DeepSeek3.2: Onboard sparse attention", What this PR does, item 4
 * (the original indexer's inputs are quantized to fp8). The page names no
 * format; the one used here: scale = amax(|row|) / 448 in float32, code =
 * round-to-nearest-even(x / scale) (float32 division), scale 0 and zero codes
 * for an all-zero row.
 *   x       [nrows, D] x_dtype (DSA_BF16 or DSA_FP32), rows contiguous
 *   codes   [nrows, D] uint8     out: E4M3 codes (s eeee mmm, bias 7)
 *   scale   [nrows]    float32   out
 * D in {64, 128, 256, 512}; x and codes 16-byte aligned. For the fp8 indexer below, q_idx [B,S,Hi,Di] is
 * B*S*Hi rows of Di and k_idx [B,S,Di] is B*S rows of Di.
 * ------------------------------------------------------------------------- */
dsa_status dsa_quant_fp8_rows(const void* x, dsa_dtype x_dtype, int64_t nrows, int D,
                              uint8_t* codes, float* scale, void* stream);

/* ---------------------------------------------------------------------------
 * dsa_index_scores_fp8 -- indexer scores from fp8 index queries and keys.
 * Source: as dsa_index_scores, with the fp8 inputs of item 4 of the same page.
 *   q8      [B,S,Hi,Di] uint8 E4M3   q_scale [B,S,Hi] float32  (q = q8 * q_scale)
 *   k8      [B,S,Di]    uint8 E4M3   k_scale [B,S]    float32  (k = k8 * k_scale)
 *   w       [B,S,Hi]    bf16
 *   seg, row0, nrows, scores, score_dtype, ld: as dsa_index_scores.
 * I[b,t,s] = sum_j w[t,j] max(0, q[t,j,:] . k[s,:]) on the dequantized values.
 * Scales must be finite and >= 0. Hi in {32, 64}, Di in {64, 128}. The code
 * products are summed by fp8 MFMAs, whose internal accumulation is coarser
 * than float32: a 64-wide partial sum was measured off by up to 2^-12.9 of the
 * largest code product in it, so a head's dot product carries an absolute
 * error of about 2^-12 of its largest code product (times q_scale * k_scale).
 * ------------------------------------------------------------------------- */
dsa_status dsa_index_scores_fp8(const uint8_t* q8, const float* q_scale, const uint8_t* k8,
                                const float* k_scale, const void* w, const int32_t* seg, int B,
                                int S, int Hi, int Di, int row0, int nrows, void* scores,
                                dsa_dtype score_dtype, int64_t ld, void* stream);

/* ---------------------------------------------------------------------------
 * dsa_indexer_rope -- partial RoPE of indexer inputs, concatenated layout.
 * Source: "DeepSeek3.2: Onboard sparse attention", What this PR does, item 1,
 * Indexer (partial RoPE on the indexer's q and k with the YaRN frequencies of
 * MLA, concatenated rather than interleaved layout).
 *   x       [B,S,nh,D] bf16   vectors to rotate (q_idx: nh = Hi; k_idx: nh = 1)
 *   cos_t, sin_t [P, rope_dim/2] float32   the frequency tables, row p for
 *           position p (the caller builds them, YaRN included)
 *   pos     [B,S] int32 or NULL   position of each token (NULL: token index t,
 *           which needs P >= S); positions outside [0, P) are clamped
 *   out     [B,S,nh,D] bf16   out; may be x itself (in place)
 * The first rope_dim dims rotate with dim i paired with i + rope_dim/2:
 *   y_i = x_i c_i - x_{i+h} s_i,  y_{i+h} = x_{i+h} c_i + x_i s_i  (h = rope_dim/2),
 * each product and sum rounded to float32 (no fused multiply-add), the result
 * rounded to bf16 (nearest, ties to even); the other dims are copied.
 * D % 8 == 0; rope_dim % 16 == 0 and 16 <= rope_dim <= D.
 * ------------------------------------------------------------------------- */
dsa_status dsa_indexer_rope(const void* x, int B, int S, int nh, int D, int rope_dim,
                            const float* cos_t, const float* sin_t, int P, const int32_t* pos,
                            void* out, void* stream);

/* ---------------------------------------------------------------------------
 * dsa_topk -- top-k selection of the rows t in [row0, row0 + nrows).
 * Source: "DeepSeek3.2: Onboard sparse attention", Background and item 1
 * (select the top-k keys of each query; get the top-k indices and the index
 * mask); "Support Ring Attention with DeepSeek DSA Sparse Indexer", Forward
 * Flow (mask [batch, S, S] combined with causal).
 *   scores  [B,nrows,ld] score_dtype, as written by dsa_index_scores. Only the
 *           entries in valid(t) are read.
 *   seg     [B,S] int32 or NULL (must match the one given to the indexer)
 *   idx     [B,S,K] int32  out: rows t of the slab get T(b,t) ascending,
 *           then -1 up to K entries. Other rows are untouched.
 *   mask    dsa_mask_bytes(B,S) bytes  out: sel_bits rows of the slab and the
 *           tile classes of the query tiles inside the slab.
 * K >= 1 (K >= S gives dense causal attention). row0 must be a multiple of
 * DSA_TILE_Q, and row0 + nrows must be a multiple of DSA_TILE_Q or equal S, so
 * that every query tile's class is built from rows of one call. Scores must be
 * finite; NaN gives an unspecified selection.
 * ------------------------------------------------------------------------- */
dsa_status dsa_topk(const void* scores, dsa_dtype score_dtype, int64_t ld,
                    const int32_t* seg, int B, int S, int K, int row0, int nrows,
                    int32_t* idx, void* mask, void* stream);

/* ---------------------------------------------------------------------------
 * dsa_build_mask -- attention mask from index lists given by the caller.
 * Source: same passages as dsa_topk (index mask shared by all heads, combined
 * with the causal and segment conditions).
 *   idx   [B,S,K] int32: entries < 0 or >= S are ignored, as are entries
 *         outside valid(t) (so the mask equals idx AND causal AND segment).
 *         Duplicates are harmless.
 *   seg   [B,S] int32 or NULL
 *   mask  dsa_mask_bytes(B,S) bytes  out: all of it.
 * ------------------------------------------------------------------------- */
dsa_status dsa_build_mask(const int32_t* idx, const int32_t* seg, int B, int S, int K,
                          void* mask, void* stream);

/* ---------------------------------------------------------------------------
 * dsa_sparse_attn_fwd -- attention of every query over its selected keys.
 * Source: "Support Ring Attention with DeepSeek DSA Sparse Indexer", Forward
 * Flow (logits are the query-key products times scale on kept entries);
 * "Integrate DeepSeek Sparse Attention with Tokamax Flash Attention",
 * Description (flash attention with a dynamic 3-D index mask).
 *   q, k  [B,S,H,Dqk] dtype;  v [B,S,H,Dv] dtype
 *   mask  from dsa_topk / dsa_build_mask for the same B, S
 *   o     [B,S,H,Dv] dtype  out
 *   lse   [B,H,S] float32   out (natural log; -inf for an empty row)
 * dtype DSA_BF16 or DSA_FP32. bf16 with (Dqk, Dv) = (192, 128) takes the MFMA
 * kernel; other dims up to 256 take a plain kernel.
 * ------------------------------------------------------------------------- */
dsa_status dsa_sparse_attn_fwd(const void* q, const void* k, const void* v, const void* mask,
                               int B, int S, int H, int Dqk, int Dv, float softmax_scale,
                               dsa_dtype dtype, void* o, float* lse, void* stream);

/* ---------------------------------------------------------------------------
 * Compressed sparse attention (CSA): the forward path over compressed keys.
 * Source: "Add Flash Attention Support to Deepseek v4", Description (CSA, at
 * compression ratio 4, attends over compressed KV blocks with block-aligned
 * causal masks); "Implement QK attention head chunking for CSA [Deepseek v4]",
 * Description (its indexer scores queries against the compressed blocks).
 * The pages give neither the compressor nor the block rule; the readings:
 *   * k_idx, k and v hold Sk = S / ratio (floor) compressed entries per batch
 *     row, made by the caller; entry c stands for tokens ratio*c .. ratio*c +
 *     ratio - 1 (tokens past ratio*Sk belong to no entry);
 *   * query t sees entry c iff ratio*c + ratio - 1 <= t (its block is
 *     complete); rows t < ratio - 1 see nothing (O = 0, LSE = -inf);
 *   * indexer, selection rule and attention are the DSA ones over the visible
 *     entries. No segment IDs, no sliding window. ratio 1 is DSA exactly.
 * Layouts follow the DSA calls with the key axis of length Sk:
 *   q_idx [B,S,Hi,Di], k_idx [B,Sk,Di], w [B,S,Hi]; scores [B,nrows,ld], ld >= Sk
 *   q [B,S,H,Dqk], k [B,Sk,H,Dqk], v [B,Sk,H,Dv]; o [B,S,H,Dv], lse [B,H,S]
 *   idx [B,S,K] int32 entry indices ascending, then -1 (dsa_csa_build_mask
 *       ignores entries < 0, >= Sk or not visible to the row; duplicates are
 *       harmless)
 *   mask  dsa_csa_mask_bytes(B,S,Sk) bytes: sel_bits uint64 [B][S][ceil(Sk/64)]
 *         then tile_cls uint8 [B][ceil(S/DSA_TILE_Q)][ceil(Sk/DSA_TILE_K)]
 * Errors: DSA_ERR_INVALID_ARG for ratio < 1, Sk != S / ratio, Sk < 1, ld < Sk
 * or the argument checks of the matching DSA call; dtype, dims, row slabs and
 * kernels (MFMA or plain) as in those calls.
 * dsa_csa_sparse_attn_bwd: gradients of sum(O * dout) w.r.t. q, k, v with the
 * forward's o, lse and mask; dq [B,S,H,Dqk], dk [B,Sk,H,Dqk], dv [B,Sk,H,Dv];
 * workspace >= dsa_bwd_workspace_min_bytes(B,S,H). It runs the prologue and the
 * key-major and query-major kernels: MFMA for bf16 192/128, with the dS handoff
 * when workspace_bytes >= dsa_csa_bwd_workspace_bytes(...) (each 32-query chunk
 * then holds all ceil(Sk/64) key tiles, 4 KB each, per (b, h); capped like the
 * token-level one) and otherwise a dQ kernel that recomputes dS (the same
 * bits); plain kernels for other dims (up to 256) and for fp32.
 * The token-level backward calls take ratio-1 masks only.
 * ------------------------------------------------------------------------- */
size_t dsa_csa_mask_bytes(int B, int S, int Sk);
size_t dsa_csa_bwd_workspace_bytes(int B, int S, int Sk, int ratio, int H, int Dqk, int Dv, dsa_dtype dtype);
dsa_status dsa_csa_index_scores(const void* q_idx, const void* k_idx, const void* w, int B, int S, int Sk,
                                int ratio, int Hi, int Di, dsa_dtype in_dtype, int row0, int nrows,
                                void* scores, dsa_dtype score_dtype, int64_t ld, void* stream);
dsa_status dsa_csa_topk(const void* scores, dsa_dtype score_dtype, int64_t ld, int B, int S, int Sk, int ratio,
                        int K, int row0, int nrows, int32_t* idx, void* mask, void* stream);
dsa_status dsa_csa_build_mask(const int32_t* idx, int B, int S, int Sk, int ratio, int K, void* mask,
                              void* stream);
dsa_status dsa_csa_sparse_attn_fwd(const void* q, const void* k, const void* v, const void* mask, int B, int S,
                                   int Sk, int ratio, int H, int Dqk, int Dv, float softmax_scale,
                                   dsa_dtype dtype, void* o, float* lse, void* stream);
dsa_status dsa_csa_sparse_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                   const float* lse, const void* mask, int B, int S, int Sk, int ratio, int H,
                                   int Dqk, int Dv, float softmax_scale, dsa_dtype dtype, void* dq, void* dk,
                                   void* dv, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * dsa_sparse_attn_bwd -- gradients of sum(O * dout) w.r.t. q, k, v.
 * Source: "Support Ring Attention with DeepSeek DSA Sparse Indexer", Backward
 * Flow (dQ = dP K, dK = dP^T Q, dV = P^T dO, each on the kept entries; dK/dV
 * run key-major).
 *   q, k, v, o, dout  as in the forward (o and lse from dsa_sparse_attn_fwd)
 *   lse       [B,H,S] float32
 *   mask      the forward's mask
 *   dq, dk    [B,S,H,Dqk] dtype out;  dv [B,S,H,Dv] dtype out
 *   workspace device scratch of workspace_bytes >= dsa_bwd_workspace_min_bytes()
 *             bytes. It receives two float32 [B,H,S] arrays: D = rowsum(dout * o),
 *             then lse * log2(e) (the row's log-sum-exp in base-2 units).
 *             With the bf16 MFMA path (Dqk = 192, Dv = 128) a larger workspace
 *             also holds, from the next 256-byte boundary, the dS tiles that the
 *             key-major kernel hands to the dQ kernel ("handoff"): 2 bytes per
 *             causal (query, key) pair of every (b, h), rounded to 32 x 64
 *             blocks, i.e. B*H*4096*T bytes with T = sum over c < ceil(S/32) of
 *             (c/2 + 1) (about B*H*S*S bytes). The handoff is used exactly when
 *             workspace_bytes covers it; otherwise the dQ kernel recomputes P
 *             and dS (same operations, same dQ, about twice the dQ time).
 *             dsa_bwd_workspace_bytes() returns the size with the handoff when
 *             the handoff is at most DSA_BWD_HANDOFF_MAX_BYTES, else the
 *             minimum, so memory stays O(B*H*S) at long sequences.
 * Same as dsa_sparse_attn_bwd_prep, _dkdv and _dq in that order on the same
 * stream. Deterministic: no atomics.
 * ------------------------------------------------------------------------- */
dsa_status dsa_sparse_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                               const void* dout, const float* lse, const void* mask,
                               int B, int S, int H, int Dqk, int Dv, float softmax_scale,
                               dsa_dtype dtype, void* dq, void* dk, void* dv,
                               void* workspace, size_t workspace_bytes, void* stream);

/* The three parts of dsa_sparse_attn_bwd, for callers that schedule them
 * separately, in this order on one workspace:
 *   _prep  D = rowsum(dout * o) and lse * log2(e) into the workspace
 *          (Backward Flow's per-row term of dS = P (dP - D)).
 *   _dkdv  key-major. Reads both; writes dk and dv, and on the MFMA path
 *          also leaves dS in the workspace.
 *   _dq    query-major. Reads the workspace; writes dq.
 * Arguments as in dsa_sparse_attn_bwd; each returns DSA_ERR_WORKSPACE for a
 * workspace below dsa_bwd_workspace_min_bytes(). The three take the route
 * (handoff or recompute) from workspace_bytes, so pass all three the same
 * workspace and size. */
dsa_status dsa_sparse_attn_bwd_prep(const void* o, const void* dout, const float* lse,
                                    int B, int S, int H, int Dqk, int Dv, dsa_dtype dtype,
                                    void* workspace, size_t workspace_bytes, void* stream);
dsa_status dsa_sparse_attn_bwd_dkdv(const void* q, const void* k, const void* v,
                                    const void* dout, const float* lse, const void* mask,
                                    int B, int S, int H, int Dqk, int Dv, float softmax_scale,
                                    dsa_dtype dtype, void* dk, void* dv, void* workspace,
                                    size_t workspace_bytes, void* stream);
dsa_status dsa_sparse_attn_bwd_dq(const void* q, const void* k, const void* v,
                                  const void* dout, const float* lse, const void* mask,
                                  int B, int S, int H, int Dqk, int Dv, float softmax_scale,
                                  dsa_dtype dtype, void* dq, const void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Largest dS handoff that dsa_bwd_workspace_bytes() asks for: 16 GiB. The
 * 2B-model shape (B 12, S 4096, 16 heads) needs 3.2 GB and the packed 8K shape
 * (B 4, S 8192, 32 heads) 8.6 GB; at S = 32768 with 128 heads it would be
 * 137 GB, so there the recompute route is the default. */
#define DSA_BWD_HANDOFF_MAX_BYTES (16ull << 30)

/* Workspace sizes of the backward calls, in bytes (0 for sizes < 1).
 *   _min_bytes: D and the base-2 LSE, 8*B*H*S rounded up to 256; the least
 *               any backward call accepts (recompute route).
 *   _bytes:     the recommended size: with the handoff where the dtype and dims
 *               take the MFMA path and the handoff is <= DSA_BWD_HANDOFF_MAX_BYTES,
 *               otherwise the minimum. */
size_t dsa_bwd_workspace_min_bytes(int B, int S, int H);
size_t dsa_bwd_workspace_bytes(int B, int S, int H, int Dqk, int Dv, dsa_dtype dtype);

/* ---------------------------------------------------------------------------
 * The indexer's KL auxiliary loss and its gradient, three calls in this order.
 * Sources: "Support Ring Attention with DeepSeek DSA Sparse Indexer", sections
 * "Isolated Flax NNX Auxiliary Loss" and "Loss Harvesting & Objective
 * Injection" (an indexer loss joins the training objective and trains the
 * indexer's query/key projections); "Implement QK attention head chunking for
 * CSA [Deepseek v4]", review of calculate_csa_indexer_loss (the teacher is a
 * float32 softmax of the attention scores, zeroed on invalid tokens, summed
 * over heads, with stop-gradient inputs). The pages give no student and no
 * divergence; the definitions taken here, with kept(t) the row's kept keys:
 *   teacher p_t(s) = (1/H) sum_h P_h(t,s), P_h head h's attention probability
 *                    over kept(t) (the heads' sum, normalised); no gradient
 *   student q_t(s) = softmax over kept(t) of I[t,s]
 *   loss = (1/N) sum_t KL(p_t || q_t), 0 log 0 = 0, over the N rows with a
 *          kept key;  dloss/dI[t,s] = (q_t(s) - p_t(s)) / N on kept pairs.
 *
 * dsa_indexer_teacher -- p_t over the kept keys, after dsa_sparse_attn_fwd.
 *   q, k    [B,S,H,Dqk] bf16, Dqk in {64, 128, 192};  lse [B,H,S] from the forward
 *   mask    the forward's mask
 *   teacher [B,S,K] float32 out: entry i of row t is p_t at the i-th smallest
 *           kept key (the i-th entry of dsa_topk's index list); 0 past them.
 *
 * dsa_indexer_kl -- student softmax, KL and the gradient w.r.t. the scores.
 *   scores  [B,S,ld] score_dtype (as given to dsa_topk)
 *   idx     [B,S,K] int32 from dsa_topk (ascending, -1 padded); teacher as above
 *   row_kl  [B,S] float32 out: KL(p_t || q_t) (0 for an empty row)
 *   loss    float32[2] out: {loss, N}
 *   dscores [B,S,ld_ds] float32 out: row t over [0, t] gets (q - p)/N at kept
 *           keys and 0 elsewhere; entries past t are untouched. With float32
 *           scores and ld_ds == ld it may be the scores buffer itself.
 * Deterministic: N is an integer count, and the loss sums row_kl in a fixed
 * order in one workgroup.
 *
 * dsa_indexer_bwd -- gradients of sum_{t,s} dscores[t,s] I[t,s] w.r.t. the
 * indexer inputs (with dscores from dsa_indexer_kl: of the loss):
 *   dw[t,j]     = sum_s g ReLU(u_j),   u_j = q_idx[t,j] . k_idx[s]
 *   dq_idx[t,j] = sum_s g w[t,j] [u_j > 0] k_idx[s]
 *   dk_idx[s]   = sum_t sum_j g w[t,j] [u_j > 0] q_idx[t,j]    (ReLU'(0) = 0)
 *   q_idx [B,S,Hi,Di], k_idx [B,S,Di], w [B,S,Hi] bf16 with Hi = 64, Di = 128
 *   dscores [B,S,ld] float32 (read over [0, t] of row t)
 *   mask    the forward's mask (its tile classes skip key tiles with no kept key)
 *   dq_idx, dk_idx, dw  out, bf16, the shapes of q_idx, k_idx, w
 * ------------------------------------------------------------------------- */
dsa_status dsa_indexer_teacher(const void* q, const void* k, const float* lse, const void* mask,
                               int B, int S, int H, int Dqk, int K, float softmax_scale,
                               dsa_dtype dtype, float* teacher, void* stream);
dsa_status dsa_indexer_kl(const void* scores, dsa_dtype score_dtype, int64_t ld, const int32_t* idx,
                          const float* teacher, const void* mask, int B, int S, int K, float* row_kl,
                          float* loss, float* dscores, int64_t ld_ds, void* stream);
dsa_status dsa_indexer_bwd(const void* q_idx, const void* k_idx, const void* w, const float* dscores,
                           int64_t ld, const void* mask, int B, int S, int Hi, int Di, dsa_dtype dtype,
                           void* dq_idx, void* dk_idx, void* dw, void* stream);

/* ---------------------------------------------------------------------------
 * dsa_sparse_attn_bwd_noalloc -- dsa_sparse_attn_bwd with no workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Arguments and results as dsa_sparse_attn_bwd, with the workspace replaced by
 * a scratch array inside the library: DSA_NOALLOC_SCRATCH_BYTES (64 MiB) of
 * device memory per GPU, held from the first call on that GPU until the
 * process ends. It covers B*H*S <= 8 Mi (D and the base-2 LSE, 8 bytes per
 * (b, h, t)); larger shapes return DSA_ERR_UNSUPPORTED before any HIP call.
 * dQ always takes the recompute route (no dS handoff), so the gradients equal
 * dsa_sparse_attn_bwd's. Nothing is allocated or freed. The scratch array is
 * shared by every call on the same GPU and keeps the last call's contents
 * (each call overwrites what it reads first), so calls that overlap in time on
 * one GPU -- on different streams or host threads -- race and must be
 * serialised by the caller. The stream must belong to the current device.
 * ------------------------------------------------------------------------- */
#define DSA_NOALLOC_SCRATCH_BYTES (64ull << 20)
dsa_status dsa_sparse_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                                       const void* dout, const float* lse, const void* mask,
                                       int B, int S, int H, int Dqk, int Dv, float softmax_scale,
                                       dsa_dtype dtype, void* dq, void* dk, void* dv, void* stream);

/* Human-readable name of a status code. Static storage. */
const char* dsa_status_string(dsa_status s);
/* Detail of the last non-OK return on this thread ("" if none). */
const char* dsa_last_error(void);
/* Library version: major * 10000 + minor * 100 + patch. */
int dsa_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H */
