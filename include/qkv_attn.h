/*
 * qkv_attn.h - C ABI of libqkvattn.so: quantized cross-loop decode attention for
 * looped Transformers on AMD Instinct MI355X (gfx950).
 *
 * What is computed (pages about "FlashLoop: Fast and Memory-Efficient Looped
 * Transformers via Lazy Updates"):
 *   - project page, The Method, STEP 03; flozi.net explainer section 3: loop 1's K/V
 *     are stored as an INT4 base and every later loop as the INT4 residual against the
 *     previous loop's reconstruction, group size 64, asymmetric scale/zero, keys grouped
 *     per channel over 64 tokens, values per token over 64 channels, the most recent
 *     tokens kept in BF16;
 *   - project page STEP 01: residual rows exist for active tokens only, inactive tokens
 *     reuse the previous loop's K/V;
 *   - project page STEP 02; explainer section 3: sparse late loops attend to the top-K
 *     key columns of the preceding loop's distribution, cache those columns' probability
 *     mass m under that full distribution, and correct the preceding loop's output for
 *     those columns only (a rank-K correction that keeps mass m);
 *   - PyPI page, Configuration: 4 loops, dense loops 1-2, 10% key budget, 4-bit, group
 *     64, 64-token BF16 tail, head dimension 128, batch one (batch > 1 is supported here).
 *
 * Conventions for every entry point
 *   - Pointers documented as "device" are HIP device memory owned by the caller; the
 *     library never allocates, frees or retains them and keeps no state between calls.
 *   - Work is queued on `stream` (a hipStream_t; NULL = the default stream) and is
 *     asynchronous: results are valid once the stream has reached that point.
 *   - Arguments are checked on the host before anything is queued; on error nothing is
 *     queued and a negative status is returned (see qkv_strerror).  Device-side contents
 *     (active lists, index lists) are trusted: they must satisfy the stated contracts.
 *   - Device buffers must be 16-byte aligned.  bf16 values are passed as uint16_t bits.
 *   - Calls that share a cache or a workspace must not overlap in time (same stream or
 *     explicit ordering).
 */
#ifndef QKV_ATTN_H
#define QKV_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QKV_MAX_LOOPS 32
#define QKV_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)  /* attn_decode_dense_noalloc's fixed scratch */
#define QKV_GROUP 64
#define QKV_TAIL_SLOTS 128

enum {
    QKV_OK = 0,
    QKV_EINVAL = -1,        /* bad argument (null pointer, size out of range, misalignment) */
    QKV_EUNSUPPORTED = -2,  /* head_dim not 64/128, loop count above QKV_MAX_LOOPS, ...     */
    QKV_ECAPACITY = -3,     /* positions or rows beyond the buffers the cache describes     */
    QKV_ELAUNCH = -4,       /* a HIP launch failed                                           */
    QKV_EWORKSPACE = -5     /* workspace missing or smaller than qkv_workspace_bytes()      */
};

/*
 * One loop's stored plane (loop p = index + 1).  Layout of `data`, device memory:
 *   [batch][heads][n_blocks][block], one block = 64 consecutive storage slots.  With
 *   c = head_dim * bits / 8 code bytes per slot (bits: see qkv_cache.residual_bits):
 *   d = 128: block = K codes [64][c] | V records [64] of (V codes [c] | (s, z) [2], fp32)
 *                    | K s[128], K z[128] (fp32)       -> 10240 bytes (4-bit), 6144 (2-bit)
 *   d = 64:  block = K codes [64][c] | V codes [64][c] | K s[64], K z[64] (fp32)
 *                    | V meta [64] of (s, z) (fp32)    -> 5120 bytes (4-bit), 3072 (2-bit)
 *   (at d = 128 a slot's value codes and value meta are adjacent, so a gather of one
 *   slot's value touches fewer 128-byte lines).
 *   4-bit codes: a byte holds channel 2i in its low nibble and channel 2i+1 in its high
 *   nibble.  2-bit codes: byte i holds channels 4i..4i+3, channel 4i+m in bits 2m, 2m+1.
 *   Key group = one block (64 consecutive slots) per channel; value group = one slot
 *   over 64 consecutive channels.  Dequantised value = fmaf(code, s, z), with
 *   s = (max - min) / (2^bits - 1).
 * A dense plane stores every body position at slot == position.  A sparse plane stores
 * the active positions in ascending order; each encode call starts on a new block and
 * pads its last block (padding slots: codes 0, value meta 0, rowpos -1).  Sparse planes
 * need the three maps below (device int32, caller-allocated; rowstart[b][0] must be 0
 * before the first encode of the plane; rowmap/rowpos need no initialisation):
 *   rowmap   [batch][cap_ctx]          position -> slot, -1 if not stored
 *   rowpos   [batch][n_blocks * 64]    slot -> position, -1 for padding
 *   rowstart [batch][cap_ctx/64 + 1]   first slot holding a position >= 64*i
 * Loop 1 (the base) must be dense.
 */
typedef struct qkv_plane {
    void* data;
    int32_t n_blocks;
    int32_t dense;
    int32_t* rowmap;
    int32_t* rowpos;
    int32_t* rowstart;
} qkv_plane;

/*
 * One layer's cross-loop cache.  Column (position) geometry, same for every sequence:
 *   body = [0, n_body) with n_body = 64 * floor((n_ctx - 64) / 64) (0 if n_ctx < 64),
 *   tail = [n_body, n_ctx), so 64 <= n_ctx - n_body < 128 once n_ctx >= 64.
 * Body positions live in the planes; tail positions in the per-loop BF16 tails
 *   tail_k[p], tail_v[p]: device bf16 [batch][heads][128][head_dim], position t at slot
 *   t % 128, holding loop p+1's value (an inactive token holds loop p's value).
 * The caller advances n_ctx; when the body boundary moves, the 64 positions that leave
 * the tail must first be encoded into every loop's plane (kv_encode_loop with
 * k_src == NULL, loops in order).
 */
typedef struct qkv_cache {
    int32_t batch, heads, head_dim, n_loops;
    int32_t cap_ctx;   /* capacity in positions, a multiple of 64 */
    int32_t n_ctx;     /* cached positions (attention columns) of every sequence */
    qkv_plane plane[QKV_MAX_LOOPS];
    uint16_t* tail_k[QKV_MAX_LOOPS];
    uint16_t* tail_v[QKV_MAX_LOOPS];
    /* NULL, or device uint32 [batch][cap_ctx], zeroed before the first encode: bit p of a
     * position's word is set iff the sparse plane of loop p+1 stores the position
     * (kv_encode_loop maintains it).  With it, a gather over a deep chain reads only the
     * planes that store a column; without it, it looks the column up in every plane. */
    uint32_t* stored_loops;
    /* Codec [project page, "Main Results": precision sweep of the KV residual quantization;
     * explainer sections 4 and 5: the "Per-loop KIVI4" ablation and the 2-bit setting]:
     *   residual_bits  code width of the planes of loops >= 2: 4 (or 0, read as 4) or 2;
     *                  loop 1's base is always 4-bit;
     *   full_state     0: loop r >= 2 stores the residual X^(r) - Xhat^(r-1) (the chain is
     *                  the sum of the stored planes); 1: every loop stores its own X^(r)
     *                  with 4-bit codes, and a position's K/V in loop r is that of the last
     *                  loop <= r that stores it (requires residual_bits 4). */
    int32_t residual_bits;
    int32_t full_state;
    /* NULL, or a device uint32 the caller zeroes: kv_encode_loop (and a flush carried by an
     * attention call) sets bit 0 (QKV_FLAG_PLANE_FULL) when a sparse plane has no block left
     * for a group of active rows; those rows are then not stored, and later reads of those
     * positions use the previous loop's values.  Size sparse planes with n_blocks >= the
     * active rows / 64 plus one block per encode call, or check this word. */
    uint32_t* error_flags;
} qkv_cache;

#define QKV_FLAG_PLANE_FULL 1u

/*
 * A 64-row tail flush carried by an attention call [project page, The Method, after STEP 03:
 * cross-loop KV updates and quantization fused into the attention kernel].  When the next
 * decode position will move the body boundary (n_ctx - n_body == 127 in this call), the
 * tail's 64 oldest positions [pos0, pos0 + 64), pos0 = n_body, must be encoded into every
 * loop's plane, loops in order.  Given to loop r's attention call of the current step, the
 * call's kernel encodes loop r's rows of that group in extra workgroups beside its readers
 * (which do not read those positions from the planes in this step); given to every loop's
 * call of the step, in loop order, it replaces the kv_encode_loop flush of the next step,
 * with identical plane contents.  The caller then advances n_ctx without flushing.
 *   pos0     must equal the body length of the current n_ctx, and pos0 + 64 <= n_ctx - 1.
 *   act_pos, n_act, ld_act  as for kv_encode_loop: the loop's active positions among the
 *            group (sparse planes); both NULL for a dense plane.
 */
typedef struct qkv_flush {
    int32_t pos0;
    int32_t ld_act;
    const int32_t* act_pos;
    const int32_t* n_act;
} qkv_flush;

/* Human-readable text of a status code (static storage). */
const char* qkv_strerror(int status);

/* Bytes of one 64-slot block for head_dim d and `bits`-bit codes (see qkv_plane), 0 if
 * unsupported.  A plane's blocks are 4-bit for loop 1 and for the full-state codec,
 * residual_bits otherwise. */
size_t qkv_block_bytes(int head_dim, int bits);

/* Body length for a context of n positions (see qkv_cache). */
int qkv_body_len(int n_ctx);

/*
 * Workspace bytes that attn_decode_dense, attn_decode_sparse and select_columns need for
 * caches of this shape with up to max_ctx positions and up to max_k selected columns.
 * The workspace is device memory owned by the caller; it needs no initialisation and
 * holds nothing between calls (calls that use one workspace must not overlap).
 */
size_t qkv_workspace_bytes(int batch, int heads, int head_dim, int max_ctx, int max_k);

/*
 * kv_encode_loop - residual-quantize encode of one loop for positions [pos0, pos0+n_pos)
 * [project page STEP 03; explainer section 3].
 *   loop     1..n_loops; loops must be encoded in order for a position range, because
 *            loop r stores X^(r) - Xhat^(r-1) and rebuilds Xhat^(r-1) from planes 1..r-1.
 *   pos0     multiple of 64; n_pos a positive multiple of 64; pos0 + n_pos <= cap_ctx.
 *   act_pos  device int32 [batch][ld_act]: ascending active positions of each sequence,
 *            all in [pos0, pos0+n_pos); n_act device int32 [batch] their counts
 *            (n_act[b] <= ld_act; a list written by select_tokens, with n_before as the
 *            counts, can be passed as it is).
 *            Both must be NULL for a dense plane (every position active).
 *   k_src, v_src  device bf16 [batch][heads][ld_src][head_dim]: row i = the i-th active
 *            position's K^(loop) / V^(loop) (post-RoPE keys).  If both are NULL the rows
 *            are read from tail_k/tail_v[loop-1] (flushing tail positions into the body).
 * Writes the plane's blocks for these slots (and, for a sparse plane, its maps).
 * Codes, scales and zeros follow the quantizer exactly: s = (max-min)/15, z = min (fp32,
 * -0 stored as +0), code = clamp(rint((x - z)/s), 0, 15), code 0 when s == 0.
 */
int kv_encode_loop(const qkv_cache* cache, int loop, int pos0, int n_pos,
                   const int32_t* act_pos, const int32_t* n_act, int ld_act,
                   const uint16_t* k_src, const uint16_t* v_src, int ld_src, void* stream);

/*
 * kv_append_tail - writes n_rows consecutive positions pos0.. of loop `loop` into the BF16
 * tail ring [PyPI Configuration: 64-token BF16 residual tail].
 *   k, v: device bf16 [batch][heads][n_rows][head_dim].  1 <= n_rows <= 128.
 *   loop == 0 writes every loop in one launch; k, v are then [n_loops][batch][heads][n_rows][head_dim].
 */
int kv_append_tail(const qkv_cache* cache, int loop, int pos0, int n_rows,
                   const uint16_t* k, const uint16_t* v, void* stream);

/*
 * attn_decode_dense - dense decode attention of loop `loop` over all n_ctx columns
 * [explainer section 1: decode reads every cached column; textbook softmax attention].
 *   Keys/values of column j are the loop's reconstruction: base plus every residual
 *   plane p <= loop in which j is stored (BF16 tail values for tail columns).
 *   q        device bf16 [batch][heads][head_dim]; sm_scale multiplies the logits.
 *   k_new, v_new  both NULL, or device bf16 [batch][heads][head_dim]: this loop's key and
 *            value of the newest position n_ctx - 1 (already counted in n_ctx).  The call
 *            stores them in the loop's BF16 tail, as kv_append_tail(cache, loop, n_ctx - 1,
 *            1, k_new, v_new) would, and attends over them in the same launch
 *            [PyPI Configuration: 64-token BF16 residual tail].
 *   o        device bf16 [batch][heads][head_dim] (may be NULL); o_f32 device fp32 same shape.
 *   scores   device fp32 [batch][heads][ld_scores]: raw logits s_j, j < n_ctx; or NULL when
 *            no later call reads them (ld_scores is then ignored).
 *   lse      device fp32 [batch][heads]: log sum_j exp(s_j).
 *   flush    NULL, or this loop's part of the next step's tail flush (see qkv_flush).
 */
int attn_decode_dense(const qkv_cache* cache, int loop, const uint16_t* q, const uint16_t* k_new,
                      const uint16_t* v_new, float sm_scale, uint16_t* o, float* o_f32, float* scores,
                      int ld_scores, float* lse, const qkv_flush* flush, void* ws, size_t ws_bytes,
                      void* stream);

/*
 * attn_decode_dense_noalloc - attn_decode_dense without a workspace argument or a tail
 * flush, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, outputs and kernels as
 * attn_decode_dense; the split partials go to a fixed device array inside the library,
 * QKV_NOALLOC_SCRATCH_BYTES (4 MiB) per GPU, held from the first call on a GPU until the
 * process ends.  The call allocates nothing.
 *   Returns QKV_EWORKSPACE (nothing queued) when the partials of this shape, i.e. the
 *   workspace attn_decode_dense would need for the current n_ctx, exceed that size (about
 *   8000 (split, sequence, head) partials at head_dim 128).
 *   Every call on one GPU shares that GPU's array: calls that overlap in time on one GPU
 *   race (the array needs no clearing: each call writes every partial it reads).
 */
int attn_decode_dense_noalloc(const qkv_cache* cache, int loop, const uint16_t* q, const uint16_t* k_new,
                              const uint16_t* v_new, float sm_scale, uint16_t* o, float* o_f32, float* scores,
                              int ld_scores, float* lse, void* stream);

/*
 * select_columns - top-k columns of each (sequence, head) under the distribution
 * exp(scores - lse) [project page STEP 02; PyPI Configuration: 10% key retention].
 *   Order: fp32 score descending, ties to the lower index (+0 and -0 are equal).  Scores
 *   should not be NaN; a NaN orders by its bit pattern (a positive NaN above +inf).
 *   0 <= k <= n (k == n takes every column); n <= ld_scores.  Writes k entries per
 *   (sequence, head):
 *   idx    device int32 [batch][heads][k]: selected columns, ascending.
 *   p_sel  device fp32 [batch][heads][k]: exp(scores[idx] - lse).
 *   mass   device fp32 [batch][heads]: sum of p_sel (cached mass m).
 */
int select_columns(const float* scores, int ld_scores, const float* lse, int batch, int heads,
                   int n, int k, int32_t* idx, float* p_sel, float* mass,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * select_tokens - the next loop's active tokens [explainer section 3, cross-loop
 * token-sparse updates: after the dense loops, each loop ranks the tokens updated in the
 * preceding loop by their normalized hidden-state change and keeps a top-k subset, so the
 * active sets nest; project page STEP 01: only active tokens write new K/V].
 *   score[t] = ||h_cur[t] - h_prev[t]||_2 / ||h_prev[t]||_2 (fp32 sums in a fixed order)
 *   for t in the preceding active set, -inf elsewhere (a zero previous state scores +inf
 *   for a nonzero change, 0 otherwise); the kept tokens are the top min(k, |set|) scores,
 *   fp32 descending, ties to the lower index, written ascending.
 *   h_cur, h_prev  device bf16 [batch][ld_tok][dm]: the preceding loop's output and input
 *            hidden states of each token (ld_tok >= n; dm a positive multiple of 8).
 *   act_prev, n_act_prev  device int32 [batch][ld_act] / [batch]: the preceding loop's
 *            active tokens, ascending, each in [0, n); both NULL when every token was
 *            active (a dense loop).  1 <= ld_act <= n.
 *   k        1..n: tokens to keep per sequence.
 *   split    act_out entries below this position are counted in n_before (e.g. the body
 *            length, so that the body part can be passed to kv_encode_loop as it is).
 *   score    device fp32 [batch][n], written.
 *   act_out  device int32 [batch][k]: the kept tokens, ascending, in the first
 *            n_act_out[b] entries (the rest is unspecified).
 *   n_act_out, n_before  device int32 [batch] (n_before may be NULL).
 *   ws       device workspace of at least qkv_token_workspace_bytes(batch, k) bytes.
 */
int select_tokens(const uint16_t* h_cur, const uint16_t* h_prev, int ld_tok, int batch, int n, int dm,
                  const int32_t* act_prev, const int32_t* n_act_prev, int ld_act, int k, int split, float* score,
                  int32_t* act_out, int32_t* n_act_out, int32_t* n_before, void* ws, size_t ws_bytes,
                  void* stream);

/* Workspace bytes select_tokens needs for `batch` sequences keeping up to k tokens. */
size_t qkv_token_workspace_bytes(int batch, int k);

/*
 * attn_decode_sparse - sparse loop `loop` (>= 2): recompute only the selected columns and
 * correct the previous loop's output [project page STEP 02; explainer section 3]:
 *   s_j = sm_scale * q . khat^(loop)_j for j in S, alpha = softmax over S of s,
 *   o = o_prev + sum_{j in S} (m * alpha_j * vhat^(loop)_j - p_sel_j * vhat^(loop-1)_j),
 *   scores[j] <- lse + log(m) + s_j - log sum_{i in S} exp(s_i)   for j in S (in place),
 * so the selected columns keep their cached mass m.  Other scores and lse are unchanged.
 *   idx, p_sel, mass as written by select_columns; k entries per (sequence, head),
 *   0 <= k <= n_ctx (k == 0: o = o_prev).
 *   o_prev   device fp32 [batch][heads][head_dim]: previous loop's output (full precision).
 *   lse      device fp32 [batch][heads]: the lse the selection used.
 *   scores   as for attn_decode_dense, updated in place; or NULL when no later selection
 *            reads them (the splice is then not stored, ld_scores ignored).
 *   k_new, v_new  as for attn_decode_dense: loop `loop`'s row of the newest position,
 *            stored in the loop's tail and used for that column if it is selected (its
 *            loop-(loop-1) value is read from that loop's tail, written by its own call).
 *   flush    NULL, or this loop's part of the next step's tail flush (see qkv_flush).
 */
int attn_decode_sparse(const qkv_cache* cache, int loop, const uint16_t* q, const uint16_t* k_new,
                       const uint16_t* v_new, float sm_scale,
                       const int32_t* idx, const float* p_sel, const float* mass, int k,
                       const float* o_prev, const float* lse, float* scores, int ld_scores,
                       uint16_t* o, float* o_f32, const qkv_flush* flush, void* ws, size_t ws_bytes,
                       void* stream);

/*
 * kv_gather_rows - compact copies of selected rows [project page, The Method, after STEP 03:
 * selected tokens and keys gathered into compact, compute-friendly buffers].
 *   src      device bf16 [batch][heads][ld_src][head_dim] (head_dim 64 or 128).
 *   idx      device int32 [batch][n_idx] (idx_per_head 0: the same rows for every head) or
 *            [batch][heads][n_idx] (idx_per_head 1); an index outside [0, ld_src) copies zeros.
 *   dst      transpose 0: device bf16 [batch][heads][n_idx][head_dim], row i = src row idx[i];
 *            transpose 1: device bf16 [batch][heads][head_dim][ld_t], ld_t = n_idx rounded up
 *            to a multiple of 32, element [c][i] = src[idx[i]][c], zero for i >= n_idx
 *            (the value layout attn_prefill_sparse takes).
 */
int kv_gather_rows(const uint16_t* src, int batch, int heads, int ld_src, int head_dim, const int32_t* idx, int n_idx,
                   int idx_per_head, int transpose, uint16_t* dst, void* stream);

/*
 * attn_prefill_sparse - prefill-side sparse loop r over compact buffers [project page, The
 * Method, after STEP 03: selected tokens and keys in compact buffers, regular GEMMs; STEP 02
 * and explainer section 3: the rank-K correction of loop r-1's output that keeps the cached
 * mass].  For each active query row i and the selected columns j at or before its position:
 *   p_ij = exp(sm q_prev_i . k_prev_j - lse_prev_i),  m_i = sum_j p_ij,
 *   alpha_ij = softmax_j(sm q_i . k_j),
 *   o_i = o_prev_i + sum_j (m_i alpha_ij v_j - p_ij v_prev_j)   (no column: o_prev_i).
 * bf16 MFMA products with fp32 accumulation.
 *   q, q_prev   device bf16 [batch][heads][n_q][head_dim]: loop r's and loop r-1's queries of
 *               the active tokens (kv_gather_rows of the full query rows).
 *   q_pos       device int32 [batch][n_q]: the active tokens' positions, ascending.
 *   lse_prev    device fp32 [batch][heads][n_q]: loop r-1's log-sum-exp of each active row.
 *   o_prev      device fp32 [batch][heads][n_q][head_dim]: loop r-1's output of those rows.
 *   k, k_prev   device bf16 [batch][heads][n_c][head_dim]: the selected columns' keys.
 *   v_t, v_prev_t  device bf16 [batch][heads][head_dim][ld_t]: their values, transposed
 *               (kv_gather_rows with transpose 1; ld_t = n_c rounded up to 32, zero-filled).
 *   c_pos       device int32 [batch][heads][n_c]: the selected columns' positions, ascending.
 *   n_c         0..: selected columns per head (0: o = o_prev).
 *   o_f32       device fp32 [batch][heads][n_q][head_dim]; o (bf16, same shape) may be NULL;
 *   mass        device fp32 [batch][heads][n_q] (m_i) or NULL.
 */
int attn_prefill_sparse(int batch, int heads, int head_dim, const uint16_t* q, const uint16_t* q_prev,
                        const int32_t* q_pos, int n_q, const float* lse_prev, const float* o_prev, const uint16_t* k,
                        const uint16_t* k_prev, const uint16_t* v_t, const uint16_t* v_prev_t, const int32_t* c_pos,
                        int n_c, float sm_scale, float* o_f32, uint16_t* o, float* mass, void* stream);

/*
 * qkv_export_plane - unpacks slots [0, n_slots) of loop `loop`'s plane for sequence b, head
 * h into plain arrays, so that a test can compare a plane's logical content with a
 * reference without decoding the packed layout above (test and inspection use; not on
 * the decode path).  All outputs are device memory owned by the caller:
 *   k_codes, v_codes  uint8 [n_slots][head_dim], one code per byte;
 *   k_scale, k_zero   fp32 [ceil(n_slots / 64)][head_dim] (one key group per block);
 *   v_scale, v_zero   fp32 [n_slots][head_dim / 64].
 * 1 <= n_slots <= the plane's n_blocks * 64.  Asynchronous on `stream`.
 */
int qkv_export_plane(const qkv_cache* cache, int loop, int b, int h, int n_slots, uint8_t* k_codes,
                     uint8_t* v_codes, float* k_scale, float* k_zero, float* v_scale, float* v_zero,
                     void* stream);

/*
 * qkv_stream_read - bandwidth reference, not part of the attention path: reads n_bytes from
 * src with a plain streaming kernel (QKV_STREAM_READ_GROUPS workgroups of 256 lanes, 8
 * 16-byte loads per lane in flight), so that the readers' rates can be set beside what a
 * read with nothing else to do reaches on the same device.
 *   src   device memory, 16-byte aligned; n_bytes > 0, a multiple of 16.
 *   sink  device uint32 [QKV_STREAM_READ_GROUPS], 16-byte aligned, caller-owned: workgroup g
 *         stores the XOR of every 32-bit word it read, where it reads the 16-byte words
 *         w with (w / 2048) % QKV_STREAM_READ_GROUPS == g.
 * Asynchronous on `stream`.  QKV_EINVAL on a bad argument (nothing launched).
 */
#define QKV_STREAM_READ_GROUPS 2048
int qkv_stream_read(const void* src, size_t n_bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QKV_ATTN_H */
