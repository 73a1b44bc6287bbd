/*
 * trimode.h -- C-ABI of libtrimode.so, the MI355X (gfx950) decode step of a
 * tri-mode language model: autoregressive (AR), block diffusion and linear
 * self-speculation served by one checkpoint.
 *
 * Sources (public write-ups of Nemotron-Labs-Diffusion):
 *   [Notes]  "Nemotron-Labs-Diffusion 技术报告：统一 AR、Diffusion 与 Self-Speculation
 *            的三模式语言模型" (ranhao.site technical notes), sections 3-7.
 *   [Digest] "Nemotron-Labs-Diffusion: A Tri-Mode Language Model Unifying
 *            Autoregressive, Diffusion, and Self-Speculation Decoding" (r9-hu
 *            paper digest), section Method.
 *   [Blog]   "Nemotron-Labs 扩散语言模型实现光速级文本生成" (shilu.ai translation of
 *            the Hugging Face blog), sections on the three generation modes and
 *            on deployment through SGLang.
 *
 * Conventions for every function:
 *   - Returns an int status: TRI_OK (0) or a negative TRI_E* code.  Nothing
 *     throws or aborts.  tri_last_error() gives a message for the calling thread.
 *   - A call that fails validation changes no state.
 *   - The library never allocates device memory.  Weights, the session
 *     workspace (KV cache and scratch) and every kernel operand are caller-owned
 *     device memory (e.g. PyTorch tensors); `stream` is a hipStream_t passed as
 *     void* (NULL = the default stream).
 *   - "device" pointers must be device memory of the current HIP device; "host"
 *     pointers are ordinary host memory.
 *   - bf16 data is stored as raw 16-bit bfloat16 (round-to-nearest-even).
 */
#ifndef TRIMODE_H
#define TRIMODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  TRI_OK = 0,
  TRI_EINVAL = -1,     /* bad argument (shape, pointer, mode, threshold ...) */
  TRI_ECAPACITY = -2,  /* a KV cache, row or workspace limit would be exceeded */
  TRI_ESTATE = -3,     /* the call does not fit the session state */
  TRI_EHIP = -4,       /* a HIP runtime call failed */
  TRI_ENUMERIC = -5    /* non-finite logits/confidence met while sampling */
};

/* Decoding modes: one checkpoint, three modes chosen by one setting
 * [Blog, deployment section; Notes §5]. */
enum { TRI_AR = 0, TRI_DIFFUSION = 1, TRI_SELFSPEC = 2, TRI_QUADSPEC = 3 };

/* Storage types: weights, activations fed to GEMMs, queries and the KV cache.
 * Accumulation, softmax, the residual stream and logits are always float32. */
enum { TRI_F32 = 0, TRI_BF16 = 1 };
/* block_causal_attn only: bf16 q/k/out with the V cache in the fp16 form a
 * bf16 session keeps (each bf16 value converted to IEEE half; exact for
 * 6.1e-5 <= |v| <= 65504, half-precision subnormals below). */
enum { TRI_BF16_V16 = 2 };

/* Decoder shape.  The embedding has vocab+1 rows; token id `vocab` is [MASK]
 * (the block's initial state in diffusion mode [Notes §5.2]).  lm_head has
 * `vocab` rows, so [MASK] is never predicted. */
typedef struct tri_model_desc {
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim, d_ffn, vocab;
  float rope_base; /* rotate-half RoPE base, e.g. 10000 */
  float rms_eps;   /* RMSNorm epsilon, e.g. 1e-6 */
  int32_t dtype;   /* TRI_F32 or TRI_BF16 */
  int32_t lora_rank; /* 0 = no adapter; else rank of the draft-only o_proj LoRA */
} tri_model_desc;

/* Per-sequence result of one tri_decode_step. */
typedef struct tri_seq_stats {
  int32_t n_committed; /* tokens committed by this step */
  int32_t n_forwards;  /* forwards executed by this step */
  int32_t accept_len;  /* self-speculation: accepted drafts a in [0, k]; else -1 */
  int32_t n_flags;     /* diffusion: commits decided within 1e-6 of the threshold */
} tri_seq_stats;

typedef struct tri_model tri_model;
typedef struct tri_session tri_session;

/* Message of the last failed call on this thread ("" if none). */
const char* tri_last_error(void);

/* ------------------------------------------------------------------------
 * Model.  `weights` is a host array of n_weights device pointers in this order
 * (element type = desc->dtype unless noted; all row-major):
 *   embed [vocab+1][d]
 *   per layer l: wq [hq*hd][d], wk [hkv*hd][d], wv [hkv*hd][d], wo [d][hq*hd],
 *                w_gate [ffn][d], w_up [ffn][d], w_down [d][ffn],
 *                attn_norm [d] (float32), ffn_norm [d] (float32)
 *   final_norm [d] (float32), lm_head [vocab][d]
 *   if lora_rank > 0, per layer l: lora_a [r][hq*hd], lora_b [d][r]
 * so n_weights = 1 + 9*n_layers + 2 + (lora_rank > 0 ? 2*n_layers : 0).
 * tri_model_create copies the embedding and norm gains into model_buf (caller
 * allocated device memory of tri_model_bytes bytes, 256-byte aligned) and
 * repacks every projection matrix there in the order the GEMM kernel streams
 * it (bf16: MFMA-fragment order).  It runs on `stream` and returns after the
 * copies are done: the caller may then free the original weights; model_buf
 * must stay alive and unchanged until tri_model_destroy.  bf16 models need d,
 * hq*hd, hkv*hd, ffn and r to be multiples of 64 and head_dim == 128; float32
 * models need head_dim <= 128; d is a multiple of 4 and ffn of 16, d <= 8192.
 * ------------------------------------------------------------------------ */
int tri_model_bytes(const tri_model_desc* desc, size_t* bytes);
int tri_model_create(const tri_model_desc* desc, const void* const* weights, int n_weights,
                     void* model_buf, size_t bytes, void* stream, tri_model** out);
int tri_model_destroy(tri_model* model);

/* ------------------------------------------------------------------------
 * Session: up to max_batch independent sequences, each with a KV cache of
 * max_ctx positions; a forward carries at most max_rows rows in total.
 * tri_session_bytes gives the size of the workspace (device memory, caller
 * allocated, >= 256-byte aligned) that tri_session_create carves into the KV
 * caches and scratch buffers.  The session launches everything on `stream`.
 * KV cache layout (per layer, per sequence): K [hkv][ctx][hd], V transposed
 * [hkv][hd][ctx], ctx = max_ctx rounded up to a multiple of 64.  bf16 models
 * store K as bf16 and V as the fp16 the attention multiplies: each value
 * rounded to bf16, then converted to fp16 with saturation at +-65504.
 * ------------------------------------------------------------------------ */
int tri_session_bytes(const tri_model* model, int max_batch, int max_ctx, int max_rows,
                      size_t* bytes);
int tri_session_create(const tri_model* model, int max_batch, int max_ctx, int max_rows,
                       void* workspace, size_t bytes, void* stream, tri_session** out);
int tri_session_destroy(tri_session* session);

/* Reset sequence `seq` to the prompt tokens[0..n) (host array, ids < vocab):
 * runs tokens[0..n-1) as causal rows into the cache and leaves tokens[n-1]
 * pending (its K/V is computed by the next forward).  Synchronous. */
int tri_prefill(tri_session* session, int seq, const int32_t* tokens, int n);

/* One decode step for every prefilled sequence, in lockstep:
 *   TRI_AR:        one forward over the pending tokens; commits the greedy
 *                  next token [Notes §5.1].  `block` and `threshold` ignored.
 *   TRI_DIFFUSION: fills one block of `block` positions starting as [MASK],
 *                  predicting in place; every forward commits the masked
 *                  positions whose max-softmax confidence is > threshold, or the
 *                  single most confident one if none is (lowest position on
 *                  ties) [Notes §5.2; Blog, FastDiffuser].  threshold in [0, 1].
 *   TRI_SELFSPEC:  one round: a draft forward (pending tokens + `block` [MASK]
 *                  rows, LoRA on the mask rows if enabled) and a causal verify
 *                  forward over the k = block drafts; commits the longest
 *                  matching prefix plus the AR token after it, 1..k+1 tokens,
 *                  lossless against greedy AR [Notes §5.3; Digest, Method].
 *   TRI_QUADSPEC:  one round of quadratic self-speculation [Notes §8.1; Blog,
 *                  performance highlights], one forward: the pending tokens
 *                  and the n drafts carried from the previous round as causal
 *                  rows (they verify the drafts: accept length a), plus for
 *                  every b = 0..n a block of k+1 = block+1 [MASK] rows at
 *                  L+b..L+b+k that sees the clean prefix [0, L+b) and itself
 *                  (LoRA rows); commits the a+1 verified tokens (lossless
 *                  against greedy AR) and carries block a's next k drafts.
 *                  n = 0 on the first round and after any other step,
 *                  prefill, kv_append or kv_rollback of the sequence.  Needs
 *                  block <= 63 and pending + n + (n+1)(block+1) rows per
 *                  sequence within max_rows; out_stats counts one forward.
 * block in [1, 64].  out_tokens: host [batch][block+1], the committed tokens
 * of each sequence, -1 padded.  out_stats: host [batch] (may be NULL).
 * Synchronous (returns after the step's results are on the host). */
int tri_decode_step(tri_session* session, int mode, int block, float threshold,
                    int32_t* out_tokens, tri_seq_stats* out_stats);

/* One mixed step: AR and self-speculation sequences share both forwards of a
 * round.  The pages let one checkpoint serve AR at high concurrency and
 * self-speculation at low [Notes §2 mode table and §11; Digest,
 * Limitations]; a mixed step lets the two coexist in one batch.
 * modes: host [max_batch], per sequence TRI_AR, TRI_SELFSPEC, or < 0 to leave
 * the sequence out of this step.  Both forwards carry every stepped sequence:
 *   TRI_SELFSPEC: the round of tri_decode_step (draft + verify, 1..k+1 tokens,
 *                 n_forwards 2, accept_len a);
 *   TRI_AR:       the pending rows in the first forward, the token it commits
 *                 as one causal row in the second: 2 greedy tokens (n_forwards
 *                 2, accept_len -1).
 * Each sequence's tokens are those of the same mode run alone (lossless:
 * the greedy AR continuation either way).  block in [1, 64]; out_tokens host
 * [max_batch][block+1], -1 padded; out_stats host [max_batch] or NULL.
 * Errors: TRI_EINVAL for a mode other than these; TRI_ESTATE for a stepped
 * sequence that is not prefilled, or for no stepped sequence; TRI_ECAPACITY when
 * a sequence would pass max_ctx (AR needs L+2, self-speculation L+block+1) or
 * either forward would pass max_rows.  Synchronous. */
int tri_decode_step_mixed(tri_session* session, const int32_t* modes, int block,
                          int32_t* out_tokens, tri_seq_stats* out_stats);

/* Speed-of-light analysis of the next block of every prefilled sequence
 * [Notes §7; Abstract]: how few forwards an ideal sampler would need to reach
 * the block that serial denoising converges to.
 *   1. Serial denoising: the diffusion block at threshold 1, one commit per
 *      forward (the most confident masked position, lowest on ties).  It
 *      fixes the target block and the serial order of its positions.
 *   2. Parallel pass from the same state: each forward commits every masked
 *      position whose greedy token already equals its target; when none does,
 *      the next position of the serial order.  Every forward commits >= 1.
 * The sequences end as after the serial block (as tri_decode_step in
 * TRI_DIFFUSION mode at threshold 1 leaves them), so calls chain over a
 * generation.  block in [1, 64].  Host outputs, [max_batch][block] and
 * [max_batch], -1 for sequences not prefilled:
 *   out_target   the target tokens;
 *   out_order    out_order[j] = the position committed by serial forward j;
 *   out_step     the parallel forward (0-based) at which each position commits;
 *   out_forwards the parallel pass's forward count (block / it = SOL tokens
 *                per forward; the serial pass always takes block forwards).
 * Errors: TRI_ESTATE (no prefilled sequence, no pending token), TRI_ECAPACITY
 * (L + block > max_ctx, or more than max_rows rows), TRI_ENUMERIC (non-finite
 * logits; the sequences are then left as before the call).  Synchronous. */
int tri_sol_block(tri_session* session, int block, int32_t* out_target, int32_t* out_order,
                  int32_t* out_step, int32_t* out_forwards);

/* Mode choice by concurrency for one mixed step (host only, no device work).
 * Chooses per sequence TRI_AR or TRI_SELFSPEC to maximise the step's expected
 * committed tokens per millisecond:
 *   tokens = 2 per AR sequence + expected[j] per self-speculation sequence;
 *   time   = t(rows of the first forward) + t(rows of the second), where the
 *            first forward has pending[j] rows per sequence (+ block for
 *            self-speculation) and the second 1 (AR) or block rows;
 *   t(r)   = the measured forward time: linear between the points
 *            (grid_rows[i], grid_ms[i]), grid_ms[0] below the first point, the
 *            line through the last two points beyond the last.
 * grid_rows: host [n_grid], strictly increasing; grid_ms: host [n_grid] > 0.
 * expected: host [n_seq], each sequence's expected tokens per self-speculation
 * round, in [1, block+1] (e.g. a running mean of accept_len + 1).  pending:
 * host [n_seq] rows >= 1, or NULL for one each.  modes: host [n_seq] out.
 * Ties go to fewer self-speculation sequences, then to lower indices.
 * TRI_EINVAL on a bad grid, block or expected value; nothing is written then. */
int tri_choose_modes(const int32_t* grid_rows, const double* grid_ms, int n_grid, int n_seq,
                     const double* expected, const int32_t* pending, int block, int32_t* modes);

/* Enable/disable the draft-only o_proj LoRA (needs lora_rank > 0).  It only
 * ever applies to the [MASK] rows of self-speculation draft forwards: the AR
 * verifier is frozen [Notes §6]. */
int tri_set_lora(tri_session* session, int enabled);

/* KV bookkeeping of sequence `seq`.  The cache holds causal K/V for positions
 * [0, kv_len).  kv_append(n) adopts n more rows that a forward has written as
 * clean (causal) rows: TRI_ESTATE if kv_len+n would pass the committed tokens or
 * the rows written, TRI_ECAPACITY past max_ctx.  kv_rollback(n) forgets the
 * last n rows (their tokens become pending again): TRI_ESTATE if n > kv_len.
 * Zero-copy: only the length moves (readings of [Notes §3.2]: prefix KV reuse). */
int kv_append(tri_session* session, int seq, int n);
int kv_rollback(tri_session* session, int seq, int n);

/* Committed length L and kv_len of `seq`, and (if tokens != NULL, host array of
 * capacity cap) the committed tokens. */
int tri_get_state(tri_session* session, int seq, int* committed, int* kv_len,
                  int32_t* tokens, int cap);

/* One forward over caller-given rows (test hook for teacher-forced parity).
 * Host arrays of n_rows: row_seq, row_tok (id <= vocab), row_pos, row_hi
 * (exclusive key limit, pos < hi <= max_ctx), row_lora (0/1).  Rows of one
 * sequence must be contiguous.  Every row's K/V is written to its cache slot;
 * kv_len is not changed.  logits: device float32 [n_rows][vocab] or NULL;
 * out_tok / out_conf: host [n_rows] greedy token and confidence, or NULL. */
int tri_forward(tri_session* session, int n_rows, const int32_t* row_seq,
                const int32_t* row_tok, const int32_t* row_pos, const int32_t* row_hi,
                const int32_t* row_lora, float* logits, int32_t* out_tok, float* out_conf);

/* Bytes of weights plus KV a forward over `rows_per_seq` rows per sequence at
 * the current state streams (the algorithmic HBM bytes used for roofline). */
int tri_forward_bytes(tri_session* session, int rows_per_seq, double* bytes);

/* ------------------------------------------------------------------------
 * Test and measurement hooks.
 * ------------------------------------------------------------------------ */

/* Record every forward of the session (rows and, when an lm_head ran, its
 * float32 logits) on the host, for teacher-forced replay through a reference.
 * Enabling or disabling clears the record.  Adds a synchronisation per forward. */
int tri_set_trace(tri_session* session, int enabled);
int tri_trace_count(tri_session* session, int* n);
/* Forward i of the record: n_rows is always set; the host arrays (capacity
 * cap_rows rows; logits cap_rows*vocab floats, may be NULL) are filled only if
 * cap_rows >= n_rows.  has_logits = 0 for forwards without an lm_head. */
int tri_trace_get(tri_session* session, int i, int* n_rows, int32_t* seq, int32_t* tok, int32_t* pos,
                  int32_t* hi, int32_t* lora, float* logits, int cap_rows, int* has_logits);

/* Controlled-acceptance replay of self-speculation: while a_star >= 0, every
 * draft forward of `seq` still runs in full, but its drafts are replaced by
 * ref[L..L+k) (the reference continuation by absolute position, e.g. an
 * earlier greedy AR run) with ref[L+a_star] changed to force a mismatch there.
 * a_star < 0 switches the replay off.  ref is copied (host, n_ref ids). */
int tri_set_draft_override(tri_session* session, int seq, const int32_t* ref, int n_ref, int a_star);

/* Controlled commit rate of diffusion mode: while set (n > 0), the t-th
 * forward of each diffusion block of `seq` commits the min(counts[t % n],
 * remaining) most confident masked positions (lowest position on ties) with
 * their greedy tokens, in place of the threshold rule; every forward still
 * runs in full.  A stand-in for a trained sampler's commit rate (the pages
 * report about 2.6x TPF for diffusion mode, [Blog] performance highlights)
 * on random-init weights, whose confidences never pass a threshold.
 * counts: host, n entries >= 1, copied; n = 0 switches it off.  tri_prefill
 * of the sequence switches it off too.  TRI_EINVAL on a bad schedule. */
int tri_set_commit_schedule(tri_session* session, int seq, const int32_t* counts, int n);

/* Time every launch of one kernel class with HIP events on the session stream:
 * 0 gate/up GEMM, 1 down GEMM, 2 QKV GEMM, 3 o_proj GEMM, 4 lm_head GEMM,
 * 5 attention (+ split combine), 6 whole forward; -1 switches timing off.
 * tri_profile resets the totals; tri_profile_read synchronises the stream and
 * returns the summed milliseconds and the number of timed launches. */
int tri_profile(tri_session* session, int kernel_class);
int tri_profile_read(tri_session* session, double* total_ms, int* launches);

/* ------------------------------------------------------------------------
 * Kernel-level entry points.  Device pointers, asynchronous on `stream`.
 * ------------------------------------------------------------------------ */

/* Block-causal grouped-query attention [Notes §3.2; Digest, Method]: every
 * query row r attends to the keys [0, row_hi[r]) of its sequence; clean rows
 * use hi = pos+1 (causal), the rows of a block [L, L+B) use hi = L+B
 * (bidirectional inside the block).  Query head h reads kv head
 * h / (hq/hkv).  softmax(q.k * scale) in float32, output = sum p v.
 *   q        [rows][hq][hd]              dtype
 *   k_cache  [n_seq][hkv][ctx][hd]       dtype
 *   v_cache  [n_seq][hkv][hd][ctx]       dtype (transposed)
 *   seq_start device int32 [n_seq+1]: rows of sequence s are [seq_start[s], seq_start[s+1])
 *   row_hi    device int32 [rows], 1 <= hi <= ctx
 *   out      [rows][hq][hd]              dtype
 *   dtype    TRI_F32, TRI_BF16, or TRI_BF16_V16 (v_cache holds IEEE-half bits;
 *            the session's own cache form)
 * ctx % 64 == 0.  bf16 needs hd == 128, float32 hd <= 128.  max_rows_per_seq
 * and max_hi bound the launch grid (host values >= the true maxima).
 * kv_split: keys per split-KV work unit, a multiple of 64 (0 = pick).  The
 * result of a row depends only on its q, its keys and kv_split.
 * ws: device workspace of at least block_causal_attn_ws_bytes(...) bytes. */
int block_causal_attn_ws_bytes(int rows, int hq, int hd, int max_hi, int kv_split, size_t* bytes);
int block_causal_attn(const void* q, const void* k_cache, const void* v_cache, int n_seq,
                      const int32_t* seq_start, const int32_t* row_hi, int rows,
                      int max_rows_per_seq, int max_hi, int hq, int hkv, int hd, int ctx,
                      float scale, int dtype, int kv_split, void* out, void* ws,
                      size_t ws_bytes, void* stream);

/* block_causal_attn for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, with the split partials in a
 * static device scratch of 32 MiB that the library holds on every GPU it
 * runs on.  No workspace argument; calls no hipMalloc/hipFree.  kv_split 0
 * picks the split as block_causal_attn does.  TRI_ECAPACITY when the
 * partials (block_causal_attn_ws_bytes) exceed 32 MiB.  Calls on one GPU
 * share its scratch: calls that overlap on one GPU (other streams, other
 * threads) race and must be serialised by the caller. */
int block_causal_attn_noalloc(const void* q, const void* k_cache, const void* v_cache, int n_seq,
                              const int32_t* seq_start, const int32_t* row_hi, int rows,
                              int max_rows_per_seq, int max_hi, int hq, int hkv, int hd, int ctx,
                              float scale, int dtype, int kv_split, void* out, void* stream);

/* Vocabulary reduction and commit decision [Notes §5.2, §5.3; Blog, FastDiffuser].
 * For every row with row_kind != 0: out_tok = argmax of logits (lowest id on
 * ties), out_conf = max softmax probability = 1/sum_j exp(l_j - max).
 *   row_kind 0: ignored; 1: greedy row, always committed (out_commit = 1);
 *            2: masked block position, eligible; 3: block position already committed.
 * Blocks: rows [block_start[b], block_start[b+1]) for b < n_blocks (device
 * int32).  In each block the eligible rows with conf > threshold are
 * committed; if none is, the eligible row with the highest confidence (lowest
 * row on ties).  out_commit[r] = 1 if committed now, else 0.
 * out_status: device int32[1], set to the number of rows with a non-finite
 * confidence (such rows are never committed).
 * logits float32 [rows][vocab]; ws >= sample_commit_ws_bytes(rows, vocab). */
int sample_commit_ws_bytes(int rows, int vocab, size_t* bytes);
int sample_commit(const float* logits, int rows, int vocab, const int32_t* row_kind,
                  const int32_t* block_start, int n_blocks, float threshold, int32_t* out_tok,
                  float* out_conf, int32_t* out_commit, int32_t* out_status, void* ws,
                  size_t ws_bytes, void* stream);

/* Self-speculation acceptance [Notes §5.3; Digest, Method]: for each of
 * `batch` sequences, a = the length of the longest prefix with
 * draft[i] == ar_tok[i] (a = k if all match); committed[b][0..a] = ar_tok[b][0..a],
 * committed[b][a+1..k] = -1; accept_len[b] = a; kv_len[b] += a (the verify rows
 * of the a accepted drafts stay in the cache, the other k - a are rolled back).
 *   draft [batch][k], ar_tok [batch][k+1], committed [batch][k+1], all device int32. */
int verify_accept(const int32_t* draft, const int32_t* ar_tok, int batch, int k,
                  int32_t* accept_len, int32_t* committed, int32_t* kv_len, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* TRIMODE_H */
