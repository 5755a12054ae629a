/*
 * dbd.h -- C ABI of libdbd, one denoise round of block-diffusion decoding on
 * an AMD Instinct MI355X (gfx950).
 *
 * A round (JetEngine README, "Block Diffusion Decoding"; JetEngine developer
 * notes (CLAUDE.md), "Entry Point & Engine": step() runs the denoise batch,
 * then postprocesses the logits) takes every active sequence's block of
 * block_length tokens through three steps:
 *   1. block-diffusion attention over the sequence's paged KV prefix and its
 *      own block (bidirectional inside the block), grouped-query heads;
 *   2. the selective LM head: only masked positions of DENOISING sequences
 *      are projected to the vocabulary, fused with the softmax, giving each
 *      such position its greedy token and confidence; logits never reach
 *      device memory;
 *   3. threshold remasking (low_confidence_dynamic), then the compact list
 *      of still-masked rows that the next round's LM head projects.
 *
 * Conventions (every entry point):
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates or frees on these calls, never synchronises and never
 *     reads device data from the host.  Work is enqueued on `stream` (a
 *     hipStream_t passed as void*; NULL = the null stream) in stream order.
 *   - Scalar arguments and pointer alignment are validated on the host
 *     before anything is enqueued; a non-OK status means nothing was
 *     enqueued, and dbd_last_error() returns a message (thread-local).
 *     Device-resident data (page ids, prefix lengths, row lists, counts) is
 *     trusted on these calls; dbd_validate_inputs() checks host copies.
 *   - bf16 tensors are passed as raw 16-bit patterns (dbd_bf16).
 *   - No exception crosses the ABI.
 */
#ifndef DBD_H
#define DBD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DBD_ABI_VERSION 4

typedef uint16_t dbd_bf16;

typedef enum {
  DBD_OK = 0,
  DBD_ERR_INVALID_ARG = 1, /* a scalar or pointer failed host validation   */
  DBD_ERR_UNSUPPORTED = 2, /* valid but outside what the kernels support   */
  DBD_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required   */
  DBD_ERR_HIP = 4          /* a HIP runtime call failed                    */
} dbd_status;

/* Sequence states, in the order of the scheduler's state machine (JetEngine
 * developer notes, "Scheduler": WAITING -> PREFILLING -> DENOISING ->
 * SAVING -> FINISHED).  A round reads DENOISING and writes SAVING. */
enum { DBD_WAITING = 0, DBD_PREFILLING = 1, DBD_DENOISING = 2,
       DBD_SAVING = 3, DBD_FINISHED = 4 };

/* dbd_remask_commit flags */
#define DBD_FALLBACK_LEFTMOST 1u /* fallback commits the leftmost masked position */
#define DBD_COMPACT_ONLY 2u      /* no commit: only rebuild the row list           */

/* Commit rules: the remasking strategies the JetEngine developer notes list
 * ("Remasking Strategies"); see dbd_remask_commit_rule. */
enum { DBD_RULE_LOW_CONF_DYNAMIC = 0, DBD_RULE_LOW_CONF_STATIC = 1,
       DBD_RULE_SEQUENTIAL = 2, DBD_RULE_ENTROPY_BOUNDED = 3 };

/* ------------------------------------------------------------------------
 * dbd_attn_paged -- block-diffusion attention over a paged KV cache.
 *
 * Defined by the denoise step's attention pattern (JetEngine developer
 * notes, "ModelRunner": prefill and denoise use different attention
 * patterns; "Layers": paged-KV denoise attention) over the paged cache with
 * per-sequence block tables (README architecture tree, "Paged KV Cache";
 * developer notes, "Chain Mechanism": positions/block tables).
 *
 * For sequence s, query head h (kv head g = h / (Hq/Hkv)), block position i:
 *   keys   = the L_s = prefix_len[s] prefix tokens, token j in page
 *            page_table[s*max_pages_per_seq + j/page_size] at slot
 *            j % page_size, followed by the B block tokens (k_blk);
 *   out    = softmax(q . keys^T * scale) . values, no mask inside the block.
 *
 * Layouts (row-major, bf16 unless noted):
 *   q, out        [S][B][Hq][D]
 *   k_blk, v_blk  [S][B][Hkv][D]
 *   k_cache,
 *   v_cache       [num_pages][Hkv][page_size][D]
 *   page_table    int32 [S][max_pages_per_seq]; entries past a prefix's
 *                 last page are not read
 *   prefix_len    int32 [S], 0 <= L_s <= max_pages_per_seq*page_size
 * softmax_scale <= 0 selects 1/sqrt(D).  Slots of a prefix's last page past
 * its end are never used (they may hold anything, NaN included).
 * Requirements: 1 <= B <= 64, D in {64,128}, Hq % Hkv == 0,
 * page_size % 16 == 0, all pointers 16-byte aligned.
 * workspace: at least dbd_attn_workspace_size(...) bytes of device memory,
 * 256-byte aligned; contents on entry are ignored.
 * ---------------------------------------------------------------------- */
dbd_status dbd_attn_paged(int S, int B, int Hq, int Hkv, int D, int page_size,
                          int max_pages_per_seq,
                          const dbd_bf16* q, const dbd_bf16* k_blk,
                          const dbd_bf16* v_blk, const dbd_bf16* k_cache,
                          const dbd_bf16* v_cache, const int32_t* page_table,
                          const int32_t* prefix_len, float softmax_scale,
                          dbd_bf16* out, void* workspace,
                          size_t workspace_bytes, void* stream);

size_t dbd_attn_workspace_size(int S, int B, int Hq, int Hkv, int D,
                               int page_size, int max_pages_per_seq);

/* ------------------------------------------------------------------------
 * dbd_attn_paged_save -- dbd_attn_paged for a batch that holds SAVING
 * sequences: the same attention for every sequence, and, in the same
 * kernel, the block keys and values of every sequence whose seq_state is
 * DBD_SAVING written into its pages.
 *
 * Defined by the SAVING forward (JetEngine developer notes, "Important
 * Patterns": a finished block runs one more forward that writes its final
 * representations into the KV cache, and skipping it corrupts the cache;
 * "Optimization History": the FA3 kernel writes the cache and attends in
 * one kernel) and the cache addressing of dbd_attn_paged:
 *   for s with seq_state[s] == DBD_SAVING, j < B, p = prefix_len[s] + j:
 *     k_cache[page_table[s][p / page_size]][g][p % page_size][:] = k_blk[s][j][g][:]
 *     v_cache[...same...]                                         = v_blk[s][j][g][:]
 *   for every kv head g.  prefix_len is not changed (dbd_commit_block
 *   advances it).
 * The caller assigns the pages that cover positions prefix_len[s] ..
 * prefix_len[s]+B-1 of each SAVING sequence before the call; a position
 * whose page index reaches max_pages_per_seq or whose page id lies outside
 * [0, num_pages) is not written (the kernel never writes outside the
 * cache).  The attention reads no slot at or past prefix_len, so the writes
 * do not affect this call's out.  seq_state: uint8 [S], read only.  Every
 * other argument, layout and requirement as dbd_attn_paged; workspace size
 * dbd_attn_workspace_size(...).
 * ---------------------------------------------------------------------- */
dbd_status dbd_attn_paged_save(int S, int B, int Hq, int Hkv, int D,
                               int page_size, int max_pages_per_seq,
                               int num_pages, const dbd_bf16* q,
                               const dbd_bf16* k_blk, const dbd_bf16* v_blk,
                               dbd_bf16* k_cache, dbd_bf16* v_cache,
                               const int32_t* page_table,
                               const int32_t* prefix_len,
                               const uint8_t* seq_state, float softmax_scale,
                               dbd_bf16* out, void* workspace,
                               size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * dbd_lmhead_conf -- selective LM head fused with the softmax.
 *
 * Defined by selective logits (README, "Selective Logits": the LM head runs
 * only for DENOISING sequences) restricted to masked positions (developer
 * notes, "Optimization History": sparse logits), with greedy decoding
 * (SDAR page, generate.py: greedy generation).
 *
 * For each r < *num_rows (device scalar), with row = row_index[r]
 * (row_index == NULL: row = r):
 *   l_v = sum_k hidden[row][k] * w_vocab[v][k]   (fp32 accumulation of the
 *         bf16 products; logits are never rounded to bf16 or stored),
 *   over every v != mask_token_id;
 *   argmax_tok[row] = the smallest v with the largest l_v;
 *   conf[row]       = exp(l_max - logsumexp_v l_v) = max probability.
 * Rows not listed are not written.
 * Layouts: hidden [rows][Hd] bf16 (row = s*B + position); w_vocab [V][Hd]
 * bf16 (row v is column v of W in R^{Hd x V}); row_index int32 [max_rows];
 * num_rows int32 device scalar, 0 <= *num_rows <= max_rows.
 * Requirements: Hd % 128 == 0, V >= 2, 0 <= mask_token_id < V.
 * workspace: dbd_lmhead_workspace_size(max_rows, V) bytes, 256-B aligned.
 * ---------------------------------------------------------------------- */
dbd_status dbd_lmhead_conf(int max_rows, int Hd, int V, int mask_token_id,
                           const dbd_bf16* hidden, const int32_t* row_index,
                           const int32_t* num_rows, const dbd_bf16* w_vocab,
                           int32_t* argmax_tok, float* conf, void* workspace,
                           size_t workspace_bytes, void* stream);

size_t dbd_lmhead_workspace_size(int max_rows, int V);

/* dbd_lmhead_conf plus each listed row's softmax entropy, the quantity the
 * entropy-bounded commit rule orders positions by (developer notes,
 * "Remasking Strategies": unmask by cumulative entropy budget):
 *   entropy[row] = -sum_{v != mask} p_v ln p_v   (nats, float32),
 * from the same fused pass (a running sum of e^(l-m) (l-m) merged like the
 * normaliser).  entropy: float [rows], written only at listed rows; every
 * other argument as dbd_lmhead_conf. */
dbd_status dbd_lmhead_conf_entropy(int max_rows, int Hd, int V,
                                   int mask_token_id, const dbd_bf16* hidden,
                                   const int32_t* row_index,
                                   const int32_t* num_rows,
                                   const dbd_bf16* w_vocab,
                                   int32_t* argmax_tok, float* conf,
                                   float* entropy, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* dbd_lmhead_conf with the token drawn from softmax(l / temperature)
 * instead of taken as the argmax (SamplingParams temperature, JetEngine
 * README usage examples; the scheduler's postprocess samples before the
 * remasking strategy selects, developer notes, "Scheduler").  Exact draw,
 * fused in the same pass, no logit stored:
 *   blocks: for chunk c (columns 32c..32c+31) and half h in {0,1}, the 16
 *     columns 32c + 8q + 4h + r (q, r in 0..3) other than the mask token;
 *   words: Philox4x32-10 (Salmon et al., "Parallel random numbers: as easy
 *     as 1, 2, 3") of counter (c, row, step, 0) and key (seed low word,
 *     seed high word), row = row_index[r]; half h uses word 2h for u and
 *     word 2h+1 for e, each as ((w >> 9) + 0.5) / 2^23;
 *   per block, with z = l / temperature: m_b = max z, S_b = sum exp(z-m_b),
 *     candidate = first column (increasing id) whose running sum of
 *     exp(z - m_b) reaches u*S_b, G_b = m_b + ln S_b - ln(-ln e);
 *   token[row] = the candidate of the block with the largest G_b (lower id
 *     on ties), which has probability exp(z_v) / sum exp(z);
 *   conf[row] = that token's probability at temperature 1 (softmax of l
 *     without the mask token), the value the commit rules compare.
 * entropy may be NULL (else as dbd_lmhead_conf_entropy).  step lets every
 * round draw fresh numbers from the same seed.  Requirements: as
 * dbd_lmhead_conf; temperature finite and > 0.  Top-k / top-p filtering is
 * not provided. */
dbd_status dbd_lmhead_sample(int max_rows, int Hd, int V, int mask_token_id,
                             const dbd_bf16* hidden, const int32_t* row_index,
                             const int32_t* num_rows, const dbd_bf16* w_vocab,
                             float temperature, uint64_t seed, uint32_t step,
                             int32_t* token, float* conf, float* entropy,
                             void* workspace, size_t workspace_bytes,
                             void* stream);

/* Top-k / top-p sampling, as a separate step after stored logits (the
 * developer notes, "Ruled-Out Optimizations", found a separate sampler
 * faster than a fused one; README usage examples: topk, topp).
 *
 * dbd_lmhead_logits: the LM head's fp32 logits of the listed rows,
 *   logits[r][v] = sum_k hidden[row_index[r]][k] * w_vocab[v][k] for
 *   r < *num_rows, with logits[r][mask_token_id] = -inf; other rows of the
 *   buffer are not written.  logits: float [max_rows][V].  Requirements as
 *   dbd_lmhead_conf; no workspace.
 *
 * dbd_sample_filtered: for each r < *num_rows (row = row_index[r], or r):
 *   rank the tokens other than the mask token by logits[r][v], higher first,
 *   the lower id first among equal logits; top_k > 0 keeps the first top_k;
 *   top_p < 1 then keeps the shortest leading run of those whose running
 *   sum of exp((l - m)/temperature) reaches top_p of their total (at least
 *   one token; m = the largest logit); token[row] is drawn from
 *   softmax(l/temperature) over the kept tokens by the block draw of
 *   dbd_lmhead_sample (same seed, step and Philox counters, the other
 *   tokens with zero weight), and conf[row] is its probability at
 *   temperature 1 over all tokens but the mask token.  top_k = 0 and
 *   top_p >= 1 give the draw of dbd_lmhead_sample.  Only finite logits
 *   are candidates (-inf ones are never ranked or drawn); a row with no
 *   candidate gets token = mask_token_id and conf = 0.  Requirements:
 *   temperature finite and > 0, top_k >= 0, top_p not NaN. */
dbd_status dbd_lmhead_logits(int max_rows, int Hd, int V, int mask_token_id,
                             const dbd_bf16* hidden, const int32_t* row_index,
                             const int32_t* num_rows, const dbd_bf16* w_vocab,
                             float* logits, void* stream);
dbd_status dbd_sample_filtered(int max_rows, int V, int mask_token_id,
                               const float* logits, const int32_t* row_index,
                               const int32_t* num_rows, float temperature,
                               int top_k, float top_p, uint64_t seed,
                               uint32_t step, int32_t* token, float* conf,
                               void* stream);

/* ------------------------------------------------------------------------
 * dbd_remask_commit -- threshold remask (low_confidence_dynamic) and the
 * next round's row list.
 *
 * Defined by the remasking strategy low_confidence_dynamic (developer notes,
 * "Remasking Strategies": unmask every position above the threshold, with a
 * fallback; README usage with dynamic_threshold) and the scheduler's state
 * machine (developer notes, "Scheduler").
 *
 * For each DENOISING sequence s with masked set M = {i : block_tokens[s][i]
 * == mask_token_id}:
 *   C = {i in M : conf[s*B+i] >= dynamic_threshold}  (float32 compare);
 *   if C is empty and M is not: C = {most confident i in M} (lowest i on
 *   ties), or with DBD_FALLBACK_LEFTMOST the leftmost i in M;
 *   block_tokens[s][i] = argmax_tok[s*B+i] for i in C;
 *   if no mask is left: seq_state[s] = DBD_SAVING.
 * Other states are untouched.  DBD_COMPACT_ONLY skips the commit and the
 * state change.  Then row_index_out receives s*B+i for every still-masked
 * position of every DENOISING sequence, sequence-major and position-minor,
 * and *num_rows_out their count.  num_committed (may be NULL) receives the
 * number committed per sequence.
 * Layouts: block_tokens int32 [S][B] in/out; seq_state uint8 [S] in/out;
 * conf float [S*B], argmax_tok int32 [S*B] (read only at masked positions
 * of DENOISING sequences); row_index_out int32 [S*B].
 * Requirements: 1 <= B <= 64, 1 <= S <= 8192, threshold not NaN.
 * ---------------------------------------------------------------------- */
dbd_status dbd_remask_commit(int S, int B, int mask_token_id,
                             float dynamic_threshold, uint32_t flags,
                             int32_t* block_tokens, uint8_t* seq_state,
                             const int32_t* argmax_tok, const float* conf,
                             int32_t* row_index_out, int32_t* num_rows_out,
                             int32_t* num_committed, void* stream);

/* ------------------------------------------------------------------------
 * dbd_remask_commit_rule -- dbd_remask_commit with the commit set chosen by
 * one of the remasking strategies of the developer notes ("Remasking
 * Strategies": sequential unmasks left to right, low_confidence_static the
 * top k by confidence, low_confidence_dynamic above a threshold with a
 * fallback, entropy_bounded by a cumulative entropy budget).  The notes
 * give one phrase per strategy; the readings taken, for a DENOISING
 * sequence with masked set M and k = min(max(tokens_per_step,1), |M|):
 *   DBD_RULE_LOW_CONF_DYNAMIC: as dbd_remask_commit (dynamic_threshold,
 *       flags);
 *   DBD_RULE_LOW_CONF_STATIC:  the k most confident positions of M (lower
 *       position first on equal confidence);
 *   DBD_RULE_SEQUENTIAL:       the k leftmost positions of M;
 *   DBD_RULE_ENTROPY_BOUNDED:  M in ascending entropy[s*B+i] (lower position
 *       first on ties); the longest leading run whose float32 running sum is
 *       <= eb_threshold, and at least its first position.
 * Then as dbd_remask_commit: committed positions take argmax_tok, SAVING
 * once no mask is left, the next round's row list.  entropy (float [S*B],
 * read at masked positions of DENOISING sequences) is required for
 * DBD_RULE_ENTROPY_BOUNDED and ignored otherwise.
 * Requirements: as dbd_remask_commit; rule one of DBD_RULE_*; eb_threshold
 * not NaN.
 * ---------------------------------------------------------------------- */
dbd_status dbd_remask_commit_rule(int S, int B, int mask_token_id, int rule,
                                  float dynamic_threshold,
                                  int tokens_per_step, float eb_threshold,
                                  uint32_t flags, int32_t* block_tokens,
                                  uint8_t* seq_state,
                                  const int32_t* argmax_tok, const float* conf,
                                  const float* entropy,
                                  int32_t* row_index_out,
                                  int32_t* num_rows_out,
                                  int32_t* num_committed, void* stream);

/* ------------------------------------------------------------------------
 * dbd_commit_block -- commit the blocks of SAVING sequences and rebuild the
 * row list.
 *
 * Defined by commit_block (JetEngine developer notes, "Sequence": a denoised
 * block is moved into the sequence's token stream) and the state machine
 * ("Scheduler": ... -> DENOISING -> SAVING -> FINISHED; "Chain Mechanism":
 * chains run across SAVING into the next block).  Call it after the SAVING
 * forward (dbd_attn_paged_save).  For each s with seq_state[s] == SAVING:
 *   token_stream[s][prefix_len[s] + j] = block_tokens[s][j]  for j < B and
 *       prefix_len[s] + j < stream_cap (token_stream may be NULL);
 *   prefix_len[s] += B;
 *   if end_len != NULL and prefix_len[s] >= end_len[s]:
 *       seq_state[s] = DBD_FINISHED (block_tokens[s] kept);
 *   else: block_tokens[s][:] = mask_token_id, seq_state[s] = DBD_DENOISING.
 * Other sequences are untouched.  Then, as dbd_remask_commit with
 * DBD_COMPACT_ONLY, row_index_out / *num_rows_out list every masked
 * position of every DENOISING sequence (the new blocks included).
 * Layouts: block_tokens int32 [S][B], seq_state uint8 [S], prefix_len int32
 * [S] (all in/out); token_stream int32 [S][stream_cap]; end_len int32 [S];
 * row_index_out int32 [S*B].
 * Requirements: as dbd_remask_commit; stream_cap >= 1 when token_stream is
 * given.
 * ---------------------------------------------------------------------- */
dbd_status dbd_commit_block(int S, int B, int mask_token_id,
                            int32_t* block_tokens, uint8_t* seq_state,
                            int32_t* prefix_len, int32_t* token_stream,
                            int stream_cap, const int32_t* end_len,
                            int32_t* row_index_out, int32_t* num_rows_out,
                            void* stream);

/* ------------------------------------------------------------------------
 * dbd_prefill_attn -- block-causal attention of a prefill over packed
 * prompts, with the prompts' K/V optionally stored into the paged cache.
 *
 * Defined by the prefill pattern of a block-diffusion model (JetEngine
 * developer notes, "ModelRunner": prefill and denoise use different
 * attention patterns; "Layers": block-sparse varlen attention for the
 * prefill, a store kernel for the cache; README, "Block Diffusion
 * Decoding": earlier blocks fully visible, bidirectional in the block):
 *   prompt s = rows cu_seqlens[s] .. cu_seqlens[s+1]-1 (L_s tokens);
 *   token i of prompt s, q head h (kv head g = h / (Hq/Hkv)) attends to the
 *   tokens j of prompt s with floor(j / block_length) <= floor(i /
 *   block_length);
 *   out = softmax(q . k^T * scale) . v over those keys.
 * block_length = 1 is causal attention; block_length >= L_s is full
 * attention.  With k_cache != NULL, token j of prompt s (every kv head) is
 * also written to page page_table[s][j / page_size], slot j % page_size
 * (positions past the table or page ids outside [0, num_pages) are not
 * written).
 * Layouts: q, out [T][Hq][D]; k, v [T][Hkv][D] (bf16, packed prompts);
 * cu_seqlens int32 [S+1], non-decreasing, cu_seqlens[0] = 0,
 * cu_seqlens[S] <= T; caches and page_table as dbd_attn_paged.
 * Requirements: D in {64, 128}, Hq % Hkv == 0, 128 % (Hq/Hkv) == 0,
 * block_length >= 1, T*Hkv*D*2 < 2^32, pointers 16-byte aligned.
 * workspace: dbd_prefill_workspace_size(S) bytes, 256-B aligned.
 * ---------------------------------------------------------------------- */
dbd_status dbd_prefill_attn(int S, int T, int Hq, int Hkv, int D,
                            int block_length, const dbd_bf16* q,
                            const dbd_bf16* k, const dbd_bf16* v,
                            const int32_t* cu_seqlens, float softmax_scale,
                            dbd_bf16* out, int page_size,
                            int max_pages_per_seq, int num_pages,
                            const int32_t* page_table, dbd_bf16* k_cache,
                            dbd_bf16* v_cache, void* workspace,
                            size_t workspace_bytes, void* stream);
size_t dbd_prefill_workspace_size(int S);

/* ------------------------------------------------------------------------
 * dbd_round -- one whole denoise round: dbd_attn_paged, then
 * dbd_lmhead_conf on the row list (row_index, *num_rows), then
 * dbd_remask_commit, which overwrites (row_index, *num_rows) with the next
 * round's list.  Build the first round's list with dbd_remask_commit and
 * DBD_COMPACT_ONLY.  With no model in the loop, `hidden` is an input of the
 * round (the state the model would have produced), not computed from
 * attn_out.
 * workspace: dbd_round_workspace_size(a) bytes.
 * ---------------------------------------------------------------------- */
typedef struct dbd_round_args {
  int S, B, Hq, Hkv, D, page_size, max_pages_per_seq;
  int Hd, V, mask_token_id;
  float dynamic_threshold;
  uint32_t flags;
  float softmax_scale;
  const dbd_bf16 *q, *k_blk, *v_blk, *k_cache, *v_cache;
  const int32_t *page_table, *prefix_len;
  dbd_bf16* attn_out;
  const dbd_bf16 *hidden, *w_vocab;
  int32_t* row_index; /* in: this round's rows; out: the next round's */
  int32_t* num_rows;  /* device scalar, same in/out rule              */
  int32_t* argmax_tok;
  float* conf;
  int32_t* block_tokens;
  uint8_t* seq_state;
  int32_t* num_committed; /* may be NULL */
  void* workspace;
  size_t workspace_bytes;
  /* commit rule (dbd_remask_commit_rule); rule 0 is the threshold rule */
  int rule;
  int tokens_per_step;
  float eb_threshold;
  float* entropy; /* float [S*B]; required for DBD_RULE_ENTROPY_BOUNDED */
  /* SAVING step.  With save_kv != 0 the round is a whole scheduler step for
   * a batch that mixes DENOISING and SAVING sequences: the attention is
   * dbd_attn_paged_save (SAVING sequences' block K/V go into their pages),
   * the LM head projects the listed rows, and the remask kernel commits
   * the rule for sequences DENOISING on entry and, for those SAVING on
   * entry, the block commit of dbd_commit_block (token_stream, stream_cap,
   * end_len as there).  A sequence that the rule fills stays SAVING until
   * the next step's SAVING forward.  k_cache, v_cache and prefix_len are
   * then written and must be writable; num_pages bounds the page ids
   * written.  save_kv == 0: none of these fields is read. */
  int save_kv;
  int num_pages;
  int32_t* token_stream; /* may be NULL */
  int stream_cap;
  const int32_t* end_len; /* may be NULL */
  /* Device-side loop control.  gate_on_rows != 0: the round's attention
   * returns at once when *num_rows is 0 on entry (no DENOISING sequence
   * has a masked position left), and the LM head and the remask then have
   * nothing to do, so the round changes nothing.  Not allowed together with
   * save_kv.  round_counter (int32 device scalar, may be NULL) is
   * incremented by every round that starts with *num_rows > 0. */
  int gate_on_rows;
  int32_t* round_counter;
  /* Temperature sampling (dbd_lmhead_sample) instead of the greedy token
   * when sample != 0: argmax_tok receives the drawn token, conf its
   * probability at temperature 1.  Give each round its own step. */
  int sample;
  float temperature;
  uint64_t seed;
  uint32_t step;
  /* Top-k / top-p filtering of the drawn token (SamplingParams topk, topp;
   * JetEngine README usage examples), with sample != 0 and filter != 0: the
   * LM head stores the listed rows' logits in `logits` (dbd_lmhead_logits;
   * float [S*B][V], caller-owned, row r = list entry r) and
   * dbd_sample_filtered draws each row's token from them with top_k and
   * top_p (the same seed and step).  Not allowed with the entropy-bounded
   * rule (no entropy is computed).  filter == 0: none of these is read. */
  int filter;
  int top_k;
  float top_p;
  float* logits;
} dbd_round_args;

dbd_status dbd_round(const dbd_round_args* a, void* stream);
size_t dbd_round_workspace_size(const dbd_round_args* a);

/* dbd_round_noalloc -- dbd_round for callers that cannot allocate device
 * memory (code under stream capture, tight serving loops, harnesses that
 * forbid allocation).  The same round with the same kernels, but the
 * workspace is the library's own static device array of
 * DBD_NOALLOC_SCRATCH_BYTES (64 MiB) on the current device, resident until
 * the process ends; a->workspace and a->workspace_bytes are not read.
 * The call makes no allocation of any kind (no hipMalloc, no library
 * routine that allocates); its first call on a device looks up that
 * device's array address once.  Returns DBD_ERR_WORKSPACE, before any HIP
 * call, when dbd_round_workspace_size(a) exceeds the array (e.g. the
 * SDAR-8B and LLaDA shapes of block 16 and 64 need 71 and 68 MiB); the
 * other checks are dbd_round's.  The array's contents are not cleared and
 * need not be: every call writes what it reads.  All calls on one device
 * share that device's array, so calls that overlap in time on one device
 * (different streams, or host threads without ordering) race; callers
 * serialise them, e.g. on one stream. */
#define DBD_NOALLOC_SCRATCH_BYTES (64u << 20)
dbd_status dbd_round_noalloc(const dbd_round_args* a, void* stream);
/* sizeof(dbd_round_args) as this library was built, so that a binding can
 * check its copy of the struct layout. */
size_t dbd_round_args_size(void);

/* Graph of n_rounds consecutive rounds (args[i] for round i, e.g. each with
 * its own per-round inputs), captured once and replayed with one launch and
 * no host work in between (dlmrt README, "Highlights": denoising loop on the
 * device; JetEngine developer notes: CUDA-graph replay of the denoise
 * batch).  The captured pointers and scalars are fixed at creation.
 *
 * A whole block as one graph, "begin -> while (not done) round -> commit"
 * (dlmrt README, "Highlights": the loop condition decided on the GPU;
 * developer notes, "Chain Mechanism": the denoise steps and the SAVING step
 * of a block in one chain, with no host synchronisation between them):
 * B rounds with gate_on_rows set, then one step with save_kv set.  Every
 * commit rule commits at least one position of every DENOISING sequence
 * with a mask left, so a block needs at most B rounds; the rounds after
 * the block is done return at once on the device.  Several such blocks may
 * follow one another in one graph. */
typedef struct dbd_graph dbd_graph;
dbd_status dbd_graph_create(const dbd_round_args* args, int n_rounds,
                            dbd_graph** out);
dbd_status dbd_graph_launch(dbd_graph* g, void* stream);
void dbd_graph_destroy(dbd_graph* g);

/* Host-side check of host copies of the device-resident inputs: page ids in
 * [0, num_pages), prefix lengths within the page table, mask id / tokens
 * within the vocabulary, states within the enum.  Makes no HIP call. */
dbd_status dbd_validate_inputs(int S, int B, int page_size,
                               int max_pages_per_seq, int num_pages, int V,
                               int mask_token_id, const int32_t* page_table,
                               const int32_t* prefix_len,
                               const int32_t* block_tokens,
                               const uint8_t* seq_state);

/* Measurement helper: reads `bytes` (a multiple of 16) of device memory
 * once (contiguous chunks per workgroup, non-temporal loads: the fastest
 * plain read found on the device) and writes a digest word per workgroup
 * to sink (dbd_stream_read_sink_words() words), so that the memory-bound
 * kernels can be compared with the device's practical read bandwidth as
 * well as with the nominal HBM peak. */
dbd_status dbd_stream_read(const void* data, size_t bytes, uint32_t* sink,
                           void* stream);
int dbd_stream_read_sink_words(void);

/* Measurement helper: a register-resident loop of bf16 matrix-core
 * multiply-adds (v_mfma_f32_32x32x16_bf16).  `operands` (device,
 * dbd_mfma_peak_operand_bytes() bytes of bf16 values, e.g. random
 * normals, 16-byte aligned) is read once; then every wave issues
 * iters * 64 of the instruction over eight independent accumulator chains
 * whose operands rotate every step, and every thread writes the sum of its
 * accumulators to sink (device, dbd_mfma_peak_sink_floats() floats).  One
 * launch performs dbd_mfma_peak_flops(iters) floating-point operations;
 * their rate is the device's practical bf16 matrix-core rate on changing
 * data, the power limit included.  iters must be in [1, 4096]. */
dbd_status dbd_mfma_peak(const void* operands, int iters, float* sink, void* stream);
size_t dbd_mfma_peak_operand_bytes(void);
int dbd_mfma_peak_sink_floats(void);
double dbd_mfma_peak_flops(int iters);

const char* dbd_last_error(void);
int dbd_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DBD_H */
