// Internal (non-ABI) declarations of libdbd: kernel argument blocks, launch
// plans and launchers.  Host and device code both include this header.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dbd {

// ---------------------------------------------------------------- attention
struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k_blk;
  const uint16_t* v_blk;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* page_table;
  const int32_t* prefix_len;
  uint16_t* out;
  float* part_o;   // [2*grid][rows][D] unnormalised sums of split segments,
                   // two slots per wave
  float2* part_ml; // [2*grid][rows] (max, sum), log2 units
  int32_t* seg_np; // [S*NHG] pieces of each segment in this launch (1: not
                   // split) | first piece's slot side << 11 | first wave << 12
  int S, B, Hq, Hkv, G, P, max_pages;
  int n_rg;        // row groups per kv head (rows = G*B split in 16*RT)
  int grid;        // workgroups (single waves) of the stream kernel
  float scale_log2;
  // SAVING forward: when save_state is set, the block keys and values of
  // every sequence whose state is SAVING are also written into its pages at
  // positions prefix_len + j (pages outside [0, num_pages) are skipped)
  const uint8_t* save_state;
  uint16_t* k_cache_out;   // the same buffers as k_cache, v_cache
  uint16_t* v_cache_out;
  int num_pages;
  // may be NULL; otherwise every attention kernel returns at once when
  // *gate <= 0 (a round with no row left to denoise)
  const int32_t* gate;
};

struct AttnPlan {
  int D, RT, n_rg, grid, ring;   // ring: LDS slots per wave
  size_t o_bytes, ml_bytes, ws_bytes;  // workspace: part_o | part_ml | seg_np
};

AttnPlan attn_plan(int S, int B, int Hq, int Hkv, int D, int page_size,
                   int max_pages);
hipError_t attn_launch(const AttnPlan& plan, const AttnArgs& a,
                       hipStream_t stream);

// ------------------------------------------------------------------ LM head
// workgroups of the persistent LM-head kernel (one per CU of an MI355X) and
// the number of (max, id, sum) partials it leaves per row
constexpr int kLmGrid = 256;
// LM-head workgroups per team for M rows: 1, 2 or 4 for M <= 256, 512 or
// more; kLmGrid / lm_team_size(M) teams each own a range of the vocabulary
__host__ __device__ inline int lm_team_size(int M) { return M <= 256 ? 1 : (M <= 512 ? 2 : 4); }

struct LmArgs {
  const uint16_t* hidden;
  const int32_t* row_index;
  const int32_t* num_rows;
  const uint16_t* w;
  int Hd, V, mask_id, max_rows;
  float* pm;       // [max_rows][kLmGrid] partial max logit
  int32_t* pa;     // [max_rows][kLmGrid] partial argmax (lowest id on ties)
  float* ps;       // [max_rows][kLmGrid] partial sum exp(l - max)
  float* pt;       // [max_rows][kLmGrid] partial sum exp(l - max) (l - max)
  int32_t* argmax_tok;
  float* conf;
  float* entropy;  // may be NULL: softmax entropy per listed row (nats)
  // temperature sampling (sample != 0): argmax_tok receives the drawn token
  int sample;
  float inv_temp;  // 1 / temperature
  uint32_t key0, key1, step;
  float* pg;       // [max_rows][kLmGrid] partial largest Gumbel value (log2 units)
  float* pl;       // [max_rows][kLmGrid] partial logit of its candidate
  float* logits;   // non-NULL: store the logits [max_rows][V] of the listed rows instead,
                   // and with pm non-NULL each team's partial row maxima in pm (the
                   // wave pair's first wave) and pa as floats (the second)
};

// ------------------------------------------------- filtered sampling
struct SampleArgs {
  const float* logits;       // [max_rows][V], row r = list entry r
  const int32_t* row_index;  // may be NULL (row id = r)
  const int32_t* num_rows;
  int V, mask_id, max_rows, top_k;
  float inv_temp, top_p;
  uint32_t key0, key1, step;
  const float* pmax;         // may be NULL: the partial row maxima of the LM head's store
  const float* pmax2;        // mode, two arrays [max_rows][kLmGrid / lm_team_size(*num_rows)];
                             // then no pass over the row looks for the maximum
  int32_t* token;            // [rows] by row id
  float* conf;
};
hipError_t sample_filtered_launch(const SampleArgs& a, hipStream_t stream);

// ------------------------------------------------------- calibration
constexpr int kStreamReadGrid = 2048;   // workgroups of the read ceiling kernel
hipError_t stream_read_launch(const void* data, size_t bytes, uint32_t* sink, int grid,
                              hipStream_t stream);
constexpr int kMfmaPeakGrid = 1024;     // workgroups of four waves
constexpr int kMfmaPeakSets = 64;       // operand sets of 16 fragments x 64 lanes x 16 bytes
constexpr int kMfmaPeakPerIter = 64;    // MFMAs per wave per iteration
hipError_t mfma_peak_launch(const void* operands, int iters, float* sink, hipStream_t stream);

// partial arrays of the LM-head workspace: pm, pa, ps, pt, pg, pl
constexpr int kLmPartArrays = 6;

size_t lmhead_ws_bytes(int max_rows, int V);
hipError_t lmhead_launch(const LmArgs& a, hipStream_t stream);

// ------------------------------------------------------------------- remask
struct RemaskArgs {
  int S, B, mask_id;
  float tau;
  uint32_t flags;
  int rule;           // 0 dynamic threshold, 1 static top-k, 2 sequential, 3 entropy-bounded
  int k;              // tokens per step (rules 1 and 2)
  float eb;           // entropy budget (rule 3)
  const float* entropy;  // [S*B] (rule 3)
  int32_t* block_tokens;
  uint8_t* seq_state;
  const int32_t* argmax_tok;
  const float* conf;
  int32_t* row_index_out;
  int32_t* num_rows_out;
  int32_t* num_committed;
  // block commit of sequences SAVING on entry (flags & kCommitSaving)
  int32_t* prefix_len;        // in/out
  int32_t* token_stream;      // [S][stream_cap], may be NULL
  int stream_cap;
  const int32_t* end_len;     // [S], may be NULL
  // may be NULL: incremented when *rows_in > 0 on entry (an active round)
  int32_t* round_counter;
  const int32_t* rows_in;
};

constexpr int kRemaskMaxSeqs = 8192;
// internal remask flag (beside the public DBD_FALLBACK_LEFTMOST = 1 and
// DBD_COMPACT_ONLY = 2): commit the blocks of sequences SAVING on entry
constexpr uint32_t kCommitSaving = 4u;
hipError_t remask_launch(const RemaskArgs& a, hipStream_t stream);

// ----------------------------------------------------------- prefill
struct PrefillArgs {
  const uint16_t* q;           // [T][Hq][D] packed prompts
  const uint16_t* k;           // [T][Hkv][D]
  const uint16_t* v;
  const int32_t* cu_seqlens;   // [S+1]
  uint16_t* out;               // [T][Hq][D]
  int32_t* plan;               // [S+1] tile prefix sums (workspace)
  int S, T_total, Hq, Hkv, G, B;
  float scale_log2;
  // optional store of the prompts' K/V into the paged cache
  const int32_t* page_table;   // [S][max_pages]
  uint16_t* k_cache_out;       // NULL: no store
  uint16_t* v_cache_out;
  int P, max_pages, num_pages;
};

size_t prefill_ws_bytes(int S);
int prefill_rows_per_wg();   // query rows per workgroup (G must divide it)
int prefill_grid(int S, int T_total, int Hkv, int G);
hipError_t prefill_launch(const PrefillArgs& a, int D, hipStream_t stream);

}  // namespace dbd
