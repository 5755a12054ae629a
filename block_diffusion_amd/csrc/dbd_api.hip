// libdbd C ABI: host-side validation, workspace carving, launches of the
// denoise-round kernels, and graph capture of whole rounds.  The contract of
// every entry point is in include/dbd.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "../../include/dbd.h"
#include "dbd_internal.hpp"

namespace {

thread_local std::string g_err;

dbd_status fail(dbd_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

dbd_status hip_fail(hipError_t e, const char* where) {
  return fail(DBD_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

#define REQUIRE(cond, ...)                                          \
  do {                                                              \
    if (!(cond)) return fail(DBD_ERR_INVALID_ARG, __VA_ARGS__);     \
  } while (0)
#define REQUIRE_PTR(p)                                                       \
  do {                                                                       \
    if ((p) == nullptr) return fail(DBD_ERR_INVALID_ARG, #p " is NULL");     \
    if (!aligned((p), 16)) return fail(DBD_ERR_INVALID_ARG, #p " is not 16-byte aligned"); \
  } while (0)

size_t round_up(size_t x) { return (x + 255) & ~(size_t)255; }

dbd_status check_attn(int S, int B, int Hq, int Hkv, int D, int page_size,
                      int max_pages) {
  REQUIRE(S >= 1, "S must be >= 1 (got %d)", S);
  REQUIRE(B >= 1 && B <= 64, "block_length must be in [1,64] (got %d)", B);
  REQUIRE(Hq >= 1 && Hkv >= 1 && Hq % Hkv == 0, "Hq (%d) must be a positive multiple of Hkv (%d)", Hq, Hkv);
  REQUIRE(page_size >= 16 && page_size % 16 == 0, "page_size must be a positive multiple of 16 (got %d)", page_size);
  REQUIRE(max_pages >= 1, "max_pages_per_seq must be >= 1 (got %d)", max_pages);
  REQUIRE(S <= 65535, "S must be <= 65535 (got %d)", S);
  REQUIRE((long)S * ((long)max_pages * page_size / 16 + 4) < (1L << 31),
          "S x max_pages_per_seq x page_size too large for 32-bit tile counts");
  if (D != 64 && D != 128) return fail(DBD_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", D);
  return DBD_OK;
}

dbd_status check_lm(int max_rows, int Hd, int V, int mask) {
  REQUIRE(max_rows >= 0, "max_rows must be >= 0 (got %d)", max_rows);
  REQUIRE(V >= 2, "vocab size must be >= 2 (got %d)", V);
  REQUIRE(mask >= 0 && mask < V, "mask_token_id %d outside [0,%d)", mask, V);
  REQUIRE(Hd >= 128 && Hd % 128 == 0, "hidden size must be a positive multiple of 128 (got %d)", Hd);
  REQUIRE((long)V * Hd < (1L << 31), "V*Hd must fit in 31 bits");
  REQUIRE((long)max_rows * Hd < (1L << 31), "max_rows*Hd must fit in 31 bits");
  return DBD_OK;
}

dbd_status check_remask(int S, int B, float tau) {
  REQUIRE(S >= 1 && S <= dbd::kRemaskMaxSeqs, "S must be in [1,%d] (got %d)", dbd::kRemaskMaxSeqs, S);
  REQUIRE(B >= 1 && B <= 64, "block_length must be in [1,64] (got %d)", B);
  REQUIRE(!isnan(tau), "dynamic_threshold is NaN");
  return DBD_OK;
}

dbd_status enqueue_attn(int S, int B, int Hq, int Hkv, int D, int P, int max_pages,
                        const dbd_bf16* q, const dbd_bf16* k_blk, const dbd_bf16* v_blk,
                        const dbd_bf16* k_cache, const dbd_bf16* v_cache,
                        const int32_t* page_table, const int32_t* prefix_len,
                        float scale, dbd_bf16* out, void* ws, size_t ws_bytes,
                        hipStream_t st, const uint8_t* save_state = nullptr,
                        dbd_bf16* kc_out = nullptr, dbd_bf16* vc_out = nullptr,
                        int num_pages = 0, const int32_t* gate = nullptr) {
  dbd::AttnPlan plan = dbd::attn_plan(S, B, Hq, Hkv, D, P, max_pages);
  if (ws == nullptr || ws_bytes < plan.ws_bytes)
    return fail(DBD_ERR_WORKSPACE, "attention workspace needs %zu bytes (got %zu)", plan.ws_bytes, ws_bytes);
  if (!aligned(ws, 256)) return fail(DBD_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  dbd::AttnArgs a{};
  a.q = q; a.k_blk = k_blk; a.v_blk = v_blk; a.k_cache = k_cache; a.v_cache = v_cache;
  a.page_table = page_table; a.prefix_len = prefix_len; a.out = out;
  char* w = static_cast<char*>(ws);
  a.part_o = reinterpret_cast<float*>(w);
  a.part_ml = reinterpret_cast<float2*>(w + plan.o_bytes);
  a.seg_np = reinterpret_cast<int32_t*>(w + plan.o_bytes + plan.ml_bytes);
  a.S = S; a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv; a.P = P; a.max_pages = max_pages;
  a.n_rg = plan.n_rg; a.grid = plan.grid;
  const float sc = scale > 0.f ? scale : 1.0f / sqrtf((float)D);
  a.scale_log2 = sc * 1.4426950408889634f;
  a.save_state = save_state; a.k_cache_out = kc_out; a.v_cache_out = vc_out;
  a.num_pages = num_pages;
  a.gate = gate;
  hipError_t e = dbd::attn_launch(plan, a, st);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return DBD_OK;
}

dbd_status enqueue_lm(int max_rows, int Hd, int V, int mask, const dbd_bf16* hidden,
                      const int32_t* row_index, const int32_t* num_rows,
                      const dbd_bf16* w, int32_t* argmax_tok, float* conf, float* entropy,
                      void* ws, size_t ws_bytes, hipStream_t st, bool sample = false,
                      float temperature = 1.f, uint64_t seed = 0, uint32_t step = 0) {
  if (max_rows == 0) return DBD_OK;
  const size_t need = dbd::lmhead_ws_bytes(max_rows, V);
  if (ws == nullptr || ws_bytes < need)
    return fail(DBD_ERR_WORKSPACE, "LM-head workspace needs %zu bytes (got %zu)", need, ws_bytes);
  if (!aligned(ws, 256)) return fail(DBD_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  dbd::LmArgs a{};
  a.hidden = hidden; a.row_index = row_index; a.num_rows = num_rows; a.w = w;
  a.Hd = Hd; a.V = V; a.mask_id = mask; a.max_rows = max_rows;
  const size_t one = need / dbd::kLmPartArrays;
  char* base = static_cast<char*>(ws);
  a.pm = reinterpret_cast<float*>(base);
  a.pa = reinterpret_cast<int32_t*>(base + one);
  a.ps = reinterpret_cast<float*>(base + 2 * one);
  a.pt = reinterpret_cast<float*>(base + 3 * one);
  a.pg = reinterpret_cast<float*>(base + 4 * one);
  a.pl = reinterpret_cast<float*>(base + 5 * one);
  a.argmax_tok = argmax_tok; a.conf = conf; a.entropy = entropy;
  a.sample = sample ? 1 : 0;
  a.inv_temp = 1.f / temperature;
  a.key0 = (uint32_t)seed; a.key1 = (uint32_t)(seed >> 32); a.step = step;
  hipError_t e = dbd::lmhead_launch(a, st);
  if (e != hipSuccess) return hip_fail(e, "LM-head launch");
  return DBD_OK;
}

// the listed rows' logits (store mode of the LM-head tile kernel)
// (pmax, pmax2 may be NULL: else each team's partial row maxima go there,
// two arrays of [max_rows][kLmGrid] floats)
dbd_status enqueue_logits(int max_rows, int Hd, int V, int mask, const dbd_bf16* hidden,
                          const int32_t* row_index, const int32_t* num_rows, const dbd_bf16* w,
                          float* logits, hipStream_t st, float* pmax = nullptr,
                          float* pmax2 = nullptr) {
  if (max_rows == 0) return DBD_OK;
  dbd::LmArgs a{};
  a.hidden = hidden; a.row_index = row_index; a.num_rows = num_rows; a.w = w;
  a.Hd = Hd; a.V = V; a.mask_id = mask; a.max_rows = max_rows;
  a.logits = logits;
  a.pm = pmax;
  a.pa = reinterpret_cast<int32_t*>(pmax2);
  hipError_t e = dbd::lmhead_launch(a, st);
  if (e != hipSuccess) return hip_fail(e, "LM-head launch");
  return DBD_OK;
}

// (pmax, pmax2: the partial row maxima enqueue_logits left for the same
// rows, or NULL)
dbd_status enqueue_filtered(int max_rows, int V, int mask, const float* logits,
                            const int32_t* row_index, const int32_t* num_rows, float temperature,
                            int top_k, float top_p, uint64_t seed, uint32_t step, int32_t* token,
                            float* conf, hipStream_t st, const float* pmax = nullptr,
                            const float* pmax2 = nullptr) {
  if (max_rows == 0) return DBD_OK;
  dbd::SampleArgs a{};
  a.logits = logits; a.row_index = row_index; a.num_rows = num_rows;
  a.V = V; a.mask_id = mask; a.max_rows = max_rows; a.top_k = top_k;
  a.inv_temp = 1.f / temperature; a.top_p = top_p;
  a.key0 = (uint32_t)seed; a.key1 = (uint32_t)(seed >> 32); a.step = step;
  a.token = token; a.conf = conf;
  a.pmax = pmax;
  a.pmax2 = pmax2;
  hipError_t e = dbd::sample_filtered_launch(a, st);
  if (e != hipSuccess) return hip_fail(e, "sampling launch");
  return DBD_OK;
}

dbd_status enqueue_remask(int S, int B, int mask, float tau, uint32_t flags, int rule, int k,
                          float eb, const float* entropy,
                          int32_t* block_tokens, uint8_t* seq_state,
                          const int32_t* argmax_tok, const float* conf,
                          int32_t* row_index_out, int32_t* num_rows_out,
                          int32_t* num_committed, hipStream_t st,
                          int32_t* prefix_len = nullptr, int32_t* token_stream = nullptr,
                          int stream_cap = 0, const int32_t* end_len = nullptr,
                          int32_t* round_counter = nullptr, const int32_t* rows_in = nullptr) {
  dbd::RemaskArgs a{};
  a.S = S; a.B = B; a.mask_id = mask; a.tau = tau; a.flags = flags;
  a.rule = rule; a.k = k < 1 ? 1 : k; a.eb = eb; a.entropy = entropy;
  a.block_tokens = block_tokens; a.seq_state = seq_state;
  a.argmax_tok = argmax_tok; a.conf = conf;
  a.row_index_out = row_index_out; a.num_rows_out = num_rows_out;
  a.num_committed = num_committed;
  a.prefix_len = prefix_len; a.token_stream = token_stream; a.stream_cap = stream_cap;
  a.end_len = end_len;
  a.round_counter = round_counter; a.rows_in = rows_in;
  hipError_t e = dbd::remask_launch(a, st);
  if (e != hipSuccess) return hip_fail(e, "remask launch");
  return DBD_OK;
}

// entropy is needed (and checked) only when the rule commits by entropy
dbd_status check_rule(int rule, float eb, const float* entropy, bool commits) {
  REQUIRE(rule >= DBD_RULE_LOW_CONF_DYNAMIC && rule <= DBD_RULE_ENTROPY_BOUNDED, "unknown rule %d", rule);
  REQUIRE(!isnan(eb), "eb_threshold is NaN");
  if (commits && rule == DBD_RULE_ENTROPY_BOUNDED) REQUIRE_PTR(entropy);
  return DBD_OK;
}

dbd_status check_round(const dbd_round_args* a, bool check_workspace = true) {
  REQUIRE(a != nullptr, "args is NULL");
  dbd_status s = check_attn(a->S, a->B, a->Hq, a->Hkv, a->D, a->page_size, a->max_pages_per_seq);
  if (s != DBD_OK) return s;
  s = check_lm(a->S * a->B, a->Hd, a->V, a->mask_token_id);
  if (s != DBD_OK) return s;
  s = check_remask(a->S, a->B, a->dynamic_threshold);
  if (s != DBD_OK) return s;
  s = check_rule(a->rule, a->eb_threshold, a->entropy, true);
  if (s != DBD_OK) return s;
  if (a->sample) REQUIRE(isfinite(a->temperature) && a->temperature > 0.f,
                         "temperature must be finite and > 0 (got %g)", (double)a->temperature);
  if (a->filter) {
    REQUIRE(a->sample, "filter needs sample");
    REQUIRE(a->top_k >= 0, "top_k must be >= 0 (got %d)", a->top_k);
    REQUIRE(!isnan(a->top_p), "top_p is NaN");
    REQUIRE(a->rule != DBD_RULE_ENTROPY_BOUNDED, "filter does not compute the entropy the rule needs");
    REQUIRE((long)a->S * a->B * a->V < (1L << 40), "S*B*V too large");
    REQUIRE_PTR(a->logits);
  }
  REQUIRE_PTR(a->q); REQUIRE_PTR(a->k_blk); REQUIRE_PTR(a->v_blk);
  REQUIRE_PTR(a->k_cache); REQUIRE_PTR(a->v_cache);
  REQUIRE_PTR(a->page_table); REQUIRE_PTR(a->prefix_len); REQUIRE_PTR(a->attn_out);
  REQUIRE_PTR(a->hidden); REQUIRE_PTR(a->w_vocab); REQUIRE_PTR(a->row_index);
  REQUIRE_PTR(a->num_rows); REQUIRE_PTR(a->argmax_tok); REQUIRE_PTR(a->conf);
  REQUIRE_PTR(a->block_tokens); REQUIRE_PTR(a->seq_state);
  if (a->save_kv) {
    REQUIRE(a->num_pages >= 1, "num_pages must be >= 1 with save_kv (got %d)", a->num_pages);
    if (a->token_stream != nullptr) {
      REQUIRE_PTR(a->token_stream);
      REQUIRE(a->stream_cap >= 1, "stream_cap must be >= 1 (got %d)", a->stream_cap);
    }
    if (a->end_len != nullptr) REQUIRE_PTR(a->end_len);
  }
  REQUIRE(!(a->save_kv && a->gate_on_rows), "gate_on_rows cannot be set on a save_kv step");
  if (a->round_counter != nullptr) REQUIRE(aligned(a->round_counter, 4), "round_counter is not 4-byte aligned");
  if (!check_workspace) return DBD_OK;
  const size_t need = dbd_round_workspace_size(a);
  if (a->workspace == nullptr || a->workspace_bytes < need)
    return fail(DBD_ERR_WORKSPACE, "round workspace needs %zu bytes (got %zu)", need, a->workspace_bytes);
  REQUIRE(aligned(a->workspace, 256), "workspace is not 256-byte aligned");
  return DBD_OK;
}

dbd_status enqueue_round(const dbd_round_args* a, hipStream_t st) {
  const dbd::AttnPlan plan = dbd::attn_plan(a->S, a->B, a->Hq, a->Hkv, a->D, a->page_size, a->max_pages_per_seq);
  const size_t attn_ws = round_up(plan.ws_bytes);
  char* ws = static_cast<char*>(a->workspace);
  // with save_kv the caller's cache and prefix lengths are writable (dbd.h)
  const bool save = a->save_kv != 0;
  dbd_status s = enqueue_attn(a->S, a->B, a->Hq, a->Hkv, a->D, a->page_size, a->max_pages_per_seq,
                              a->q, a->k_blk, a->v_blk, a->k_cache, a->v_cache, a->page_table,
                              a->prefix_len, a->softmax_scale, a->attn_out, ws, plan.ws_bytes, st,
                              save ? a->seq_state : nullptr,
                              save ? const_cast<dbd_bf16*>(a->k_cache) : nullptr,
                              save ? const_cast<dbd_bf16*>(a->v_cache) : nullptr, a->num_pages,
                              a->gate_on_rows ? a->num_rows : nullptr);
  if (s != DBD_OK) return s;
  const int max_rows = a->S * a->B;
  float* ent = a->rule == DBD_RULE_ENTROPY_BOUNDED ? a->entropy : nullptr;
  if (a->sample && a->filter) {
    // the LM head's partial-maximum array of the round workspace carries
    // each row's maximum to the filtered draw (one pass fewer over the row)
    const size_t one = dbd::lmhead_ws_bytes(max_rows, a->V) / dbd::kLmPartArrays;
    float* pmax = reinterpret_cast<float*>(ws + attn_ws);
    float* pmax2 = reinterpret_cast<float*>(ws + attn_ws + one);
    s = enqueue_logits(max_rows, a->Hd, a->V, a->mask_token_id, a->hidden, a->row_index,
                       a->num_rows, a->w_vocab, a->logits, st, pmax, pmax2);
    if (s != DBD_OK) return s;
    s = enqueue_filtered(max_rows, a->V, a->mask_token_id, a->logits, a->row_index, a->num_rows,
                         a->temperature, a->top_k, a->top_p, a->seed, a->step, a->argmax_tok,
                         a->conf, st, pmax, pmax2);
  } else {
    s = enqueue_lm(max_rows, a->Hd, a->V, a->mask_token_id, a->hidden, a->row_index, a->num_rows,
                   a->w_vocab, a->argmax_tok, a->conf, ent, ws + attn_ws, a->workspace_bytes - attn_ws,
                   st, a->sample != 0, a->temperature, a->seed, a->step);
  }
  if (s != DBD_OK) return s;
  const uint32_t fl = (a->flags & ~DBD_COMPACT_ONLY) | (save ? dbd::kCommitSaving : 0u);
  return enqueue_remask(a->S, a->B, a->mask_token_id, a->dynamic_threshold, fl,
                        a->rule, a->tokens_per_step, a->eb_threshold, ent,
                        a->block_tokens, a->seq_state, a->argmax_tok, a->conf, a->row_index,
                        a->num_rows, a->num_committed, st,
                        save ? const_cast<int32_t*>(a->prefix_len) : nullptr,
                        save ? a->token_stream : nullptr, a->stream_cap,
                        save ? a->end_len : nullptr, a->round_counter, a->num_rows);
}

// The round workspace of dbd_round_noalloc: one array per device, resident
// for the life of the process.  In host code `scratch` names a host-side
// stand-in, not device memory: only the address hipGetSymbolAddress returns
// on a device may be handed to kernels.
constexpr size_t kScratchBytes = (size_t)DBD_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// scratch's device address on the current device, looked up once per device
dbd_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(DBD_ERR_UNSUPPORTED, "device index %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr || !aligned(p, 256)) return fail(DBD_ERR_HIP, "scratch has no 256-byte aligned device address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DBD_OK;
}

}  // namespace

struct dbd_graph {
  hipStream_t stream;
  hipGraph_t graph;
  hipGraphExec_t exec;
};

extern "C" {

int dbd_abi_version(void) { return DBD_ABI_VERSION; }

size_t dbd_round_args_size(void) { return sizeof(dbd_round_args); }

const char* dbd_last_error(void) { return g_err.c_str(); }

size_t dbd_attn_workspace_size(int S, int B, int Hq, int Hkv, int D, int page_size,
                               int max_pages_per_seq) {
  if (check_attn(S, B, Hq, Hkv, D, page_size, max_pages_per_seq) != DBD_OK) return 0;
  return dbd::attn_plan(S, B, Hq, Hkv, D, page_size, max_pages_per_seq).ws_bytes;
}

size_t dbd_lmhead_workspace_size(int max_rows, int V) {
  if (max_rows <= 0 || V < 2) return 0;
  return dbd::lmhead_ws_bytes(max_rows, V);
}

size_t dbd_round_workspace_size(const dbd_round_args* a) {
  if (a == nullptr) return 0;
  const size_t attn = dbd_attn_workspace_size(a->S, a->B, a->Hq, a->Hkv, a->D, a->page_size,
                                              a->max_pages_per_seq);
  return round_up(attn) + dbd_lmhead_workspace_size(a->S * a->B, a->V);
}

dbd_status dbd_attn_paged(int S, int B, int Hq, int Hkv, int D, int page_size,
                          int max_pages_per_seq, const dbd_bf16* q, const dbd_bf16* k_blk,
                          const dbd_bf16* v_blk, const dbd_bf16* k_cache,
                          const dbd_bf16* v_cache, const int32_t* page_table,
                          const int32_t* prefix_len, float softmax_scale, dbd_bf16* out,
                          void* workspace, size_t workspace_bytes, void* stream) {
  dbd_status s = check_attn(S, B, Hq, Hkv, D, page_size, max_pages_per_seq);
  if (s != DBD_OK) return s;
  REQUIRE_PTR(q); REQUIRE_PTR(k_blk); REQUIRE_PTR(v_blk); REQUIRE_PTR(k_cache);
  REQUIRE_PTR(v_cache); REQUIRE_PTR(page_table); REQUIRE_PTR(prefix_len); REQUIRE_PTR(out);
  REQUIRE(!isnan(softmax_scale), "softmax_scale is NaN");
  return enqueue_attn(S, B, Hq, Hkv, D, page_size, max_pages_per_seq, q, k_blk, v_blk, k_cache,
                      v_cache, page_table, prefix_len, softmax_scale, out, workspace,
                      workspace_bytes, static_cast<hipStream_t>(stream));
}

dbd_status dbd_attn_paged_save(int S, int B, int Hq, int Hkv, int D, int page_size,
                               int max_pages_per_seq, int num_pages, const dbd_bf16* q,
                               const dbd_bf16* k_blk, const dbd_bf16* v_blk, dbd_bf16* k_cache,
                               dbd_bf16* v_cache, const int32_t* page_table,
                               const int32_t* prefix_len, const uint8_t* seq_state,
                               float softmax_scale, dbd_bf16* out, void* workspace,
                               size_t workspace_bytes, void* stream) {
  dbd_status s = check_attn(S, B, Hq, Hkv, D, page_size, max_pages_per_seq);
  if (s != DBD_OK) return s;
  REQUIRE(num_pages >= 1, "num_pages must be >= 1 (got %d)", num_pages);
  REQUIRE_PTR(q); REQUIRE_PTR(k_blk); REQUIRE_PTR(v_blk); REQUIRE_PTR(k_cache);
  REQUIRE_PTR(v_cache); REQUIRE_PTR(page_table); REQUIRE_PTR(prefix_len);
  REQUIRE_PTR(seq_state); REQUIRE_PTR(out);
  REQUIRE(!isnan(softmax_scale), "softmax_scale is NaN");
  return enqueue_attn(S, B, Hq, Hkv, D, page_size, max_pages_per_seq, q, k_blk, v_blk, k_cache,
                      v_cache, page_table, prefix_len, softmax_scale, out, workspace,
                      workspace_bytes, static_cast<hipStream_t>(stream), seq_state, k_cache,
                      v_cache, num_pages);
}

dbd_status dbd_commit_block(int S, int B, int mask_token_id, int32_t* block_tokens,
                            uint8_t* seq_state, int32_t* prefix_len, int32_t* token_stream,
                            int stream_cap, const int32_t* end_len, int32_t* row_index_out,
                            int32_t* num_rows_out, void* stream) {
  dbd_status s = check_remask(S, B, 0.f);
  if (s != DBD_OK) return s;
  REQUIRE_PTR(block_tokens); REQUIRE_PTR(seq_state); REQUIRE_PTR(prefix_len);
  REQUIRE_PTR(row_index_out); REQUIRE_PTR(num_rows_out);
  if (token_stream != nullptr) {
    REQUIRE_PTR(token_stream);
    REQUIRE(stream_cap >= 1, "stream_cap must be >= 1 (got %d)", stream_cap);
  }
  if (end_len != nullptr) REQUIRE_PTR(end_len);
  return enqueue_remask(S, B, mask_token_id, 0.f, DBD_COMPACT_ONLY | dbd::kCommitSaving,
                        DBD_RULE_LOW_CONF_DYNAMIC, 1, 0.f, nullptr, block_tokens, seq_state,
                        nullptr, nullptr, row_index_out, num_rows_out, nullptr,
                        static_cast<hipStream_t>(stream), prefix_len, token_stream, stream_cap,
                        end_len);
}

dbd_status dbd_lmhead_conf(int max_rows, int Hd, int V, int mask_token_id,
                           const dbd_bf16* hidden, const int32_t* row_index,
                           const int32_t* num_rows, const dbd_bf16* w_vocab,
                           int32_t* argmax_tok, float* conf, void* workspace,
                           size_t workspace_bytes, void* stream) {
  dbd_status s = check_lm(max_rows, Hd, V, mask_token_id);
  if (s != DBD_OK) return s;
  REQUIRE_PTR(hidden); REQUIRE_PTR(num_rows); REQUIRE_PTR(w_vocab);
  REQUIRE_PTR(argmax_tok); REQUIRE_PTR(conf);
  if (row_index != nullptr) REQUIRE_PTR(row_index);
  return enqueue_lm(max_rows, Hd, V, mask_token_id, hidden, row_index, num_rows, w_vocab,
                    argmax_tok, conf, nullptr, workspace, workspace_bytes,
                    static_cast<hipStream_t>(stream));
}

dbd_status dbd_lmhead_conf_entropy(int max_rows, int Hd, int V, int mask_token_id,
                                   const dbd_bf16* hidden, const int32_t* row_index,
                                   const int32_t* num_rows, const dbd_bf16* w_vocab,
                                   int32_t* argmax_tok, float* conf, float* entropy,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  dbd_status s = check_lm(max_rows, Hd, V, mask_token_id);
  if (s != DBD_OK) return s;
  REQUIRE_PTR(hidden); REQUIRE_PTR(num_rows); REQUIRE_PTR(w_vocab);
  REQUIRE_PTR(argmax_tok); REQUIRE_PTR(conf); REQUIRE_PTR(entropy);
  if (row_index != nullptr) REQUIRE_PTR(row_index);
  return enqueue_lm(max_rows, Hd, V, mask_token_id, hidden, row_index, num_rows, w_vocab,
                    argmax_tok, conf, entropy, workspace, workspace_bytes,
                    static_cast<hipStream_t>(stream));
}

dbd_status dbd_lmhead_sample(int max_rows, int Hd, int V, int mask_token_id,
                             const dbd_bf16* hidden, const int32_t* row_index,
                             const int32_t* num_rows, const dbd_bf16* w_vocab, float temperature,
                             uint64_t seed, uint32_t step, int32_t* token, float* conf,
                             float* entropy, void* workspace, size_t workspace_bytes,
                             void* stream) {
  dbd_status s = check_lm(max_rows, Hd, V, mask_token_id);
  if (s != DBD_OK) return s;
  REQUIRE(isfinite(temperature) && temperature > 0.f, "temperature must be finite and > 0 (got %g)",
          (double)temperature);
  REQUIRE_PTR(hidden); REQUIRE_PTR(num_rows); REQUIRE_PTR(w_vocab);
  REQUIRE_PTR(token); REQUIRE_PTR(conf);
  if (row_index != nullptr) REQUIRE_PTR(row_index);
  if (entropy != nullptr) REQUIRE_PTR(entropy);
  return enqueue_lm(max_rows, Hd, V, mask_token_id, hidden, row_index, num_rows, w_vocab, token,
                    conf, entropy, workspace, workspace_bytes, static_cast<hipStream_t>(stream), true,
                    temperature, seed, step);
}

dbd_status dbd_lmhead_logits(int max_rows, int Hd, int V, int mask_token_id,
                             const dbd_bf16* hidden, const int32_t* row_index,
                             const int32_t* num_rows, const dbd_bf16* w_vocab, float* logits,
                             void* stream) {
  dbd_status s = check_lm(max_rows, Hd, V, mask_token_id);
  if (s != DBD_OK) return s;
  REQUIRE((long)max_rows * V < (1L << 40), "max_rows*V too large");
  REQUIRE_PTR(hidden); REQUIRE_PTR(num_rows); REQUIRE_PTR(w_vocab); REQUIRE_PTR(logits);
  if (row_index != nullptr) REQUIRE_PTR(row_index);
  return enqueue_logits(max_rows, Hd, V, mask_token_id, hidden, row_index, num_rows, w_vocab, logits,
                        static_cast<hipStream_t>(stream));
}

dbd_status dbd_sample_filtered(int max_rows, int V, int mask_token_id, const float* logits,
                               const int32_t* row_index, const int32_t* num_rows,
                               float temperature, int top_k, float top_p, uint64_t seed,
                               uint32_t step, int32_t* token, float* conf, void* stream) {
  REQUIRE(max_rows >= 0, "max_rows must be >= 0 (got %d)", max_rows);
  REQUIRE(V >= 2, "vocab size must be >= 2 (got %d)", V);
  REQUIRE(mask_token_id >= 0 && mask_token_id < V, "mask_token_id %d outside [0,%d)", mask_token_id, V);
  REQUIRE(isfinite(temperature) && temperature > 0.f, "temperature must be finite and > 0 (got %g)",
          (double)temperature);
  REQUIRE(!isnan(top_p), "top_p is NaN");
  REQUIRE(top_k >= 0, "top_k must be >= 0 (got %d)", top_k);
  REQUIRE_PTR(logits); REQUIRE_PTR(num_rows); REQUIRE_PTR(token); REQUIRE_PTR(conf);
  if (row_index != nullptr) REQUIRE_PTR(row_index);
  return enqueue_filtered(max_rows, V, mask_token_id, logits, row_index, num_rows, temperature, top_k,
                          top_p, seed, step, token, conf, static_cast<hipStream_t>(stream));
}

dbd_status dbd_remask_commit(int S, int B, int mask_token_id, float dynamic_threshold,
                             uint32_t flags, int32_t* block_tokens, uint8_t* seq_state,
                             const int32_t* argmax_tok, const float* conf,
                             int32_t* row_index_out, int32_t* num_rows_out,
                             int32_t* num_committed, void* stream) {
  dbd_status s = check_remask(S, B, dynamic_threshold);
  if (s != DBD_OK) return s;
  REQUIRE((flags & ~(DBD_FALLBACK_LEFTMOST | DBD_COMPACT_ONLY)) == 0, "unknown flags 0x%x", flags);
  REQUIRE_PTR(block_tokens); REQUIRE_PTR(seq_state); REQUIRE_PTR(row_index_out);
  REQUIRE_PTR(num_rows_out);
  if (!(flags & DBD_COMPACT_ONLY)) {
    REQUIRE_PTR(argmax_tok);
    REQUIRE_PTR(conf);
  }
  if (num_committed != nullptr) REQUIRE_PTR(num_committed);
  return enqueue_remask(S, B, mask_token_id, dynamic_threshold, flags, DBD_RULE_LOW_CONF_DYNAMIC, 1,
                        0.f, nullptr, block_tokens, seq_state, argmax_tok, conf, row_index_out,
                        num_rows_out, num_committed, static_cast<hipStream_t>(stream));
}

dbd_status dbd_remask_commit_rule(int S, int B, int mask_token_id, int rule,
                                  float dynamic_threshold, int tokens_per_step,
                                  float eb_threshold, uint32_t flags, int32_t* block_tokens,
                                  uint8_t* seq_state, const int32_t* argmax_tok,
                                  const float* conf, const float* entropy,
                                  int32_t* row_index_out, int32_t* num_rows_out,
                                  int32_t* num_committed, void* stream) {
  dbd_status s = check_remask(S, B, dynamic_threshold);
  if (s != DBD_OK) return s;
  REQUIRE((flags & ~(DBD_FALLBACK_LEFTMOST | DBD_COMPACT_ONLY)) == 0, "unknown flags 0x%x", flags);
  const bool commit = !(flags & DBD_COMPACT_ONLY);
  s = check_rule(rule, eb_threshold, entropy, commit);
  if (s != DBD_OK) return s;
  REQUIRE_PTR(block_tokens); REQUIRE_PTR(seq_state); REQUIRE_PTR(row_index_out);
  REQUIRE_PTR(num_rows_out);
  if (commit) {
    REQUIRE_PTR(argmax_tok);
    if (rule == DBD_RULE_LOW_CONF_DYNAMIC || rule == DBD_RULE_LOW_CONF_STATIC) REQUIRE_PTR(conf);
  }
  if (num_committed != nullptr) REQUIRE_PTR(num_committed);
  return enqueue_remask(S, B, mask_token_id, dynamic_threshold, flags, rule, tokens_per_step,
                        eb_threshold, entropy, block_tokens, seq_state, argmax_tok, conf,
                        row_index_out, num_rows_out, num_committed,
                        static_cast<hipStream_t>(stream));
}

size_t dbd_prefill_workspace_size(int S) {
  if (S < 1) return 0;
  return dbd::prefill_ws_bytes(S);
}

dbd_status dbd_prefill_attn(int S, int T, int Hq, int Hkv, int D, int block_length,
                            const dbd_bf16* q, const dbd_bf16* k, const dbd_bf16* v,
                            const int32_t* cu_seqlens, float softmax_scale, dbd_bf16* out,
                            int page_size, int max_pages_per_seq, int num_pages,
                            const int32_t* page_table, dbd_bf16* k_cache, dbd_bf16* v_cache,
                            void* workspace, size_t workspace_bytes, void* stream) {
  REQUIRE(S >= 1 && S <= 65535, "S must be in [1,65535] (got %d)", S);
  REQUIRE(T >= 0, "T must be >= 0 (got %d)", T);
  REQUIRE(Hq >= 1 && Hkv >= 1 && Hq % Hkv == 0, "Hq (%d) must be a positive multiple of Hkv (%d)", Hq, Hkv);
  REQUIRE(dbd::prefill_rows_per_wg() % (Hq / Hkv) == 0, "Hq/Hkv must divide %d (got %d)",
          dbd::prefill_rows_per_wg(), Hq / Hkv);
  REQUIRE(block_length >= 1, "block_length must be >= 1 (got %d)", block_length);
  if (D != 64 && D != 128) return fail(DBD_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", D);
  REQUIRE((long)T * Hkv * D * 2 < (1L << 32), "T*Hkv*D*2 must be below 2^32");
  REQUIRE((long)T * (Hq / Hkv) < (1L << 31), "T*Hq/Hkv too large");
  REQUIRE(!isnan(softmax_scale), "softmax_scale is NaN");
  REQUIRE_PTR(cu_seqlens);
  if (T > 0) {
    REQUIRE_PTR(q); REQUIRE_PTR(k); REQUIRE_PTR(v); REQUIRE_PTR(out);
  }
  if (k_cache != nullptr) {
    REQUIRE_PTR(k_cache); REQUIRE_PTR(v_cache); REQUIRE_PTR(page_table);
    REQUIRE(page_size >= 1 && max_pages_per_seq >= 1 && num_pages >= 1,
            "page_size, max_pages_per_seq and num_pages must be >= 1 with a cache");
  }
  const size_t need = dbd::prefill_ws_bytes(S);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(DBD_ERR_WORKSPACE, "prefill workspace needs %zu bytes (got %zu)", need, workspace_bytes);
  REQUIRE(aligned(workspace, 256), "workspace is not 256-byte aligned");
  dbd::PrefillArgs a{};
  a.q = q; a.k = k; a.v = v; a.cu_seqlens = cu_seqlens; a.out = out;
  a.plan = static_cast<int32_t*>(workspace);
  a.S = S; a.T_total = T; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv; a.B = block_length;
  const float sc = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)D);
  a.scale_log2 = sc * 1.4426950408889634f;
  a.page_table = page_table; a.k_cache_out = k_cache; a.v_cache_out = k_cache ? v_cache : nullptr;
  a.P = page_size; a.max_pages = max_pages_per_seq; a.num_pages = num_pages;
  hipError_t e = dbd::prefill_launch(a, D, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  return DBD_OK;
}

dbd_status dbd_stream_read(const void* data, size_t bytes, uint32_t* sink, void* stream) {
  REQUIRE_PTR(data); REQUIRE_PTR(sink);
  REQUIRE(bytes % 16 == 0, "bytes must be a multiple of 16 (got %zu)", bytes);
  hipError_t e = dbd::stream_read_launch(data, bytes, sink, dbd::kStreamReadGrid,
                                         static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "stream read launch");
  return DBD_OK;
}

int dbd_stream_read_sink_words(void) { return dbd::kStreamReadGrid; }

size_t dbd_mfma_peak_operand_bytes(void) { return (size_t)dbd::kMfmaPeakSets * 16 * 64 * 16; }
int dbd_mfma_peak_sink_floats(void) { return dbd::kMfmaPeakGrid * 256; }
double dbd_mfma_peak_flops(int iters) {
  // 2 * 32 * 32 * 16 per instruction
  return iters <= 0 ? 0.0
                    : (double)dbd::kMfmaPeakGrid * 4 * iters * dbd::kMfmaPeakPerIter * 32768.0;
}

dbd_status dbd_mfma_peak(const void* operands, int iters, float* sink, void* stream) {
  REQUIRE(iters >= 1 && iters <= 4096, "iters must be in [1, 4096] (got %d)", iters);
  REQUIRE_PTR(operands);
  REQUIRE_PTR(sink);
  hipError_t e = dbd::mfma_peak_launch(operands, iters, sink, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "MFMA ceiling launch");
  return DBD_OK;
}

dbd_status dbd_round(const dbd_round_args* a, void* stream) {
  dbd_status s = check_round(a);
  if (s != DBD_OK) return s;
  return enqueue_round(a, static_cast<hipStream_t>(stream));
}

dbd_status dbd_round_noalloc(const dbd_round_args* a, void* stream) {
  dbd_status s = check_round(a, false);
  if (s != DBD_OK) return s;
  const size_t need = dbd_round_workspace_size(a);
  if (need > kScratchBytes)
    return fail(DBD_ERR_WORKSPACE,
                "round workspace needs %zu bytes, beyond the %zu-byte static scratch of dbd_round_noalloc",
                need, kScratchBytes);
  void* ws = nullptr;
  s = scratch_for_current_device(&ws);
  if (s != DBD_OK) return s;
  dbd_round_args b = *a;
  b.workspace = ws;
  b.workspace_bytes = kScratchBytes;
  return enqueue_round(&b, static_cast<hipStream_t>(stream));
}

dbd_status dbd_graph_create(const dbd_round_args* args, int n_rounds, dbd_graph** out) {
  REQUIRE(out != nullptr, "out is NULL");
  REQUIRE(args != nullptr && n_rounds >= 1, "need at least one round");
  *out = nullptr;
  for (int i = 0; i < n_rounds; ++i) {
    dbd_status s = check_round(&args[i]);
    if (s != DBD_OK) return s;
  }
  dbd_graph* g = new dbd_graph{};
  hipError_t e = hipStreamCreateWithFlags(&g->stream, hipStreamNonBlocking);
  if (e != hipSuccess) {
    delete g;
    return hip_fail(e, "hipStreamCreateWithFlags");
  }
  e = hipStreamBeginCapture(g->stream, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) {
    (void)hipStreamDestroy(g->stream);
    delete g;
    return hip_fail(e, "hipStreamBeginCapture");
  }
  dbd_status st = DBD_OK;
  for (int i = 0; i < n_rounds && st == DBD_OK; ++i) st = enqueue_round(&args[i], g->stream);
  hipGraph_t graph = nullptr;
  e = hipStreamEndCapture(g->stream, &graph);
  if (st != DBD_OK || e != hipSuccess) {
    if (graph) (void)hipGraphDestroy(graph);
    (void)hipStreamDestroy(g->stream);
    delete g;
    return st != DBD_OK ? st : hip_fail(e, "hipStreamEndCapture");
  }
  g->graph = graph;
  e = hipGraphInstantiate(&g->exec, graph, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(graph);
    (void)hipStreamDestroy(g->stream);
    delete g;
    return hip_fail(e, "hipGraphInstantiate");
  }
  *out = g;
  return DBD_OK;
}

dbd_status dbd_graph_launch(dbd_graph* g, void* stream) {
  REQUIRE(g != nullptr, "graph is NULL");
  hipError_t e = hipGraphLaunch(g->exec, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "hipGraphLaunch");
  return DBD_OK;
}

void dbd_graph_destroy(dbd_graph* g) {
  if (!g) return;
  if (g->exec) (void)hipGraphExecDestroy(g->exec);
  if (g->graph) (void)hipGraphDestroy(g->graph);
  if (g->stream) (void)hipStreamDestroy(g->stream);
  delete g;
}

dbd_status dbd_validate_inputs(int S, int B, int page_size, int max_pages_per_seq, int num_pages,
                               int V, int mask_token_id, const int32_t* page_table,
                               const int32_t* prefix_len, const int32_t* block_tokens,
                               const uint8_t* seq_state) {
  REQUIRE(S >= 1 && B >= 1 && B <= 64 && page_size >= 1 && max_pages_per_seq >= 1 && num_pages >= 0,
          "bad sizes");
  REQUIRE(V >= 2 && mask_token_id >= 0 && mask_token_id < V, "mask_token_id %d outside [0,%d)",
          mask_token_id, V);
  if (prefix_len) {
    for (int s = 0; s < S; ++s) {
      const long L = prefix_len[s];
      if (L < 0 || L > (long)max_pages_per_seq * page_size)
        return fail(DBD_ERR_INVALID_ARG, "prefix_len[%d] = %ld outside [0,%ld]", s, L,
                    (long)max_pages_per_seq * page_size);
      if (page_table) {
        const long npg = (L + page_size - 1) / page_size;
        for (long j = 0; j < npg; ++j) {
          const int p = page_table[(size_t)s * max_pages_per_seq + j];
          if (p < 0 || p >= num_pages)
            return fail(DBD_ERR_INVALID_ARG, "page_table[%d][%ld] = %d outside [0,%d)", s, j, p,
                        num_pages);
        }
      }
    }
  }
  if (block_tokens) {
    for (long i = 0; i < (long)S * B; ++i)
      if (block_tokens[i] < 0 || block_tokens[i] >= V)
        return fail(DBD_ERR_INVALID_ARG, "block_tokens[%ld] = %d outside [0,%d)", i, block_tokens[i], V);
  }
  if (seq_state) {
    for (int s = 0; s < S; ++s)
      if (seq_state[s] > DBD_FINISHED)
        return fail(DBD_ERR_INVALID_ARG, "seq_state[%d] = %d is not a state", s, seq_state[s]);
  }
  return DBD_OK;
}

}  // extern "C"
