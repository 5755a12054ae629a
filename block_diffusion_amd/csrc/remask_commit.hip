// Remask by a commit rule, and row compaction, gfx950.
//
// The remasking strategies of JetEngine's scheduler (developer notes,
// "Remasking Strategies"), applied to DENOISING sequences, and the state
// change to SAVING once a block holds no mask (developer notes,
// "Scheduler"):
//   rule 0, low_confidence_dynamic: every masked position with confidence
//     >= the threshold; if none, the most confident (lowest position on
//     ties), or the leftmost with DBD_FALLBACK_LEFTMOST;
//   rule 1, low_confidence_static: the k most confident masked positions
//     (lower position first on ties);
//   rule 2, sequential: the k leftmost masked positions;
//   rule 3, entropy_bounded: masked positions in ascending entropy (lower
//     position first on ties), the longest leading run whose float32 running
//     sum stays within the budget, at least one.
// Confidences, entropies and the threshold are compared in float32.  A NaN
// confidence ranks below every number, a NaN entropy after every number; a
// position stays masked while it holds the mask token, also when a commit
// wrote the mask token itself (the LM head's answer for a row with no
// candidate token).
//
// Block commit (kCommitSaving): a sequence that is SAVING on entry has had
// its SAVING forward (the attention launch wrote its block into the KV
// cache), so its block is committed (developer notes, "Sequence":
// commit_block puts the block into the token stream): the block goes to
// token_stream[s][prefix_len .. prefix_len+B-1] (positions past the
// stream's capacity are dropped), prefix_len grows by B, and the sequence
// starts a new all-mask block in DENOISING, or is FINISHED (keeping its
// block) once prefix_len reaches end_len[s].  A sequence that the rule
// fills in this launch stays SAVING until its own SAVING forward.
//
// One workgroup of 16 waves.  Pass 1: a wave holds 64/SEGW sequences at
// once (SEGW = the power of two >= B), one per segment of lanes, lane =
// block position within it: ballots of the masked set; the rule's choice is
// built one segment-wide selection at a time (max or min, then the lowest
// position).
// The still-masked set of each sequence is kept as a 64-bit mask in LDS.
// Pass 2: exclusive scan of the per-sequence counts.  Pass 3: each
// still-masked position writes s*B+i at its rank, so the list is
// sequence-major and position-minor, the same on every run.
#include "dbd_device.hpp"
#include "dbd_internal.hpp"

namespace dbd {

constexpr uint32_t kFallbackLeftmost = 1u;
constexpr uint32_t kCompactOnly = 2u;
constexpr uint8_t kDenoising = 2, kSaving = 3, kFinished = 4;

__global__ __launch_bounds__(1024) void remask_kernel(RemaskArgs a) {
  __shared__ unsigned long long s_left[kRemaskMaxSeqs];
  __shared__ int s_off[kRemaskMaxSeqs];
  __shared__ int s_wsum[16];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int S = a.S, B = a.B;
  // rows_in may alias num_rows_out: read it before pass 2 writes the count
  if (a.round_counter != nullptr && tid == 0 && *a.rows_in > 0) *a.round_counter += 1;

  // A wave holds NSEG sequences at once, one per segment of SEGW lanes
  // (SEGW = the power of two >= B); lane = segment * SEGW + position.
  // Ballots are cut to the segment's bits, and reductions shuffle with
  // offsets below SEGW, so they stay inside the segment; every branch on a
  // sequence's data is taken by all lanes of its segment together.
  const int SEGW = B <= 1 ? 1 : 1 << (32 - __clz(B - 1));
  const int NSEG = 64 / SEGW;
  const int seg = lane / SEGW, pos = lane % SEGW;
  const unsigned long long segmask = SEGW == 64 ? ~0ull : ((1ull << SEGW) - 1ull);
  auto sball = [&](bool p) { return (__ballot(p) >> (seg * SEGW)) & segmask; };
  auto seg_max = [&](float x) {
    for (int off = SEGW >> 1; off >= 1; off >>= 1) x = fmaxf(x, shfl_xor_f(x, off));
    return x;
  };
  auto seg_min = [&](float x) {
    for (int off = SEGW >> 1; off >= 1; off >>= 1) x = fminf(x, shfl_xor_f(x, off));
    return x;
  };

  // pass 1: commit, state, still-masked set
  for (int base = wave * NSEG; base < S; base += 16 * NSEG) {
    const int s = base + seg;
    const bool live = s < S;
    const uint8_t st = live ? a.seq_state[s] : (uint8_t)0;   // same on the segment's lanes
    const bool in = live && pos < B;
    if (live && st == kSaving && (a.flags & kCommitSaving)) {
      const int L = a.prefix_len[s];
      if (a.token_stream != nullptr && in && L + pos >= 0 && L + pos < a.stream_cap)
        a.token_stream[(size_t)s * a.stream_cap + L + pos] = a.block_tokens[s * B + pos];
      const int L2 = L + B;
      const bool fin = a.end_len != nullptr && L2 >= a.end_len[s];
      if (in && !fin) a.block_tokens[s * B + pos] = a.mask_id;
      if (pos == 0) {
        a.prefix_len[s] = L2;
        a.seq_state[s] = fin ? kFinished : kDenoising;
        if (a.num_committed && !(a.flags & kCompactOnly)) a.num_committed[s] = 0;
      }
      const unsigned long long fresh = sball(in && !fin);
      if (pos == 0) s_left[s] = fresh;
      continue;
    }
    const bool den = st == kDenoising;
    const bool masked = in && den && a.block_tokens[s * B + pos] == a.mask_id;
    const unsigned long long mball = sball(masked);
    bool still = masked;
    if (live && den && !(a.flags & kCompactOnly)) {
      unsigned long long cball = 0ull;
      if (a.rule == 0) {
        const float c = masked ? a.conf[s * B + pos] : -INFINITY;
        cball = sball(masked && c >= a.tau);
        if (cball == 0ull && mball != 0ull) {
          if (a.flags & kFallbackLeftmost) {
            cball = mball & (~mball + 1ull);  // lowest set bit
          } else {
            // NaN ranks below every number; with every masked value NaN
            // the tie is empty and the lowest masked position is taken
            const float best = seg_max(c);
            unsigned long long tie = sball(masked && c == best);
            if (tie == 0ull) tie = mball;
            cball = tie & (~tie + 1ull);
          }
        }
      } else if (a.rule == 2) {
        // the k lowest set bits of the masked set
        unsigned long long rest = mball;
        for (int r = 0; r < a.k && rest != 0ull; ++r) {
          const unsigned long long low = rest & (~rest + 1ull);
          cball |= low;
          rest ^= low;
        }
      } else if (a.rule == 1) {
        // k times: the most confident remaining position, lowest on ties
        const float c = masked ? a.conf[s * B + pos] : -INFINITY;
        unsigned long long rest = mball;
        for (int r = 0; r < a.k && rest != 0ull; ++r) {
          const bool cand = (rest >> pos) & 1ull;
          const float best = seg_max(cand ? c : -INFINITY);
          unsigned long long tie = sball(cand && c == best);
          if (tie == 0ull) tie = rest;   // every remaining value is -inf or NaN
          const unsigned long long pick = tie & (~tie + 1ull);
          cball |= pick;
          rest ^= pick;
        }
      } else {
        // ascending entropy; stop before the running sum passes the budget
        const float e = masked ? a.entropy[s * B + pos] : INFINITY;
        unsigned long long rest = mball;
        float run = 0.f;
        while (rest != 0ull) {
          const bool cand = (rest >> pos) & 1ull;
          const float lo = seg_min(cand ? e : INFINITY);
          unsigned long long tie = sball(cand && e == lo);
          if (tie == 0ull) tie = rest;   // every remaining value is +inf or NaN
          const unsigned long long pick = tie & (~tie + 1ull);
          const float nxt = run + lo;
          if (cball != 0ull && nxt > a.eb) break;
          cball |= pick;
          rest ^= pick;
          run = nxt;
        }
      }
      const bool commit = (cball >> pos) & 1ull;
      int tok = 0;
      if (commit) {
        tok = a.argmax_tok[s * B + pos];
        a.block_tokens[s * B + pos] = tok;
      }
      // a commit of the mask token itself (a row with no candidate) leaves
      // the position masked
      still = masked && (!commit || tok == a.mask_id);
      const unsigned long long left = sball(still);
      if (pos == 0) {
        if (left == 0ull) a.seq_state[s] = kSaving;
        if (a.num_committed) a.num_committed[s] = __popcll(cball);
      }
    } else if (live && !(a.flags & kCompactOnly) && a.num_committed && pos == 0) {
      a.num_committed[s] = 0;
    }
    const unsigned long long left = sball(still);
    if (live && pos == 0) s_left[s] = left;
  }
  __syncthreads();

  // pass 2: exclusive scan of per-sequence counts
  const int per = (S + 1023) / 1024;
  const int b0 = tid * per;
  int local = 0;
  for (int j = 0; j < per; ++j)
    if (b0 + j < S) local += __popcll(s_left[b0 + j]);
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  int wpre = 0;
  for (int w = 0; w < wave; ++w) wpre += s_wsum[w];
  int run = wpre + incl - local;
  for (int j = 0; j < per; ++j)
    if (b0 + j < S) {
      s_off[b0 + j] = run;
      run += __popcll(s_left[b0 + j]);
    }
  if (tid == 1023) *a.num_rows_out = wpre + incl;
  __syncthreads();

  // pass 3: scatter row ids, NSEG sequences per wave as in pass 1
  for (int base = wave * NSEG; base < S; base += 16 * NSEG) {
    const int s = base + seg;
    if (s >= S || pos >= B) continue;
    const unsigned long long left = s_left[s];
    if ((left >> pos) & 1ull) {
      const unsigned long long below = pos ? (left & ((1ull << pos) - 1ull)) : 0ull;
      a.row_index_out[s_off[s] + __popcll(below)] = s * B + pos;
    }
  }
}

hipError_t remask_launch(const RemaskArgs& a, hipStream_t st) {
  remask_kernel<<<1, 1024, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace dbd
