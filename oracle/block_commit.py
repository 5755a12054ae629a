"""The SAVING step and the block commit (test infrastructure only).

A block whose masks are all gone is not finished yet: its sequence sits in
SAVING, and one more forward over the final tokens writes their keys and
values into the paged cache (JetEngine developer notes, "Important
Patterns": the SAVING forward writes the final block's representations into
the KV cache, and skipping it corrupts the cache; "Optimization History":
the FA3 kernel writes the cache and attends in one kernel).  Then
commit_block moves the block into the sequence's token stream (developer
notes, "Sequence"), and the sequence starts a new all-mask block
(developer notes, "Scheduler": WAITING -> PREFILLING -> DENOISING -> SAVING
-> FINISHED; "Chain Mechanism": one chain holds the denoise steps and the
SAVING step, and chains run across SAVING).

Readings of points the pages leave open:
  * the block's tokens occupy absolute positions prefix_len .. prefix_len+B-1
    of the sequence, so their keys and values go to logical cache positions
    prefix_len + j, found through the page table like prefix tokens
    (page page_table[s][p // P], offset p % P); the caller has assigned the
    pages that cover them;
  * the keys and values written are the SAVING forward's own (an input
    here, as every forward's keys and values are: no model is in the loop);
  * that forward's attention is the ordinary denoise attention (prefix plus
    block, bidirectional in the block): kv_save changes nothing it reads;
  * the token stream holds token p of the sequence at index p; commit_block
    writes the block at prefix_len .. prefix_len+B-1 (indices past the
    stream's capacity are dropped), adds B to prefix_len, refills the block
    with the mask token and sets the state back to DENOISING, or to
    FINISHED once prefix_len reaches the sequence's end length (prompt plus
    max_tokens, SamplingParams in the README's usage examples); a FINISHED
    sequence keeps its last block;
  * in one step, a sequence that is SAVING when the step starts is committed,
    and a DENOISING one goes through the commit rule; a sequence that the
    rule moves to SAVING is committed only in the next step, after its own
    SAVING forward.
"""
import numpy as np

from .remask import DENOISING, SAVING, remask_rule, compact_rows

FINISHED = 4


def kv_save(k_cache, v_cache, page_table, prefix_len, seq_state, k_blk, v_blk):
    """Copies of the caches with each SAVING sequence's block keys and values
    written at its positions prefix_len+j.  Caches are [pages][Hkv][P][D]
    bf16 bits; k_blk, v_blk are [S][B][Hkv][D] bf16 bits."""
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    P = kc.shape[2]
    S, B = k_blk.shape[:2]
    for s in range(S):
        if seq_state[s] != SAVING:
            continue
        L = int(prefix_len[s])
        for j in range(B):
            p = L + j
            page = int(page_table[s][p // P])
            kc[page, :, p % P, :] = k_blk[s, j]
            vc[page, :, p % P, :] = v_blk[s, j]
    return kc, vc


def commit_block(block_tokens, seq_state, prefix_len, mask_id, token_stream=None,
                 end_len=None):
    """Commits every SAVING sequence's block.  Returns (tokens, state,
    prefix_len, token_stream); the inputs are not modified."""
    toks = np.array(block_tokens, dtype=np.int64, copy=True)
    state = np.array(seq_state, copy=True)
    L = np.array(prefix_len, dtype=np.int64, copy=True)
    ts = None if token_stream is None else np.array(token_stream, copy=True)
    S, B = toks.shape
    for s in range(S):
        if state[s] != SAVING:
            continue
        if ts is not None:
            for j in range(B):
                if L[s] + j < ts.shape[1]:
                    ts[s, L[s] + j] = toks[s, j]
        L[s] += B
        if end_len is not None and L[s] >= end_len[s]:
            state[s] = FINISHED
        else:
            toks[s, :] = mask_id
            state[s] = DENOISING
    return toks, state, L, ts


def step_commit(block_tokens, seq_state, prefix_len, conf, argmax_tok, mask_id, rule,
                tau=0.9, tokens_per_step=1, eb=0.0, entropy=None, flags=0,
                token_stream=None, end_len=None):
    """The end of one step: the commit rule for sequences DENOISING on entry,
    the block commit for those SAVING on entry.  Returns (tokens, state,
    prefix_len, token_stream, committed, next_rows)."""
    saving0 = np.asarray(seq_state) == SAVING
    toks, state, committed = remask_rule(block_tokens, seq_state, conf, argmax_tok,
                                         mask_id, rule, tau=tau,
                                         tokens_per_step=tokens_per_step, eb=eb,
                                         entropy=entropy, flags=flags)
    # commit only the sequences that were SAVING on entry
    only = np.where(saving0, SAVING, 0).astype(state.dtype)
    t2, st2, L2, ts2 = commit_block(toks, only, prefix_len, mask_id, token_stream, end_len)
    state = np.where(saving0, st2, state).astype(state.dtype)
    toks = np.where(saving0[:, None], t2, toks)
    return toks, state, L2, ts2, committed, compact_rows(toks, state, mask_id)
