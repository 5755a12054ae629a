"""One denoise round: attention, selective LM head, threshold remask
(test infrastructure only).

The round as the JetEngine developer notes describe a denoise step (Engine:
step() runs the batch through the model, then postprocesses logits through
the scheduler; ModelRunner: the LM head runs only where needed).  Attention
runs for every sequence of the batch; the LM head and the remask only for
DENOISING sequences, on their masked positions.  With no model in the loop,
the hidden states the LM head projects are round inputs, not a function of
the attention output.
"""
import numpy as np

from .attention import attention
from .lmhead import lmhead_rows
from .remask import remask, compact_rows


def denoise_round(inp, fixed, mask_id, tau, flags=0, block_tokens=None,
                  seq_state=None, scale=None, with_attention=True):
    """inp: per-round inputs (q, k_blk, v_blk, hidden as bf16 bits);
    fixed: prefix_len, page_table, k_cache, v_cache, w_vocab.
    Starts from (block_tokens, seq_state) if given, else fixed's initial
    block.  Returns a dict of every intermediate."""
    toks = fixed.block_tokens0 if block_tokens is None else block_tokens
    state = fixed.seq_state0 if seq_state is None else seq_state
    S, B = toks.shape
    out = None
    if with_attention:
        out = attention(inp.q, inp.k_blk, inp.v_blk, fixed.k_cache,
                        fixed.v_cache, fixed.page_table, fixed.prefix_len,
                        scale)
    rows = compact_rows(toks, state, mask_id)
    conf = np.full(S * B, np.nan)
    arg = np.full(S * B, -1, dtype=np.int64)
    p2 = np.full(S * B, np.nan)
    if rows.size:
        a, x1, x2 = lmhead_rows(inp.hidden[rows], fixed.w_vocab, mask_id)
        arg[rows], conf[rows], p2[rows] = a, x1, x2
    new_toks, new_state, committed = remask(toks, state, conf, arg, mask_id,
                                            tau, flags)
    return dict(attn=out, rows=rows, argmax=arg, p1=conf, p2=p2,
                tokens=new_toks, state=new_state, committed=committed,
                next_rows=compact_rows(new_toks, new_state, mask_id))
