"""Threshold remasking, literally (test infrastructure only).

The rule is JetEngine's low_confidence_dynamic (developer notes, "Remasking
Strategies": unmask every position above the threshold, with a fallback;
README usage examples with dynamic_threshold 0.90; dInfer blog, threshold
decoding), applied to DENOISING sequences only; a sequence whose block has
no mask left moves to SAVING (developer notes, "Scheduler" state machine).

Per DENOISING sequence with masked set M (positions holding mask_id):
  C = { i in M : conf_i >= tau }
  if C is empty and M is not: C = { the most confident i in M }, lowest i on
      ties (flags & FALLBACK_LEFTMOST: the leftmost i in M, the "fallback
      to sequential" the developer notes name);
  tok_i <- argmax_i for i in C;
  if no mask_id is left in the block: state <- SAVING.
A DENOISING sequence with M empty on entry goes to SAVING with no commit;
other states are untouched.

conf is compared as given (the caller decides its precision; the GPU path
passes float32 confidences and a float32 threshold).
"""
import numpy as np

DENOISING, SAVING = 2, 3
FALLBACK_LEFTMOST = 1


def remask(block_tokens, seq_state, conf, argmax_tok, mask_id, tau, flags=0):
    """Returns (new_tokens [S][B], new_state [S], committed [S][B] bool).

    conf, argmax_tok: [S*B] (row s*B+i); only masked positions of DENOISING
    sequences are read."""
    S, B = block_tokens.shape
    toks = np.array(block_tokens, dtype=np.int64, copy=True)
    state = np.array(seq_state, copy=True)
    committed = np.zeros((S, B), dtype=bool)
    conf = np.asarray(conf).reshape(S, B)
    argm = np.asarray(argmax_tok).reshape(S, B)
    for s in range(S):
        if state[s] != DENOISING:
            continue
        masked = [i for i in range(B) if toks[s, i] == mask_id]
        if masked:
            chosen = [i for i in masked if conf[s, i] >= tau]
            if not chosen:
                if flags & FALLBACK_LEFTMOST:
                    chosen = [masked[0]]
                else:
                    best = masked[0]
                    for i in masked[1:]:
                        if conf[s, i] > conf[s, best]:
                            best = i
                    chosen = [best]
            for i in chosen:
                toks[s, i] = argm[s, i]
                committed[s, i] = True
        if not np.any(toks[s] == mask_id):
            state[s] = SAVING
    return toks, state, committed


def compact_rows(block_tokens, seq_state, mask_id):
    """Rows s*B+i of still-masked positions of DENOISING sequences, in
    sequence-major, position-minor order: the row set the next round's LM
    head projects."""
    S, B = block_tokens.shape
    rows = [s * B + i for s in range(S) if seq_state[s] == DENOISING
            for i in range(B) if block_tokens[s, i] == mask_id]
    return np.asarray(rows, dtype=np.int64)
