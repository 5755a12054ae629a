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

remask_rule adds the other strategies the developer notes list under
"Remasking Strategies" (sequential: unmask left to right;
low_confidence_static: unmask the top k by confidence; entropy_bounded:
unmask by a cumulative entropy budget).  The pages give no formula beyond
those phrases; the readings taken are:
  * static: C = the k = min(tokens_per_step, |M|) most confident positions
    of M, the lower position first among equal confidences;
  * sequential: C = the k leftmost positions of M;
  * entropy_bounded: M in ascending entropy order (lower position first on
    ties); C = the longest leading run whose running sum stays <= the
    budget eb, and never less than its first position.  The running sum is
    taken in the precision of the entropy array given, in that order.
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


RULE_DYNAMIC, RULE_STATIC, RULE_SEQUENTIAL, RULE_ENTROPY = 0, 1, 2, 3


def remask_rule(block_tokens, seq_state, conf, argmax_tok, mask_id, rule,
                tau=0.9, tokens_per_step=1, eb=0.0, entropy=None, flags=0):
    """Commit by one of the four rules; returns (new_tokens, new_state,
    committed) like remask().  conf / entropy / argmax_tok: [S*B]."""
    if rule == RULE_DYNAMIC:
        return remask(block_tokens, seq_state, conf, argmax_tok, mask_id, tau, flags)
    S, B = block_tokens.shape
    toks = np.array(block_tokens, dtype=np.int64, copy=True)
    state = np.array(seq_state, copy=True)
    committed = np.zeros((S, B), dtype=bool)
    conf = np.asarray(conf).reshape(S, B)
    argm = np.asarray(argmax_tok).reshape(S, B)
    ent = None if entropy is None else np.asarray(entropy).reshape(S, B)
    for s in range(S):
        if state[s] != DENOISING:
            continue
        masked = [i for i in range(B) if toks[s, i] == mask_id]
        chosen = []
        if masked:
            k = min(max(int(tokens_per_step), 1), len(masked))
            if rule == RULE_SEQUENTIAL:
                chosen = masked[:k]
            elif rule == RULE_STATIC:
                # repeatedly take the most confident remaining position
                rest = list(masked)
                for _ in range(k):
                    best = rest[0]
                    for i in rest[1:]:
                        if conf[s, i] > conf[s, best]:
                            best = i
                    chosen.append(best)
                    rest.remove(best)
            elif rule == RULE_ENTROPY:
                order = sorted(masked, key=lambda i: (ent[s, i], i))
                cum = ent.dtype.type(0)
                budget = ent.dtype.type(eb)
                for i in order:
                    nxt = ent.dtype.type(cum + ent[s, i])
                    if chosen and nxt > budget:
                        break
                    chosen.append(i)
                    cum = nxt
            else:
                raise ValueError(f"unknown rule {rule}")
            for i in chosen:
                toks[s, i] = argm[s, i]
                committed[s, i] = True
        if not np.any(toks[s] == mask_id):
            state[s] = SAVING
    return toks, state, committed
