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
passes float32 confidences and a float32 threshold).  A NaN confidence is
never >= tau and ranks below every number (-inf included) in the fallback
and in the static rule; when every masked confidence is NaN the fallback
takes the lowest masked position.  Likewise a NaN entropy ranks after every
number (+inf included) and counts as +inf in the entropy budget.  The pages
never produce NaN; this only fixes what the rule does with one.

A position is masked while it holds mask_id, also after a commit that wrote
mask_id itself (a row with no candidate token; lmhead_rows gives it the mask
id with confidence 0): such a sequence stays DENOISING.

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
                    chosen = [_most_confident(masked, conf[s])]
            for i in chosen:
                toks[s, i] = argm[s, i]
                committed[s, i] = True
        if not np.any(toks[s] == mask_id):
            state[s] = SAVING
    return toks, state, committed


def _most_confident(positions, conf_row):
    """The position of the largest confidence, the lowest position among
    equal ones; NaN ranks below every number, and when every confidence is
    NaN the lowest position is taken."""
    best = None
    for i in positions:
        if np.isnan(conf_row[i]):
            continue
        if best is None or conf_row[i] > conf_row[best]:
            best = i
    return positions[0] if best is None else best


def _entropy_order(positions, ent_row):
    """Positions by ascending entropy, the lower position first among equal
    ones; NaN entropies after every number (+inf included), by position."""
    nums = sorted((i for i in positions if not np.isnan(ent_row[i])), key=lambda i: (ent_row[i], i))
    return nums + [i for i in positions if np.isnan(ent_row[i])]


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
                    best = _most_confident(rest, conf[s])
                    chosen.append(best)
                    rest.remove(best)
            elif rule == RULE_ENTROPY:
                order = _entropy_order(masked, ent[s])
                cum = ent.dtype.type(0)
                budget = ent.dtype.type(eb)
                for i in order:
                    e_i = ent.dtype.type(np.inf) if np.isnan(ent[s, i]) else ent[s, i]
                    with np.errstate(invalid="ignore"):        # inf + -inf stays NaN
                        nxt = ent.dtype.type(cum + e_i)
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
