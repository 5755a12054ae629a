"""Selective LM head with greedy confidence (test infrastructure only).

The pages run the LM head only for sequences still denoising (JetEngine
README, "Selective Logits"; developer notes, "ModelRunner": selective
logits) and only on still-masked positions (developer notes, "Optimization
History": sparse logits).  Each projected row gives the greedy token and its
confidence, the largest probability of the softmax over the vocabulary
(sampling at temperature 1 with greedy choice; SDAR page, generate.py runs
greedy generation).

Readings:
  * logits l_v = sum_k h[k] W[k][v], W stored as its transpose [V][Hd];
  * the mask token is never a candidate: its logit is treated as -inf, so it
    is out of both the argmax and the normaliser;
  * ties in the argmax go to the lowest token id;
  * confidence max_p = exp(m - lse), m = max logit, lse = log-sum-exp.

A row with no candidate (every logit other than the mask token's is -inf)
has no distribution; it gives the mask token itself with confidence 0 (and
p2 = 0), so a commit of it leaves the position masked, and entropy +inf.

Also returns the runner-up probability p2, which the tests use only to
decide which rows are near-ties.

lmhead_entropy gives each row's entropy -sum_v p_v ln p_v over the same
distribution (mask token excluded); the entropy-bounded commit rule
(developer notes, "Remasking Strategies": unmask by cumulative entropy
budget) orders positions by it.
"""
import numpy as np

from .bf16 import widen


def lmhead_logits(h_rows, w_vocab_bits, mask_id, vchunk=512):
    """float64 logits [M][V] with the mask column at -inf.

    W is widened a few hundred vocabulary rows at a time (each logit is the
    same dot product; this only bounds the float64 copy of W in memory)."""
    H = widen(h_rows)                            # [M][Hd]
    V = w_vocab_bits.shape[0]
    logits = np.empty((H.shape[0], V))
    for v0 in range(0, V, vchunk):
        W = widen(w_vocab_bits[v0:v0 + vchunk])  # [vchunk][Hd]
        logits[:, v0:v0 + vchunk] = H @ W.T
    logits[:, mask_id] = -np.inf
    return logits


def _reduce(logits, mask_id):
    m = logits.max(axis=1)
    arg = logits.argmax(axis=1)                  # first maximum = lowest id
    none = m == -np.inf                          # rows with no candidate
    e = np.exp(logits - np.where(none, 0.0, m)[:, None])
    ssum = e.sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        p1 = 1.0 / ssum                          # exp(m - lse)
        part = np.partition(e, -2, axis=1)[:, -2]
        p2 = part / ssum
    arg = np.where(none, mask_id, arg)
    p1 = np.where(none, 0.0, p1)
    p2 = np.where(none, 0.0, p2)
    return arg.astype(np.int64), p1, p2


def lmhead_rows(h_rows, w_vocab_bits, mask_id, chunk=256):
    """Greedy token, confidence and runner-up probability for each row.

    h_rows: [M][Hd] bf16 bits; w_vocab_bits: [V][Hd] bf16 bits.
    Returns (argmax [M] int64, p1 [M] float64, p2 [M] float64)."""
    M = h_rows.shape[0]
    args = np.empty(M, dtype=np.int64)
    p1 = np.empty(M)
    p2 = np.empty(M)
    for i in range(0, M, chunk):
        logits = lmhead_logits(h_rows[i:i + chunk], w_vocab_bits, mask_id)
        a, x1, x2 = _reduce(logits, mask_id)
        args[i:i + chunk], p1[i:i + chunk], p2[i:i + chunk] = a, x1, x2
    return args, p1, p2


def lmhead_entropy(h_rows, w_vocab_bits, mask_id, chunk=256):
    """Entropy in nats of each row's softmax over the vocabulary without the
    mask token: H = -sum_v p_v ln p_v, written as lse - sum_v p_v l_v.

    h_rows: [M][Hd] bf16 bits; w_vocab_bits: [V][Hd] bf16 bits.
    Returns H [M] float64."""
    M = h_rows.shape[0]
    H = np.empty(M)
    for i in range(0, M, chunk):
        logits = lmhead_logits(h_rows[i:i + chunk], w_vocab_bits, mask_id)
        m = logits.max(axis=1, keepdims=True)
        none = m[:, 0] == -np.inf                 # rows with no candidate
        z = logits - np.where(none[:, None], 0.0, m)    # -inf at the mask column
        e = np.exp(z)
        ssum = e.sum(axis=1)
        zfin = np.where(np.isfinite(z), z, 0.0)   # the mask column has p = 0
        with np.errstate(divide="ignore", invalid="ignore"):
            H[i:i + chunk] = np.log(ssum) - (e * zfin).sum(axis=1) / ssum
        H[i:i + chunk][none] = np.inf
    return H
