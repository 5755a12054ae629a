"""Temperature sampling of each masked position's token (test
infrastructure only).

The pages' SamplingParams carry a temperature (JetEngine README usage
examples: temperature 1.0 with topk 0 and topp 1.0, i.e. no filtering;
developer notes, "Benchmarking": 0.6), and the scheduler's postprocess
samples a token for every masked position before a remasking strategy picks
which to commit (developer notes, "Scheduler": postprocessing is sampling
plus token selection).  The pages give no formula.  Readings taken:
  * the token is drawn from softmax(l / T) over the vocabulary without the
    mask token;
  * the confidence the commit rules read is the model's probability of
    that token, softmax(l) at temperature 1 without the mask token (so as
    T -> 0 the pair becomes the greedy token and max_p);
  * random numbers come from Philox4x32-10 (Salmon, Moraes, Dror, Shaw,
    "Parallel random numbers: as easy as 1, 2, 3", SC 2011), key = the
    64-bit seed (low word, high word), counter = (chunk, row id, step, 0),
    where the row id is s*B + position and step is the caller's round
    number; a 32-bit word w gives the uniform ((w >> 9) + 0.5) / 2^23 in
    (0, 1), exact in float32;
  * the draw is exact and hierarchical (a reading: the pages name no
    sampler).  Every token v belongs to one *block* (c, h) with
    c = v div 32 and h = (v div 4) mod 2: each aligned run of 32 ids is cut
    into the two interleaved sets of ids whose bit 2 is 0 or 1, 16 ids each
    (fewer at the end of the vocabulary).  Philox(c, row, step, 0) gives
    four words per c; block (c, h) uses word 2h for u and word 2h+1 for e.
    Per block, with z = l / T and the mask token at weight 0:
      m_b = max z,  S_b = sum exp(z - m_b)   (members in increasing id),
      candidate = the first member whose running sum of exp(z - m_b)
                  reaches u * S_b (inverse CDF inside the block; if
                  rounding leaves none, the last member with weight),
      G_b = m_b + ln S_b - ln(-ln e)   (a Gumbel draw located at the
                                        block's log-sum-exp);
    the token is the candidate of the block with the largest G_b (lower
    candidate id on equal G_b).  The largest of independent Gumbel variables
    located at log-sum-exps falls on block b with probability proportional
    to its sum of exp(z), independently of its value, so the token has
    probability exp(z_v) / sum exp(z) -- the Gumbel-max trick applied to
    blocks instead of single tokens (16 times fewer random numbers).  Any
    partition of the vocabulary into blocks gives that distribution; this
    one fixes which random words decide which token, so that a draw does
    not depend on how the vocabulary is split among workers.
  * a row with no candidate (every weight 0) draws the mask token with
    confidence 0.

Top-k / top-p filtering (README usage examples: topk, topp; developer
notes, "Benchmarking": top_p 0.95; "Ruled-Out Optimizations": a separate
sampler after the logits was faster than a fused one).  Readings:
  * tokens other than the mask token are ranked by logit, higher first, the
    lower id first among equal logits; only finite logits take part (the
    mask column arrives as -inf from the LM head, so it never does);
  * top_k > 0 keeps the first top_k of that ranking (all if fewer);
  * top_p < 1 then keeps the shortest leading run of the kept tokens whose
    running sum of exp((l - m) / T) reaches top_p times their total (at
    least one token), i.e. top-p applies to the top-k distribution;
  * the draw is the block draw above with every token outside the kept set
    given zero weight; the confidence is unchanged (the model's
    probability of the drawn token at temperature 1).
"""
import math

import numpy as np

from .lmhead import lmhead_logits

_MASK32 = np.uint64(0xFFFFFFFF)
_M0, _M1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
_W0, _W1 = np.uint64(0x9E3779B9), np.uint64(0xBB67AE85)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32 with 10 rounds, elementwise over arrays of 32-bit values
    (held in uint64).  Each round multiplies words 0 and 2 by the two
    multipliers, takes the high and low halves of the 64-bit products and
    mixes them with words 1 and 3 and the key; the key is bumped by the two
    Weyl constants between rounds."""
    c = [np.asarray(x, dtype=np.uint64) & _MASK32 for x in (c0, c1, c2, c3)]
    k = [np.asarray(x, dtype=np.uint64) & _MASK32 for x in (k0, k1)]
    for _ in range(10):
        p0 = _M0 * c[0]
        p1 = _M1 * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c = [hi1 ^ c[1] ^ k[0], lo1, hi0 ^ c[3] ^ k[1], lo0]
        k = [(k[0] + _W0) & _MASK32, (k[1] + _W1) & _MASK32]
    return c


def uniform01(words):
    """23-bit uniform in (0, 1): ((w >> 9) + 0.5) / 2^23."""
    w = np.asarray(words, dtype=np.uint64)
    return ((w >> np.uint64(9)).astype(np.float64) + 0.5) / float(1 << 23)


def block_of(v):
    """The sampling block (c, h) of token id v (ints or integer arrays)."""
    return v // 32, (v // 4) % 2


def block_members(c, h, V):
    """Token ids of block (c, h) in increasing order, ids >= V left out."""
    return [v for v in range(32 * c, min(32 * c + 32, V)) if block_of(v) == (c, h)]


def block_words(seed, row_id, step, nchunks):
    """Philox words [nchunks][4] of counter (c, row id, step, 0), key = seed."""
    w = philox4x32_10(np.arange(nchunks), np.full(nchunks, row_id), np.full(nchunks, step),
                      np.zeros(nchunks), np.full(nchunks, seed & 0xFFFFFFFF),
                      np.full(nchunks, (seed >> 32) & 0xFFFFFFFF))
    return np.stack(w, axis=1)


def _inverse_cdf(wt, members, u):
    """The draw inside one block: wt [V] are the weights exp(z - m_b) (0 for
    no weight); the first member, in id order, whose running sum reaches
    u * S_b, or the last member with weight if rounding leaves none.
    Returns (candidate, margin of u * S_b from the candidate's interval,
    relative to S_b)."""
    S_b = 0.0
    for v in members:
        S_b += wt[v]
    target = u * S_b
    cum, cand, last, lo_c, hi_c = 0.0, None, None, 0.0, 0.0
    for v in members:
        before = cum
        cum += wt[v]
        if wt[v] > 0.0:
            last = v
            if cand is None and cum >= target:
                cand, lo_c, hi_c = v, before, cum
    if cand is None:
        cand, lo_c, hi_c = last, target, target
    return cand, min(abs(target - lo_c), abs(hi_c - target)) / S_b


def sample_row(logits, temperature, seed, row_id, step, keep=None, words=None, mask_id=-1):
    """One row: logits [V] float64 (mask token at -inf).  Returns
    (token, conf, info) where info holds what the tests need to recognise
    draws that float32 rounding could decide otherwise: the gap between the
    two largest G_b, the runner-up block's candidate, the winning block's
    distance from its inverse-CDF boundaries (relative to S_b), and that
    block's members of nonzero weight.  keep (bool [V], optional): only
    these tokens can be drawn.  words ([chunks][4] uint32, optional): the
    random words to use instead of Philox's (hand-worked cases).  A row
    with no candidate gives (mask_id, 0)."""
    V = logits.shape[0]
    z = np.asarray(logits, dtype=np.float64) / temperature
    if keep is not None:
        z = np.where(np.asarray(keep, dtype=bool), z, -np.inf)
    nc = -(-V // 32)
    if words is None:
        words = block_words(seed, row_id, step, nc)
    words = np.asarray(words, dtype=np.uint64)
    # block of every token, as one index 2c + h
    c_of, h_of = block_of(np.arange(V))
    b_of = 2 * c_of + h_of
    # block maxima, then block sums of exp(z - m_b) accumulated in id order
    # (np.add.at applies its additions in index order, unbuffered)
    m = np.full(2 * nc, -np.inf)
    np.maximum.at(m, b_of, z)
    with np.errstate(invalid="ignore"):
        wt = np.where(z > -np.inf, np.exp(z - m[b_of]), 0.0)
    S = np.zeros(2 * nc)
    np.add.at(S, b_of, wt)
    live = m > -np.inf
    info = dict(g_gap=np.inf, runner_up=-1, cdf_margin=np.inf, block=set())
    if not live.any():
        return int(mask_id), 0.0, info
    # block (c, h): u from word 2h, e from word 2h + 1 of chunk c
    blocks = np.arange(2 * nc)
    u = uniform01(words[blocks // 2, 2 * (blocks % 2)])
    e = uniform01(words[blocks // 2, 2 * (blocks % 2) + 1])
    with np.errstate(divide="ignore"):
        G = np.where(live, m + np.log(np.where(live, S, 1.0)) - np.log(-np.log(e)), -np.inf)
    cands = {}

    def cand_of(b):
        if b not in cands:
            cands[b] = _inverse_cdf(wt, block_members(b // 2, b % 2, V), float(u[b]))
        return cands[b][0]
    # largest G_b first, the lower candidate first among equal G_b
    g1 = G.max()
    win = min(np.nonzero(G == g1)[0].tolist(), key=cand_of)
    tok = cand_of(win)
    rest = np.nonzero(live & (blocks != win))[0]
    if rest.size:
        g2 = G[rest].max()
        ru = min(rest[G[rest] == g2].tolist(), key=cand_of)
        info["g_gap"] = float(g1 - g2)
        info["runner_up"] = int(cand_of(ru))
    info["cdf_margin"] = float(cands[win][1])
    info["block"] = set(v for v in block_members(win // 2, win % 2, V) if wt[v] > 0.0)
    fin = logits[np.isfinite(logits)]
    lmax = fin.max()
    lse = lmax + math.log(float(np.sum(np.exp(fin - lmax))))
    conf = float(math.exp(logits[tok] - lse))
    return int(tok), conf, info


def lmhead_sample(h_rows, w_vocab_bits, mask_id, row_ids, temperature, seed, step, chunk=64):
    """Sampled token and confidence of each row (h_rows [M][Hd] bf16 bits,
    row_ids [M] = s*B + position).  Returns (tokens [M], conf [M], infos)."""
    M = h_rows.shape[0]
    toks = np.empty(M, dtype=np.int64)
    conf = np.empty(M)
    infos = []
    for i0 in range(0, M, chunk):
        L = lmhead_logits(h_rows[i0:i0 + chunk], w_vocab_bits, mask_id)
        for j in range(L.shape[0]):
            t, c, inf = sample_row(L[j], temperature, seed, int(row_ids[i0 + j]), step,
                                   mask_id=mask_id)
            toks[i0 + j], conf[i0 + j] = t, c
            infos.append(inf)
    return toks, conf, infos


def topk_topp_keep(logits, temperature, top_k, top_p):
    """The kept set of the filtering readings above: bool [V], and info on
    the top-p boundary (its margin relative to the kept total, and the kept
    sets one token shorter and one longer) for the tests."""
    V = logits.shape[0]
    cand = np.nonzero(np.isfinite(logits))[0]
    order = cand[np.lexsort((cand, -logits[cand]))]      # higher logit, then lower id
    n = order.size
    k = n if (top_k <= 0 or top_k >= n) else int(top_k)
    kept = order[:k]
    info = dict(margin=np.inf, shorter=None, longer=None)
    if top_p < 1.0 and n > 0:
        m = logits[order[0]]
        w = np.exp((logits[kept] - m) / temperature)
        cum = np.cumsum(w)
        target = top_p * cum[-1]
        j = min(int(np.searchsorted(cum, target, side="left")), k - 1)
        lo = cum[j - 1] if j > 0 else 0.0
        info["margin"] = float(min(abs(target - lo), abs(cum[j] - target)) / cum[-1])
        mk = lambda jj: np.isin(np.arange(V), kept[:jj + 1])
        info["shorter"] = mk(max(j - 1, 0))
        info["longer"] = mk(min(j + 1, k - 1))
        kept = kept[:j + 1]
    keep = np.zeros(V, dtype=bool)
    keep[kept] = True
    return keep, info


def sample_filtered(logits, temperature, top_k, top_p, seed, row_id, step, mask_id=-1):
    """One row drawn after top-k / top-p filtering.  Returns (token, conf,
    info) like sample_row, info also holding the filter's boundary info.  A
    row with no candidate gives (mask_id, 0)."""
    keep, finfo = topk_topp_keep(logits, temperature, top_k, top_p)
    tok, conf, info = sample_row(logits, temperature, seed, row_id, step, keep, mask_id=mask_id)
    info["filter"] = finfo
    info["keep"] = keep
    return tok, conf, info
