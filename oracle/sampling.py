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
  * the draw is exact and hierarchical.  The vocabulary is cut into blocks:
    chunk c = tokens 32c .. 32c+31, and its half h in {0, 1} holds the 16
    tokens 32c + 8q + 4h + r (q, r in 0..3), in increasing id, without the
    mask token and ids >= V.  Philox(c, row, step, 0) gives four words; half
    h uses word 2h for u and word 2h+1 for e.  Per block, with z = l / T:
      m_b = max z,  S_b = sum exp(z - m_b),
      candidate = the first member whose running sum of exp(z - m_b)
                  reaches u * S_b (inverse CDF inside the block),
      G_b = m_b + ln S_b - ln(-ln e)   (a Gumbel draw located at the
                                        block's log-sum-exp);
    the token is the candidate of the block with the largest G_b (lower
    candidate id on equal G_b).  The largest of independent Gumbel variables
    located at log-sum-exps falls on block b with probability proportional
    to its sum of exp(z), independently of its value, so the token has
    probability exp(z_v) / sum exp(z) -- the Gumbel-max trick applied to
    blocks instead of single tokens (16 times fewer random numbers).

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


def sample_row(logits, temperature, seed, row_id, step, keep=None):
    """One row: logits [V] float64 (mask token at -inf).  Returns
    (token, conf, info) where info holds what the tests need to recognise
    draws that float32 rounding could decide otherwise: the gap between the
    two largest G_b, the runner-up block's candidate, and the winning
    block's distance from its inverse-CDF boundaries (relative to S_b) with
    the neighbouring candidates.  keep (bool [V], optional): only these
    tokens can be drawn."""
    V = logits.shape[0]
    nc = -(-V // 32)
    z = np.full(nc * 32, -np.inf)
    z[:V] = logits / temperature
    if keep is not None:
        z[:V][~np.asarray(keep, dtype=bool)] = -np.inf
    ids = np.arange(nc * 32)
    # [chunk][q][h][r] -> [chunk][h][16 members in (q, r) order]
    zb = z.reshape(nc, 4, 2, 4).transpose(0, 2, 1, 3).reshape(nc, 2, 16)
    ib = ids.reshape(nc, 4, 2, 4).transpose(0, 2, 1, 3).reshape(nc, 2, 16)
    m = zb.max(axis=2)                                   # [nc][2]
    live = np.isfinite(m)
    e = np.where(live[:, :, None], np.exp(zb - np.where(live, m, 0.0)[:, :, None]), 0.0)
    S = e.sum(axis=2)
    w = philox4x32_10(np.arange(nc), np.full(nc, row_id), np.full(nc, step), np.zeros(nc),
                      np.full(nc, seed & 0xFFFFFFFF), np.full(nc, (seed >> 32) & 0xFFFFFFFF))
    u = np.stack([uniform01(w[0]), uniform01(w[2])], axis=1)      # [nc][2]
    eu = np.stack([uniform01(w[1]), uniform01(w[3])], axis=1)
    G = np.where(live, m + np.log(np.where(live, S, 1.0)) - np.log(-np.log(eu)), -np.inf)
    cum = np.cumsum(e, axis=2)
    target = u * S
    reach = cum >= target[:, :, None]
    reach[:, :, 15] |= live                              # rounding guard: the last member
    first = reach.argmax(axis=2)
    # the first member reached may have zero weight only through the guard;
    # step back to the last member with weight
    cand = np.take_along_axis(ib, first[:, :, None], axis=2)[:, :, 0]
    for c, h in zip(*np.nonzero(live & (np.take_along_axis(e, first[:, :, None], 2)[:, :, 0] == 0))):
        j = int(np.nonzero(e[c, h] > 0)[0][-1])
        cand[c, h] = ib[c, h, j]
    Gf = G.ravel()
    cf = cand.ravel()
    order = np.lexsort((cf, -Gf))                        # largest G, then lower candidate
    win = order[0]
    tok = int(cf[win])
    lse = np.max(logits) + np.log(np.sum(np.exp(logits - np.max(logits))))
    conf = float(np.exp(logits[tok] - lse))
    c, h = divmod(int(win), 2)
    j = int(first[c, h])
    lo = cum[c, h, j - 1] if j > 0 else 0.0
    margin = min(abs(target[c, h] - lo), abs(cum[c, h, j] - target[c, h])) / S[c, h]
    neighbours = set(int(x) for x in ib[c, h][e[c, h] > 0])
    info = dict(g_gap=float(Gf[win] - Gf[order[1]]) if np.isfinite(Gf[order[1]]) else np.inf,
                runner_up=int(cf[order[1]]), cdf_margin=float(margin), block=neighbours)
    return tok, conf, info


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
            t, c, inf = sample_row(L[j], temperature, seed, int(row_ids[i0 + j]), step)
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
    if top_p < 1.0:
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


def sample_filtered(logits, temperature, top_k, top_p, seed, row_id, step):
    """One row drawn after top-k / top-p filtering.  Returns (token, conf,
    info) like sample_row, info also holding the filter's boundary info."""
    keep, finfo = topk_topp_keep(logits, temperature, top_k, top_p)
    tok, conf, info = sample_row(logits, temperature, seed, row_id, step, keep)
    info["filter"] = finfo
    info["keep"] = keep
    return tok, conf, info
