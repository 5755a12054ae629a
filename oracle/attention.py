"""Block-diffusion attention over a paged KV cache (test infrastructure only).

Follows the pages' description of the denoise forward: the denoise step has
its own attention pattern (JetEngine developer notes, "ModelRunner": prefill
and denoise use different attention patterns), served from a paged KV cache
with per-sequence block tables (JetEngine README architecture tree, "Paged
KV Cache"; developer notes, "Chain Mechanism": block tables reused across
steps).  Each query of the block sees every committed prefix token of its
own sequence and every token of its own block, with no causal mask inside
the block (bidirectional within the block).

Readings of points the pages leave open:
  * softmax scale 1/sqrt(D) unless given;
  * grouped-query attention: query head h reads kv head h // (Hq/Hkv);
  * cache layout [num_pages][Hkv][page_size][D]; logical token j of
    sequence s lives in page page_table[s][j // P] at offset j % P;
  * the block's own keys/values are passed densely as [S][B][Hkv][D].

Everything is float64: softmax with the maximum subtracted, then a weighted
sum of value rows.
"""
import numpy as np

from .bf16 import widen


def _prefix_rows(cache_bits, page_table_s, L, g, P):
    """The first L token rows of kv head g for one sequence, in logical order."""
    if L == 0:
        return np.zeros((0, cache_bits.shape[-1]), dtype=np.float64)
    npg = -(-L // P)
    pages = np.asarray(page_table_s[:npg], dtype=np.int64)
    rows = cache_bits[pages, g]                  # [npg][P][D]
    return widen(rows.reshape(npg * P, -1)[:L])


def attention_group(s, g, q, k_blk, v_blk, k_cache, v_cache, page_table,
                    prefix_len, scale=None):
    """Outputs of the G query heads of kv group g of sequence s, [B][G][D]."""
    S, B, Hq, D = q.shape
    Hkv = k_blk.shape[2]
    G = Hq // Hkv
    P = k_cache.shape[2]
    L = int(prefix_len[s])
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(D)
    keys = np.concatenate([_prefix_rows(k_cache, page_table[s], L, g, P),
                           widen(k_blk[s, :, g, :])], axis=0)      # [L+B][D]
    vals = np.concatenate([_prefix_rows(v_cache, page_table[s], L, g, P),
                           widen(v_blk[s, :, g, :])], axis=0)
    out = np.empty((B, G, D), dtype=np.float64)
    for gi in range(G):
        h = g * G + gi
        qh = widen(q[s, :, h, :])                 # [B][D]
        z = (qh @ keys.T) * scale                 # [B][L+B]
        z -= z.max(axis=1, keepdims=True)
        p = np.exp(z)
        p /= p.sum(axis=1, keepdims=True)
        out[:, gi, :] = p @ vals
    return out


def attention(q, k_blk, v_blk, k_cache, v_cache, page_table, prefix_len,
              scale=None):
    """Full output [S][B][Hq][D] in float64."""
    S, B, Hq, D = q.shape
    Hkv = k_blk.shape[2]
    G = Hq // Hkv
    out = np.empty((S, B, Hq, D), dtype=np.float64)
    for s in range(S):
        for g in range(Hkv):
            out[s, :, g * G:(g + 1) * G, :] = attention_group(
                s, g, q, k_blk, v_blk, k_cache, v_cache, page_table,
                prefix_len, scale)
    return out
