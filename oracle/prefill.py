"""Block-causal prefill attention and the prompt's K/V store (test
infrastructure only).

A prompt enters the engine through a prefill forward whose attention
pattern differs from the denoise step's (JetEngine developer notes,
"ModelRunner": prefill and denoise use different attention patterns;
"Layers": a block-sparse Triton attention, sparse_attn_varlen, serves the
prefill of packed variable-length prompts; a Triton store_kvcache kernel
writes the keys and values into the paged cache).  A block-diffusion model
decodes a block with every earlier block fully visible and bidirectional
attention inside the block (README, "Block Diffusion Decoding"), so the
prompt is read the same way, block by block.

Readings of points the pages leave open:
  * block-causal mask: token i of a prompt attends to token j of the same
    prompt iff floor(j / B) <= floor(i / B), B = block_length (B = 1 is the
    usual causal mask; B >= L is full bidirectional attention);
  * prompts are packed: rows cu_seqlens[s] .. cu_seqlens[s+1]-1 of q, k, v
    ([T][H][D]) are prompt s, positions 0 .. L_s-1;
  * grouped-query heads as in the denoise attention: q head h reads kv head
    h // (Hq / Hkv); scale 1/sqrt(D) unless given;
  * the store writes token j of prompt s at logical cache position j (page
    page_table[s][j // P], offset j % P), every kv head.
Everything is float64.
"""
import numpy as np

from .bf16 import widen


def prefill_attention(q, k, v, cu_seqlens, block_len, scale=None):
    """q [T][Hq][D], k, v [T][Hkv][D] bf16 bits; returns out [T][Hq][D]."""
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((T, Hq, D))
    for s in range(len(cu_seqlens) - 1):
        a, b = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
        L = b - a
        if L == 0:
            continue
        blk = np.arange(L) // block_len
        allowed = blk[None, :] <= blk[:, None]               # [query i][key j]
        for g in range(Hkv):
            keys = widen(k[a:b, g, :])
            vals = widen(v[a:b, g, :])
            for gi in range(G):
                h = g * G + gi
                z = (widen(q[a:b, h, :]) @ keys.T) * scale
                z = np.where(allowed, z, -np.inf)
                z -= z.max(axis=1, keepdims=True)
                p = np.exp(z)
                p /= p.sum(axis=1, keepdims=True)
                out[a:b, h, :] = p @ vals
    return out


def prefill_store(k_cache, v_cache, page_table, k, v, cu_seqlens):
    """Copies of the caches with every prompt token's keys and values at its
    position."""
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    P = kc.shape[2]
    for s in range(len(cu_seqlens) - 1):
        a, b = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
        for j in range(b - a):
            page = int(page_table[s][j // P])
            kc[page, :, j % P, :] = k[a + j]
            vc[page, :, j % P, :] = v[a + j]
    return kc, vc
