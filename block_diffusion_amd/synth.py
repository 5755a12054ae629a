"""Seeded synthetic inputs for the denoise round.

This module is the only code shared by the checking side (the CPU oracle
and the tests) and the GPU side (bench, smoke).  It holds random draws, the
bf16 encoding of those draws, the paged layout of the prefix cache and the
planted-token construction of the hidden states; it holds none of the
round's arithmetic (no attention, no softmax, no commit rule).

Every stream is keyed ``[1234, seed_id, round, stream]`` (large arrays add
a block index, see normal_bf16) so any array can be regenerated on its own.  Values are drawn in float32
and rounded to bf16 (round to nearest even); both sides consume the same
16-bit patterns.
"""
from __future__ import annotations

import os
from dataclasses import dataclass

import numpy as np

from .workloads import DENOISING, Workload

# stream ids
ST_PREFIX, ST_PAGES, ST_KCACHE, ST_VCACHE, ST_W = 0, 1, 2, 3, 4
ST_Q, ST_KBLK, ST_VBLK, ST_G, ST_T, ST_A, ST_INIT = 5, 6, 7, 8, 9, 10, 11

BF16_QNAN = np.uint16(0x7FC0)


def rng(w: Workload, rnd: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([1234, w.seed_id, rnd, stream])


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (NaN -> qNaN)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    nan = np.isnan(x)
    if nan.any():
        u = np.where(nan, np.uint32(0), u)
    # finite inputs: u + 0x7FFF + lsb cannot wrap past 0xFF807FFF
    out = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        out[nan] = BF16_QNAN
    return out


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


CHUNK = 1 << 22


def _fill_chunk(out, key, i, std):
    n = out.size
    lo, hi = i * CHUNK, min(n, (i + 1) * CHUNK)
    v = np.random.default_rng(key + [i]).standard_normal(hi - lo, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    out[lo:hi] = f32_to_bf16(v)


def normal_bf16(g, shape, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) draws in float32, rounded to bf16.

    g is either a Generator (one sequential stream) or a seed key (list of
    ints): then element block i (of CHUNK elements) is drawn from
    default_rng(key + [i]), block by block on a thread pool, so multi-GB
    caches are generated in parallel and still the same on every run."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    if isinstance(g, np.random.Generator):
        for i in range(0, n, CHUNK):
            m = min(CHUNK, n - i)
            v = g.standard_normal(m, dtype=np.float32)
            if std != 1.0:
                v *= np.float32(std)
            out[i:i + m] = f32_to_bf16(v)
        return out.reshape(shape)
    nchunks = -(-n // CHUNK)
    if nchunks <= 2:
        for i in range(nchunks):
            _fill_chunk(out, list(g), i, std)
    else:
        from concurrent.futures import ThreadPoolExecutor
        workers = min(16, len(os.sched_getaffinity(0)), nchunks)
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(lambda i: _fill_chunk(out, list(g), i, std), range(nchunks)))
    return out.reshape(shape)


def key(w: Workload, rnd: int, stream: int) -> list:
    return [1234, w.seed_id, rnd, stream]


@dataclass
class Fixed:
    """Per-block inputs that stay fixed across the rounds of one block."""
    prefix_len: np.ndarray     # [S] int32
    page_table: np.ndarray     # [S][max_pages] int32, -1 = unused
    k_cache: np.ndarray        # [num_pages][Hkv][P][D] bf16 bits
    v_cache: np.ndarray        # [num_pages][Hkv][P][D] bf16 bits
    w_vocab: np.ndarray        # [V][Hd] bf16 bits (row v = column v of W)
    block_tokens0: np.ndarray  # [S][B] int32, initial block
    seq_state0: np.ndarray     # [S] uint8


@dataclass
class RoundInputs:
    """Fresh inputs of one round (no model feeds committed tokens back)."""
    q: np.ndarray       # [S][B][Hq][D] bf16 bits
    k_blk: np.ndarray   # [S][B][Hkv][D] bf16 bits
    v_blk: np.ndarray   # [S][B][Hkv][D] bf16 bits
    hidden: np.ndarray  # [S*B][Hd] bf16 bits, row = s*B + position


def prefix_lengths(w: Workload) -> np.ndarray:
    if w.prefix_fixed:
        assert len(w.prefix_fixed) == w.S
        return np.asarray(w.prefix_fixed, dtype=np.int32)
    g = rng(w, 0, ST_PREFIX)
    return g.integers(w.prefix_lo, w.prefix_hi + 1, size=w.S).astype(np.int32)


def page_layout(w: Workload, prefix_len: np.ndarray, reserve_tokens: int = 0):
    """Physical page ids: a seeded permutation of all pages the prefixes
    need (plus room for reserve_tokens more tokens per sequence, for blocks
    that later steps append), so that logical order and physical order
    differ."""
    npg = [(-(-(int(L) + reserve_tokens) // w.P)) for L in prefix_len]
    total = int(sum(npg))
    perm = rng(w, 0, ST_PAGES).permutation(total).astype(np.int32)
    table = np.full((w.S, max(w.max_pages, max(npg))), -1, dtype=np.int32)
    o = 0
    for s, n in enumerate(npg):
        table[s, :n] = perm[o:o + n]
        o += n
    return table, total


def make_fixed(w: Workload, poison_tail: bool = True, with_w: bool = True,
               reserve_tokens: int = 0) -> Fixed:
    L = prefix_lengths(w)
    table, npages = page_layout(w, L, reserve_tokens)
    shape = (npages, w.Hkv, w.P, w.D)
    kc = normal_bf16(key(w, 0, ST_KCACHE), shape)
    vc = normal_bf16(key(w, 0, ST_VCACHE), shape)
    if poison_tail:
        # slots past a prefix's end (the rest of its last page and any
        # reserved page) are not part of the prefix; fill them with NaN so
        # any read of them shows up.
        for s in range(w.S):
            n = (-(-int(L[s]) // w.P))
            tail = int(L[s]) - (n - 1) * w.P
            if n and tail < w.P:
                p = table[s, n - 1]
                kc[p, :, tail:, :] = BF16_QNAN
                vc[p, :, tail:, :] = BF16_QNAN
            for p in table[s, n:]:
                if p >= 0:
                    kc[p] = BF16_QNAN
                    vc[p] = BF16_QNAN
    wv = normal_bf16(key(w, 0, ST_W), (w.V, w.Hd), std=1.0 / np.sqrt(w.Hd)) if with_w else None
    toks = np.full((w.S, w.B), w.mask_id, dtype=np.int32)
    if w.init_committed_max > 0:
        g = rng(w, 0, ST_INIT)
        for s in range(w.S):
            k = int(g.integers(0, w.init_committed_max + 1))
            pos = g.choice(w.B, size=k, replace=False)
            t = g.integers(0, w.V - 1, size=k)
            t = np.where(t >= w.mask_id, t + 1, t)   # uniform over [0,V) \ {mask}
            toks[s, pos] = t
    state = np.full(w.S, DENOISING, dtype=np.uint8)
    return Fixed(L, table, kc, vc, wv, toks, state)


def make_hidden(w: Workload, rnd: int, w_vocab: np.ndarray) -> np.ndarray:
    """h = g + a * w_t / ||w_t||: g ~ N(0,1)^Hd, t ~ U[0,V), a ~ U[0,a_max],
    w_t = column t of W (row t of the stored [V][Hd]); the norm is taken in
    float64 over the bf16 values; h is rounded to bf16 at the end.  The
    planted direction makes confidences span low to near one."""
    n = w.S * w.B
    g = rng(w, rnd, ST_G).standard_normal((n, w.Hd), dtype=np.float32).astype(np.float64)
    t = rng(w, rnd, ST_T).integers(0, w.V, size=n)
    a = rng(w, rnd, ST_A).uniform(0.0, w.a_max, size=n)
    wt = bf16_to_f32(w_vocab[t]).astype(np.float64)
    wt /= np.linalg.norm(wt, axis=1, keepdims=True)
    h = g + a[:, None] * wt
    return f32_to_bf16(h.astype(np.float32))


def make_round(w: Workload, rnd: int, w_vocab: np.ndarray | None) -> RoundInputs:
    q = normal_bf16(key(w, rnd, ST_Q), (w.S, w.B, w.Hq, w.D))
    kb = normal_bf16(key(w, rnd, ST_KBLK), (w.S, w.B, w.Hkv, w.D))
    vb = normal_bf16(key(w, rnd, ST_VBLK), (w.S, w.B, w.Hkv, w.D))
    h = make_hidden(w, rnd, w_vocab) if w_vocab is not None else None
    return RoundInputs(q, kb, vb, h)
