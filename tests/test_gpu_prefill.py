"""Block-causal prefill attention (dbd_prefill_attn) against the CPU oracle
on seeded packed prompts, through the C ABI: whole outputs at small sizes,
sampled rows at SDAR-4B head shapes with prompts up to 4096 tokens, and
the K/V store into a NaN-poisoned paged cache bit for bit.  Tolerances are
the attention ones (max abs 2e-2, relative L2 5e-3; bf16 output)."""
import math

import numpy as np
import pytest
import torch

import oracle
from block_diffusion_amd import api, synth
from gpu_util import (ATTN_MAX_ABS, ATTN_REL_L2, attn_errors, dev_bf16, dev_i32, host_bits,
                      widen_bits)

pytestmark = pytest.mark.gpu


def _prompts(seed, lens, Hq, Hkv, D):
    g = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q = synth.normal_bf16(g, (T, Hq, D))
    k = synth.normal_bf16(g, (T, Hkv, D))
    v = synth.normal_bf16(g, (T, Hkv, D))
    return q, k, v, cu


def _paged(seed, lens, Hkv, D, P):
    """A page table covering every prompt (a seeded permutation of pages,
    one spare) and NaN-filled caches."""
    g = np.random.default_rng(seed)
    npg = [max(1, -(-L // P)) for L in lens]
    total = sum(npg) + 1
    perm = g.permutation(total)
    pt = np.full((len(lens), max(npg)), -1, dtype=np.int32)
    o = 0
    for s, n in enumerate(npg):
        pt[s, :n] = perm[o:o + n]
        o += n
    kc = np.full((total, Hkv, P, D), synth.BF16_QNAN, dtype=np.uint16)
    return pt, kc, kc.copy()


def _run(q, k, v, cu, B, store=None):
    T, Hq, D = q.shape
    out = torch.full((T, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    kw = {}
    if store is not None:
        pt, kc, vc = store
        kw = dict(page_table=dev_i32(pt), k_cache=dev_bf16(kc), v_cache=dev_bf16(vc))
    api.dbd_prefill_attn(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_i32(cu), out, B, **kw)
    torch.cuda.synchronize()
    caches = (host_bits(kw["k_cache"]), host_bits(kw["v_cache"])) if store is not None else None
    return host_bits(out), caches


CASES = {
    # name: (lens, Hq, Hkv, D, B, P)
    "tiny_d64": ((16, 37, 0, 5, 100), 4, 2, 64, 4, 16),
    "g4_d128_b4": ((300, 1, 257, 640), 32, 8, 128, 4, 256),
    "g4_d128_b16": ((129, 511, 64), 32, 8, 128, 16, 256),
    "causal_b1": ((70, 200), 8, 2, 128, 1, 64),
    "full_bL": ((90, 33), 8, 4, 64, 128, 32),
    "mha_g1": ((260, 17), 4, 4, 128, 8, 64),
}


@pytest.mark.parametrize("name", list(CASES))
def test_prefill_parity(name):
    lens, Hq, Hkv, D, B, P = CASES[name]
    print(f"{name}: lens {lens} Hq={Hq} Hkv={Hkv} D={D} B={B}", flush=True)
    q, k, v, cu = _prompts(sum(name.encode()), lens, Hq, Hkv, D)
    store = _paged(3, lens, Hkv, D, P)
    out, (kc, vc) = _run(q, k, v, cu, B, store)
    ref = oracle.prefill_attention(q, k, v, cu, B)
    mx, rl = attn_errors(widen_bits(out), ref)
    print(f"  max abs {mx:.3g}, rel L2 {rl:.3g}", flush=True)
    assert mx <= ATTN_MAX_ABS and rl <= ATTN_REL_L2
    ek, ev = oracle.prefill_store(store[1], store[2], store[0], k, v, cu)
    assert np.array_equal(kc, ek) and np.array_equal(vc, ev)
    # without a cache: the same outputs
    out2, _ = _run(q, k, v, cu, B)
    assert np.array_equal(out, out2)


def _rows_ref(q, k, v, cu, B, picks):
    """Oracle rows one by one: picks of (prompt, token, q head)."""
    T, Hq, D = q.shape
    G = Hq // k.shape[1]
    refs = []
    for s, i, h in picks:
        a = int(cu[s])
        n = (i // B + 1) * B
        n = min(n, int(cu[s + 1]) - a)
        keys = widen_bits(k[a:a + n, h // G])
        vals = widen_bits(v[a:a + n, h // G])
        z = keys @ widen_bits(q[a + i, h]) / math.sqrt(D)
        p = np.exp(z - z.max())
        refs.append(p @ vals / p.sum())
    return np.stack(refs)


def test_prefill_sdar4b_sampled():
    """SDAR-4B heads (32 q, 8 kv, D = 128), block 4, 24 prompts of 256..4096
    tokens: sampled rows, always including each prompt's first and last."""
    g = np.random.default_rng(12)
    lens = tuple(int(x) for x in g.integers(256, 4097, 24))
    q, k, v, cu = _prompts(13, lens, 32, 8, 128)
    out, _ = _run(q, k, v, cu, 4)
    picks = []
    for s, L in enumerate(lens):
        for i in {0, L - 1, int(g.integers(0, L)), int(g.integers(0, L))}:
            picks.append((s, i, int(g.integers(0, 32))))
    ref = _rows_ref(q, k, v, cu, 4, picks)
    got = np.stack([widen_bits(out[int(cu[s]) + i, h]) for s, i, h in picks])
    mx, rl = attn_errors(got, ref)
    print(f"{len(picks)} rows: max abs {mx:.3g}, rel L2 {rl:.3g}", flush=True)
    assert mx <= ATTN_MAX_ABS and rl <= ATTN_REL_L2
    assert not np.any(np.isnan(widen_bits(out)))


def test_prefill_deterministic_and_empty():
    lens = (0, 45, 0, 0, 300, 0)
    q, k, v, cu = _prompts(21, lens, 8, 2, 128)
    a, _ = _run(q, k, v, cu, 4)
    b, _ = _run(q, k, v, cu, 4)
    assert np.array_equal(a, b)
    ref = oracle.prefill_attention(q, k, v, cu, 4)
    mx, rl = attn_errors(widen_bits(a), ref)
    assert mx <= ATTN_MAX_ABS and rl <= ATTN_REL_L2


def test_prefill_many_short_prompts():
    """300 prompts of 0..40 tokens (most workgroups hold one partial tile),
    D = 64, G = 2, block 8, with the store."""
    g = np.random.default_rng(31)
    lens = tuple(int(x) for x in g.integers(0, 41, 300))
    q, k, v, cu = _prompts(32, lens, 4, 2, 64)
    store = _paged(33, lens, 2, 64, 16)
    out, (kc, vc) = _run(q, k, v, cu, 8, store)
    ref = oracle.prefill_attention(q, k, v, cu, 8)
    mx, rl = attn_errors(widen_bits(out), ref)
    assert mx <= ATTN_MAX_ABS and rl <= ATTN_REL_L2, (mx, rl)
    ek, ev = oracle.prefill_store(store[1], store[2], store[0], k, v, cu)
    assert np.array_equal(kc, ek) and np.array_equal(vc, ev)


def _random_prefill_shapes(n, seed=4242):
    """Seeded random shapes within the boundary's limits: G a power of two
    dividing the 128 query rows of a workgroup, D 64 or 128, blocks of 1 to
    64 tokens, page sizes 16 to 256; prompt lengths from empty through one
    token, a block minus one and whole blocks to about 1200 tokens."""
    g = np.random.default_rng(seed)
    shapes = []
    for i in range(n):
        D = int(g.choice([64, 128]))
        Hkv = int(g.integers(1, 9))
        G = int(g.choice([1, 2, 4, 8, 16]))
        B = int(g.choice([1, 2, 3, 4, 7, 16, 64]))
        P = int(g.choice([16, 32, 64, 128, 256]))
        S = int(g.integers(1, 9))
        lens = g.integers(0, 1200, S)
        pick = g.integers(0, 5, S)
        lens = np.where(pick == 1, 0, np.where(pick == 2, 1, np.where(pick == 3, np.maximum(B - 1, 0),
                                                                        np.where(pick == 4, (lens // B) * B, lens))))
        shapes.append((f"rand{i}_s{S}_g{G}x{Hkv}_d{D}_b{B}_p{P}", tuple(int(x) for x in lens), G * Hkv, Hkv, D, B,
                       P))
    return shapes


@pytest.mark.parametrize("case", _random_prefill_shapes(8), ids=lambda c: c[0])
def test_prefill_random_shapes(case):
    """Seeded random shapes: sampled rows (each prompt's first and last
    among them) against the oracle, and the K/V store bit for bit."""
    name, lens, Hq, Hkv, D, B, P = case
    print(f"{name}: lens {lens}", flush=True)
    q, k, v, cu = _prompts(sum(name.encode()), lens, Hq, Hkv, D)
    store = _paged(7, lens, Hkv, D, P)
    out, (kc, vc) = _run(q, k, v, cu, B, store)
    g = np.random.default_rng(len(name))
    picks = []
    for s, L in enumerate(lens):
        if L == 0:
            continue
        for i in {0, L - 1, int(g.integers(0, L)), int(g.integers(0, L))}:
            picks.append((s, i, int(g.integers(0, Hq))))
    if picks:
        ref = _rows_ref(q, k, v, cu, B, picks)
        got = np.stack([widen_bits(out[int(cu[s]) + i, h]) for s, i, h in picks])
        mx, rl = attn_errors(got, ref)
        print(f"  {len(picks)} rows: max abs {mx:.3g}, rel L2 {rl:.3g}", flush=True)
        assert mx <= ATTN_MAX_ABS and rl <= ATTN_REL_L2
    assert not np.any(np.isnan(widen_bits(out)))
    ek, ev = oracle.prefill_store(store[1], store[2], store[0], k, v, cu)
    assert np.array_equal(kc, ek) and np.array_equal(vc, ev)
