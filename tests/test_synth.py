"""The seeded input generator: determinism, bf16 rounding, page layout."""
import numpy as np
import torch

from block_diffusion_amd import synth
from block_diffusion_amd.workloads import ALL, TINY, SDAR_8B, DENOISING


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1e-40, 3.0e38, -3.0e38, np.inf, -np.inf], np.float32)])
    ours = synth.f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert synth.f32_to_bf16(np.array([np.nan], np.float32))[0] == 0x7FC0
    back = synth.bf16_to_f32(ours)
    assert np.array_equal(synth.f32_to_bf16(back), ours)


def test_deterministic():
    a = synth.make_fixed(TINY)
    b = synth.make_fixed(TINY)
    for k in ("prefix_len", "page_table", "k_cache", "v_cache", "w_vocab", "block_tokens0"):
        assert np.array_equal(getattr(a, k), getattr(b, k))
    r1 = synth.make_round(TINY, 1, a.w_vocab)
    r2 = synth.make_round(TINY, 1, a.w_vocab)
    r3 = synth.make_round(TINY, 2, a.w_vocab)
    assert np.array_equal(r1.hidden, r2.hidden) and np.array_equal(r1.q, r2.q)
    assert not np.array_equal(r1.q, r3.q)


def test_page_layout():
    for w in ALL:
        L = synth.prefix_lengths(w)
        assert L.shape == (w.S,)
        if not w.prefix_fixed:
            assert L.min() >= w.prefix_lo and L.max() <= w.prefix_hi
        table, n = synth.page_layout(w, L)
        used = table[table >= 0]
        assert sorted(used.tolist()) == list(range(n))           # a permutation
        for s in range(w.S):
            k = -(-int(L[s]) // w.P)
            assert np.all(table[s, :k] >= 0) and np.all(table[s, k:] == -1)


def test_tiny_fixed_contents():
    f = synth.make_fixed(TINY)
    assert f.prefix_len.tolist() == [16, 37]
    assert f.k_cache.shape == (1 + 3, TINY.Hkv, TINY.P, TINY.D)
    assert np.all(f.block_tokens0 == TINY.mask_id) and np.all(f.seq_state0 == DENOISING)
    # the tail of sequence 1's last page (37 = 2*16 + 5) is poisoned
    p = f.page_table[1, 2]
    assert np.all(f.k_cache[p, :, 5:] == 0x7FC0) and not np.any(f.k_cache[p, :, :5] == 0x7FC0)


def test_initial_commits():
    w = SDAR_8B.with_(V=1000, mask_id=999, Hd=8, prefix_lo=1, prefix_hi=2, Hkv=1, Hq=1, D=8, P=16)
    f = synth.make_fixed(w)
    committed = (f.block_tokens0 != w.mask_id).sum(1)
    assert committed.min() >= 0 and committed.max() <= 12
    assert np.all(f.block_tokens0[f.block_tokens0 != w.mask_id] < w.V)


def test_hidden_planted_direction():
    f = synth.make_fixed(TINY)
    r = synth.make_round(TINY, 1, f.w_vocab)
    assert r.hidden.shape == (TINY.S * TINY.B, TINY.Hd)
    assert r.q.shape == (TINY.S, TINY.B, TINY.Hq, TINY.D)
