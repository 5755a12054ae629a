"""Parity of the HIP path (through the C ABI) with the CPU oracle on seeded
inputs, element by element, at sizes the oracle finishes in seconds and, at
the full SDAR-4B shapes, on sampled outputs.  Tolerances: attention max abs
2e-2 and relative L2 5e-3 (bf16 output); confidence 1e-3 absolute; greedy
tokens and committed sets exact outside the near-tie and near-threshold
bands (tests/gpu_util.py)."""
import numpy as np
import pytest
import torch

import oracle
from block_diffusion_amd import api, synth
from block_diffusion_amd.workloads import (LLADA_LONG, SDAR_1P7B, SDAR_4B, SDAR_4B_HIGHCONF,
                                           SDAR_8B, SDAR_8B_HIGHCONF, TINY, Workload)
from gpu_util import (ATTN_MAX_ABS, ATTN_REL_L2, RoundState, check_commits, check_lm_rows,
                      check_rows_against, compare_attn, dev_bf16, dev_i32, dev_u8, host_bits,
                      oracle_attn_groups, oracle_rows_with_ties, round_inputs_dev, run_attn, tie_set,
                      widen_bits)

pytestmark = pytest.mark.gpu


def _custom(name, seed, **kw):
    base = dict(name=name, seed_id=seed, S=1, B=4, Hq=4, Hkv=2, D=64, P=16, Hd=128, V=1000,
                mask_id=999, prefix_lo=0, prefix_hi=0, tau=0.9, rounds=4, a_max=12.0)
    base.update(kw)
    return Workload(**base)


ATTN_SMALL = [
    TINY,
    # several prefix chunks, an empty prefix and a one-token prefix; 9 rows (G=3, B=3)
    _custom("multichunk_p16_d64", 101, S=3, B=3, Hq=6, Hkv=2, D=64, P=16,
            prefix_fixed=(0, 1, 1500), prefix_hi=1500),
    # 32 rows per kv head (two 16-row tiles), D=128
    _custom("rows32_d128", 102, S=4, B=8, Hq=8, Hkv=2, D=128, P=32,
            prefix_fixed=(33, 700, 0, 1025), prefix_hi=1025),
    # 128 rows per kv head: two row groups of 64
    _custom("rows128_two_groups", 103, S=2, B=16, Hq=16, Hkv=2, D=128, P=16,
            prefix_fixed=(2100, 17), prefix_hi=2100),
    # MHA with the largest block, 64 rows
    _custom("mha_b64", 104, S=2, B=64, Hq=4, Hkv=4, D=128, P=256,
            prefix_fixed=(3000, 255), prefix_hi=3000),
    # block of one token, D=64, 64 rows from G=64
    _custom("g64_b1", 105, S=2, B=1, Hq=64, Hkv=1, D=64, P=64,
            prefix_fixed=(64, 129), prefix_hi=129),
    # page tables that hold 65568 tiles: the three-slot ring, with 9 rows per
    # segment (padded to 16) and one 64 K-token prefix cut over many waves
    _custom("deep_ring_rows9_d128", 106, S=4, B=3, Hq=24, Hkv=8, D=128, P=256,
            prefix_fixed=(0, 5, 65536, 300), prefix_hi=65536),
    # the same at D=64, where the three-slot ring still leaves four waves per CU
    _custom("deep_ring_rows8_d64", 107, S=4, B=4, Hq=16, Hkv=8, D=64, P=256,
            prefix_fixed=(0, 5, 65536, 300), prefix_hi=65536),
]


def _random_attn_shapes(n, seed=2024):
    """Seeded random shapes within the boundary's limits (B <= 64, D 64 or
    128, page size a multiple of 16): GQA widths 1..16, several page sizes,
    prefixes from empty through page-aligned to a few thousand tokens."""
    g = np.random.default_rng(seed)
    shapes = []
    for i in range(n):
        D = int(g.choice([64, 128]))
        Hkv = int(g.integers(1, 9))
        G = int(g.choice([1, 2, 3, 4, 6, 8, 16]))
        B = int(g.choice([1, 2, 3, 4, 5, 8, 16, 31, 64]))
        while G * B > 256:
            B = max(1, B // 2)
        P = int(g.choice([16, 32, 64, 128, 256]))
        S = int(g.integers(1, 12))
        L = g.integers(0, 2500, S)
        pick = g.integers(0, 4, S)            # 0: as drawn, 1: empty, 2: whole pages, 3: a page minus one
        L = np.where(pick == 1, 0, np.where(pick == 2, (L // P) * P,
                                            np.where(pick == 3, np.maximum(P - 1, (L // P) * P - 1), L)))
        if L.max() == 0:
            L[0] = P + 1                      # the cache needs a page; one prefix crosses into a second
        shapes.append(_custom(f"rand{i}_s{S}_b{B}_g{G}x{Hkv}_d{D}_p{P}", 300 + i, S=S, B=B, Hq=G * Hkv,
                              Hkv=Hkv, D=D, P=P, prefix_fixed=tuple(int(x) for x in L),
                              prefix_hi=max(1, int(L.max()))))
    return shapes


@pytest.mark.parametrize("w", _random_attn_shapes(12), ids=lambda w: w.name)
def test_attention_parity_random_shapes(w):
    """Seeded random shapes: up to 8 (sequence, kv head) groups, among them
    the first and the last, against the oracle."""
    fx = synth.make_fixed(w, with_w=False)
    rin = synth.make_round(w, 1, None)
    out = run_attn(fx, rin)
    allg = [(s, g) for s in range(w.S) for g in range(w.Hkv)]
    rng = np.random.default_rng(w.seed_id)
    idx = sorted(set([0, len(allg) - 1] + list(rng.choice(len(allg), min(6, len(allg)), replace=False))))
    ref = oracle_attn_groups(fx, rin, [allg[i] for i in idx])
    mx, rl2 = compare_attn(out, ref, w.G)
    print(f"{w.name} prefixes {list(w.prefix_fixed)}: max abs {mx:.3e} rel L2 {rl2:.3e}", flush=True)
    assert mx <= ATTN_MAX_ABS and rl2 <= ATTN_REL_L2


@pytest.mark.parametrize("w", ATTN_SMALL, ids=lambda w: w.name)
def test_attention_parity_small(w):
    fx = synth.make_fixed(w, with_w=False)
    rin = synth.make_round(w, 1, None)
    out = run_attn(fx, rin)
    groups = [(s, g) for s in range(w.S) for g in range(w.Hkv)]
    ref = oracle_attn_groups(fx, rin, groups)
    mx, rl2 = compare_attn(out, ref, w.G)
    print(f"{w.name}: max abs {mx:.3e} rel L2 {rl2:.3e}")
    assert mx <= ATTN_MAX_ABS and rl2 <= ATTN_REL_L2


def test_attention_parity_sdar1p7b_full():
    w = SDAR_1P7B
    fx = synth.make_fixed(w, with_w=False)
    rin = synth.make_round(w, 1, None)
    out = run_attn(fx, rin)
    ref = oracle_attn_groups(fx, rin, [(s, g) for s in range(w.S) for g in range(w.Hkv)])
    mx, rl2 = compare_attn(out, ref, w.G)
    print(f"{w.name}: max abs {mx:.3e} rel L2 {rl2:.3e}")
    assert mx <= ATTN_MAX_ABS and rl2 <= ATTN_REL_L2


@pytest.fixture(scope="module")
def sdar4b_fixed(big_fixed):
    return big_fixed(SDAR_4B)


def test_attention_parity_sdar4b_sampled(sdar4b_fixed):
    w, fx = SDAR_4B, sdar4b_fixed
    rin = synth.make_round(w, 1, None)
    out = run_attn(fx, rin)
    g = np.random.default_rng(7)
    L = fx.prefix_len
    # the longest and shortest prefixes plus a random sample
    ss = sorted(set([int(np.argmax(L)), int(np.argmin(L))] + g.choice(w.S, 22, replace=False).tolist()))
    groups = [(s, int(k)) for s in ss for k in g.choice(w.Hkv, 3, replace=False)]
    ref = oracle_attn_groups(fx, rin, groups)
    mx, rl2 = compare_attn(out, ref, w.G)
    print(f"{w.name}: {len(groups)} groups, max abs {mx:.3e} rel L2 {rl2:.3e}")
    assert mx <= ATTN_MAX_ABS and rl2 <= ATTN_REL_L2
    assert np.all(np.isfinite(widen_bits(out)))


def test_attention_page_relabel_bitwise():
    """Physical page ids do not change the traversal order, so relabelling
    the pages gives the same bits."""
    w = ATTN_SMALL[1]
    fx = synth.make_fixed(w, with_w=False)
    rin = synth.make_round(w, 1, None)
    base = run_attn(fx, rin)
    n = fx.k_cache.shape[0]
    pi = np.random.default_rng(3).permutation(n)
    kc = np.empty_like(fx.k_cache); vc = np.empty_like(fx.v_cache)
    kc[pi] = fx.k_cache; vc[pi] = fx.v_cache
    pt = fx.page_table.copy()
    pt[pt >= 0] = pi[pt[pt >= 0]]
    fx2 = synth.Fixed(fx.prefix_len, pt, kc, vc, None, fx.block_tokens0, fx.seq_state0)
    assert np.array_equal(run_attn(fx2, rin), base)


def test_attention_deterministic():
    w = ATTN_SMALL[3]
    fx = synth.make_fixed(w, with_w=False)
    rin = synth.make_round(w, 1, None)
    assert np.array_equal(run_attn(fx, rin), run_attn(fx, rin))


def test_side_stream_binding_workspace():
    """Attention and the LM head launched on a stream the caller names (a
    torch stream, then its raw handle), with the workspace the binding
    allocates itself, while the current stream allocates and fills memory
    right after each launch: the same bits as the launches on the current
    stream."""
    w = SDAR_1P7B
    fx = synth.make_fixed(w)
    rin = synth.make_round(w, 1, fx.w_vocab)
    ref = run_attn(fx, rin)
    rows = np.arange(w.S * w.B, dtype=np.int32)
    arg_ref, conf_ref = _lm_run(rin.hidden, fx.w_vocab, w.mask_id, rows)
    q, kb, vb = dev_bf16(rin.q), dev_bf16(rin.k_blk), dev_bf16(rin.v_blk)
    kc, vc = dev_bf16(fx.k_cache), dev_bf16(fx.v_cache)
    pt, pl = dev_i32(fx.page_table), dev_i32(fx.prefix_len)
    h, wv, ri, nr = dev_bf16(rin.hidden), dev_bf16(fx.w_vocab), dev_i32(rows), dev_i32([rows.size])
    side = torch.cuda.Stream()
    for handle in (False, True):
        st = side.cuda_stream if handle else side
        out = torch.empty((w.S, w.B, w.Hq, w.D), dtype=torch.bfloat16, device="cuda")
        arg = torch.full((rows.size,), -7, dtype=torch.int32, device="cuda")
        conf = torch.full((rows.size,), float("nan"), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        api.dbd_attn_paged(q, kb, vb, kc, vc, pt, pl, out, stream=st)
        # sizes that fit the freed workspaces' blocks (the attention's in
        # the large pool, the LM head's in the small one)
        junk = [torch.full((n,), 7.0, device="cuda") for n in (1 << 19, 1 << 17) * 4]
        api.dbd_lmhead_conf(h, wv, nr, arg, conf, w.mask_id, row_index=ri, max_rows=rows.size, stream=st)
        junk += [torch.full((n,), 9.0, device="cuda") for n in (1 << 19, 1 << 17) * 4]
        torch.cuda.synchronize()
        del junk
        assert np.array_equal(host_bits(out), ref), f"attention, handle={handle}"
        assert np.array_equal(arg.cpu().numpy(), arg_ref[rows]), f"LM head tokens, handle={handle}"
        assert np.array_equal(conf.cpu().numpy(), conf_ref[rows]), f"LM head conf, handle={handle}"


@pytest.fixture(scope="module")
def big_fixed():
    """Fixed inputs of the SDAR-8B (B=16) and LLaDA (B=64, 16K-32K prefix)
    shapes, generated once per module."""
    cache = {}

    def get(w):
        key = (w.seed_id, w.S, w.B, w.prefix_lo, w.prefix_hi)   # a_max changes only the hidden rows
        if key not in cache:
            cache[key] = synth.make_fixed(w)
        return cache[key]
    return get


def _sample_groups(w, L, n_seq, n_head, seed):
    g = np.random.default_rng(seed)
    ss = sorted(set([int(np.argmax(L)), int(np.argmin(L))] +
                    g.choice(w.S, min(n_seq, w.S), replace=False).tolist()))
    return [(s, int(k)) for s in ss for k in g.choice(w.Hkv, min(n_head, w.Hkv), replace=False)]


@pytest.mark.parametrize("w", [SDAR_8B, LLADA_LONG], ids=lambda w: w.name)
def test_attention_parity_large_sampled(w, big_fixed):
    """Full-size SDAR-8B (64 rows per kv head, prefixes to 8K) and LLaDA
    (MHA, 64 rows, prefixes to 32K) attention on sampled (sequence, head)
    groups, always including the longest and shortest prefixes."""
    fx = big_fixed(w)
    rin = synth.make_round(w, 1, None)
    out = run_attn(fx, rin)
    groups = _sample_groups(w, fx.prefix_len, 6, 3, 11)
    ref = oracle_attn_groups(fx, rin, groups)
    mx, rl2 = compare_attn(out, ref, w.G)
    print(f"{w.name}: {len(groups)} groups, max abs {mx:.3e} rel L2 {rl2:.3e}")
    assert mx <= ATTN_MAX_ABS and rl2 <= ATTN_REL_L2
    assert np.all(np.isfinite(widen_bits(out)))


# ------------------------------------------------------------------- LM head

def _lm_run(hidden_bits, w_bits, mask_id, rows, max_rows=None, use_index=True):
    n = hidden_bits.shape[0]
    h = dev_bf16(hidden_bits)
    wv = dev_bf16(w_bits)
    M = len(rows)
    if max_rows is None:
        max_rows = M
    ri = np.zeros(max(max_rows, 1), np.int32)
    ri[:M] = rows
    ri_d = dev_i32(ri) if use_index else None
    nr = dev_i32([M])
    arg = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    conf = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    api.dbd_lmhead_conf(h, wv, nr, arg, conf, mask_id, row_index=ri_d, max_rows=max_rows)
    torch.cuda.synchronize()
    return arg.cpu().numpy(), conf.cpu().numpy()


def test_lmhead_parity_tiny_all_rows():
    w = TINY
    fx = synth.make_fixed(w)
    rin = synth.make_round(w, 1, fx.w_vocab)
    rows = np.arange(w.S * w.B)
    arg, conf = _lm_run(rin.hidden, fx.w_vocab, w.mask_id, rows, use_index=False)
    _, p1, _, nt = check_lm_rows(rows, arg, conf, rin.hidden, fx.w_vocab, w.mask_id)
    print("tiny p1:", np.round(p1, 3), "tie-exempt", nt)


@pytest.mark.parametrize("V,Hd,mask,n,M,max_rows", [
    (1000, 128, 500, 64, 37, 50),      # ragged last vocab tile, listed rows < max_rows
    (300, 128, 0, 300, 300, 300),      # two row tiles (256 + 44), mask id 0
    (2048, 256, 2047, 40, 0, 40),      # no rows this round
    (129, 128, 128, 5, 5, 5),          # one column past a 128 tile
])
def test_lmhead_parity_ragged(V, Hd, mask, n, M, max_rows):
    g = np.random.default_rng(V + M)
    wv = synth.normal_bf16(g, (V, Hd), std=1.0 / np.sqrt(Hd))
    t = g.integers(0, V, n)
    a = g.uniform(0, 10, n)
    wt = widen_bits(wv[t]); wt /= np.linalg.norm(wt, axis=1, keepdims=True)
    h = synth.f32_to_bf16((g.standard_normal((n, Hd)) + a[:, None] * wt).astype(np.float32))
    rows = g.permutation(n)[:M]
    arg, conf = _lm_run(h, wv, mask, rows, max_rows=max_rows)
    if M:
        check_lm_rows(rows, arg, conf, h, wv, mask)
    untouched = np.setdiff1d(np.arange(n), rows)
    assert np.all(arg[untouched] == -7) and np.all(np.isnan(conf[untouched]))


def test_lmhead_no_candidate_rows():
    """Rows with no candidate token (W all -inf against positive hidden rows,
    so every logit is -inf) give the mask token with confidence 0 and
    entropy +inf, greedy and sampled, as the oracle does; rows of the same
    launch with finite logits are unaffected."""
    V, Hd, mask = 1000, 128, 7
    g = np.random.default_rng(4)
    wv = synth.f32_to_bf16(np.full((V, Hd), -np.inf, np.float32))
    h = synth.f32_to_bf16(np.abs(g.standard_normal((6, Hd))).astype(np.float32) + 0.5)
    rows = np.array([1, 4])
    arg, conf = _lm_run(h, wv, mask, rows)
    a, p1, _ = oracle.lmhead_rows(h[rows], wv, mask)
    assert np.all(arg[rows] == mask) and np.all(a == mask)
    assert np.all(conf[rows] == 0.0) and np.all(p1 == 0.0)
    ent = torch.full((6,), float("nan"), dtype=torch.float32, device="cuda")
    nr = dev_i32([2])
    arg_d = torch.full((6,), -7, dtype=torch.int32, device="cuda")
    conf_d = torch.full((6,), float("nan"), dtype=torch.float32, device="cuda")
    api.dbd_lmhead_conf(dev_bf16(h), dev_bf16(wv), nr, arg_d, conf_d, mask, row_index=dev_i32(rows),
                        max_rows=2, entropy=ent)
    tok_s = torch.full((6,), -7, dtype=torch.int32, device="cuda")
    conf_s = torch.full((6,), float("nan"), dtype=torch.float32, device="cuda")
    api.dbd_lmhead_sample(dev_bf16(h), dev_bf16(wv), nr, tok_s, conf_s, mask, 0.7, 5, 1,
                          row_index=dev_i32(rows), max_rows=2)
    torch.cuda.synchronize()
    assert np.all(ent.cpu().numpy()[rows] == np.inf)
    assert np.all(oracle.lmhead_entropy(h[rows], wv, mask) == np.inf)
    assert np.all(tok_s.cpu().numpy()[rows] == mask) and np.all(conf_s.cpu().numpy()[rows] == 0.0)
    # finite rows beside them: W finite except one -inf row
    wv2 = synth.normal_bf16(g, (V, Hd), std=1.0 / np.sqrt(Hd))
    wv2[11] = wv[0]
    arg2, conf2 = _lm_run(h, wv2, mask, rows)
    check_lm_rows(rows, arg2, conf2, h, wv2, mask)


def test_lmhead_parity_sdar1p7b_all_rows():
    w = SDAR_1P7B
    fx = synth.make_fixed(w)
    rin = synth.make_round(w, 1, fx.w_vocab)
    rows = np.arange(w.S * w.B)
    arg, conf = _lm_run(rin.hidden, fx.w_vocab, w.mask_id, rows)
    _, p1, _, nt = check_lm_rows(rows, arg, conf, rin.hidden, fx.w_vocab, w.mask_id)
    print(f"{w.name}: {(p1 >= w.tau).sum()} rows >= tau, tie-exempt {nt}")


@pytest.mark.parametrize("w", [SDAR_4B, SDAR_4B_HIGHCONF], ids=lambda w: w.name)
def test_lmhead_parity_sdar4b_sampled(w, sdar4b_fixed):
    fx = sdar4b_fixed
    rin = synth.make_round(w, 1, fx.w_vocab)
    for M in (512, 384):
        rows = np.arange(M)
        arg, conf = _lm_run(rin.hidden, fx.w_vocab, w.mask_id, rows, max_rows=512)
        g = np.random.default_rng(M)
        samp = np.sort(np.concatenate([g.choice(M, 40, replace=False), [0, M - 1]]))
        samp = np.unique(samp)
        check_lm_rows(samp, arg, conf, rin.hidden, fx.w_vocab, w.mask_id)
        assert np.all(arg[M:] == -7)


@pytest.mark.parametrize("w", [SDAR_8B, LLADA_LONG], ids=lambda w: w.name)
def test_lmhead_parity_large_sampled(w, big_fixed):
    """Round-1 masked rows of the SDAR-8B shapes (about 640 rows: two row
    tiles of the LM head, hidden 4096) and of LLaDA (512 rows, vocabulary
    126464), through the compact row list; sampled rows against the oracle."""
    fx = big_fixed(w)
    rin = synth.make_round(w, 1, fx.w_vocab)
    rows = oracle.compact_rows(fx.block_tokens0, fx.seq_state0, w.mask_id)
    M = rows.size
    arg, conf = _lm_run(rin.hidden, fx.w_vocab, w.mask_id, rows, max_rows=w.S * w.B)
    g = np.random.default_rng(M)
    samp = np.unique(np.concatenate([rows[g.choice(M, 24, replace=False)], rows[[0, M - 1]]]))
    _, p1, _, nt = check_lm_rows(samp, arg, conf, rin.hidden, fx.w_vocab, w.mask_id)
    print(f"{w.name}: M={M}, {len(samp)} sampled rows, tie-exempt {nt}")
    untouched = np.setdiff1d(np.arange(w.S * w.B), rows)
    assert np.all(arg[untouched] == -7)


# -------------------------------------------------------------------- remask

@pytest.mark.parametrize("S,B,flags", [(1, 1, 0), (3, 4, 0), (128, 4, 0), (64, 16, 0),
                                       (8, 64, 0), (50, 7, 1), (8192, 4, 0), (1000, 64, 0)])
def test_remask_parity(S, B, flags):
    g = np.random.default_rng(S * 131 + B)
    mask = 151669
    tau = np.float32(0.9)
    levels = np.array([0.1, 0.5, 0.9, 0.9, 0.95, 0.3, 0.3], dtype=np.float32)
    toks = np.where(g.random((S, B)) < 0.7, mask, g.integers(0, mask, (S, B))).astype(np.int32)
    state = g.choice(np.array([2, 2, 2, 3, 0, 4], np.uint8), size=S)
    conf = np.where(g.random(S * B) < 0.5, g.choice(levels, S * B), g.random(S * B)).astype(np.float32)
    argm = g.integers(0, mask, S * B).astype(np.int32)
    t_d, s_d = dev_i32(toks), dev_u8(state)
    ri = torch.full((S * B,), -1, dtype=torch.int32, device="cuda")
    nr = torch.zeros(1, dtype=torch.int32, device="cuda")
    nc = torch.full((S,), -1, dtype=torch.int32, device="cuda")
    api.dbd_remask_commit(t_d, s_d, dev_i32(argm), torch.from_numpy(conf).cuda(), ri, nr, mask,
                          float(tau), flags=flags, num_committed=nc)
    torch.cuda.synchronize()
    et, es, com = oracle.remask(toks, state, conf.astype(np.float64), argm, mask,
                                float(tau), flags)
    assert np.array_equal(t_d.cpu().numpy(), et)
    assert np.array_equal(s_d.cpu().numpy(), es)
    rows = oracle.compact_rows(et, es, mask)
    assert nr.item() == rows.size
    assert np.array_equal(ri.cpu().numpy()[:rows.size], rows)
    den = state == 2
    assert np.array_equal(nc.cpu().numpy()[den], com.sum(1)[den])


def test_remask_nan_and_mask_commit():
    """Hand-built cases: every masked confidence NaN (the lowest masked
    position commits), NaN below -inf, a NaN first position losing the
    fallback to a number, and a commit of the mask token itself (the
    position stays masked and the sequence DENOISING); exact against the
    oracle, row list included."""
    mask, tau = 9, 0.875
    nan, inf = np.nan, np.inf
    toks = np.array([[5, 9, 9, 9], [9, 9, 9, 9], [9, 9, 9, 9], [9, 1, 2, 3], [9, 9, 4, 9]], np.int32)
    state = np.full(5, 2, np.uint8)
    conf = np.array([0.75, nan, nan, nan, nan, -inf, nan, -inf, nan, 0.25, 0.5, 0.125,
                     0.95, 0, 0, 0, 0.9, 0.1, 0, nan], np.float32)
    argm = np.array([0, 121, 122, 123, 130, 131, 132, 133, 140, 141, 142, 143, 9, 0, 0, 0,
                     150, 151, 0, 153], np.int32)
    t_d, s_d = dev_i32(toks), dev_u8(state)
    ri = torch.full((20,), -1, dtype=torch.int32, device="cuda")
    nr = torch.zeros(1, dtype=torch.int32, device="cuda")
    api.dbd_remask_commit(t_d, s_d, dev_i32(argm), torch.from_numpy(conf).cuda(), ri, nr, mask, tau)
    torch.cuda.synchronize()
    et, es, _ = oracle.remask(toks, state, conf.astype(np.float64), argm, mask, float(np.float32(tau)))
    assert et.tolist() == [[5, 121, 9, 9], [9, 131, 9, 9], [9, 9, 142, 9], [9, 1, 2, 3], [150, 9, 4, 9]]
    assert np.array_equal(t_d.cpu().numpy(), et) and np.array_equal(s_d.cpu().numpy(), es)
    rows = oracle.compact_rows(et, es, mask)
    assert nr.item() == rows.size and np.array_equal(ri.cpu().numpy()[:rows.size], rows)
    assert 12 in rows.tolist()          # the position that received the mask token


def test_remask_compact_only():
    S, B, mask = 37, 5, 9
    g = np.random.default_rng(1)
    toks = np.where(g.random((S, B)) < 0.5, mask, 1).astype(np.int32)
    state = g.choice(np.array([2, 3], np.uint8), size=S)
    t_d, s_d = dev_i32(toks), dev_u8(state)
    ri = torch.full((S * B,), -1, dtype=torch.int32, device="cuda")
    nr = torch.zeros(1, dtype=torch.int32, device="cuda")
    api.dbd_remask_commit(t_d, s_d, None, None, ri, nr, mask, 0.9, flags=api.DBD_COMPACT_ONLY)
    rows = oracle.compact_rows(toks, state, mask)
    assert nr.item() == rows.size and np.array_equal(ri.cpu().numpy()[:rows.size], rows)
    assert np.array_equal(t_d.cpu().numpy(), toks) and np.array_equal(s_d.cpu().numpy(), state)


# --------------------------------------------------------------- whole round

def _setup_rounds(w, fx, n_rounds):
    st = RoundState(w, fx)
    st.init_rows()
    attn_out = torch.empty((w.S, w.B, w.Hq, w.D), dtype=torch.bfloat16, device="cuda")
    rins = [synth.make_round(w, r, fx.w_vocab) for r in range(1, n_rounds + 1)]
    devs = [round_inputs_dev(r) for r in rins]
    args = [st.args(d, attn_out) for d in devs]
    return st, rins, devs, args, attn_out


def _run_rounds(w, fx, n_rounds, check_lm_full):
    """Eager rounds with teacher forcing: each round is checked from the
    GPU's state at its start."""
    st, rins, devs, args, _ = _setup_rounds(w, fx, n_rounds)
    history = []
    toks = fx.block_tokens0.copy()
    state = fx.seq_state0.copy()
    for r in range(n_rounds):
        rows0 = oracle.compact_rows(toks, state, w.mask_id)
        assert st.bufs.num_rows.item() == rows0.size
        assert np.array_equal(st.bufs.row_index.cpu().numpy()[:rows0.size], rows0)
        api.dbd_round(args[r])
        torch.cuda.synchronize()
        t1 = st.bufs.block_tokens.cpu().numpy()
        s1 = st.bufs.seq_state.cpu().numpy()
        arg = st.bufs.argmax_tok.cpu().numpy()
        conf = st.bufs.conf.cpu().numpy()
        history.append((t1.copy(), s1.copy()))
        if rows0.size:
            if check_lm_full:
                a, p1, p2, _ = check_lm_rows(rows0, arg, conf, rins[r].hidden, fx.w_vocab, w.mask_id)
                p1_by_row = np.full(w.S * w.B, np.nan); p1_by_row[rows0] = p1
                a_by_row = np.full(w.S * w.B, -1); a_by_row[rows0] = a
                p2_by_row = np.full(w.S * w.B, np.nan); p2_by_row[rows0] = p2
                hid = rins[r].hidden

                def arg_ok(row, tok):
                    if p1_by_row[row] - p2_by_row[row] >= 1e-4:
                        return tok == a_by_row[row]
                    return tok in tie_set(hid[row], fx.w_vocab, w.mask_id, p1_by_row[row])
                check_commits(toks, state, t1, s1, p1_by_row, arg_ok, w.mask_id, w.tau)
            # exact: the commit rule applied by the oracle to the GPU's own
            # float32 confidences and tokens gives the GPU's result
            et, es, _ = oracle.remask(toks, state, conf.astype(np.float64), arg, w.mask_id,
                                      float(np.float32(w.tau)))
            assert np.array_equal(t1, et) and np.array_equal(s1, es)
        else:
            assert np.array_equal(t1, toks)
        toks, state = t1, s1       # teacher forcing: the next round starts from the GPU state
    return st, history


@pytest.mark.parametrize("w", [TINY, SDAR_1P7B], ids=lambda w: w.name)
def test_round_parity_teacher_forced(w):
    fx = synth.make_fixed(w)
    st, hist = _run_rounds(w, fx, w.rounds, check_lm_full=True)
    assert np.all(hist[-1][1] == oracle.SAVING)


def _sample_seqs(rows, B, min_rows, g):
    """Sequences whose listed rows are checked against the oracle: those of
    the first and the last listed row, then random others until at least
    min_rows rows (or every row) are covered."""
    seqs_all = np.unique(rows // B)
    pick = {int(rows[0] // B), int(rows[-1] // B)}
    for s in g.permutation(seqs_all):
        if sum(int(np.sum(rows // B == x)) for x in pick) >= min_rows:
            break
        pick.add(int(s))
    return sorted(pick)


def _round_block(w, fx, min_rows=64, attn_rounds=2, seed=0):
    """Rounds of one block on the GPU until every sequence is SAVING (at most
    the workload's round cap), teacher forced: each round starts from the
    GPU's state.  Every round: the row list is the oracle's compaction of
    that state, and the commits are exactly the rule applied to the GPU's
    own float32 confidences.  Sampled sequences covering at least min_rows
    rows (those of the first and the last listed row among them) are checked
    against the oracle: every row's confidence and token, and the commits
    by the acceptance rule on the oracle's confidences.  The oracle's LM
    head runs once over the sampled rows of all rounds.  Attention is
    checked against the oracle on two (sequence, head) groups in the first
    attn_rounds rounds and the last."""
    g = np.random.default_rng(seed)
    st = RoundState(w, fx)
    st.init_rows()
    attn_out = torch.empty((w.S, w.B, w.Hq, w.D), dtype=torch.bfloat16, device="cuda")
    toks, state = fx.block_tokens0.copy(), fx.seq_state0.copy()
    recs = []
    last_rin = None
    for r in range(1, w.rounds + 1):
        rows0 = oracle.compact_rows(toks, state, w.mask_id)
        assert st.bufs.num_rows.item() == rows0.size
        assert np.array_equal(st.bufs.row_index.cpu().numpy()[:rows0.size], rows0)
        if rows0.size == 0:
            break
        rin = synth.make_round(w, r, fx.w_vocab)
        api.dbd_round(st.args(round_inputs_dev(rin), attn_out))
        torch.cuda.synchronize()
        t1 = st.bufs.block_tokens.cpu().numpy()
        s1 = st.bufs.seq_state.cpu().numpy()
        arg = st.bufs.argmax_tok.cpu().numpy()
        conf = st.bufs.conf.cpu().numpy()
        et, es, _ = oracle.remask(toks, state, conf.astype(np.float64), arg, w.mask_id,
                                  float(np.float32(w.tau)))
        assert np.array_equal(t1, et) and np.array_equal(s1, es), f"round {r}"
        seqs = _sample_seqs(rows0, w.B, min_rows, g)
        srows = np.array([x for x in rows0 if x // w.B in seqs])
        recs.append(dict(r=r, toks=toks, state=state, t1=t1, s1=s1, seqs=seqs, rows=srows,
                         arg=arg[srows], conf=conf[srows], hidden=rin.hidden[srows]))
        if r <= attn_rounds:
            groups = _sample_groups(w, fx.prefix_len, 1, 1, 100 + r)[:2]
            mx, rl2 = compare_attn(host_bits(attn_out), oracle_attn_groups(fx, rin, groups), w.G)
            assert mx <= ATTN_MAX_ABS and rl2 <= ATTN_REL_L2, (r, mx, rl2)
        last_rin = rin
        toks, state = t1, s1
    assert np.all(state == oracle.SAVING), "block not finished within the round cap"
    if len(recs) > attn_rounds:
        groups = _sample_groups(w, fx.prefix_len, 1, 1, 999)[:2]
        mx, rl2 = compare_attn(host_bits(attn_out), oracle_attn_groups(fx, last_rin, groups), w.G)
        assert mx <= ATTN_MAX_ABS and rl2 <= ATTN_REL_L2, ("last", mx, rl2)
    # the oracle over every round's sampled rows at once
    H = np.concatenate([x["hidden"] for x in recs])
    a, p1, p2, ties = oracle_rows_with_ties(H, fx.w_vocab, w.mask_id)
    o = 0
    n_tie = n_ex = 0
    for x in recs:
        n = x["rows"].size
        sl = slice(o, o + n)
        sub_ties = {i - o: t for i, t in ties.items() if o <= i < o + n}
        n_tie += check_rows_against(x["arg"], x["conf"], a[sl], p1[sl], p2[sl], sub_ties,
                                    label=f"round {x['r']}")
        p1_by_row = np.full(w.S * w.B, np.nan)
        p1_by_row[x["rows"]] = p1[sl]
        ok = {int(rw): (int(a[o + j]), p1[o + j] - p2[o + j], sub_ties.get(j))
              for j, rw in enumerate(x["rows"])}

        def arg_ok(row, tok, ok=ok):
            aa, gap, ts = ok[row]
            return tok == aa if gap >= 1e-4 else tok in ts
        n_ex += check_commits(x["toks"], x["state"], x["t1"], x["s1"], p1_by_row, arg_ok, w.mask_id,
                              w.tau, seqs=x["seqs"])
        o += n
    thr = sum(int(((x["t1"] != x["toks"]).sum(1) > 1).sum()) for x in recs)
    print(f"{w.name}: {len(recs)} rounds, {H.shape[0]} oracle rows, tie-exempt {n_tie}, "
          f"band-exempt sequences {n_ex}, sequence-rounds with several commits {thr}", flush=True)
    return recs


@pytest.mark.timeout(900)
@pytest.mark.parametrize("w", [SDAR_4B, SDAR_4B_HIGHCONF, SDAR_8B, SDAR_8B_HIGHCONF, LLADA_LONG],
                         ids=lambda w: w.name)
def test_round_whole_block_sampled(w, big_fixed):
    """Whole blocks at the SDAR-4B (literal and a <= 16), SDAR-8B (block
    16, initial commits, threshold 0.75; literal and a <= 16) and LLaDA
    (block 64, 16K-32K prefixes) shapes: every round until the block is
    full, each against the oracle on at least 64 sampled rows."""
    fx = big_fixed(w)
    recs = _round_block(w, fx)
    masked = [(x["toks"] == w.mask_id).sum() for x in recs] + [(recs[-1]["t1"] == w.mask_id).sum()]
    assert all(b < a for a, b in zip(masked, masked[1:]))
    if w.a_max >= 16.0:
        # the threshold branch fires: some sequence commits several positions in a round
        assert any(((x["t1"] != x["toks"]).sum(1) > 1).any() for x in recs)


@pytest.mark.parametrize("w", [TINY, SDAR_1P7B], ids=lambda w: w.name)
def test_graph_matches_eager(w):
    """One graph of all rounds, replayed three times with eager resets and
    host syncs in between; every replay equals the eager rounds bit for bit."""
    fx = synth.make_fixed(w)
    st_e, hist = _run_rounds(w, fx, w.rounds, check_lm_full=False)
    ref = [st_e.bufs.block_tokens.cpu().numpy(), st_e.bufs.seq_state.cpu().numpy(),
           st_e.bufs.conf.cpu().numpy(), st_e.bufs.argmax_tok.cpu().numpy()]
    st, rins, devs, args, attn_out = _setup_rounds(w, fx, w.rounds)
    gr = api.dbd_graph_create(args)
    try:
        for rep in range(3):
            st.bufs.block_tokens.copy_(dev_i32(fx.block_tokens0))
            st.bufs.seq_state.copy_(dev_u8(fx.seq_state0))
            st.bufs.conf.fill_(float("nan"))
            st.bufs.argmax_tok.fill_(-1)
            st.init_rows()
            torch.cuda.synchronize()
            gr.launch()
            torch.cuda.synchronize()
            got = [st.bufs.block_tokens.cpu().numpy(), st.bufs.seq_state.cpu().numpy(),
                   st.bufs.conf.cpu().numpy(), st.bufs.argmax_tok.cpu().numpy()]
            for a, b in zip(got, ref):
                assert np.array_equal(a, b, equal_nan=True), rep
            assert st.bufs.num_rows.item() == st_e.bufs.num_rows.item()
    finally:
        gr.close()
