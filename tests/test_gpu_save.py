"""Parity of the SAVING step through the C ABI: the K/V write fused into the
attention kernel (dbd_attn_paged_save), the block commit
(dbd_commit_block), and whole multi-block runs of dbd_round steps with
save_kv set, against the CPU oracle on seeded inputs.

The cache, tokens, states, prefix lengths, token stream and row lists are
integer or bit data: compared exactly.  Attention outputs use the usual
attention tolerances (max abs 2e-2, relative L2 5e-3 against the float64
oracle) and must equal dbd_attn_paged's bit for bit (same arithmetic)."""
import numpy as np
import pytest
import torch

import oracle
from block_diffusion_amd import api, synth
from block_diffusion_amd.workloads import SDAR_1P7B, SDAR_4B, TINY, Workload
from gpu_util import (ATTN_MAX_ABS, ATTN_REL_L2, RoundState, attn_errors, check_lm_rows,
                      dev_bf16, dev_i32, dev_u8, host_bits, round_inputs_dev, widen_bits)

pytestmark = pytest.mark.gpu

WAITING, DEN, SAV, FIN = 0, 2, 3, 4


def _states(g, S):
    st = g.choice(np.array([DEN, SAV, SAV, FIN, WAITING], np.uint8), size=S)
    st[0] = SAV
    return st


def _save_case(name):
    """(workload, fixed inputs with room for two more blocks, round inputs)"""
    if name == "tiny":
        w = TINY
    elif name == "ragged_d128":
        # blocks that cross pages (L % P near P), an empty prefix, 5-token blocks
        w = Workload(name="save_ragged", seed_id=40, S=7, B=5, Hq=8, Hkv=2, D=128, P=16,
                     Hd=256, V=1024, mask_id=7, prefix_lo=0, prefix_hi=64, tau=0.9, rounds=5,
                     a_max=12.0, prefix_fixed=(14, 16, 0, 31, 47, 3, 64))
    elif name == "llada_b64":
        # LLaDA heads (MHA, 32 x 128) and 64-token blocks that span pages
        w = Workload(name="save_llada", seed_id=42, S=3, B=64, Hq=32, Hkv=32, D=128, P=256,
                     Hd=256, V=1024, mask_id=7, prefix_lo=0, prefix_hi=600, tau=0.9, rounds=64,
                     a_max=12.0, prefix_fixed=(230, 0, 511))
    elif name == "rt4_d64":
        # G*B = 80 query rows per kv head: two row groups, only the first writes
        w = Workload(name="save_rt4", seed_id=41, S=5, B=5, Hq=32, Hkv=2, D=64, P=32,
                     Hd=256, V=1024, mask_id=7, prefix_lo=0, prefix_hi=90, tau=0.9, rounds=5,
                     a_max=12.0, prefix_fixed=(30, 1, 90, 0, 63))
    elif name == "deep_ring_ragged":
        # page tables that can hold 66 K tiles (the attention takes its
        # three-slot ring) over mostly short, empty and page-crossing
        # prefixes: short tile streams per wave
        lens = (0, 1, 15, 16, 17, 31, 32, 33, 255, 256, 257, 300, 511, 512, 1000, 4000) * 4
        w = Workload(name="save_deep_ring", seed_id=43, S=64, B=4, Hq=32, Hkv=8, D=128, P=256,
                     Hd=256, V=1024, mask_id=7, prefix_lo=0, prefix_hi=4000, tau=0.9, rounds=4,
                     a_max=12.0, prefix_fixed=lens)
    elif name == "sdar4b":
        w = SDAR_4B
    else:
        w = SDAR_1P7B
    fx = synth.make_fixed(w, with_w=False, reserve_tokens=2 * w.B)
    rin = synth.make_round(w, 1, None)
    return w, fx, rin


@pytest.mark.parametrize("name", ["tiny", "ragged_d128", "rt4_d64", "llada_b64", "sdar1p7b",
                                  "deep_ring_ragged", "sdar4b"])
def test_attn_save_parity(name):
    w, fx, rin = _save_case(name)
    g = np.random.default_rng(w.seed_id + 77)
    state = _states(g, w.S)
    print(f"{name}: S={w.S} B={w.B} states {np.bincount(state, minlength=5).tolist()}", flush=True)
    q, kb, vb = dev_bf16(rin.q), dev_bf16(rin.k_blk), dev_bf16(rin.v_blk)
    kc, vc = dev_bf16(fx.k_cache), dev_bf16(fx.v_cache)
    pt, pl, st = dev_i32(fx.page_table), dev_i32(fx.prefix_len), dev_u8(state)
    out = torch.empty((w.S, w.B, w.Hq, w.D), dtype=torch.bfloat16, device="cuda")
    api.dbd_attn_paged_save(q, kb, vb, kc, vc, pt, pl, st, out)
    torch.cuda.synchronize()
    ek, ev = oracle.kv_save(fx.k_cache, fx.v_cache, fx.page_table, fx.prefix_len, state,
                            rin.k_blk, rin.v_blk)
    assert np.array_equal(host_bits(kc), ek)
    assert np.array_equal(host_bits(vc), ev)
    assert np.array_equal(pl.cpu().numpy(), fx.prefix_len)
    assert np.array_equal(st.cpu().numpy(), state)
    # the attention is that of dbd_attn_paged, bit for bit, and the oracle's
    out2 = torch.empty_like(out)
    api.dbd_attn_paged(q, kb, vb, dev_bf16(fx.k_cache), dev_bf16(fx.v_cache), pt, pl, out2)
    torch.cuda.synchronize()
    ob = host_bits(out)
    assert np.array_equal(ob, host_bits(out2))
    groups = [(s, gk) for s in range(w.S) for gk in range(w.Hkv)]
    if len(groups) > 24:
        groups = [groups[i] for i in g.choice(len(groups), 24, replace=False)]
    got, ref = [], []
    for s, gk in groups:
        ref.append(oracle.attention_group(s, gk, rin.q, rin.k_blk, rin.v_blk, fx.k_cache,
                                          fx.v_cache, fx.page_table, fx.prefix_len))
        got.append(widen_bits(ob[s, :, gk * w.G:(gk + 1) * w.G, :]))
    mx, rl = attn_errors(np.stack(got), np.stack(ref))
    assert mx <= ATTN_MAX_ABS and rl <= ATTN_REL_L2, (mx, rl)


@pytest.mark.parametrize("S,B", [(1, 1), (5, 4), (128, 4), (64, 16), (8, 64), (3000, 7)])
def test_commit_block_parity(S, B):
    g = np.random.default_rng(S * 31 + B)
    mask = 151669
    toks = np.where(g.random((S, B)) < 0.4, mask, g.integers(0, mask, (S, B))).astype(np.int32)
    state = g.choice(np.array([DEN, SAV, SAV, FIN, WAITING, 1], np.uint8), size=S)
    L = g.integers(0, 4000, S).astype(np.int32)
    cap = 4000 + B // 2 + 1            # some blocks end past the stream's capacity
    ts = np.full((S, cap), -5, dtype=np.int32)
    end = (L + g.choice([B, 2 * B, 10 ** 6], S)).astype(np.int32)
    for with_stream, with_end in ((True, True), (False, False), (True, False)):
        t_d, s_d, l_d = dev_i32(toks), dev_u8(state), dev_i32(L)
        ts_d = dev_i32(ts) if with_stream else None
        ri = torch.full((S * B,), -1, dtype=torch.int32, device="cuda")
        nr = torch.zeros(1, dtype=torch.int32, device="cuda")
        api.dbd_commit_block(t_d, s_d, l_d, ri, nr, mask, token_stream=ts_d,
                             end_len=dev_i32(end) if with_end else None)
        torch.cuda.synchronize()
        et, es, eL, ets = oracle.commit_block(toks, state, L, mask, ts if with_stream else None,
                                              end if with_end else None)
        assert np.array_equal(t_d.cpu().numpy(), et)
        assert np.array_equal(s_d.cpu().numpy(), es)
        assert np.array_equal(l_d.cpu().numpy(), eL)
        if with_stream:
            assert np.array_equal(ts_d.cpu().numpy(), ets)
        rows = oracle.compact_rows(et, es, mask)
        assert nr.item() == rows.size and np.array_equal(ri.cpu().numpy()[:rows.size], rows)


@pytest.mark.parametrize("w", [TINY, SDAR_1P7B], ids=lambda w: w.name)
def test_multiblock_steps_teacher_forced(w):
    """Steps of dbd_round with save_kv over three blocks per sequence, each
    step checked against the oracle from the GPU's own state: the cache after
    the SAVING writes (bit exact), the attention over the grown prefixes
    (sampled), the LM-head rows (sampled), and the step's commits, prefix
    lengths, states and token stream (exact, the oracle's rule applied to
    the GPU's float32 confidences)."""
    nb = 3
    fx = synth.make_fixed(w, reserve_tokens=nb * w.B)
    st = RoundState(w, fx)
    st.init_rows()
    L0 = fx.prefix_len.copy()
    end = (L0 + nb * w.B).astype(np.int32)
    cap = int(end.max())
    ts_d = torch.full((w.S, cap), -1, dtype=torch.int32, device="cuda")
    end_d = dev_i32(end)
    attn_out = torch.empty((w.S, w.B, w.Hq, w.D), dtype=torch.bfloat16, device="cuda")
    kc, vc = fx.k_cache.copy(), fx.v_cache.copy()
    toks, state, L = fx.block_tokens0.copy(), fx.seq_state0.copy(), L0.copy()
    ts = np.full((w.S, cap), -1, dtype=np.int64)
    g = np.random.default_rng(5)
    max_steps = nb * (w.B + 1) + 2
    for step in range(1, max_steps + 1):
        rin = synth.make_round(w, step, fx.w_vocab)
        a = st.args(round_inputs_dev(rin), attn_out)
        a.save_kv, a.num_pages = 1, int(fx.k_cache.shape[0])
        a.token_stream, a.stream_cap, a.end_len = api._ptr(ts_d), cap, api._ptr(end_d)
        rows0 = oracle.compact_rows(toks, state, w.mask_id)
        print(f"{w.name} step {step}: states {np.bincount(state, minlength=5).tolist()} "
              f"rows {rows0.size}", flush=True)
        api.dbd_round(a)
        torch.cuda.synchronize()
        # SAVING forward: the cache
        kc, vc = oracle.kv_save(kc, vc, fx.page_table, L, state, rin.k_blk, rin.v_blk)
        assert np.array_equal(host_bits(st.fixed["k_cache"]), kc), f"step {step}: k_cache"
        assert np.array_equal(host_bits(st.fixed["v_cache"]), vc), f"step {step}: v_cache"
        # attention over the prefixes as they were at the step's start
        ob = host_bits(attn_out)
        groups = [(s, gk) for s in range(w.S) for gk in range(w.Hkv)]
        if len(groups) > 12:
            groups = [groups[i] for i in g.choice(len(groups), 12, replace=False)]
        got, ref = [], []
        for s, gk in groups:
            ref.append(oracle.attention_group(s, gk, rin.q, rin.k_blk, rin.v_blk, kc, vc,
                                              fx.page_table, L))
            got.append(widen_bits(ob[s, :, gk * w.G:(gk + 1) * w.G, :]))
        mx, rl = attn_errors(np.stack(got), np.stack(ref))
        assert mx <= ATTN_MAX_ABS and rl <= ATTN_REL_L2, (step, mx, rl)
        # LM head on the step's rows
        arg, conf = st.bufs.argmax_tok.cpu().numpy(), st.bufs.conf.cpu().numpy()
        if rows0.size:
            samp = rows0 if w is TINY else rows0[:: max(1, rows0.size // 16)]
            check_lm_rows(samp, arg, conf, rin.hidden, fx.w_vocab, w.mask_id)
        # the step's commits
        et, es, eL, ets, _, erows = oracle.step_commit(toks, state, L, conf, arg, w.mask_id, 0,
                                                       tau=np.float32(w.tau), token_stream=ts,
                                                       end_len=end)
        t1 = st.bufs.block_tokens.cpu().numpy()
        s1 = st.bufs.seq_state.cpu().numpy()
        l1 = st.fixed["prefix_len"].cpu().numpy()
        assert np.array_equal(t1, et) and np.array_equal(s1, es), f"step {step}: commits"
        assert np.array_equal(l1, eL), f"step {step}: prefix_len"
        assert np.array_equal(ts_d.cpu().numpy(), ets), f"step {step}: token stream"
        nr = st.bufs.num_rows.item()
        assert nr == erows.size and np.array_equal(st.bufs.row_index.cpu().numpy()[:nr], erows)
        toks, state, L, ts = t1, s1, l1, ets
        if np.all(state == FIN):
            break
    assert np.all(state == FIN), f"not finished after {max_steps} steps"
    assert np.array_equal(L, end)
    # every position of the stream past the prompt holds a committed token
    for s in range(w.S):
        assert np.all(ts[s, :L0[s]] == -1)
        assert np.all((ts[s, L0[s]:end[s]] >= 0) & (ts[s, L0[s]:end[s]] != w.mask_id))


def _random_save_cases(n, seed=5150):
    """Seeded random SAVING-step shapes: GQA widths 1..16, D 64/128, blocks
    1..64, page sizes 16..256, prefixes empty, page-aligned (the block
    starts a page), a page minus one (the block crosses into the next) or
    drawn, with room for two blocks past each prefix."""
    g = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        D = int(g.choice([64, 128]))
        Hkv = int(g.integers(1, 9))
        G = int(g.choice([1, 2, 4, 6, 16]))
        B = int(g.choice([1, 3, 4, 16, 31, 64]))
        while G * B > 256:
            B = max(1, B // 2)
        P = int(g.choice([16, 32, 64, 256]))
        S = int(g.integers(1, 10))
        L = g.integers(0, 1500, S)
        pick = g.integers(0, 4, S)
        L = np.where(pick == 1, 0, np.where(pick == 2, (L // P) * P,
                                            np.where(pick == 3, np.maximum(P - 1, (L // P) * P - 1), L)))
        cases.append(Workload(name=f"save_rand{i}_s{S}_b{B}_g{G}x{Hkv}_d{D}_p{P}", seed_id=500 + i, S=S, B=B,
                              Hq=G * Hkv, Hkv=Hkv, D=D, P=P, Hd=256, V=1024, mask_id=7, prefix_lo=0,
                              prefix_hi=max(1, int(L.max())), tau=0.9, rounds=B, a_max=12.0,
                              prefix_fixed=tuple(int(x) for x in L)))
    return cases


@pytest.mark.parametrize("w", _random_save_cases(8), ids=lambda w: w.name)
def test_attn_save_random(w):
    """The K/V write of SAVING sequences bit for bit against the oracle, the
    outputs bit for bit against dbd_attn_paged and within the attention
    tolerances of the oracle on sampled groups."""
    fx = synth.make_fixed(w, with_w=False, reserve_tokens=2 * w.B)
    rin = synth.make_round(w, 1, None)
    g = np.random.default_rng(w.seed_id)
    state = _states(g, w.S)
    q, kb, vb = dev_bf16(rin.q), dev_bf16(rin.k_blk), dev_bf16(rin.v_blk)
    kc, vc = dev_bf16(fx.k_cache), dev_bf16(fx.v_cache)
    pt, pl, st = dev_i32(fx.page_table), dev_i32(fx.prefix_len), dev_u8(state)
    out = torch.empty((w.S, w.B, w.Hq, w.D), dtype=torch.bfloat16, device="cuda")
    api.dbd_attn_paged_save(q, kb, vb, kc, vc, pt, pl, st, out)
    torch.cuda.synchronize()
    ek, ev = oracle.kv_save(fx.k_cache, fx.v_cache, fx.page_table, fx.prefix_len, state, rin.k_blk, rin.v_blk)
    assert np.array_equal(host_bits(kc), ek) and np.array_equal(host_bits(vc), ev)
    out2 = torch.empty_like(out)
    api.dbd_attn_paged(q, kb, vb, dev_bf16(fx.k_cache), dev_bf16(fx.v_cache), pt, pl, out2)
    torch.cuda.synchronize()
    ob = host_bits(out)
    assert np.array_equal(ob, host_bits(out2))
    groups = [(s, gk) for s in range(w.S) for gk in range(w.Hkv)]
    groups = [groups[i] for i in sorted(set([0, len(groups) - 1] + list(
        g.choice(len(groups), min(6, len(groups)), replace=False))))]
    got, ref = [], []
    for s, gk in groups:
        ref.append(oracle.attention_group(s, gk, rin.q, rin.k_blk, rin.v_blk, fx.k_cache, fx.v_cache,
                                          fx.page_table, fx.prefix_len))
        got.append(widen_bits(ob[s, :, gk * w.G:(gk + 1) * w.G, :]))
    mx, rl = attn_errors(np.stack(got), np.stack(ref))
    print(f"{w.name} prefixes {list(w.prefix_fixed)} states {state.tolist()}: max abs {mx:.3e} rel L2 {rl:.3e}",
          flush=True)
    assert mx <= ATTN_MAX_ABS and rl <= ATTN_REL_L2
