"""Parity of the other commit rules (static top-k, sequential, entropy
bounded) and of the LM head's softmax entropy, through the C ABI, with the
CPU oracle on seeded inputs.

Entropy tolerance: 1e-3 absolute.  The logits accumulate in fp32; an error
delta_v in logit v moves the entropy by sum_v p_v (l_v - mean_p l) delta_v,
at most max|delta| * E_p|l - mean_p l|, which is below 1e-4 for these
workloads (|delta| ~ 1e-5, logit spread < 20).  Commit decisions are exact:
the oracle's rule is applied to the same float32 confidences and entropies
the kernel read."""
import numpy as np
import pytest
import torch

import oracle
from block_diffusion_amd import api, synth
from block_diffusion_amd.workloads import SDAR_1P7B, TINY
from gpu_util import (RoundState, check_lm_rows, dev_bf16, dev_i32, dev_u8, round_inputs_dev,
                      widen_bits)

pytestmark = pytest.mark.gpu

ENT_TOL = 1e-3


def _lm_run_ent(hidden_bits, w_bits, mask_id, rows, max_rows=None):
    n = hidden_bits.shape[0]
    M = len(rows)
    max_rows = M if max_rows is None else max_rows
    ri = np.zeros(max(max_rows, 1), np.int32)
    ri[:M] = rows
    nr = dev_i32([M])
    arg = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    conf = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    ent = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    h, wv, ri_d = dev_bf16(hidden_bits), dev_bf16(w_bits), dev_i32(ri)
    api.dbd_lmhead_conf(h, wv, nr, arg, conf, mask_id, row_index=ri_d, max_rows=max_rows,
                        entropy=ent)
    # the same call without entropy gives the same tokens and confidences
    arg2 = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    conf2 = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    api.dbd_lmhead_conf(h, wv, nr, arg2, conf2, mask_id, row_index=ri_d, max_rows=max_rows)
    torch.cuda.synchronize()
    assert torch.equal(arg, arg2) and torch.equal(conf.nan_to_num(-1), conf2.nan_to_num(-1))
    return arg.cpu().numpy(), conf.cpu().numpy(), ent.cpu().numpy()


@pytest.mark.parametrize("case", ["tiny", "ragged", "sdar1p7b"])
def test_lmhead_entropy_parity(case):
    if case == "tiny":
        w = TINY
        fx = synth.make_fixed(w)
        h, wv, mask = synth.make_round(w, 1, fx.w_vocab).hidden, fx.w_vocab, w.mask_id
        rows = np.arange(w.S * w.B)
    elif case == "ragged":
        g = np.random.default_rng(5)
        V, Hd, n, mask = 1000, 256, 70, 3
        wv = synth.normal_bf16(g, (V, Hd), std=1.0 / np.sqrt(Hd))
        t = g.integers(0, V, n)
        a = g.uniform(0, 14, n)
        wt = widen_bits(wv[t]); wt /= np.linalg.norm(wt, axis=1, keepdims=True)
        h = synth.f32_to_bf16((g.standard_normal((n, Hd)) + a[:, None] * wt).astype(np.float32))
        rows = g.permutation(n)[:51]
    else:
        w = SDAR_1P7B
        fx = synth.make_fixed(w)
        h, wv, mask = synth.make_round(w, 1, fx.w_vocab).hidden, fx.w_vocab, w.mask_id
        rows = np.random.default_rng(7).choice(w.S * w.B, 32, replace=False)
    arg, conf, ent = _lm_run_ent(h, wv, mask, rows)
    check_lm_rows(rows, arg, conf, h, wv, mask)
    ref = oracle.lmhead_entropy(h[rows], wv, mask)
    err = np.abs(ent[rows].astype(np.float64) - ref).max()
    print(f"{case}: entropy range [{ref.min():.3f}, {ref.max():.3f}], max abs err {err:.2e}")
    assert err <= ENT_TOL
    others = np.setdiff1d(np.arange(h.shape[0]), rows)
    assert np.all(np.isnan(ent[others]))


@pytest.mark.parametrize("rule", [1, 3])
def test_remask_rule_nan(rule):
    """NaN confidences and entropies (with -inf and +inf beside them) under
    the static and entropy-bounded rules: exact against the oracle's reading
    (NaN below every confidence, after every entropy, +inf in the budget)."""
    g = np.random.default_rng(40 + rule)
    S, B, mask = 300, 8, 151669
    toks = np.where(g.random((S, B)) < 0.8, mask, g.integers(0, mask, (S, B))).astype(np.int32)
    state = np.full(S, 2, np.uint8)
    vals = np.array([np.nan, np.nan, -np.inf, np.inf, 0.5, 0.25, 0.5, 2.0], dtype=np.float32)
    conf = g.choice(vals, S * B).astype(np.float32)
    ent = g.choice(vals, S * B).astype(np.float32)
    argm = g.integers(0, mask, S * B).astype(np.int32)
    for k, eb in ((1, 10.0), (3, 1.0), (2, float("inf"))):
        t_d, s_d = dev_i32(toks), dev_u8(state)
        ri = torch.full((S * B,), -1, dtype=torch.int32, device="cuda")
        nr = torch.zeros(1, dtype=torch.int32, device="cuda")
        api.dbd_remask_commit_rule(t_d, s_d, dev_i32(argm), torch.from_numpy(conf).cuda(), ri, nr,
                                   mask, rule, tokens_per_step=k, eb_threshold=eb,
                                   entropy=torch.from_numpy(ent).cuda())
        torch.cuda.synchronize()
        et, es, _ = oracle.remask_rule(toks, state, conf, argm, mask, rule, tokens_per_step=k, eb=eb,
                                       entropy=ent)
        assert np.array_equal(t_d.cpu().numpy(), et), (rule, k, eb)
        assert np.array_equal(s_d.cpu().numpy(), es)
        rows = oracle.compact_rows(et, es, mask)
        assert nr.item() == rows.size and np.array_equal(ri.cpu().numpy()[:rows.size], rows)


@pytest.mark.parametrize("rule", [1, 2, 3])
@pytest.mark.parametrize("S,B", [(1, 1), (3, 4), (128, 4), (64, 16), (8, 64), (1000, 64)])
def test_remask_rule_parity(rule, S, B):
    g = np.random.default_rng(S * 7 + B + 1000 * rule)
    mask = 151669
    toks = np.where(g.random((S, B)) < 0.7, mask, g.integers(0, mask, (S, B))).astype(np.int32)
    state = g.choice(np.array([2, 2, 2, 3, 0, 4], np.uint8), size=S)
    levels = np.array([0.1, 0.5, 0.9, 0.9, 0.3, 0.3], dtype=np.float32)
    conf = np.where(g.random(S * B) < 0.5, g.choice(levels, S * B), g.random(S * B)).astype(np.float32)
    elev = np.array([0.05, 0.3, 0.3, 1.25, 2.5, 0.7], dtype=np.float32)
    ent = np.where(g.random(S * B) < 0.5, g.choice(elev, S * B), 4 * g.random(S * B)).astype(np.float32)
    argm = g.integers(0, mask, S * B).astype(np.int32)
    k = int(g.integers(1, 5))
    eb = float(np.float32(g.choice([0.0, 0.35, 1.0, 3.0])))
    t_d, s_d = dev_i32(toks), dev_u8(state)
    ri = torch.full((S * B,), -1, dtype=torch.int32, device="cuda")
    nr = torch.zeros(1, dtype=torch.int32, device="cuda")
    nc = torch.full((S,), -1, dtype=torch.int32, device="cuda")
    api.dbd_remask_commit_rule(t_d, s_d, dev_i32(argm), torch.from_numpy(conf).cuda(), ri, nr, mask,
                               rule, tokens_per_step=k, eb_threshold=eb,
                               entropy=torch.from_numpy(ent).cuda(), num_committed=nc)
    torch.cuda.synchronize()
    et, es, com = oracle.remask_rule(toks, state, conf, argm, mask, rule, tokens_per_step=k,
                                     eb=eb, entropy=ent)
    assert np.array_equal(t_d.cpu().numpy(), et)
    assert np.array_equal(s_d.cpu().numpy(), es)
    rows = oracle.compact_rows(et, es, mask)
    assert nr.item() == rows.size
    assert np.array_equal(ri.cpu().numpy()[:rows.size], rows)
    den = state == 2
    assert np.array_equal(nc.cpu().numpy()[den], com.sum(1)[den])


@pytest.mark.parametrize("w", [TINY, SDAR_1P7B], ids=lambda w: w.name)
@pytest.mark.parametrize("rule,k,eb", [(1, 1, 0.0), (2, 2, 0.0), (3, 1, 2.0)])
def test_round_rule_teacher_forced(w, rule, k, eb):
    """Whole rounds under a commit rule, from the GPU's state each round: the
    commits are exactly the rule applied to the GPU's own tokens, confidences
    and entropies; those entropies match the oracle's; the block fills."""
    fx = synth.make_fixed(w)
    st = RoundState(w, fx)
    st.init_rows()
    attn_out = torch.empty((w.S, w.B, w.Hq, w.D), dtype=torch.bfloat16, device="cuda")
    ent_d = torch.full((w.S * w.B,), float("nan"), dtype=torch.float32, device="cuda")
    toks, state = fx.block_tokens0.copy(), fx.seq_state0.copy()
    for r in range(1, w.B + 1):
        rin = synth.make_round(w, r, fx.w_vocab)
        a = st.args(round_inputs_dev(rin), attn_out)
        a.rule, a.tokens_per_step, a.eb_threshold = rule, k, eb
        a.entropy = api._ptr(ent_d)
        rows0 = oracle.compact_rows(toks, state, w.mask_id)
        api.dbd_round(a)
        torch.cuda.synchronize()
        t1, s1 = st.bufs.block_tokens.cpu().numpy(), st.bufs.seq_state.cpu().numpy()
        arg, conf = st.bufs.argmax_tok.cpu().numpy(), st.bufs.conf.cpu().numpy()
        ent = ent_d.cpu().numpy()
        if rows0.size:
            samp = rows0 if w is TINY else rows0[:: max(1, rows0.size // 24)]
            check_lm_rows(samp, arg, conf, rin.hidden, fx.w_vocab, w.mask_id)
            if rule == 3:
                ref = oracle.lmhead_entropy(rin.hidden[samp], fx.w_vocab, w.mask_id)
                assert np.abs(ent[samp].astype(np.float64) - ref).max() <= ENT_TOL
        et, es, _ = oracle.remask_rule(toks, state, conf, arg, w.mask_id, rule,
                                       tokens_per_step=k, eb=eb,
                                       entropy=ent if rule == 3 else None)
        assert np.array_equal(t1, et) and np.array_equal(s1, es), f"round {r}"
        toks, state = t1, s1
        if not np.any(state == oracle.DENOISING):
            break
    assert np.all(state == oracle.SAVING)


def _random_remask_cases(n, seed=31337):
    """Seeded random remask inputs: every rule, batches of 1..2500 sequences,
    block lengths 1..64 including odd ones (segments padded to the next power
    of two), thresholds below 0 and above 1, the leftmost fallback, NaN
    confidences and entropies, argmax tokens equal to the mask token."""
    g = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        rule = i % 4
        S = int(g.choice([1, 2, 5, 63, 300, 2500]))
        B = int(g.choice([1, 2, 3, 5, 13, 16, 33, 47, 64]))
        tau = float(np.float32(g.choice([-0.5, 0.0, 0.3, 0.9, 0.999, 1.5])))
        flags = int(g.integers(0, 2)) if rule == 0 else 0
        k = int(g.integers(1, 9))
        eb = float(np.float32(g.choice([0.0, 0.35, 1.0, 5.0])))
        cases.append((f"rand{i}_rule{rule}_s{S}_b{B}", rule, S, B, tau, flags, k, eb))
    return cases


@pytest.mark.parametrize("case", _random_remask_cases(16), ids=lambda c: c[0])
def test_remask_random(case):
    """Bit-exact tokens, states, row list and commit counts against the
    oracle's rule on seeded random inputs."""
    name, rule, S, B, tau, flags, k, eb = case
    g = np.random.default_rng(sum(name.encode()))
    mask = 151669
    toks = np.where(g.random((S, B)) < 0.6, mask, g.integers(0, mask, (S, B))).astype(np.int32)
    state = g.choice(np.array([2, 2, 2, 2, 3, 0, 4], np.uint8), size=S)
    levels = np.array([0.1, 0.5, tau, tau, 0.3, 0.3, np.nan], dtype=np.float32)
    conf = np.where(g.random(S * B) < 0.4, g.choice(levels, S * B), g.random(S * B)).astype(np.float32)
    elev = np.array([0.05, 0.3, 0.3, 1.25, np.nan, 0.7], dtype=np.float32)
    ent = np.where(g.random(S * B) < 0.4, g.choice(elev, S * B), 4 * g.random(S * B)).astype(np.float32)
    argm = np.where(g.random(S * B) < 0.03, mask, g.integers(0, mask, S * B)).astype(np.int32)
    t_d, s_d = dev_i32(toks), dev_u8(state)
    ri = torch.full((S * B,), -1, dtype=torch.int32, device="cuda")
    nr = torch.zeros(1, dtype=torch.int32, device="cuda")
    nc = torch.full((S,), -1, dtype=torch.int32, device="cuda")
    api.dbd_remask_commit_rule(t_d, s_d, dev_i32(argm), torch.from_numpy(conf).cuda(), ri, nr, mask, rule,
                               dynamic_threshold=tau, tokens_per_step=k, eb_threshold=eb,
                               entropy=torch.from_numpy(ent).cuda(), flags=flags, num_committed=nc)
    torch.cuda.synchronize()
    et, es, com = oracle.remask_rule(toks, state, conf, argm, mask, rule, tau=tau, tokens_per_step=k, eb=eb,
                                     entropy=ent, flags=flags)
    assert np.array_equal(t_d.cpu().numpy(), et)
    assert np.array_equal(s_d.cpu().numpy(), es)
    rows = oracle.compact_rows(et, es, mask)
    assert nr.item() == rows.size
    assert np.array_equal(ri.cpu().numpy()[:rows.size], rows)
    den = state == 2
    assert np.array_equal(nc.cpu().numpy()[den], com.sum(1)[den])
    print(f"{name}: {int(com.sum())} commits, {rows.size} rows left", flush=True)
