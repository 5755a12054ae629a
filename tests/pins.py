"""Pins for the CPU oracle: checks against brute force, closed forms, library
special cases and invariants.  Each check takes the implementation (a module
exposing the oracle's functions) so that the same checks can be run on
deliberately broken copies of the oracle (test_oracle_mutants.py) and shown
to fail there.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np

from block_diffusion_amd.synth import f32_to_bf16

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def bf(x):
    return f32_to_bf16(np.asarray(x, dtype=np.float32))


def wid(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ----------------------------------------------------------------- attention

def tiny_attn_case(seed=0, S=2, B=3, Hq=4, Hkv=2, D=8, P=4, L=(7, 0), extra_pages=2):
    g = np.random.default_rng(seed)
    npg = [-(-l // P) for l in L]
    total = sum(npg) + extra_pages
    perm = g.permutation(total)
    maxp = max(max(npg), 1)
    pt = np.full((S, maxp), -1, dtype=np.int32)
    o = 0
    for s, n in enumerate(npg):
        pt[s, :n] = perm[o:o + n]
        o += n
    kc = bf(g.standard_normal((total, Hkv, P, D)))
    vc = bf(g.standard_normal((total, Hkv, P, D)))
    q = bf(g.standard_normal((S, B, Hq, D)))
    kb = bf(g.standard_normal((S, B, Hkv, D)))
    vb = bf(g.standard_normal((S, B, Hkv, D)))
    return dict(q=q, k_blk=kb, v_blk=vb, k_cache=kc, v_cache=vc,
                page_table=pt, prefix_len=np.asarray(L, dtype=np.int32))


def attn_bruteforce(c, scale=None):
    """Scalar loops and math.fsum, walking the page table token by token."""
    q, kb, vb, kc, vc, pt, Ls = (c["q"], c["k_blk"], c["v_blk"], c["k_cache"],
                                 c["v_cache"], c["page_table"], c["prefix_len"])
    S, B, Hq, D = q.shape
    Hkv = kb.shape[2]
    P = kc.shape[2]
    G = Hq // Hkv
    sc = 1.0 / math.sqrt(D) if scale is None else scale
    out = np.zeros((S, B, Hq, D))
    for s in range(S):
        for h in range(Hq):
            g = h // G
            keys, vals = [], []
            for j in range(int(Ls[s])):
                page = int(pt[s][j // P])
                keys.append([float(x) for x in wid(kc[page, g, j % P])])
                vals.append([float(x) for x in wid(vc[page, g, j % P])])
            for j in range(B):
                keys.append([float(x) for x in wid(kb[s, j, g])])
                vals.append([float(x) for x in wid(vb[s, j, g])])
            for i in range(B):
                qi = [float(x) for x in wid(q[s, i, h])]
                z = [math.fsum(a * b for a, b in zip(qi, k)) * sc for k in keys]
                mz = max(z)
                e = [math.exp(t - mz) for t in z]
                den = math.fsum(e)
                for d in range(D):
                    out[s, i, h, d] = math.fsum(e[j] * vals[j][d] for j in range(len(keys))) / den
    return out


def _call_attn(impl, c, scale=None):
    return impl.attention(c["q"], c["k_blk"], c["v_blk"], c["k_cache"], c["v_cache"],
                          c["page_table"], c["prefix_len"], scale)


def check_attn_bruteforce(impl):
    for seed, L, P, B in [(0, (7, 0), 4, 3), (1, (16, 9), 4, 4), (2, (1, 13), 8, 2)]:
        c = tiny_attn_case(seed=seed, L=L, P=P, B=B)
        ref = attn_bruteforce(c)
        got = _call_attn(impl, c)
        assert np.max(np.abs(got - ref)) < 1e-12, (seed, np.max(np.abs(got - ref)))


def check_attn_sdpa(impl):
    """Library special case: after resolving pages, each sequence is plain
    unmasked scaled-dot-product attention over [prefix ++ block], with kv
    heads repeated for the query groups."""
    import torch
    import torch.nn.functional as F
    c = tiny_attn_case(seed=5, S=3, B=4, Hq=6, Hkv=3, D=16, P=4, L=(9, 4, 0))
    got = _call_attn(impl, c)
    S, B, Hq, D = c["q"].shape
    Hkv = c["k_blk"].shape[2]
    P = c["k_cache"].shape[2]
    for s in range(S):
        L = int(c["prefix_len"][s])
        ks, vs = [], []
        for j in range(L):
            p = c["page_table"][s][j // P]
            ks.append(wid(c["k_cache"][p, :, j % P]))
            vs.append(wid(c["v_cache"][p, :, j % P]))
        K = np.concatenate([np.stack(ks, 0) if ks else np.zeros((0, Hkv, D)), wid(c["k_blk"][s])], 0)
        Vv = np.concatenate([np.stack(vs, 0) if vs else np.zeros((0, Hkv, D)), wid(c["v_blk"][s])], 0)
        qt = torch.from_numpy(wid(c["q"][s])).permute(1, 0, 2)[None]          # [1,Hq,B,D]
        kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)[None]
        vt = torch.from_numpy(Vv).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)[None]
        ref = F.scaled_dot_product_attention(qt, kt, vt)[0].permute(1, 0, 2).numpy()
        assert np.max(np.abs(got[s] - ref)) < 1e-12


def check_attn_closed_forms(impl):
    # Q = 0: uniform weights, the mean of all L+B value rows of the group.
    c = tiny_attn_case(seed=3, L=(11, 5), P=4, B=3)
    c["q"] = np.zeros_like(c["q"])
    got = _call_attn(impl, c)
    S, B, Hq, D = c["q"].shape
    Hkv = c["k_blk"].shape[2]
    P = c["k_cache"].shape[2]
    for s in range(S):
        L = int(c["prefix_len"][s])
        for h in range(Hq):
            g = h // (Hq // Hkv)
            rows = [wid(c["v_cache"][c["page_table"][s][j // P], g, j % P]) for j in range(L)]
            rows += [wid(c["v_blk"][s, j, g]) for j in range(B)]
            mean = np.mean(np.stack(rows), 0)
            for i in range(B):
                assert np.max(np.abs(got[s, i, h] - mean)) < 1e-12
    # L = 0, B = 1: the only key is the token itself, O = its value row.
    c = tiny_attn_case(seed=4, S=2, L=(0, 0), B=1)
    got = _call_attn(impl, c)
    G = c["q"].shape[2] // c["k_blk"].shape[2]
    for h in range(c["q"].shape[2]):
        assert np.array_equal(got[:, 0, h], wid(c["v_blk"][:, 0, h // G]))
    # identical keys everywhere: weights uniform whatever q is.
    c = tiny_attn_case(seed=6, L=(6, 3), P=4, B=2)
    one = c["k_blk"][0, 0, 0].copy()
    c["k_cache"][...] = one
    c["k_blk"][...] = one
    got = _call_attn(impl, c)
    c0 = dict(c)
    c0["q"] = np.zeros_like(c["q"])
    assert np.max(np.abs(got - _call_attn(impl, c0))) < 1e-12


def check_attn_block_permutation(impl):
    """Bidirectional within the block: permuting the block's positions
    (queries, keys and values together) permutes the outputs."""
    c = tiny_attn_case(seed=7, L=(5, 10), P=4, B=4)
    base = _call_attn(impl, c)
    perm = np.array([2, 0, 3, 1])
    c2 = dict(c)
    for k in ("q", "k_blk", "v_blk"):
        c2[k] = c[k][:, perm]
    got = _call_attn(impl, c2)
    assert np.max(np.abs(got - base[:, perm])) < 1e-12


def check_attn_page_relabel(impl):
    c = tiny_attn_case(seed=8, L=(13, 6), P=4, B=3, extra_pages=3)
    base = _call_attn(impl, c)
    n = c["k_cache"].shape[0]
    pi = np.random.default_rng(9).permutation(n)
    c2 = dict(c)
    kc = np.empty_like(c["k_cache"]); vc = np.empty_like(c["v_cache"])
    kc[pi] = c["k_cache"]; vc[pi] = c["v_cache"]
    pt = c["page_table"].copy()
    pt[pt >= 0] = pi[pt[pt >= 0]]
    c2.update(k_cache=kc, v_cache=vc, page_table=pt)
    assert np.array_equal(_call_attn(impl, c2), base)


def check_attn_gqa_as_mha(impl):
    c = tiny_attn_case(seed=10, S=2, B=3, Hq=6, Hkv=2, D=8, P=4, L=(9, 2))
    base = _call_attn(impl, c)
    G = 3
    c2 = dict(c)
    for k in ("k_blk", "v_blk"):
        c2[k] = np.repeat(c[k], G, axis=2)
    for k in ("k_cache", "v_cache"):
        c2[k] = np.repeat(c[k], G, axis=1)
    assert np.max(np.abs(_call_attn(impl, c2) - base)) < 1e-12


def check_attn_golden(impl):
    with open(os.path.join(GOLDEN, "closed_form_cases.json")) as f:
        cases = json.load(f)["attention"]
    for c in cases:
        arr = {k: bf(np.array(c[k], dtype=np.float32)) for k in
               ("q", "k_blk", "v_blk", "k_cache", "v_cache")}
        got = impl.attention(arr["q"], arr["k_blk"], arr["v_blk"], arr["k_cache"],
                             arr["v_cache"], np.array(c["page_table"], dtype=np.int32),
                             np.array(c["prefix_len"], dtype=np.int32))
        assert np.max(np.abs(got - np.array(c["expect"]))) < 1e-15, c["name"]


ATTN_CHECKS = [check_attn_golden, check_attn_bruteforce, check_attn_sdpa, check_attn_closed_forms,
               check_attn_block_permutation, check_attn_page_relabel,
               check_attn_gqa_as_mha]


# ------------------------------------------------------------------- LM head

def lm_bruteforce(h_bits, w_bits, mask_id):
    H = wid(h_bits); W = wid(w_bits)
    out = []
    for r in range(H.shape[0]):
        logit = {}
        for v in range(W.shape[0]):
            if v == mask_id:
                continue
            logit[v] = math.fsum(float(a) * float(b) for a, b in zip(H[r], W[v]))
        m = max(logit.values())
        arg = min(v for v, x in logit.items() if x == m)
        e = sorted((math.exp(x - m) for x in logit.values()), reverse=True)
        den = math.fsum(e)
        out.append((arg, 1.0 / den, e[1] / den))
    return out


def check_lm_bruteforce(impl):
    g = np.random.default_rng(11)
    for V, Hd, mask in [(12, 4, 11), (17, 8, 0), (9, 16, 4)]:
        h = bf(g.standard_normal((5, Hd)) * 2)
        w = bf(g.standard_normal((V, Hd)))
        a, p1, p2 = impl.lmhead_rows(h, w, mask)
        for r, (ea, e1, e2) in enumerate(lm_bruteforce(h, w, mask)):
            assert a[r] == ea
            assert abs(p1[r] - e1) < 1e-13 and abs(p2[r] - e2) < 1e-13


def check_lm_zero_hidden(impl):
    """h = 0: every candidate logit is 0, so max_p = 1/(V-1) and the argmax is
    the smallest id that is not the mask."""
    for V, mask in [(10, 9), (10, 0), (33, 5)]:
        w = bf(np.random.default_rng(V).standard_normal((V, 8)))
        h = np.zeros((3, 8), dtype=np.uint16)
        a, p1, p2 = impl.lmhead_rows(h, w, mask)
        assert np.all(a == (1 if mask == 0 else 0))
        assert np.allclose(p1, 1.0 / (V - 1), rtol=0, atol=1e-15)
        assert np.allclose(p2, 1.0 / (V - 1), rtol=0, atol=1e-15)


def check_lm_one_hot(impl):
    """W column t = c*e_k, every other column 0, h = e_k: logit c at t, 0
    elsewhere, so max_p = e^c / (e^c + V - 2)."""
    V, Hd, mask = 20, 6, 19
    for t, k, c in [(3, 2, 2.5), (0, 5, 7.0), (18, 0, 0.75)]:
        w = np.zeros((V, Hd), dtype=np.float32)
        w[t, k] = c
        h = np.zeros((1, Hd), dtype=np.float32)
        h[0, k] = 1.0
        a, p1, _ = impl.lmhead_rows(bf(h), bf(w), mask)
        assert a[0] == t
        assert abs(p1[0] - math.exp(c) / (math.exp(c) + V - 2)) < 1e-14


def check_lm_vocab_permutation(impl):
    g = np.random.default_rng(12)
    V, Hd, mask = 40, 8, 7
    h = bf(g.standard_normal((6, Hd)) * 3)
    w = bf(g.standard_normal((V, Hd)))
    a, p1, p2 = impl.lmhead_rows(h, w, mask)
    pi = g.permutation(V)                    # new id of old id v is pi[v]
    w2 = np.empty_like(w); w2[pi] = w
    a2, q1, q2 = impl.lmhead_rows(h, w2, int(pi[mask]))
    assert np.array_equal(a2, pi[a])
    assert np.max(np.abs(q1 - p1)) < 1e-12 and np.max(np.abs(q2 - p2)) < 1e-12


def check_lm_mask_never_chosen(impl):
    g = np.random.default_rng(13)
    V, Hd, mask = 30, 8, 12
    h = g.standard_normal((4, Hd)).astype(np.float32)
    w = g.standard_normal((V, Hd)).astype(np.float32) * 0.1
    w[mask] = 50.0 * h[0] / np.linalg.norm(h[0])
    a, p1, _ = impl.lmhead_rows(bf(h), bf(w), mask)
    assert not np.any(a == mask)
    # the normaliser leaves the mask out too (brute force skips its column).
    ref = lm_bruteforce(bf(h), bf(w), mask)
    for r, (ea, e1, _) in enumerate(ref):
        assert a[r] == ea and abs(p1[r] - e1) < 1e-13


def check_lm_ties_lowest(impl):
    V, Hd, mask = 16, 4, 15
    w = np.zeros((V, Hd), dtype=np.float32)
    w[9, 1] = 3.0
    w[4, 1] = 3.0
    w[12, 1] = 3.0
    h = np.zeros((1, Hd), dtype=np.float32); h[0, 1] = 1.0
    a, p1, p2 = impl.lmhead_rows(bf(h), bf(w), mask)
    assert a[0] == 4 and p1[0] == p2[0]


def check_lm_scipy(impl):
    from scipy.special import softmax
    g = np.random.default_rng(14)
    V, Hd, mask = 300, 32, 123
    h = bf(g.standard_normal((8, Hd)) * 2)
    w = bf(g.standard_normal((V, Hd)) / np.sqrt(Hd))
    a, p1, p2 = impl.lmhead_rows(h, w, mask)
    logit = wid(h) @ wid(w).T
    keep = np.array([v for v in range(V) if v != mask])
    p = softmax(logit[:, keep], axis=1)
    assert np.array_equal(a, keep[np.argmax(p, axis=1)])
    assert np.max(np.abs(p1 - p.max(1))) < 1e-14
    assert np.max(np.abs(p2 - np.sort(p, 1)[:, -2])) < 1e-14


def check_lm_golden(impl):
    with open(os.path.join(GOLDEN, "closed_form_cases.json")) as f:
        cases = json.load(f)["lmhead"]
    for c in cases:
        a, p1, p2 = impl.lmhead_rows(bf(np.array(c["hidden"], dtype=np.float32)),
                                     bf(np.array(c["w_vocab"], dtype=np.float32)), c["mask_id"])
        assert a.tolist() == c["expect_argmax"], c["name"]
        assert np.max(np.abs(p1 - np.array(c["expect_p1"]))) < 1e-15, c["name"]
        assert np.max(np.abs(p2 - np.array(c["expect_p2"]))) < 1e-15, c["name"]


def lm_entropy_bruteforce(h_bits, w_bits, mask_id):
    H = wid(h_bits); W = wid(w_bits)
    out = []
    for r in range(H.shape[0]):
        logit = [math.fsum(float(a) * float(b) for a, b in zip(H[r], W[v]))
                 for v in range(W.shape[0]) if v != mask_id]
        m = max(logit)
        e = [math.exp(x - m) for x in logit]
        den = math.fsum(e)
        out.append(-math.fsum((t / den) * math.log(t / den) for t in e if t > 0))
    return out


def check_lm_entropy_bruteforce(impl):
    g = np.random.default_rng(21)
    for V, Hd, mask in [(12, 4, 11), (17, 8, 0), (9, 16, 4)]:
        h = bf(g.standard_normal((5, Hd)) * 2)
        w = bf(g.standard_normal((V, Hd)))
        H = impl.lmhead_entropy(h, w, mask)
        for r, e in enumerate(lm_entropy_bruteforce(h, w, mask)):
            assert abs(H[r] - e) < 1e-12


def check_lm_entropy_closed_forms(impl):
    """h = 0: uniform over the V-1 candidates, H = ln(V-1).  One-hot W with
    logit c at t: p_t = e^c/(e^c+V-2), the rest share 1-p_t equally, so
    H = -p_t ln p_t - (1-p_t) ln((1-p_t)/(V-2))."""
    for V, mask in [(10, 9), (33, 5)]:
        w = bf(np.random.default_rng(V).standard_normal((V, 8)))
        H = impl.lmhead_entropy(np.zeros((2, 8), dtype=np.uint16), w, mask)
        assert np.allclose(H, math.log(V - 1), rtol=0, atol=1e-13)
    V, Hd, mask = 20, 6, 19
    for t, k, c in [(3, 2, 2.5), (0, 5, 7.0)]:
        w = np.zeros((V, Hd), dtype=np.float32)
        w[t, k] = c
        h = np.zeros((1, Hd), dtype=np.float32)
        h[0, k] = 1.0
        pt = math.exp(c) / (math.exp(c) + V - 2)
        want = -pt * math.log(pt) - (1 - pt) * math.log((1 - pt) / (V - 2))
        assert abs(impl.lmhead_entropy(bf(h), bf(w), mask)[0] - want) < 1e-13


def check_lm_entropy_scipy(impl):
    from scipy.special import softmax
    from scipy.stats import entropy
    g = np.random.default_rng(22)
    V, Hd, mask = 300, 32, 123
    h = bf(g.standard_normal((8, Hd)) * 2)
    w = bf(g.standard_normal((V, Hd)) / np.sqrt(Hd))
    logit = wid(h) @ wid(w).T
    keep = np.array([v for v in range(V) if v != mask])
    p = softmax(logit[:, keep], axis=1)
    assert np.max(np.abs(impl.lmhead_entropy(h, w, mask) - entropy(p, axis=1))) < 1e-12


def check_lm_no_candidate(impl):
    """A row with no candidate (every logit but the mask's is -inf: W all
    -inf against a positive hidden row) gives the mask token, confidence 0
    and runner-up 0, and entropy +inf; other rows are unaffected."""
    V, Hd, mask = 10, 4, 3
    h = bf(np.ones((2, Hd)))
    w = bf(np.full((V, Hd), -np.inf))
    a, p1, p2 = impl.lmhead_rows(h, w, mask)
    assert np.all(a == mask) and np.all(p1 == 0.0) and np.all(p2 == 0.0), (a, p1, p2)
    assert np.all(impl.lmhead_entropy(h, w, mask) == np.inf)
    g = np.random.default_rng(12)
    w2 = bf(g.standard_normal((V, Hd)))
    a2, q1, _ = impl.lmhead_rows(h, w2, mask)
    ref = lm_bruteforce(h, w2, mask)
    assert a2[0] == ref[0][0] and abs(q1[0] - ref[0][1]) < 1e-13


LM_CHECKS = [check_lm_no_candidate, check_lm_entropy_bruteforce, check_lm_entropy_closed_forms, check_lm_entropy_scipy,
             check_lm_golden, check_lm_bruteforce, check_lm_zero_hidden, check_lm_one_hot,
             check_lm_vocab_permutation, check_lm_mask_never_chosen,
             check_lm_ties_lowest, check_lm_scipy]


# -------------------------------------------------------------------- remask

DEN, SAV = 2, 3


def remask_bruteforce(toks, state, conf, argm, mask_id, tau):
    """Enumerate every subset C of the masked set and keep the one that the
    rule characterises: if some masked confidence reaches tau, C is exactly
    the set of those positions (every member reaches tau, and every position
    that reaches tau is a member); otherwise C is a singleton {j} with conf_j
    >= every masked confidence and j lower than any other position of equal
    confidence."""
    S, B = toks.shape
    conf = np.asarray(conf).reshape(S, B)
    argm = np.asarray(argm).reshape(S, B)
    nt = toks.copy(); ns = state.copy()
    for s in range(S):
        if state[s] != DEN:
            continue
        M = [i for i in range(B) if toks[s, i] == mask_id]
        sols = []
        for r in range(1, len(M) + 1):
            for C in itertools.combinations(M, r):
                above = [i for i in M if conf[s, i] >= tau]
                if above:
                    ok = set(C) == set(above) and all(conf[s, i] >= tau for i in C)
                else:
                    j = C[0]
                    ok = (len(C) == 1 and all(conf[s, j] >= conf[s, i] for i in M)
                          and all(not (conf[s, i] == conf[s, j] and i < j) for i in M))
                if ok:
                    sols.append(C)
        assert len(sols) == (1 if M else 0)
        for C in sols:
            for i in C:
                nt[s, i] = argm[s, i]
        if not np.any(nt[s] == mask_id):
            ns[s] = SAV
    return nt, ns


def random_remask_case(g, S, B, mask_id, tau, exact=True):
    toks = np.where(g.random((S, B)) < 0.7, mask_id, g.integers(0, mask_id, (S, B))).astype(np.int64)
    state = np.where(g.random(S) < 0.85, DEN, SAV).astype(np.uint8)
    levels = np.array([0.1, 0.3, tau, tau, 0.5, 0.95, 0.95, 0.2]) if exact else None
    conf = (g.choice(levels, size=S * B) if exact else g.random(S * B))
    argm = g.integers(0, mask_id, S * B)
    return toks, state, conf, argm


def check_remask_bruteforce(impl):
    g = np.random.default_rng(15)
    for B in (1, 2, 3, 4, 5, 6):
        for _ in range(40):
            tau = float(g.choice([0.5, 0.75, 0.9]))
            toks, state, conf, argm = random_remask_case(g, 4, B, 99, tau)
            et, es = remask_bruteforce(toks, state, conf, argm, 99, tau)
            nt, ns, _ = impl.remask(toks, state, conf, argm, 99, tau)
            assert np.array_equal(nt, et) and np.array_equal(ns, es)


def check_remask_invariants(impl):
    """Over whole blocks: committed tokens never change, each round of a
    DENOISING sequence with a mask left commits at least one, the masked
    count strictly falls, SAVING iff no mask is left, and a block finishes
    within |M_1| rounds."""
    g = np.random.default_rng(16)
    mask = 50
    for B in (1, 4, 16, 64):
        S = 5
        toks = np.where(g.random((S, B)) < 0.8, mask, g.integers(0, mask, (S, B))).astype(np.int64)
        state = np.full(S, DEN, dtype=np.uint8)
        m0 = (toks == mask).sum(1)
        rounds = 0
        while np.any(state == DEN):
            conf = g.random(S * B)
            argm = g.integers(0, mask, S * B)
            nt, ns, com = impl.remask(toks, state, conf, argm, mask, 0.9)
            was = toks != mask
            assert np.array_equal(nt[was], toks[was])
            for s in range(S):
                if state[s] == DEN:
                    before = (toks[s] == mask).sum(); after = (nt[s] == mask).sum()
                    if before:
                        assert after < before and com[s].sum() >= 1
                    assert (ns[s] == SAV) == (after == 0)
                else:
                    assert np.array_equal(nt[s], toks[s]) and ns[s] == state[s]
            toks, state = nt, ns
            rounds += 1
            assert rounds <= max(1, m0.max())


def check_remask_special_thresholds(impl):
    """tau > 1: exactly one commit per round, the most confident (the static
    one-token-per-step schedule of block 4 / 4 steps); tau <= 0: every masked
    position commits in the first round."""
    g = np.random.default_rng(17)
    mask, S, B = 77, 3, 4
    toks = np.full((S, B), mask, dtype=np.int64)
    state = np.full(S, DEN, dtype=np.uint8)
    for r in range(B):
        conf = g.random(S * B)
        argm = g.integers(0, mask, S * B)
        nt, ns, com = impl.remask(toks, state, conf, argm, mask, 1.5)
        c2 = conf.reshape(S, B)
        for s in range(S):
            assert com[s].sum() == 1
            M = np.where(toks[s] == mask)[0]
            j = M[np.argmax(c2[s, M])]
            assert com[s, j]
        toks, state = nt, ns
    assert np.all(state == SAV)
    toks = np.full((S, B), mask, dtype=np.int64)
    state = np.full(S, DEN, dtype=np.uint8)
    nt, ns, com = impl.remask(toks, state, g.random(S * B), g.integers(0, mask, S * B), mask, 0.0)
    assert com.all() and np.all(ns == SAV)


def check_remask_golden(impl):
    with open(os.path.join(GOLDEN, "remask_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        toks = np.array(c["block_tokens"], dtype=np.int64)
        state = np.array(c["seq_state"], dtype=np.uint8)
        nt, ns, _ = impl.remask(toks, state, np.array(c["conf"], dtype=np.float64),
                                np.array(c["argmax"]), c["mask_id"], c["tau"],
                                c.get("flags", 0))
        assert nt.tolist() == c["expect_tokens"], c["name"]
        assert ns.tolist() == c["expect_state"], c["name"]


def check_compact_rows(impl):
    mask = 9
    toks = np.array([[9, 1, 9, 9], [2, 3, 4, 5], [9, 9, 0, 9], [9, 9, 9, 9]])
    state = np.array([DEN, DEN, SAV, DEN], dtype=np.uint8)
    assert impl.compact_rows(toks, state, mask).tolist() == [0, 2, 3, 12, 13, 14, 15]


REMASK_CHECKS = [check_remask_bruteforce, check_remask_invariants,
                 check_remask_special_thresholds, check_remask_golden,
                 check_compact_rows]


# -------------------------------------------------------------- commit rules

def rule_bruteforce(toks, state, conf, ent, argm, mask_id, rule, k, eb):
    """Enumerate every subset C of the masked set and keep the ones the
    rule's characterisation admits:
      static:     |C| = min(k,|M|), and no position outside C beats one in C
                  (higher confidence, or equal and lower position);
      sequential: |C| = min(k,|M|), and no position outside C lies left of
                  one in C;
      entropy:    C is a leading run of M sorted by (entropy, position), its
                  running sum (float32, in that order) is within eb unless
                  |C| = 1, and adding the next position would exceed eb.
    Exactly one subset must qualify."""
    S, B = toks.shape
    conf = np.asarray(conf).reshape(S, B)
    ent = np.asarray(ent, dtype=np.float32).reshape(S, B)
    argm = np.asarray(argm).reshape(S, B)
    nt = toks.copy(); ns = state.copy()
    for s in range(S):
        if state[s] != DEN:
            continue
        M = [i for i in range(B) if toks[s, i] == mask_id]
        kk = min(max(k, 1), len(M))
        order = sorted(M, key=lambda i: (ent[s, i], i))
        sols = []
        for r in range(1, len(M) + 1):
            for C in itertools.combinations(M, r):
                out = [i for i in M if i not in C]
                if rule == 1:
                    ok = r == kk and not any(
                        conf[s, o] > conf[s, c] or (conf[s, o] == conf[s, c] and o < c)
                        for o in out for c in C)
                elif rule == 2:
                    ok = r == kk and not any(o < c for o in out for c in C)
                else:
                    ok = sorted(C, key=lambda i: (ent[s, i], i)) == order[:r]
                    run = np.float32(0)
                    for i in order[:r]:
                        run = np.float32(run + ent[s, i])
                    ok = ok and (r == 1 or run <= np.float32(eb))
                    if ok and r < len(M):
                        ok = np.float32(run + ent[s, order[r]]) > np.float32(eb)
                if ok:
                    sols.append(C)
        assert len(sols) == (1 if M else 0), (rule, sols)
        for C in sols:
            for i in C:
                nt[s, i] = argm[s, i]
        if not np.any(nt[s] == mask_id):
            ns[s] = SAV
    return nt, ns


def _rule_case(g, S, B, mask_id):
    toks, state, conf, argm = random_remask_case(g, S, B, mask_id, 0.5)
    ent = g.choice(np.array([0.05, 0.3, 0.3, 1.2, 2.5, 0.7], dtype=np.float32), size=S * B)
    return toks, state, conf, ent, argm


def check_rule_bruteforce(impl):
    g = np.random.default_rng(23)
    for rule in (1, 2, 3):
        for B in (1, 2, 3, 4, 5, 6):
            for _ in range(25):
                toks, state, conf, ent, argm = _rule_case(g, 3, B, 99)
                k = int(g.integers(1, 4))
                eb = float(g.choice([0.0, 0.35, 1.0, 3.0, 100.0]))
                et, es = rule_bruteforce(toks, state, conf, ent, argm, 99, rule, k, eb)
                nt, ns, _ = impl.remask_rule(toks, state, conf, argm, 99, rule,
                                             tokens_per_step=k, eb=eb, entropy=ent)
                assert np.array_equal(nt, et) and np.array_equal(ns, es), (rule, B)


def check_rule_special_cases(impl):
    """static with k = 1 is the dynamic rule with tau > 1; sequential with
    k = 1 is the dynamic rule with tau > 1 and the leftmost fallback; an
    unbounded entropy budget commits every masked position, a negative one
    exactly the lowest-entropy position."""
    g = np.random.default_rng(24)
    for _ in range(30):
        toks, state, conf, ent, argm = _rule_case(g, 5, 6, 77)
        a = impl.remask_rule(toks, state, conf, argm, 77, 1, tokens_per_step=1)
        b = impl.remask(toks, state, conf, argm, 77, 1.5)
        assert all(np.array_equal(x, y) for x, y in zip(a, b))
        a = impl.remask_rule(toks, state, conf, argm, 77, 2, tokens_per_step=1)
        b = impl.remask(toks, state, conf, argm, 77, 1.5, 1)
        assert all(np.array_equal(x, y) for x, y in zip(a, b))
        nt, ns, com = impl.remask_rule(toks, state, conf, argm, 77, 3, eb=1e30, entropy=ent)
        den = state == DEN
        assert np.array_equal(com[den], toks[den] == 77)
        nt, ns, com = impl.remask_rule(toks, state, conf, argm, 77, 3, eb=-1.0, entropy=ent)
        e2 = ent.reshape(5, 6)
        for s in np.where(den)[0]:
            M = np.where(toks[s] == 77)[0]
            if M.size:
                j = min(M, key=lambda i: (e2[s, i], i))
                assert com[s].sum() == 1 and com[s, j]


def check_rule_invariants(impl):
    """Whole blocks under each rule: committed tokens never change, at least
    one commit per round while a mask is left, SAVING iff no mask left,
    static / sequential commit exactly min(k, |M|)."""
    g = np.random.default_rng(25)
    mask = 50
    for rule in (1, 2, 3):
        for B in (1, 4, 16, 64):
            S = 4
            toks = np.where(g.random((S, B)) < 0.8, mask, g.integers(0, mask, (S, B))).astype(np.int64)
            state = np.full(S, DEN, dtype=np.uint8)
            while np.any(state == DEN):
                conf = g.random(S * B)
                ent = (g.random(S * B) * 3).astype(np.float32)
                k = int(g.integers(1, 5))
                nt, ns, com = impl.remask_rule(toks, state, conf, g.integers(0, mask, S * B), mask,
                                               rule, tokens_per_step=k, eb=2.0, entropy=ent)
                assert np.array_equal(nt[toks != mask], toks[toks != mask])
                for s in range(S):
                    if state[s] != DEN:
                        continue
                    before = (toks[s] == mask).sum()
                    if before:
                        assert com[s].sum() >= 1
                        if rule in (1, 2):
                            assert com[s].sum() == min(k, before)
                    assert (ns[s] == SAV) == ((nt[s] == mask).sum() == 0)
                toks, state = nt, ns


def check_rule_nan_cases(impl):
    """Hand-worked cases of the NaN readings: a NaN confidence ranks below
    every number (the static rule takes numbers first, then NaN positions
    from the left); a NaN entropy ranks after every number, +inf included,
    and counts as +inf in the budget."""
    mask, nan, inf = 9, np.nan, np.inf
    toks = np.full((1, 4), mask, dtype=np.int64)
    st = np.array([DEN], dtype=np.uint8)
    argm = np.array([10, 11, 12, 13])
    cases = [  # (rule, k, eb, conf, entropy, committed positions)
        (1, 2, 0.0, [nan, 0.2, nan, 0.1], None, [1, 3]),
        (1, 2, 0.0, [nan, nan, 0.3, nan], None, [0, 2]),
        (1, 1, 0.0, [nan, -inf, nan, nan], None, [1]),
        (3, 1, 10.0, None, [nan, 0.5, inf, 0.25], [1, 3]),
        (3, 1, 10.0, None, [nan, nan, nan, nan], [0]),
        (3, 1, inf, None, [nan, 1.0, nan, 2.0], [0, 1, 2, 3]),
        (3, 1, 10.0, None, [nan, inf, nan, 2.0], [3]),
    ]
    for rule, k, eb, conf, ent, exp in cases:
        c = np.zeros(4) if conf is None else np.array(conf)
        e = None if ent is None else np.array(ent, dtype=np.float32)
        nt, ns, com = impl.remask_rule(toks, st, c, argm, mask, rule, tokens_per_step=k, eb=eb,
                                       entropy=e)
        assert np.nonzero(com[0])[0].tolist() == exp, (rule, conf, ent, com[0])
        assert all(nt[0, i] == argm[i] for i in exp)


RULE_CHECKS = [check_rule_bruteforce, check_rule_special_cases, check_rule_invariants,
               check_rule_nan_cases]


# ------------------------------------------------- SAVING step, block commit
# The checks take the implementation for kv_save / commit_block / step_commit
# and the real (separately pinned) oracle for attention and the rules.

FIN = 4


def _saving_case(seed, S=3, B=3, Hq=4, Hkv=2, D=8, P=4, L=(7, 0, 5), blocks=2):
    """A paged cache whose tables already cover `blocks` more blocks, with
    the slots past each prefix filled with NaN."""
    g = np.random.default_rng(seed)
    npg = [-(-(l + blocks * B) // P) for l in L]
    total = sum(npg) + 2
    perm = g.permutation(total)
    pt = np.full((S, max(npg)), -1, dtype=np.int32)
    o = 0
    for s, n in enumerate(npg):
        pt[s, :n] = perm[o:o + n]
        o += n
    kc = bf(g.standard_normal((total, Hkv, P, D)))
    vc = bf(g.standard_normal((total, Hkv, P, D)))
    for s in range(S):
        for p in range(L[s], npg[s] * P):
            kc[pt[s, p // P], :, p % P] = 0x7FC0
            vc[pt[s, p // P], :, p % P] = 0x7FC0

    def blk():
        return (bf(g.standard_normal((S, B, Hq, D))), bf(g.standard_normal((S, B, Hkv, D))),
                bf(g.standard_normal((S, B, Hkv, D))))
    return g, dict(k_cache=kc, v_cache=vc, page_table=pt, prefix_len=np.asarray(L, np.int32)), blk


def _attn_lists(q, keys, vals, sc):
    """Attention of q [B][Hq][D] (float64) over explicit per-kv-head key and
    value lists keys[g] = [n][D]: scalar loops and math.fsum."""
    B, Hq, D = q.shape
    G = Hq // len(keys)
    out = np.zeros((B, Hq, D))
    for h in range(Hq):
        K, V = keys[h // G], vals[h // G]
        for i in range(B):
            z = [math.fsum(a * b for a, b in zip(q[i, h], k)) * sc for k in K]
            mz = max(z)
            e = [math.exp(t - mz) for t in z]
            den = math.fsum(e)
            for d in range(D):
                out[i, h, d] = math.fsum(e[j] * V[j][d] for j in range(len(K))) / den
    return out


def check_kvsave_attention(impl):
    """After the SAVING step and the commit, the next block's attention over
    the cache equals attention over an explicit key list: the old prefix
    (walked through the page table), the saved block, the new block; for a
    sequence that was not SAVING, the old prefix and the new block."""
    import oracle as real
    for seed, L, P, B in [(0, (7, 0, 5), 4, 3), (1, (3, 8, 1), 4, 2), (2, (16, 9, 4), 8, 4)]:
        g, c, blk = _saving_case(seed, B=B, P=P, L=L)
        S = len(L)
        state = np.array([SAV, SAV, DEN], dtype=np.uint8)
        q1, kb1, vb1 = blk()
        kc2, vc2 = impl.kv_save(c["k_cache"], c["v_cache"], c["page_table"], c["prefix_len"],
                                state, kb1, vb1)
        toks = g.integers(0, 50, (S, B))
        toks[2, 0] = 99
        t2, s2, L2, _ = impl.commit_block(toks, state, c["prefix_len"], 99)
        q2, kb2, vb2 = blk()
        got = real.attention(q2, kb2, vb2, kc2, vc2, c["page_table"], L2)
        Hkv, D = kb1.shape[2], kb1.shape[3]
        for s in range(S):
            keys, vals = [], []
            for gk in range(Hkv):
                K, V = [], []
                for j in range(int(L[s])):
                    page = int(c["page_table"][s][j // P])
                    K.append(list(wid(c["k_cache"][page, gk, j % P])))
                    V.append(list(wid(c["v_cache"][page, gk, j % P])))
                if state[s] == SAV:
                    K += [list(wid(kb1[s, j, gk])) for j in range(B)]
                    V += [list(wid(vb1[s, j, gk])) for j in range(B)]
                K += [list(wid(kb2[s, j, gk])) for j in range(B)]
                V += [list(wid(vb2[s, j, gk])) for j in range(B)]
                keys.append(K)
                vals.append(V)
            ref = _attn_lists(wid(q2[s]), keys, vals, 1.0 / math.sqrt(D))
            assert np.max(np.abs(got[s] - ref)) < 1e-12, (seed, s)


def check_kvsave_untouched(impl):
    """Exactly the slots at positions prefix_len..prefix_len+B-1 of SAVING
    sequences change, to the block's bits; every other bit (NaN tails
    included) is unchanged; the inputs are not modified."""
    for seed, L, P, B in [(3, (7, 0, 5), 4, 3), (4, (4, 12, 2), 4, 4), (5, (0, 1, 30), 16, 5)]:
        g, c, blk = _saving_case(seed, B=B, P=P, L=L)
        for state in ([SAV, DEN, SAV], [DEN, DEN, DEN], [SAV, SAV, SAV], [0, SAV, FIN]):
            state = np.array(state, dtype=np.uint8)
            _, kb, vb = blk()
            k0, v0 = c["k_cache"].copy(), c["v_cache"].copy()
            kc2, vc2 = impl.kv_save(c["k_cache"], c["v_cache"], c["page_table"], c["prefix_len"],
                                    state, kb, vb)
            assert np.array_equal(c["k_cache"], k0) and np.array_equal(c["v_cache"], v0)
            touched = np.zeros(k0.shape[:1] + k0.shape[2:3], dtype=bool)   # [page][slot]
            for s in np.where(state == SAV)[0]:
                for j in range(B):
                    p = int(L[s]) + j
                    pg = int(c["page_table"][s][p // P])
                    touched[pg, p % P] = True
                    assert np.array_equal(kc2[pg, :, p % P], kb[s, j])
                    assert np.array_equal(vc2[pg, :, p % P], vb[s, j])
            assert touched.sum() == (state == SAV).sum() * B
            keep = ~touched
            assert np.array_equal(kc2.transpose(0, 2, 1, 3)[keep], k0.transpose(0, 2, 1, 3)[keep])
            assert np.array_equal(vc2.transpose(0, 2, 1, 3)[keep], v0.transpose(0, 2, 1, 3)[keep])


def check_commit_block_worked(impl):
    """A hand-worked case.  Sequence 0 SAVING commits its block at 5..7 and
    restarts; 1 DENOISING is untouched; 2 SAVING reaches its end length
    (8 + 3 >= 11) and finishes, keeping its block; 3 WAITING is untouched;
    4 SAVING near the stream's end keeps only the positions that fit."""
    toks = np.array([[4, 5, 6], [9, 9, 1], [7, 8, 2], [9, 9, 9], [3, 1, 4]])
    state = np.array([SAV, DEN, SAV, 0, SAV], dtype=np.uint8)
    L = np.array([5, 2, 8, 0, 11], dtype=np.int32)
    ts = np.full((5, 13), -1, dtype=np.int64)
    end = np.array([100, 100, 11, 100, 100], dtype=np.int32)
    nt, ns, nL, nts = impl.commit_block(toks, state, L, 9, ts, end)
    assert np.array_equal(nt, [[9, 9, 9], [9, 9, 1], [7, 8, 2], [9, 9, 9], [9, 9, 9]])
    assert np.array_equal(ns, [DEN, DEN, FIN, 0, DEN])
    assert np.array_equal(nL, [8, 2, 11, 0, 14])
    exp = np.full((5, 13), -1)
    exp[0, 5:8] = [4, 5, 6]
    exp[2, 8:11] = [7, 8, 2]
    exp[4, 11:13] = [3, 1]
    assert np.array_equal(nts, exp)
    # without a stream or end lengths nothing finishes
    nt, ns, nL, nts = impl.commit_block(toks, state, L, 9)
    assert nts is None and np.array_equal(ns, [DEN, DEN, DEN, 0, DEN])


def check_step_commit_order(impl):
    """One step commits the sequences that were SAVING on entry, and only
    those: a sequence that the rule fills in this step stays SAVING (its
    SAVING forward comes first); the next row list holds the fresh blocks."""
    B, mask = 4, 99
    toks = np.array([[1, 2, 3, 4], [mask, 5, 6, 7], [mask, mask, 8, 9]])
    state = np.array([SAV, DEN, DEN], dtype=np.uint8)
    L = np.array([8, 4, 0], dtype=np.int32)
    conf = np.full(3 * B, 0.5)
    argm = np.arange(3 * B) + 100
    nt, ns, nL, _, com, rows = impl.step_commit(toks, state, L, conf, argm, mask, 2,
                                                tokens_per_step=1)
    assert np.array_equal(ns, [DEN, SAV, DEN])
    assert np.array_equal(nL, [12, 4, 0])
    assert np.array_equal(nt, [[mask] * 4, [104, 5, 6, 7], [108, mask, 8, 9]])
    assert np.array_equal(rows, [0, 1, 2, 3, 9])
    assert com.sum() == 2


def check_multiblock_stream(impl):
    """Several whole blocks, each B rounds of the sequential rule (k = 1)
    and one SAVING step, with argmax = 1000*step + row: position j of block
    b is committed at step (B+1)*b + j, so the stream holds a closed form."""
    S, B, mask, L0, nb = 3, 3, 999, np.array([2, 5, 0], np.int32), 3
    toks = np.full((S, B), mask)
    state = np.full(S, DEN, dtype=np.uint8)
    L = L0.copy()
    ts = np.full((S, 20), -1, dtype=np.int64)
    for t in range((B + 1) * nb):
        argm = 1000 * t + np.arange(S * B)
        toks, state, L, ts, _, _ = impl.step_commit(toks, state, L, np.zeros(S * B), argm, mask, 2,
                                                    tokens_per_step=1, token_stream=ts)
    assert np.all(state == DEN) and np.array_equal(L, L0 + nb * B)
    for s in range(S):
        for b in range(nb):
            for j in range(B):
                assert ts[s, L0[s] + b * B + j] == 1000 * ((B + 1) * b + j) + s * B + j
        assert np.all(ts[s, :L0[s]] == -1) and np.all(ts[s, L0[s] + nb * B:] == -1)


SAVE_CHECKS = [check_kvsave_attention, check_kvsave_untouched, check_commit_block_worked,
               check_step_commit_order, check_multiblock_stream]


# ------------------------------------------------------------------ sampling

def check_philox_known_answers(impl):
    """Philox4x32-10 against the known-answer vectors published with the
    Random123 library (zero counter and key; all-ones; the digits of pi)."""
    cases = [((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
             ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
             ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
              (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1))]
    for ctr, key, out in cases:
        got = impl.philox4x32_10(*[np.array([x]) for x in ctr], *[np.array([x]) for x in key])
        assert [int(g[0]) for g in got] == list(out), [hex(int(g[0])) for g in got]


def check_uniform01(impl):
    u = impl.uniform01(np.array([0, 511, 512, 0xFFFFFFFF], dtype=np.uint64))
    assert u[0] == 2.0 ** -24 and u[1] == 2.0 ** -24 and u[2] == 3 * 2.0 ** -24
    assert u[3] == 1 - 2.0 ** -24
    assert np.all(u.astype(np.float32).astype(np.float64) == u)      # exact in float32


def _chi2_sf(x, k):
    from scipy.stats import chi2
    return chi2.sf(x, k)


def check_sampler_distribution(impl):
    """Many draws (steps 0..N-1) of one row follow softmax(l / T): a
    chi-square test over the tokens with expected count >= 5 (fixed seeds,
    so the outcome is fixed too).  Catches a dropped block normaliser, a
    Gumbel of the wrong sign, u and e sharing a word, the wrong temperature
    in either stage."""
    g = np.random.default_rng(31)
    V, N = 77, 4000
    for T, spread in ((1.0, 1.5), (0.6, 1.0), (2.0, 3.0)):
        l = g.normal(0, spread, V)
        l[5] = -np.inf                                  # the mask token
        p = np.exp((l - l[np.isfinite(l)].max()) / T)
        p /= p.sum()
        cnt = np.zeros(V)
        for step in range(N):
            t, _, _ = impl.sample_row(l, T, 0x1234_5678_9ABC, 3, step)
            cnt[t] += 1
        assert cnt[5] == 0
        keep = p * N >= 5
        x = np.sum((cnt[keep] - N * p[keep]) ** 2 / (N * p[keep])) + \
            (cnt[~keep].sum() - N * p[~keep].sum()) ** 2 / max(N * p[~keep].sum(), 1e-9)
        pv = _chi2_sf(x, keep.sum())
        assert pv > 1e-4, (T, x, pv)


def check_sampler_block_choice(impl):
    """Which block wins follows the blocks' shares of the mass, and inside a
    block the candidate follows the members' shares: a row whose mass sits
    in two tokens of different blocks, and one whose mass sits in two tokens
    of one block, each drawn N times."""
    V, N = 64, 3000
    for a, b in ((3, 36), (3, 6)):          # 3 and 36: chunks 0 and 1; 3 and 6: one block
        l = np.full(V, -40.0)
        l[a], l[b] = 0.0, np.log(3.0)       # p = 1/4, 3/4
        hits = sum(impl.sample_row(l, 1.0, 99, 1, s)[0] == b for s in range(N))
        assert abs(hits / N - 0.75) < 4 * np.sqrt(0.75 * 0.25 / N), (a, b, hits)


def check_sampler_greedy_limit(impl):
    """At T -> 0 the draw is the greedy token, and the confidence is the
    greedy max_p (at temperature 1) for every temperature."""
    g = np.random.default_rng(32)
    for _ in range(20):
        l = g.normal(0, 2, 300)
        l[7] = -np.inf
        top = np.argsort(-l)
        if l[top[0]] - l[top[1]] < 0.05:
            continue
        t, c, _ = impl.sample_row(l, 1e-3, int(g.integers(1 << 40)), 5, 0)
        p = np.exp(l - l[top[0]])
        assert t == top[0] and abs(c - 1.0 / p.sum()) < 1e-12
        t2, c2, _ = impl.sample_row(l, 1.7, 11, 5, 2)
        assert abs(c2 - np.exp(l[t2] - l[top[0]]) / p.sum()) < 1e-12


def check_sampler_seeds(impl):
    """The same (seed, row, step) gives the same token; rows, steps and
    seeds each give independent draws (a near-uniform row: about 1/V
    agreement between two streams)."""
    l = np.zeros(512)
    same = [impl.sample_row(l, 1.0, 5, 9, s)[0] for s in range(50)]
    again = [impl.sample_row(l, 1.0, 5, 9, s)[0] for s in range(50)]
    assert same == again
    for kw in (dict(seed=6, row=9), dict(seed=5, row=10), dict(seed=5 + (1 << 32), row=9)):
        other = [impl.sample_row(l, 1.0, kw["seed"], kw["row"], s)[0] for s in range(50)]
        assert sum(x == y for x, y in zip(same, other)) <= 3
    assert len(set(same)) >= 40


def check_filter_bruteforce(impl):
    """The kept set against a direct reading: rank by (higher logit, lower
    id), keep the first top_k, then the shortest run reaching top_p of the
    kept mass; ties at the boundary included."""
    g = np.random.default_rng(41)
    # equal logits: the running mass hits top_p times the total exactly
    for top_p, n in ((0.25, 1), (0.5, 2), (0.75, 3)):
        keep, _ = impl.topk_topp_keep(np.zeros(4), 1.0, 0, top_p)
        assert np.array_equal(np.nonzero(keep)[0], np.arange(n)), (top_p, keep)
    for trial in range(300):
        V = int(g.integers(2, 14))
        l = np.round(g.normal(0, 1.5, V), 1)            # rounding makes ties common
        l[int(g.integers(0, V))] = -np.inf              # the mask token
        T = float(g.choice([0.5, 1.0, 2.0]))
        top_k = int(g.integers(0, V + 2))
        top_p = float(g.choice([0.0, 0.3, 0.6, 0.9, 0.95, 1.0]))
        keep, _ = impl.topk_topp_keep(l, T, top_k, top_p)
        ranked = sorted([v for v in range(V) if np.isfinite(l[v])], key=lambda v: (-l[v], v))
        if 0 < top_k < len(ranked):
            ranked = ranked[:top_k]
        if top_p < 1.0:
            m = max(l[v] for v in ranked)
            w = [math.exp((l[v] - m) / T) for v in ranked]
            tot = math.fsum(w)
            run, out = 0.0, []
            for v, x in zip(ranked, w):
                out.append(v)
                run += x
                if run >= top_p * tot:
                    break
            ranked = out
        assert set(np.nonzero(keep)[0].tolist()) == set(ranked), (trial, l, T, top_k, top_p)


def check_filtered_distribution(impl):
    """Draws after filtering follow softmax(l/T) restricted to the kept set
    (chi-square), and never leave it."""
    from scipy.stats import chi2
    g = np.random.default_rng(42)
    V, N = 60, 3000
    for T, top_k, top_p in ((1.0, 6, 1.0), (0.7, 0, 0.8), (1.3, 20, 0.9)):
        l = g.normal(0, 1.2, V)
        l[3] = -np.inf
        keep, _ = impl.topk_topp_keep(l, T, top_k, top_p)
        p = np.where(keep, np.exp((l - l[np.isfinite(l)].max()) / T), 0.0)
        p /= p.sum()
        cnt = np.zeros(V)
        for step in range(N):
            cnt[impl.sample_filtered(l, T, top_k, top_p, 77, 2, step)[0]] += 1
        assert np.all(cnt[~keep] == 0)
        x = np.sum((cnt[keep] - N * p[keep]) ** 2 / (N * p[keep]))
        assert chi2.sf(x, keep.sum() - 1) > 1e-4, (T, top_k, top_p, x)


def check_filter_special_cases(impl):
    """No filtering draws exactly what the plain sampler draws; top_p = 0 or
    top_k = 1 leaves the greedy token; top_k beyond the vocabulary is no
    filter."""
    g = np.random.default_rng(43)
    for step in range(40):
        l = g.normal(0, 2, 200)
        l[9] = -np.inf
        a = impl.sample_filtered(l, 0.9, 0, 1.0, 5, 1, step)[0]
        assert a == impl.sample_row(l, 0.9, 5, 1, step)[0]
        assert impl.sample_filtered(l, 0.9, 1000, 1.0, 5, 1, step)[0] == a
        top = int(np.argmax(l))
        assert impl.sample_filtered(l, 0.9, 0, 0.0, 5, 1, step)[0] == top
        assert impl.sample_filtered(l, 0.9, 1, 1.0, 5, 1, step)[0] == top


def check_sampler_hand_cases(impl):
    """Hand-worked draws with given random words (tests/golden/
    sampling_hand_cases.json): which block wins, the inverse CDF inside it,
    the temperature, each chunk's own words, the tie rule, no candidate."""
    with open(os.path.join(GOLDEN, "sampling_hand_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        l = np.full(c["V"], -np.inf)
        for v, x in c["logits"]:
            l[v] = x
        words = np.array(c["words"], dtype=np.uint64)
        t, conf, _ = impl.sample_row(l, c["T"], 0, 0, 0, words=words, mask_id=c["mask_id"])
        assert t == c["expect_token"], (c["name"], t)
        assert abs(conf - c["expect_conf"]) < 1e-12, (c["name"], conf)


def check_sampler_counter_layout(impl):
    """The random words of chunk c are Philox4x32-10 (pinned by its known
    answers) at counter (c, row id, step, 0) with key (seed low word, seed
    high word): a draw equals the draw with those words given."""
    g = np.random.default_rng(34)
    V = 200
    nc = -(-V // 32)
    for seed, row, step in ((0x1234_5678_9ABC, 7, 3), (5, 1000, 0), ((1 << 40) + 17, 3, 99)):
        l = g.normal(0, 2, V)
        l[11] = -np.inf
        w = impl.philox4x32_10(np.arange(nc), np.full(nc, row), np.full(nc, step), np.zeros(nc),
                               np.full(nc, seed & 0xFFFFFFFF), np.full(nc, seed >> 32))
        words = np.stack([np.asarray(x, dtype=np.uint64) for x in w], axis=1)
        for T in (0.5, 1.0, 3.0):
            a = impl.sample_row(l, T, seed, row, step)
            b = impl.sample_row(l, T, 0, 0, 0, words=words)
            assert a[0] == b[0] and a[1] == b[1], (seed, row, step, T)


def check_lmhead_sample_rows(impl):
    """lmhead_sample is the block draw of each row's brute-force logits
    (mask column excluded) with that row's own id: tokens and confidences
    equal sample_row on scalar-loop logits, for rows listed out of order."""
    g = np.random.default_rng(33)
    V, Hd, mask = 70, 8, 12
    h = bf(g.standard_normal((12, Hd)) * 1.5)
    w = bf(g.standard_normal((V, Hd)))
    row_ids = np.array([13, 2, 40, 7, 21, 5, 0, 33, 9, 18, 27, 44])
    H, W = wid(h), wid(w)
    for T, seed, step in ((0.8, 0xABCDEF12345, 4), (1.5, 3, 0), (0.4, 77, 9)):
        toks, conf, _ = impl.lmhead_sample(h, w, mask, row_ids, T, seed, step)
        for j in range(h.shape[0]):
            l = np.array([math.fsum(float(a) * float(b) for a, b in zip(H[j], W[v])) for v in range(V)])
            l[mask] = -np.inf
            t, c, _ = impl.sample_row(l, T, seed, int(row_ids[j]), step)
            assert toks[j] == t and abs(conf[j] - c) < 1e-12, (T, j, toks[j], t)
            assert toks[j] != mask


SAMPLE_CHECKS = [check_sampler_hand_cases, check_sampler_counter_layout, check_lmhead_sample_rows,
                 check_philox_known_answers, check_uniform01, check_sampler_distribution,
                 check_sampler_block_choice, check_sampler_greedy_limit, check_sampler_seeds,
                 check_filter_bruteforce, check_filtered_distribution, check_filter_special_cases]


# ------------------------------------------------------------ whole round

def check_round_composition(impl):
    """denoise_round is the composition of the separately pinned parts:
    attention of every sequence by scalar loops, the LM head by scalar loops
    on exactly the masked rows of DENOISING sequences (sequence-major,
    position-minor), results scattered to those rows, the commit rule by
    subset enumeration on those confidences, and the next row list from the
    new state.  Sequences in every state and partly committed blocks make a
    misaligned gather or scatter visible; three thresholds exercise both
    branches of the rule."""
    from types import SimpleNamespace
    c = tiny_attn_case(seed=5, S=3, B=4, Hq=4, Hkv=2, D=8, P=4, L=(6, 0, 9))
    V, Hd, mask = 40, 8, 39
    g = np.random.default_rng(51)
    w = bf(g.standard_normal((V, Hd)))
    hid = bf(g.standard_normal((12, Hd)) * 3)
    toks0 = np.array([[39, 7, 39, 39], [39, 39, 39, 39], [39, 1, 2, 39]], dtype=np.int64)
    state0 = np.array([DEN, SAV, DEN], dtype=np.uint8)
    fixed = SimpleNamespace(block_tokens0=toks0, seq_state0=state0, prefix_len=c["prefix_len"],
                            page_table=c["page_table"], k_cache=c["k_cache"], v_cache=c["v_cache"],
                            w_vocab=w)
    inp = SimpleNamespace(q=c["q"], k_blk=c["k_blk"], v_blk=c["v_blk"], hidden=hid)
    attn_ref = attn_bruteforce(c)
    rows = [0, 2, 3, 8, 11]
    lm = lm_bruteforce(hid[rows], w, mask)
    conf = np.full(12, np.nan)
    argm = np.full(12, -1, dtype=np.int64)
    for r, (a, p1, _) in zip(rows, lm):
        conf[r], argm[r] = p1, a
    for tau in (0.0, 0.35, 2.0):
        res = impl.denoise_round(inp, fixed, mask, tau)
        assert np.max(np.abs(res["attn"] - attn_ref)) < 1e-12
        assert res["rows"].tolist() == rows
        for r, (a, p1, p2) in zip(rows, lm):
            assert res["argmax"][r] == a and abs(res["p1"][r] - p1) < 1e-13 and abs(res["p2"][r] - p2) < 1e-13
        others = [r for r in range(12) if r not in rows]
        assert np.all(res["argmax"][others] == -1) and np.all(np.isnan(res["p1"][others]))
        et, es = remask_bruteforce(toks0, state0, conf, argm, mask, tau)
        assert np.array_equal(res["tokens"], et) and np.array_equal(res["state"], es), tau
        assert np.array_equal(res["committed"], et != toks0)
        nxt = [s * 4 + i for s in range(3) if es[s] == DEN for i in range(4) if et[s, i] == mask]
        assert res["next_rows"].tolist() == nxt
    # a round from a given state: the state passed in, not the initial one, decides the rows
    t1 = np.array([[5, 7, 39, 6], [39, 39, 39, 39], [39, 1, 2, 3]], dtype=np.int64)
    s1 = np.array([DEN, DEN, SAV], dtype=np.uint8)
    res = impl.denoise_round(inp, fixed, mask, 0.35, block_tokens=t1, seq_state=s1)
    assert res["rows"].tolist() == [2, 4, 5, 6, 7]


ROUND_CHECKS = [check_round_composition]


# ------------------------------------------------- block-causal prefill

def _prefill_case(seed, lens=(7, 0, 12, 5), Hq=4, Hkv=2, D=8):
    g = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q = bf(g.standard_normal((T, Hq, D)))
    k = bf(g.standard_normal((T, Hkv, D)))
    v = bf(g.standard_normal((T, Hkv, D)))
    return q, k, v, cu


def check_prefill_bruteforce(impl):
    """Scalar loops over the mask's definition."""
    for seed, B in ((0, 3), (1, 1), (2, 5), (3, 16)):
        q, k, v, cu = _prefill_case(seed)
        got = impl.prefill_attention(q, k, v, cu, B)
        T, Hq, D = q.shape
        G = Hq // k.shape[1]
        sc = 1.0 / math.sqrt(D)
        for s in range(len(cu) - 1):
            a, b = int(cu[s]), int(cu[s + 1])
            for i in range(b - a):
                for h in range(Hq):
                    keys = [j for j in range(b - a) if j // B <= i // B]
                    qi = [float(x) for x in wid(q[a + i, h])]
                    z = [math.fsum(x * y for x, y in zip(qi, wid(k[a + j, h // G]))) * sc for j in keys]
                    mz = max(z)
                    e = [math.exp(t - mz) for t in z]
                    den = math.fsum(e)
                    for d in range(D):
                        ref = math.fsum(e[n] * float(wid(v[a + j, h // G])[d]) for n, j in enumerate(keys)) / den
                        assert abs(got[a + i, h, d] - ref) < 1e-12, (seed, B, s, i, h)


def _sdpa(q, k, v, causal):
    import torch
    qt = torch.from_numpy(wid(q)).permute(1, 0, 2)       # [H][L][D]
    G = q.shape[1] // k.shape[1]
    kt = torch.from_numpy(wid(k)).permute(1, 0, 2).repeat_interleave(G, 0)
    vt = torch.from_numpy(wid(v)).permute(1, 0, 2).repeat_interleave(G, 0)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal)
    return o.permute(1, 0, 2).numpy()


def check_prefill_special_cases(impl):
    """A block at least as long as the prompt is full attention; a block of
    one token is causal attention (PyTorch's float64 SDPA, per prompt)."""
    q, k, v, cu = _prefill_case(4, lens=(9, 13, 1))
    full = impl.prefill_attention(q, k, v, cu, 64)
    causal = impl.prefill_attention(q, k, v, cu, 1)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        assert np.max(np.abs(full[a:b] - _sdpa(q[a:b], k[a:b], v[a:b], False))) < 1e-12
        assert np.max(np.abs(causal[a:b] - _sdpa(q[a:b], k[a:b], v[a:b], True))) < 1e-12


def check_prefill_matches_denoise(impl):
    """Each full block of a prompt sees exactly what a denoise step of that
    block sees once the earlier blocks are in the cache: the prefill rows of
    block b equal the (separately pinned) denoise attention with prefix
    length b*B over a cache filled by the store."""
    import oracle as real
    B, P, Hq, Hkv, D = 3, 4, 4, 2, 8
    lens = (9, 6, 12)
    q, k, v, cu = _prefill_case(5, lens=lens, Hq=Hq, Hkv=Hkv, D=D)
    got = impl.prefill_attention(q, k, v, cu, B)
    S = len(lens)
    npg = [-(-L // P) for L in lens]
    pt = np.full((S, max(npg)), -1, dtype=np.int32)
    perm = np.random.default_rng(6).permutation(sum(npg))
    o = 0
    for s, n in enumerate(npg):
        pt[s, :n] = perm[o:o + n]
        o += n
    kc = np.zeros((sum(npg), Hkv, P, D), dtype=np.uint16)
    vc = np.zeros_like(kc)
    kc, vc = impl.prefill_store(kc, vc, pt, k, v, cu)
    for s, L in enumerate(lens):
        a = int(cu[s])
        for b0 in range(0, L, B):
            blk = slice(a + b0, a + b0 + B)
            ref = real.attention(q[None, blk], k[None, blk], v[None, blk], kc, vc, pt[s:s + 1],
                                 np.array([b0], np.int32))
            assert np.max(np.abs(got[blk] - ref[0])) < 1e-12, (s, b0)


def check_prefill_store(impl):
    q, k, v, cu = _prefill_case(7, lens=(5, 0, 9), Hq=4, Hkv=2, D=8)
    P = 4
    pt = np.array([[3, 0, -1], [-1, -1, -1], [1, 4, 2]], dtype=np.int32)
    kc0 = bf(np.random.default_rng(8).standard_normal((6, 2, P, 8)))
    vc0 = bf(np.random.default_rng(9).standard_normal((6, 2, P, 8)))
    kc, vc = impl.prefill_store(kc0, vc0, pt, k, v, cu)
    touched = np.zeros((6, P), dtype=bool)
    for s in range(3):
        a = int(cu[s])
        for j in range(int(cu[s + 1]) - a):
            pg = pt[s, j // P]
            assert np.array_equal(kc[pg, :, j % P], k[a + j]) and np.array_equal(vc[pg, :, j % P], v[a + j])
            touched[pg, j % P] = True
    keep = ~touched
    assert np.array_equal(kc.transpose(0, 2, 1, 3)[keep], kc0.transpose(0, 2, 1, 3)[keep])
    assert np.array_equal(vc.transpose(0, 2, 1, 3)[keep], vc0.transpose(0, 2, 1, 3)[keep])


def check_prefill_packing(impl):
    """Prompts do not see each other: packed results equal per-prompt ones."""
    q, k, v, cu = _prefill_case(10, lens=(4, 7, 0, 3))
    got = impl.prefill_attention(q, k, v, cu, 2)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        one = impl.prefill_attention(q[a:b], k[a:b], v[a:b], np.array([0, b - a]), 2)
        assert np.array_equal(got[a:b], one)


PREFILL_CHECKS = [check_prefill_bruteforce, check_prefill_special_cases, check_prefill_matches_denoise,
                  check_prefill_store, check_prefill_packing]
