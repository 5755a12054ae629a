"""Temperature sampling in the fused LM head (dbd_lmhead_sample, and
dbd_round with sample set) against the CPU oracle's sampler on seeded
inputs, through the C ABI.

Tokens are compared exactly, with two exemptions that float32 rounding of
the logits can decide either way (the oracle computes in float64): a draw
whose two best blocks have Gumbel values within G_BAND of each other may
give the runner-up's candidate, and a draw within CDF_BAND (relative to the
block's mass) of an inverse-CDF boundary may give any member of the winning
block.  The confidence of the drawn token is checked to 1e-3 like the greedy
one.  A distribution test draws 4096 tokens of one row in one launch (the
same hidden state under 4096 row ids) and compares their histogram with
softmax(l/T)."""
import numpy as np
import pytest
import torch

import oracle
from block_diffusion_amd import api, synth
from block_diffusion_amd.workloads import SDAR_1P7B, TINY
from gpu_util import (CONF_ABS, RoundState, check_filtered_rows, check_lm_rows, dev_bf16, dev_i32,
                      round_inputs_dev, widen_bits)

pytestmark = pytest.mark.gpu

G_BAND = 1e-3
CDF_BAND = 1e-4
ENT_TOL = 1e-3


def _case(name):
    if name == "tiny":
        w = TINY
        fx = synth.make_fixed(w)
        return synth.make_round(w, 1, fx.w_vocab).hidden, fx.w_vocab, w.mask_id, np.arange(w.S * w.B)
    if name == "ragged":
        g = np.random.default_rng(15)
        V, Hd, n, mask = 1000, 256, 90, 999        # V not a multiple of 32, mask in the last chunk
        wv = synth.normal_bf16(g, (V, Hd), std=1.0 / np.sqrt(Hd))
        t = g.integers(0, V, n)
        a = g.uniform(0, 6, n)
        wt = widen_bits(wv[t])
        wt /= np.linalg.norm(wt, axis=1, keepdims=True)
        h = synth.f32_to_bf16((g.standard_normal((n, Hd)) + a[:, None] * wt).astype(np.float32))
        return h, wv, mask, g.permutation(n)[:61]
    w = SDAR_1P7B
    fx = synth.make_fixed(w)
    return (synth.make_round(w, 1, fx.w_vocab).hidden, fx.w_vocab, w.mask_id,
            np.random.default_rng(8).choice(w.S * w.B, 24, replace=False))


def _run(h, wv, mask, rows, T, seed, step, entropy=False):
    n = h.shape[0]
    M = len(rows)
    ri = dev_i32(rows)
    nr = dev_i32([M])
    tok = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    conf = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    ent = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda") if entropy else None
    api.dbd_lmhead_sample(dev_bf16(h), dev_bf16(wv), nr, tok, conf, mask, T, seed, step,
                          row_index=ri, max_rows=M, entropy=ent)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), conf.cpu().numpy(), (ent.cpu().numpy() if entropy else None)


def check_draws(rows, tok, conf, h, wv, mask, T, seed, step):
    """Exact tokens up to the rounding exemptions; confidences to 1e-3.
    Returns the number of exempt rows."""
    ref, _, infos = oracle.lmhead_sample(h[rows], wv, mask, rows, T, seed, step)
    logits = oracle.lmhead_logits(h[rows], wv, mask)
    exempt = 0
    for j, r in enumerate(rows):
        t = int(tok[r])
        inf = infos[j]
        if t != ref[j]:
            ok = (inf["g_gap"] < G_BAND and t == inf["runner_up"]) or \
                 (inf["cdf_margin"] < CDF_BAND and t in inf["block"])
            assert ok, f"row {r}: gpu {t} oracle {ref[j]} info {inf}"
            exempt += 1
        lse = logits[j].max() + np.log(np.exp(logits[j] - logits[j].max()).sum())
        p = np.exp(logits[j][t] - lse)
        assert abs(float(conf[r]) - p) <= CONF_ABS, (r, conf[r], p)
    return exempt


@pytest.mark.parametrize("name", ["tiny", "ragged", "sdar1p7b"])
@pytest.mark.parametrize("T,seed,step", [(1.0, 1, 0), (0.6, 0xDEADBEEF12345, 7), (1.7, 42, 3)])
def test_lmhead_sample_parity(name, T, seed, step):
    h, wv, mask, rows = _case(name)
    tok, conf, _ = _run(h, wv, mask, rows, T, seed, step)
    ex = check_draws(rows, tok, conf, h, wv, mask, T, seed, step)
    print(f"{name} T={T}: {len(rows)} rows, {ex} exempt", flush=True)
    assert ex <= max(1, len(rows) // 20)
    others = np.setdiff1d(np.arange(h.shape[0]), rows)
    assert np.all(tok[others] == -7)
    # the same call again draws the same tokens
    tok2, conf2, _ = _run(h, wv, mask, rows, T, seed, step)
    assert np.array_equal(tok, tok2) and np.array_equal(conf, conf2, equal_nan=True)


def test_lmhead_sample_with_entropy():
    h, wv, mask, rows = _case("ragged")
    tok, conf, ent = _run(h, wv, mask, rows, 0.8, 5, 1, entropy=True)
    tok0, conf0, _ = _run(h, wv, mask, rows, 0.8, 5, 1)
    assert np.array_equal(tok, tok0) and np.array_equal(conf, conf0, equal_nan=True)
    ref = oracle.lmhead_entropy(h[rows], wv, mask)
    assert np.abs(ent[rows].astype(np.float64) - ref).max() <= ENT_TOL


@pytest.mark.parametrize("T", [1.0, 0.5])
def test_lmhead_sample_distribution(T):
    """4096 draws of one row (4096 row ids, same hidden state) in one launch:
    chi-square against softmax(l/T) over tokens with expected count >= 5."""
    from scipy.stats import chi2
    g = np.random.default_rng(77)
    V, Hd, N, mask = 300, 128, 4096, 17
    wv = synth.normal_bf16(g, (V, Hd), std=1.0 / np.sqrt(Hd))
    h1 = synth.normal_bf16(g, (1, Hd), std=1.5)
    h = np.repeat(h1, N, axis=0)
    tok, _, _ = _run(h, wv, mask, np.arange(N), T, 2024, 0)
    l = oracle.lmhead_logits(h1, wv, mask)[0]
    p = np.exp((l - l.max()) / T)
    p /= p.sum()
    cnt = np.bincount(tok, minlength=V).astype(np.float64)
    assert cnt[mask] == 0
    keep = p * N >= 5
    x = np.sum((cnt[keep] - N * p[keep]) ** 2 / (N * p[keep]))
    rest = N * p[~keep].sum()
    if rest > 0:
        x += (cnt[~keep].sum() - rest) ** 2 / rest
    pv = chi2.sf(x, keep.sum())
    print(f"T={T}: chi2 {x:.1f} over {keep.sum()} cells, p-value {pv:.3g}", flush=True)
    assert pv > 1e-4


@pytest.mark.parametrize("w", [TINY, SDAR_1P7B], ids=lambda w: w.name)
def test_round_sampling_teacher_forced(w):
    """Whole blocks of rounds with sample set (a fresh step per round): the
    drawn tokens match the oracle's sampler, and the commits are exactly the
    threshold rule applied to the GPU's own tokens and confidences."""
    fx = synth.make_fixed(w)
    st = RoundState(w, fx)
    st.init_rows()
    attn_out = torch.empty((w.S, w.B, w.Hq, w.D), dtype=torch.bfloat16, device="cuda")
    toks, state = fx.block_tokens0.copy(), fx.seq_state0.copy()
    T, seed = 0.8, 0x5EED
    for r in range(1, w.B + 1):
        rin = synth.make_round(w, r, fx.w_vocab)
        a = st.args(round_inputs_dev(rin), attn_out)
        a.sample, a.temperature, a.seed, a.step = 1, T, seed, r
        rows0 = oracle.compact_rows(toks, state, w.mask_id)
        api.dbd_round(a)
        torch.cuda.synchronize()
        arg, conf = st.bufs.argmax_tok.cpu().numpy(), st.bufs.conf.cpu().numpy()
        if rows0.size:
            samp = rows0 if w is TINY else rows0[:: max(1, rows0.size // 24)]
            check_draws(samp, arg, conf, rin.hidden, fx.w_vocab, w.mask_id, T, seed, r)
        t1, s1 = st.bufs.block_tokens.cpu().numpy(), st.bufs.seq_state.cpu().numpy()
        et, es, _ = oracle.remask(toks, state, conf, arg, w.mask_id, np.float32(w.tau))
        assert np.array_equal(t1, et) and np.array_equal(s1, es), f"round {r}"
        toks, state = t1, s1
        if not np.any(state == oracle.DENOISING):
            break
    assert np.all(state == oracle.SAVING)


@pytest.mark.parametrize("w", [TINY, SDAR_1P7B], ids=lambda w: w.name)
@pytest.mark.parametrize("k,p", [(0, 0.95), (20, 0.9)])
def test_round_filtered_teacher_forced(w, k, p):
    """Whole blocks of rounds with top-k / top-p filtering inside the round
    (the LM head stores the listed rows' logits, the filtered draw reads
    them): every drawn token matches the oracle's filtered draw on the
    round's own stored logits, and the commits are exactly the threshold
    rule applied to the GPU's tokens and confidences."""
    fx = synth.make_fixed(w)
    st = RoundState(w, fx)
    st.init_rows()
    attn_out = torch.empty((w.S, w.B, w.Hq, w.D), dtype=torch.bfloat16, device="cuda")
    logits = torch.full((w.S * w.B, w.V), float("nan"), dtype=torch.float32, device="cuda")
    toks, state = fx.block_tokens0.copy(), fx.seq_state0.copy()
    T, seed = 0.7, 0xF17 + k
    for r in range(1, w.B + 1):
        rin = synth.make_round(w, r, fx.w_vocab)
        a = st.args(round_inputs_dev(rin), attn_out)
        a.sample, a.temperature, a.seed, a.step = 1, T, seed, r
        a.filter, a.top_k, a.top_p, a.logits = 1, k, p, logits.data_ptr()
        rows0 = oracle.compact_rows(toks, state, w.mask_id)
        api.dbd_round(a)
        torch.cuda.synchronize()
        arg, conf = st.bufs.argmax_tok.cpu().numpy(), st.bufs.conf.cpu().numpy()
        if rows0.size:
            step_sel = 1 if w is TINY else max(1, rows0.size // 16)
            sel = np.arange(0, rows0.size, step_sel)
            lg = logits[torch.from_numpy(sel).cuda()].cpu().numpy()
            ex = check_filtered_rows(lg, rows0[sel], arg, conf, w.mask_id, T, k, p, seed, r)
            print(f"round {r}: {sel.size} rows checked, {ex} exempt", flush=True)
            assert ex <= max(1, sel.size // 20)
        t1, s1 = st.bufs.block_tokens.cpu().numpy(), st.bufs.seq_state.cpu().numpy()
        et, es, _ = oracle.remask(toks, state, conf, arg, w.mask_id, np.float32(w.tau))
        assert np.array_equal(t1, et) and np.array_equal(s1, es), f"round {r}"
        toks, state = t1, s1
        if not np.any(state == oracle.DENOISING):
            break
    assert np.all(state == oracle.SAVING)



@pytest.mark.parametrize("M", [1025, 1500, 2100])
def test_lmhead_modes_many_rows(M):
    """More than 1024 listed rows: the tile kernel runs passes of 1024 rows
    with four-member teams, the last pass ragged.  The greedy head with the
    entropy, and the temperature-sampling head, on sampled rows (the first
    and last of each pass among them) against the oracle; every listed row
    written, the other rows untouched."""
    g = np.random.default_rng(M)
    V, Hd, n, mask = 2003, 256, M + 100, 77     # V not a multiple of 32
    wv = synth.normal_bf16(g, (V, Hd), std=1.0 / np.sqrt(Hd))
    t = g.integers(0, V, n)
    a = g.uniform(0, 14, n)
    wt = widen_bits(wv[t])
    wt /= np.linalg.norm(wt, axis=1, keepdims=True)
    h = synth.f32_to_bf16((g.standard_normal((n, Hd)) + a[:, None] * wt).astype(np.float32))
    rows = g.permutation(n)[:M].astype(np.int32)
    ends = [0, 1023, 1024, M - 1] + ([2047, 2048] if M > 2048 else [])
    samp = np.unique(np.concatenate([rows[g.choice(M, 30, replace=False)], rows[ends]]))
    others = np.setdiff1d(np.arange(n), rows)
    ri, nr = dev_i32(rows), dev_i32([M])

    # greedy, with the entropy
    arg = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    conf = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    ent = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    api.dbd_lmhead_conf(dev_bf16(h), dev_bf16(wv), nr, arg, conf, mask, row_index=ri, max_rows=M, entropy=ent)
    torch.cuda.synchronize()
    arg, conf, ent = arg.cpu().numpy(), conf.cpu().numpy(), ent.cpu().numpy()
    check_lm_rows(samp, arg, conf, h, wv, mask)
    ref = oracle.lmhead_entropy(h[samp], wv, mask)
    assert np.abs(ent[samp].astype(np.float64) - ref).max() <= ENT_TOL
    assert np.all((arg[rows] >= 0) & (arg[rows] < V) & (arg[rows] != mask))
    assert np.all(arg[others] == -7) and np.all(np.isnan(conf[others])) and np.all(np.isnan(ent[others]))

    # temperature sampling
    T, seed, step = 0.8, 0x5A17 + M, 3
    tok, sconf, _ = _run(h, wv, mask, rows, T, seed, step)
    ex = check_draws(samp, tok, sconf, h, wv, mask, T, seed, step)
    print(f"M={M}: {len(samp)} sampled rows, {ex} draws exempt", flush=True)
    assert ex <= 2
    assert np.all((tok[rows] >= 0) & (tok[rows] < V) & (tok[rows] != mask))
    assert np.all(tok[others] == -7)


def _random_lm_shapes(n, seed=777):
    """Seeded random LM-head shapes: hidden sizes 128..1024 (multiples of
    128), vocabularies from 2 (one candidate) to 40000 (ragged ends), any
    mask id, 1..1300 listed rows out of a larger buffer."""
    g = np.random.default_rng(seed)
    shapes = []
    for i in range(n):
        # vocabularies and row counts cycle through their lists, the rest is drawn
        Hd = int(g.choice([128, 256, 384, 640, 1024]))
        V = (2, 33, 257, 1000, 4099, 40000)[i % 6]
        mask = int(g.integers(0, V))
        M = (1, 1300, 64, 1025, 257, 600, 7, 255)[i % 8]
        extra = int(g.integers(0, 40))
        shapes.append((f"rand{i}_hd{Hd}_v{V}_m{M}", Hd, V, mask, M, M + extra))
    return shapes


@pytest.mark.parametrize("case", _random_lm_shapes(8), ids=lambda c: c[0])
def test_lmhead_random_shapes(case):
    """Seeded random shapes: greedy token and confidence, entropy, and the
    temperature draw on sampled rows (the first and last listed among them)
    against the oracle; rows outside the list untouched."""
    name, Hd, V, mask, M, nbuf = case
    g = np.random.default_rng(sum(name.encode()))
    wv = synth.normal_bf16(g, (V, Hd), std=1.0 / np.sqrt(Hd))
    t = g.integers(0, V, nbuf)
    a = g.uniform(0, 14, nbuf)
    wt = widen_bits(wv[t])
    wt /= np.linalg.norm(wt, axis=1, keepdims=True)
    h = synth.f32_to_bf16((g.standard_normal((nbuf, Hd)) + a[:, None] * wt).astype(np.float32))
    rows = g.permutation(nbuf)[:M].astype(np.int32)
    samp = np.unique(np.concatenate([rows[g.choice(M, min(M, 20), replace=False)], rows[[0, M - 1]]]))
    others = np.setdiff1d(np.arange(nbuf), rows)
    ri, nr = dev_i32(rows), dev_i32([M])
    arg = torch.full((nbuf,), -7, dtype=torch.int32, device="cuda")
    conf = torch.full((nbuf,), float("nan"), dtype=torch.float32, device="cuda")
    ent = torch.full((nbuf,), float("nan"), dtype=torch.float32, device="cuda")
    api.dbd_lmhead_conf(dev_bf16(h), dev_bf16(wv), nr, arg, conf, mask, row_index=ri, max_rows=M, entropy=ent)
    torch.cuda.synchronize()
    arg, conf, ent = arg.cpu().numpy(), conf.cpu().numpy(), ent.cpu().numpy()
    check_lm_rows(samp, arg, conf, h, wv, mask)
    ref = oracle.lmhead_entropy(h[samp], wv, mask)
    assert np.abs(ent[samp].astype(np.float64) - ref).max() <= ENT_TOL
    assert np.all(arg[others] == -7) and np.all(np.isnan(conf[others]))
    T, seed, step = 0.9, 0x77 + M, 2
    tok, sconf, _ = _run(h, wv, mask, rows, T, seed, step)
    ex = check_draws(samp, tok, sconf, h, wv, mask, T, seed, step)
    print(f"{name}: {len(samp)} rows, {ex} draws exempt", flush=True)
    assert ex <= 2
    assert np.all(tok[others] == -7)
