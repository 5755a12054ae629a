"""Top-k / top-p sampling through the C ABI: the stored logits of
dbd_lmhead_logits against the oracle's, and dbd_sample_filtered against the
oracle's filtered draw applied to the kernel's own float32 logits (so every
ranking decision is taken on the same values).  Tokens are exact except
where float32 sums could decide otherwise: a top-p boundary within 1e-5 of
the kept mass (the token may then come from the kept set one shorter or
longer), and the block-draw bands of the plain sampler."""
import numpy as np
import pytest
import torch

import oracle
from block_diffusion_amd import api, synth
from block_diffusion_amd.workloads import SDAR_1P7B, TINY
from gpu_util import check_filtered_rows, dev_bf16, dev_i32, widen_bits

pytestmark = pytest.mark.gpu

def _case(name):
    if name == "tiny":
        w = TINY
        fx = synth.make_fixed(w)
        return synth.make_round(w, 1, fx.w_vocab).hidden, fx.w_vocab, w.mask_id, np.arange(w.S * w.B)
    if name == "ragged":
        g = np.random.default_rng(25)
        V, Hd, n, mask = 1003, 256, 70, 1001
        wv = synth.normal_bf16(g, (V, Hd), std=1.0 / np.sqrt(Hd))
        t = g.integers(0, V, n)
        a = g.uniform(0, 6, n)
        wt = widen_bits(wv[t])
        wt /= np.linalg.norm(wt, axis=1, keepdims=True)
        h = synth.f32_to_bf16((g.standard_normal((n, Hd)) + a[:, None] * wt).astype(np.float32))
        return h, wv, mask, g.permutation(n)[:45]
    w = SDAR_1P7B
    fx = synth.make_fixed(w)
    return (synth.make_round(w, 1, fx.w_vocab).hidden, fx.w_vocab, w.mask_id,
            np.random.default_rng(9).choice(w.S * w.B, 16, replace=False))


def _logits(h, wv, mask, rows):
    M = len(rows)
    V = wv.shape[0]
    lg = torch.full((M + 2, V), float("nan"), dtype=torch.float32, device="cuda")
    api.dbd_lmhead_logits(dev_bf16(h), dev_bf16(wv), dev_i32([M]), lg, mask, row_index=dev_i32(rows),
                          max_rows=M)
    torch.cuda.synchronize()
    return lg


@pytest.mark.parametrize("name", ["tiny", "ragged", "sdar1p7b"])
def test_lmhead_logits_parity(name):
    h, wv, mask, rows = _case(name)
    lg = _logits(h, wv, mask, rows).cpu().numpy()
    M = len(rows)
    ref = oracle.lmhead_logits(h[rows], wv, mask)
    assert np.all(np.isneginf(lg[:M, mask]))
    fin = np.isfinite(ref)
    err = np.abs(lg[:M][fin].astype(np.float64) - ref[fin]).max()
    print(f"{name}: max abs logit error {err:.2e}", flush=True)
    assert err <= 2e-3
    assert np.all(np.isnan(lg[M:]))


@pytest.mark.parametrize("name", ["tiny", "ragged", "sdar1p7b"])
@pytest.mark.parametrize("T,k,p", [(1.0, 0, 1.0), (0.6, 0, 0.95), (1.0, 50, 1.0), (0.8, 20, 0.9),
                                   (1.0, 1, 1.0), (0.7, 0, 0.0), (1.3, 3, 0.5)])
def test_sample_filtered_parity(name, T, k, p):
    h, wv, mask, rows = _case(name)
    M = len(rows)
    lg = _logits(h, wv, mask, rows)
    n = h.shape[0]
    tok = torch.full((n,), -9, dtype=torch.int32, device="cuda")
    conf = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    seed, step = 0xC0FFEE + k, 3
    api.dbd_sample_filtered(lg, dev_i32([M]), tok, conf, mask, T, k, p, seed, step,
                            row_index=dev_i32(rows), max_rows=M)
    torch.cuda.synchronize()
    ex = check_filtered_rows(lg.cpu().numpy(), rows, tok.cpu().numpy(), conf.cpu().numpy(), mask,
                             T, k, p, seed, step)
    print(f"{name} T={T} k={k} p={p}: {M} rows, {ex} exempt", flush=True)
    assert ex <= max(1, M // 20)
    if k == 0 and p >= 1.0:
        # no filter: the fused sampler draws the same tokens
        tok2 = torch.full((n,), -9, dtype=torch.int32, device="cuda")
        conf2 = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
        api.dbd_lmhead_sample(dev_bf16(h), dev_bf16(wv), dev_i32([M]), tok2, conf2, mask, T, seed,
                              step, row_index=dev_i32(rows), max_rows=M)
        torch.cuda.synchronize()
        assert np.array_equal(tok.cpu().numpy(), tok2.cpu().numpy())


@pytest.mark.parametrize("k,p", [(10, 1.0), (0, 0.8)])
def test_sample_filtered_distribution(k, p):
    """4096 draws of one row (4096 row ids) after filtering: never outside
    the kept set, and chi-square against softmax(l/T) on it."""
    from scipy.stats import chi2
    g = np.random.default_rng(88)
    V, Hd, N, mask, T = 300, 128, 4096, 11, 0.9
    wv = synth.normal_bf16(g, (V, Hd), std=1.0 / np.sqrt(Hd))
    h1 = synth.normal_bf16(g, (1, Hd), std=1.5)
    lg1 = _logits(h1, wv, mask, np.array([0]))[:1]
    lg = lg1.repeat(N, 1).contiguous()
    tok = torch.full((N,), -9, dtype=torch.int32, device="cuda")
    conf = torch.empty((N,), dtype=torch.float32, device="cuda")
    api.dbd_sample_filtered(lg, dev_i32([N]), tok, conf, mask, T, k, p, 2024, 0)
    torch.cuda.synchronize()
    l = lg1[0].double().cpu().numpy()
    keep, _ = oracle.topk_topp_keep(l, T, k, p)
    pr = np.where(keep, np.exp((l - l.max()) / T), 0.0)
    pr /= pr.sum()
    cnt = np.bincount(tok.cpu().numpy(), minlength=V).astype(np.float64)
    assert np.all(cnt[~keep] == 0)
    x = np.sum((cnt[keep] - N * pr[keep]) ** 2 / (N * pr[keep]))
    pv = chi2.sf(x, keep.sum() - 1)
    print(f"k={k} p={p}: {keep.sum()} kept, chi2 {x:.1f}, p-value {pv:.3g}", flush=True)
    assert pv > 1e-4


def test_lmhead_logits_many_rows():
    """1500 listed rows (two passes of the tile kernel at four-member teams)
    of a ragged vocabulary: sampled rows against the oracle's logits, every
    mask column -inf, rows past the list untouched."""
    g = np.random.default_rng(61)
    V, Hd, n, mask = 2003, 256, 1600, 77
    wv = synth.normal_bf16(g, (V, Hd), std=1.0 / np.sqrt(Hd))
    h = synth.normal_bf16(g, (n, Hd))
    rows = g.permutation(n)[:1500]
    lg = _logits(h, wv, mask, rows).cpu().numpy()
    M = len(rows)
    samp = np.sort(g.choice(M, 40, replace=False))
    ref = oracle.lmhead_logits(h[rows[samp]], wv, mask)
    fin = np.isfinite(ref)
    assert np.abs(lg[samp][fin].astype(np.float64) - ref[fin]).max() <= 2e-3
    assert np.all(np.isneginf(lg[:M, mask]))
    assert np.all(np.isnan(lg[M:]))


def _direct_rows(V, mask, seed):
    """Logit rows that stress the boundary search: long runs of equal logits
    (6000 and 1500 tokens at one value), a plain spread, -inf tokens, an
    all-equal row, a row with five tokens far above the rest, and a row
    whose top 3000 are 1600 tokens at +0 and 1600 at -0 (equal logits, so
    ranked by id); the mask column is -inf as the LM head stores it."""
    g = np.random.default_rng(seed)
    rows = []
    for n_tie in (6000, 1500):
        x = (g.standard_normal(V) * 2).astype(np.float32)
        x[g.choice(V, n_tie, replace=False)] = 3.0
        rows.append(x)
    rows.append((g.standard_normal(V) * 3).astype(np.float32))
    x = (g.standard_normal(V) * 2).astype(np.float32)
    x[g.choice(V, 100, replace=False)] = -np.inf
    rows.append(x)
    rows.append(np.zeros(V, np.float32))
    x = g.standard_normal(V).astype(np.float32)
    x[:5] = 12.0
    rows.append(x)
    x = -np.abs(g.standard_normal(V)).astype(np.float32) - 1.0
    z = g.choice(V, 3200, replace=False)
    x[z[:1600]] = 0.0
    x[z[1600:]] = -0.0
    rows.append(x)
    lg = np.stack(rows)
    lg[:, mask] = -np.inf
    return lg


@pytest.mark.parametrize("V", [20000, 20003])
@pytest.mark.parametrize("T,k,p", [(1.0, 0, 0.9), (1.0, 3000, 1.0), (1.0, 3000, 0.9), (0.7, 1500, 0.95),
                                   (50.0, 0, 0.5), (0.05, 0, 0.99), (1.0, 19990, 0.999), (0.6, 0, 0.95),
                                   (1.0, 0, 0.0), (1.3, 3, 0.5)])
def test_sample_filtered_boundary_rows(V, T, k, p):
    """Stored-logit rows whose filter boundary falls inside a run of equal
    logits too long for the in-LDS sort (the radix path), inside a shorter
    run (the sorted path), at extreme temperatures (everything in one value
    bin, or almost nothing near the top), and with top_k above the number
    of finite logits (keep them all)."""
    mask = 7
    lg_h = _direct_rows(V, mask, 400 + V % 7)
    M = lg_h.shape[0]
    lg = torch.from_numpy(lg_h).to("cuda")
    tok = torch.full((M,), -9, dtype=torch.int32, device="cuda")
    conf = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    seed, step = 77 + k, 5
    api.dbd_sample_filtered(lg, dev_i32([M]), tok, conf, mask, T, k, p, seed, step)
    torch.cuda.synchronize()
    ex = check_filtered_rows(lg_h, np.arange(M), tok.cpu().numpy(), conf.cpu().numpy(), mask,
                             T, k, p, seed, step)
    print(f"V={V} T={T} k={k} p={p}: {M} rows, {ex} exempt", flush=True)
    assert ex <= 1


def test_sample_filtered_no_candidate():
    """A row whose only finite logit is the mask token's draws the mask
    token with confidence 0; the other rows are unaffected."""
    V, mask = 4096, 3
    lg_h = np.full((2, V), -np.inf, np.float32)
    lg_h[0, mask] = 5.0
    lg_h[1] = np.random.default_rng(2).standard_normal(V).astype(np.float32)
    lg_h[1, mask] = -np.inf
    lg = torch.from_numpy(lg_h).to("cuda")
    tok = torch.full((2,), -9, dtype=torch.int32, device="cuda")
    conf = torch.full((2,), float("nan"), dtype=torch.float32, device="cuda")
    api.dbd_sample_filtered(lg, dev_i32([2]), tok, conf, mask, 1.0, 10, 0.9, 5, 0)
    torch.cuda.synchronize()
    t, c = tok.cpu().numpy(), conf.cpu().numpy()
    assert t[0] == mask and c[0] == 0.0
    ex = check_filtered_rows(lg_h[1:], np.array([1]), t, c, mask, 1.0, 10, 0.9, 5, 0)
    assert ex <= 1


@pytest.mark.parametrize("T,k,p", [(1.0, 0, 0.5), (0.6, 0, 0.95), (1.0, 60000, 1.0), (1.0, 30000, 0.9)])
def test_sample_filtered_full_vocab_overflow(T, k, p):
    """Full-vocabulary rows whose boundary bin spans most of the row (all
    logits equal; 60000 tied at the top of a spread), so that more blocks
    are deferred than the draw can list: the boundary is then resolved from
    the whole row (radix select) and the row drawn again."""
    V, mask = 151936, 151669
    g = np.random.default_rng(1207)
    rows = [np.zeros(V, np.float32)]
    x = (g.standard_normal(V) * 2 - 6).astype(np.float32)
    x[g.choice(V, 60000, replace=False)] = 1.5
    rows.append(x)
    lg_h = np.stack(rows)
    lg_h[:, mask] = -np.inf
    M = lg_h.shape[0]
    lg = torch.from_numpy(lg_h).to("cuda")
    tok = torch.full((M,), -9, dtype=torch.int32, device="cuda")
    conf = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    seed, step = 31 + k, 2
    api.dbd_sample_filtered(lg, dev_i32([M]), tok, conf, mask, T, k, p, seed, step)
    torch.cuda.synchronize()
    ex = check_filtered_rows(lg_h, np.arange(M), tok.cpu().numpy(), conf.cpu().numpy(), mask,
                             T, k, p, seed, step)
    print(f"T={T} k={k} p={p}: {M} rows, {ex} exempt", flush=True)
    assert ex <= 1


def _random_filter_cases(n, seed=909):
    """Seeded random draws: vocabularies with ragged ends, 1..300 rows,
    temperatures 0.2..3, top_k off or 1..V, top_p off or 0..1; logits as
    Gaussians of random spread, some rows with ties and -inf entries."""
    g = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        V = (997, 5003, 20000, 151936)[i % 4]
        M = int(g.choice([1, 3, 17, 128, 300]))
        T = float(np.round(g.uniform(0.2, 3.0), 3))
        k = int(g.choice([0, 0, 1, 5, 200, V // 2]))
        p = float(g.choice([1.0, 0.5, 0.9, 0.95, 0.999, 0.0]))
        cases.append((f"rand{i}_v{V}_m{M}_t{T}_k{k}_p{p}", V, M, T, k, p))
    return cases


@pytest.mark.parametrize("case", _random_filter_cases(8), ids=lambda c: c[0])
def test_sample_filtered_random(case):
    name, V, M, T, k, p = case
    g = np.random.default_rng(sum(name.encode()))
    mask = int(g.integers(0, V))
    spread = g.uniform(0.3, 4.0, M)[:, None]
    lg_h = (g.standard_normal((M, V)) * spread).astype(np.float32)
    for r in range(0, M, 3):                          # every third row: a run of ties and some -inf
        lg_h[r, g.choice(V, max(2, V // 50), replace=False)] = np.float32(lg_h[r].max() * 0.5)
        lg_h[r, g.choice(V, max(1, V // 100), replace=False)] = -np.inf
    lg_h[:, mask] = -np.inf
    rows = g.permutation(M + 5)[:M].astype(np.int32)
    lg = torch.from_numpy(lg_h).to("cuda")
    tok = torch.full((M + 5,), -9, dtype=torch.int32, device="cuda")
    conf = torch.full((M + 5,), float("nan"), dtype=torch.float32, device="cuda")
    seed, step = 0xF11 + M, 9
    api.dbd_sample_filtered(lg, dev_i32([M]), tok, conf, mask, T, k, p, seed, step, row_index=dev_i32(rows),
                            max_rows=M)
    torch.cuda.synchronize()
    t, c = tok.cpu().numpy(), conf.cpu().numpy()
    samp = np.unique(np.concatenate([np.arange(min(M, 6)), [M - 1], g.choice(M, min(M, 10), replace=False)]))
    ex = check_filtered_rows(lg_h[samp], rows[samp], t, c, mask, T, k, p, seed, step)
    print(f"{name}: {len(samp)} rows checked, {ex} exempt", flush=True)
    assert ex <= max(1, len(samp) // 10)
    assert np.all(t[np.setdiff1d(np.arange(M + 5), rows)] == -9)
