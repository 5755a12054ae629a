"""Plants plausible mistakes in copies of the oracle (on the CPU) and checks
that at least one pin fails for each: the pins are strong enough to notice a
dropped term, a wrong sign or index, or a swapped rule."""
import importlib.util
import os
import sys
import types

import pytest

from pins import (ATTN_CHECKS, LM_CHECKS, REMASK_CHECKS, PREFILL_CHECKS, ROUND_CHECKS, RULE_CHECKS, SAMPLE_CHECKS,
                  SAVE_CHECKS)

ORACLE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")

# (file, original text, replacement, which pin family must catch it)
MUTANTS = [
    ("attention.py", "scale = 1.0 / np.sqrt(D)", "scale = 1.0 / D", "attn"),
    ("attention.py", "h = g * G + gi", "h = gi * Hkv + g", "attn"),
    ("attention.py", "reshape(npg * P, -1)[:L]", "reshape(npg * P, -1)[:max(L - 1, 0)]", "attn"),
    ("attention.py", "z -= z.max(axis=1, keepdims=True)",
     "z[:, L:] += np.triu(np.full((B, B), -np.inf), 1)\n        z -= z.max(axis=1, keepdims=True)", "attn"),
    ("attention.py", "pages = np.asarray(page_table_s[:npg], dtype=np.int64)",
     "pages = np.sort(np.asarray(page_table_s[:npg], dtype=np.int64))", "attn"),
    ("attention.py", "out[:, gi, :] = p @ vals", "out[:, gi, :] = p @ keys", "attn"),
    ("lmhead.py", "    logits[:, mask_id] = -np.inf\n    return logits",
     "    return logits", "lm"),
    ("lmhead.py", "arg = logits.argmax(axis=1)",
     "arg = logits.shape[1] - 1 - logits[:, ::-1].argmax(axis=1)", "lm"),
    ("lmhead.py", "logits[:, v0:v0 + vchunk] = H @ W.T",
     "logits[:, v0:v0 + vchunk] = (H @ W.T) / np.sqrt(H.shape[1])", "lm"),
    ("lmhead.py", "part = np.partition(e, -2, axis=1)[:, -2]",
     "part = np.sort(e, axis=1)[:, -2] * 0 + np.sort(e, axis=1)[:, -3]", "lm"),
    ("remask.py", "conf[s, i] >= tau", "conf[s, i] > tau", "remask"),
    ("remask.py", "if best is None or conf_row[i] > conf_row[best]:",
     "if best is None or conf_row[i] >= conf_row[best]:", "remask"),
    ("remask.py", "if flags & FALLBACK_LEFTMOST:", "if True:", "remask"),
    ("remask.py", "            state[s] = SAVING", "            pass", "remask"),
    ("remask.py", "for s in range(S) if seq_state[s] == DENOISING\n            for i in range(B)",
     "for i in range(B) for s in range(S) if seq_state[s] == DENOISING", "remask"),
    ("lmhead.py", "H[i:i + chunk] = np.log(ssum) - (e * zfin).sum(axis=1) / ssum",
     "H[i:i + chunk] = np.log(ssum) + (e * zfin).sum(axis=1) / ssum", "lm"),
    ("lmhead.py", "H[i:i + chunk] = np.log(ssum) - (e * zfin).sum(axis=1) / ssum",
     "H[i:i + chunk] = np.log2(ssum) - (e * zfin).sum(axis=1) / ssum", "lm"),
    ("lmhead.py", "zfin = np.where(np.isfinite(z), z, 0.0)   # the mask column has p = 0",
     "zfin = np.where(np.isfinite(z), z, 0.0); ssum = ssum + np.exp(-1.0)", "lm"),
    ("remask.py", "chosen = masked[:k]", "chosen = masked[-k:]", "rule"),
    ("remask.py", "k = min(max(int(tokens_per_step), 1), len(masked))",
     "k = max(min(max(int(tokens_per_step), 1), len(masked)) - 1, 1)", "rule"),
    ("remask.py", "best = _most_confident(rest, conf[s])", "best = _most_confident(rest, -conf[s])", "rule"),
    ("remask.py", "if chosen and nxt > budget:", "if nxt > budget:", "rule"),
    ("remask.py", "if chosen and nxt > budget:", "if chosen and nxt >= budget:", "rule"),
    ("remask.py", "key=lambda i: (ent_row[i], i))", "key=lambda i: (ent_row[i], -i))", "rule"),
    ("block_commit.py", "            p = L + j\n", "            p = L + j + 1\n", "save"),
    ("block_commit.py", "kc[page, :, p % P, :] = k_blk[s, j]", "kc[page, :, j % P, :] = k_blk[s, j]", "save"),
    ("block_commit.py", "page = int(page_table[s][p // P])", "page = int(page_table[s][j // P])", "save"),
    ("block_commit.py", "vc[page, :, p % P, :] = v_blk[s, j]", "vc[page, :, p % P, :] = k_blk[s, j]", "save"),
    ("block_commit.py", "        if seq_state[s] != SAVING:\n            continue\n        L = int",
     "        if seq_state[s] == 0:\n            continue\n        L = int", "save"),
    ("block_commit.py", "        L[s] += B\n", "        L[s] += B - 1\n", "save"),
    ("block_commit.py", "            toks[s, :] = mask_id\n", "            pass\n", "save"),
    ("block_commit.py", "if end_len is not None and L[s] >= end_len[s]:",
     "if end_len is not None and L[s] > end_len[s]:", "save"),
    ("block_commit.py", "ts[s, L[s] + j] = toks[s, j]", "ts[s, L[s] + j] = toks[s, B - 1 - j]", "save"),
    ("block_commit.py", "only = np.where(saving0, SAVING, 0).astype(state.dtype)", "only = state", "save"),
    ("sampling.py", "m + np.log(np.where(live, S, 1.0)) - np.log(-np.log(e))", "m - np.log(-np.log(e))",
     "sample"),
    ("sampling.py", "m + np.log(np.where(live, S, 1.0)) - np.log(-np.log(e))",
     "m + np.log(np.where(live, S, 1.0)) + np.log(-np.log(e))", "sample"),
    ("sampling.py", "e = uniform01(words[blocks // 2, 2 * (blocks % 2) + 1])", "e = u", "sample"),
    ("sampling.py", "target = u * S_b\n", "target = u * S_b * 0.5\n", "sample"),
    ("sampling.py", "z = np.asarray(logits, dtype=np.float64) / temperature",
     "z = np.asarray(logits, dtype=np.float64)", "sample"),
    ("sampling.py", "lse = lmax + math.log(float(np.sum(np.exp(fin - lmax))))", "lse = lmax", "sample"),
    ("sampling.py", "return v // 32, (v // 4) % 2", "return v // 32, (v // 8) % 2", "sample"),
    ("sampling.py", "u = uniform01(words[blocks // 2, 2 * (blocks % 2)])",
     "u = uniform01(words[blocks // 2, 2 * (1 - blocks % 2)])", "sample"),
    ("sampling.py", "if cand is None and cum >= target:", "if cum >= target:", "sample"),
    ("sampling.py", "win = min(np.nonzero(G == g1)[0].tolist(), key=cand_of)",
     "win = max(np.nonzero(G == g1)[0].tolist(), key=cand_of)", "sample"),
    ("sampling.py", "return int(mask_id), 0.0, info", "return 0, 0.0, info", "sample"),
    ("sampling.py", "w = philox4x32_10(np.arange(nchunks), np.full(nchunks, row_id), np.full(nchunks, step),",
     "w = philox4x32_10(np.arange(nchunks), np.full(nchunks, step), np.full(nchunks, row_id),", "sample"),
    ("sampling.py", "t, c, inf = sample_row(L[j], temperature, seed, int(row_ids[i0 + j]), step,",
     "t, c, inf = sample_row(L[j], temperature, seed, i0 + j, step,", "sample"),
    ("sampling.py", "t, c, inf = sample_row(L[j], temperature, seed, int(row_ids[i0 + j]), step,",
     "t, c, inf = sample_row(L[j], 1.0, seed, int(row_ids[i0 + j]), step,", "sample"),
    ("sampling.py", "    for _ in range(10):", "    for _ in range(9):", "sample"),
    ("sampling.py", "c = [hi1 ^ c[1] ^ k[0], lo1, hi0 ^ c[3] ^ k[1], lo0]",
     "c = [lo1 ^ c[1] ^ k[0], hi1, hi0 ^ c[3] ^ k[1], lo0]", "sample"),
    ("sampling.py", "return ((w >> np.uint64(9)).astype(np.float64) + 0.5) / float(1 << 23)",
     "return ((w >> np.uint64(8)).astype(np.float64) + 0.5) / float(1 << 24)", "sample"),
    ("sampling.py", "order = cand[np.lexsort((cand, -logits[cand]))]",
     "order = cand[np.lexsort((cand, logits[cand]))]", "sample"),
    ("sampling.py", "order = cand[np.lexsort((cand, -logits[cand]))]",
     "order = cand[np.lexsort((-cand, -logits[cand]))]", "sample"),
    ("sampling.py", "j = min(int(np.searchsorted(cum, target, side=\"left\")), k - 1)",
     "j = min(int(np.searchsorted(cum, target, side=\"right\")), k - 1)", "sample"),
    ("sampling.py", "w = np.exp((logits[kept] - m) / temperature)",
     "w = np.exp((logits[order] - m) / temperature)", "sample"),
    ("sampling.py", "z = np.where(np.asarray(keep, dtype=bool), z, -np.inf)", "z = z", "sample"),
    ("remask.py", "        if np.isnan(conf_row[i]):\n            continue", "        if False:\n            continue",
     "remask"),
    ("remask.py", "return positions[0] if best is None else best",
     "return positions[-1] if best is None else best", "remask"),
    ("remask.py", "e_i = ent.dtype.type(np.inf) if np.isnan(ent[s, i]) else ent[s, i]", "e_i = ent[s, i]",
     "rule"),
    ("remask.py", "return nums + [i for i in positions if np.isnan(ent_row[i])]",
     "return [i for i in positions if np.isnan(ent_row[i])] + nums", "rule"),
    ("lmhead.py", "arg = np.where(none, mask_id, arg)", "arg = arg", "lm"),
    ("lmhead.py", "p1 = np.where(none, 0.0, p1)", "p1 = p1", "lm"),
    ("lmhead.py", "H[i:i + chunk][none] = np.inf", "H[i:i + chunk][none] = 0.0", "lm"),
    ("round.py", "arg[rows], conf[rows], p2[rows] = a, x1, x2",
     "arg[rows], conf[rows], p2[rows] = a[::-1], x1[::-1], x2[::-1]", "round"),
    ("round.py", "arg[rows], conf[rows], p2[rows] = a, x1, x2",
     "arg[rows[::-1]], conf[rows[::-1]], p2[rows[::-1]] = a, x1, x2", "round"),
    ("round.py", "lmhead_rows(inp.hidden[rows], fixed.w_vocab, mask_id)",
     "lmhead_rows(inp.hidden[:rows.size], fixed.w_vocab, mask_id)", "round"),
    ("round.py", "next_rows=compact_rows(new_toks, new_state, mask_id)",
     "next_rows=compact_rows(toks, state, mask_id)", "round"),
    ("round.py", "rows = compact_rows(toks, state, mask_id)",
     "rows = compact_rows(toks, np.full_like(state, 2), mask_id)", "round"),
    ("round.py", "tau, flags)", "tau, flags | 1)", "round"),
    ("round.py", "toks = fixed.block_tokens0 if block_tokens is None else block_tokens",
     "toks = fixed.block_tokens0", "round"),
    ("prefill.py", "allowed = blk[None, :] <= blk[:, None]", "allowed = blk[None, :] < blk[:, None]",
     "prefill"),
    ("prefill.py", "allowed = blk[None, :] <= blk[:, None]",
     "allowed = np.arange(L)[None, :] <= np.arange(L)[:, None]", "prefill"),
    ("prefill.py", "blk = np.arange(L) // block_len", "blk = (np.arange(L) + 1) // block_len", "prefill"),
    ("prefill.py", "scale = 1.0 / np.sqrt(D)", "scale = 1.0 / D", "prefill"),
    ("prefill.py", "h = g * G + gi", "h = gi * Hkv + g", "prefill"),
    ("prefill.py", "kc[page, :, j % P, :] = k[a + j]", "kc[page, :, (j + 1) % P, :] = k[a + j]", "prefill"),
    ("prefill.py", "vc[page, :, j % P, :] = v[a + j]", "vc[page, :, j % P, :] = k[a + j]", "prefill"),
]


def load_mutant(fname, old, new):
    pkg = types.ModuleType("oracle_mut")
    pkg.__path__ = []
    sys.modules["oracle_mut"] = pkg
    for dep in ("bf16.py", "remask.py", "lmhead.py", "attention.py"):
        if dep == fname:
            continue
        spec = importlib.util.spec_from_file_location("oracle_mut." + dep[:-3], os.path.join(ORACLE, dep))
        m = importlib.util.module_from_spec(spec)
        sys.modules[spec.name] = m
        spec.loader.exec_module(m)
    src = open(os.path.join(ORACLE, fname)).read()
    assert old in src, (fname, old)
    src = src.replace(old, new)
    name = "oracle_mut." + fname[:-3]
    mod = types.ModuleType(name)
    mod.__package__ = "oracle_mut"
    sys.modules[name] = mod
    exec(compile(src, f"<mutant {fname}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("mut", MUTANTS, ids=lambda m: f"{m[0]}:{m[1][:30]}")
def test_mutant_is_caught(mut):
    fname, old, new, fam = mut
    mod = load_mutant(fname, old, new)
    checks = {"attn": ATTN_CHECKS, "lm": LM_CHECKS, "remask": REMASK_CHECKS, "rule": RULE_CHECKS,
              "save": SAVE_CHECKS, "sample": SAMPLE_CHECKS, "prefill": PREFILL_CHECKS,
              "round": ROUND_CHECKS}[fam]
    caught = []
    for chk in checks:
        try:
            chk(mod)
        except Exception:          # an assertion or a crash both count
            caught.append(chk.__name__)
    assert caught, f"no pin notices mutant {old!r} -> {new!r}"
