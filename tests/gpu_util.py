"""Helpers for the GPU parity tests: device copies of the seeded inputs, the
oracle comparisons and the acceptance rule of a round's commits."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from block_diffusion_amd import api, synth

ATTN_MAX_ABS = 2e-2
ATTN_REL_L2 = 5e-3
CONF_ABS = 1e-3
TAU_BAND = 1e-3
TIE_BAND = 1e-4
# filtered sampling: float32 bands within which the draw may differ
G_BAND = 1e-3
CDF_BAND = 1e-4
P_BAND = 1e-5


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def dev_i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def dev_u8(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def widen_bits(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def attn_errors(got, ref):
    """max abs error and relative L2 error over everything compared."""
    d = got - ref
    return float(np.max(np.abs(d))), float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300))


def run_attn(fx, rin, stream=None):
    """Device copies + one dbd_attn_paged call; returns (out bits, device tensors)."""
    S, B, Hq, D = rin.q.shape
    q, kb, vb = dev_bf16(rin.q), dev_bf16(rin.k_blk), dev_bf16(rin.v_blk)
    kc, vc = dev_bf16(fx.k_cache), dev_bf16(fx.v_cache)
    pt, pl = dev_i32(fx.page_table), dev_i32(fx.prefix_len)
    out = torch.empty((S, B, Hq, D), dtype=torch.bfloat16, device="cuda")
    api.dbd_attn_paged(q, kb, vb, kc, vc, pt, pl, out, stream=stream)
    torch.cuda.synchronize()
    return host_bits(out)


def oracle_attn_groups(fx, rin, groups):
    """Oracle output for the listed (s, g) pairs: dict -> [B][G][D]."""
    return {(s, g): oracle.attention_group(s, g, rin.q, rin.k_blk, rin.v_blk, fx.k_cache,
                                           fx.v_cache, fx.page_table, fx.prefix_len)
            for s, g in groups}


def compare_attn(out_bits, ref_groups, G):
    got, ref = [], []
    for (s, g), r in ref_groups.items():
        got.append(widen_bits(out_bits[s, :, g * G:(g + 1) * G, :]))
        ref.append(r)
    return attn_errors(np.stack(got), np.stack(ref))


def tie_set(h_row_bits, w_bits, mask_id, p1):
    """Token ids whose probability is within TIE_BAND of the top one."""
    logits = oracle.lmhead_logits(h_row_bits[None], w_bits, mask_id)[0]
    m = logits.max()
    p = np.exp(logits - m)
    p /= p.sum()
    return set(np.nonzero(p >= p1 - TIE_BAND)[0].tolist())


def check_lm_rows(rows, gpu_arg, gpu_conf, hidden_bits, w_bits, mask_id, ref=None):
    """conf within CONF_ABS of the oracle's max probability on every row;
    argmax equal to the oracle's unless the top two are within TIE_BAND, and
    then inside the tie set.  Returns (a, p1, p2, n_tie_exempt)."""
    if ref is None:
        ref = oracle.lmhead_rows(hidden_bits[rows], w_bits, mask_id)
    a, p1, p2 = ref
    g_arg = np.asarray(gpu_arg)[rows]
    g_conf = np.asarray(gpu_conf, dtype=np.float64)[rows]
    err = np.abs(g_conf - p1)
    assert np.all(err <= CONF_ABS), f"conf error {err.max():.3g} at row {rows[int(np.argmax(err))]}"
    clear = (p1 - p2) >= TIE_BAND
    bad = np.nonzero(clear & (g_arg != a))[0]
    assert bad.size == 0, f"argmax mismatch at rows {[int(rows[i]) for i in bad[:8]]}: " \
                          f"gpu {g_arg[bad[:8]]} oracle {a[bad[:8]]}"
    for i in np.nonzero(~clear)[0]:
        ts = tie_set(hidden_bits[rows[i]], w_bits, mask_id, p1[i])
        assert int(g_arg[i]) in ts, (rows[i], g_arg[i], ts)
    return a, p1, p2, int((~clear).sum())


def oracle_rows_with_ties(hidden_rows, w_bits, mask_id, chunk=1024):
    """Oracle (argmax, p1, p2) of the given hidden rows ([M][Hd] bits) in a
    few batched calls, and the tie set (tokens within TIE_BAND of the top
    probability) of every row whose top two are that close, from one more
    batched call on those rows only.  Returns (a, p1, p2, ties: dict)."""
    a, p1, p2 = oracle.lmhead_rows(hidden_rows, w_bits, mask_id, chunk=chunk)
    ties = {}
    near = np.nonzero((p1 - p2) < TIE_BAND)[0]
    for i0 in range(0, near.size, chunk):
        idx = near[i0:i0 + chunk]
        L = oracle.lmhead_logits(hidden_rows[idx], w_bits, mask_id)
        for j, i in enumerate(idx):
            m = L[j].max()
            if m == -np.inf:
                ties[int(i)] = {int(mask_id)}
                continue
            p = np.exp(L[j] - m)
            p /= p.sum()
            ties[int(i)] = set(np.nonzero(p >= p1[i] - TIE_BAND)[0].tolist())
    return a, p1, p2, ties


def check_rows_against(gpu_arg, gpu_conf, a, p1, p2, ties, label=""):
    """GPU argmax / confidence of rows against the oracle's (aligned
    arrays): conf within CONF_ABS everywhere; argmax exact where the top two
    are at least TIE_BAND apart, else inside the tie set."""
    g_arg = np.asarray(gpu_arg)
    err = np.abs(np.asarray(gpu_conf, dtype=np.float64) - p1)
    assert np.all(err <= CONF_ABS), f"{label} conf error {err.max():.3g} at {int(np.argmax(err))}"
    clear = (p1 - p2) >= TIE_BAND
    bad = np.nonzero(clear & (g_arg != a))[0]
    assert bad.size == 0, f"{label} argmax mismatch at {bad[:8]}: gpu {g_arg[bad[:8]]} oracle {a[bad[:8]]}"
    for i in np.nonzero(~clear)[0]:
        assert int(g_arg[i]) in ties[int(i)], (label, i, g_arg[i])
    return int((~clear).sum())


def check_commits(toks0, state0, toks1, state1, p1_by_row, arg_ok, mask_id, tau, seqs=None):
    """The acceptance rule of one round's commits, per DENOISING sequence.

    R = robust commits (p1 >= tau + band), A = ambiguous (|p1 - tau| < band),
    F = fallback ties (p1 within TIE_BAND of the masked maximum).  The GPU
    commit set C is valid iff C != {} and R <= C <= R|A, or R == {} and C is
    one position of F.  Committed tokens must have passed arg_ok(row, tok).
    seqs: the sequences to check (all by default).  Returns the number of
    sequences that used an exemption."""
    S, B = toks0.shape
    exempt = 0
    for s in (range(S) if seqs is None else seqs):
        if state0[s] != oracle.DENOISING:
            assert np.array_equal(toks1[s], toks0[s]) and state1[s] == state0[s], s
            continue
        M = [i for i in range(B) if toks0[s, i] == mask_id]
        keep = [i for i in range(B) if toks0[s, i] != mask_id]
        assert np.array_equal(toks1[s, keep], toks0[s, keep]), f"seq {s}: committed token changed"
        C = {i for i in M if toks1[s, i] != mask_id}
        if M:
            p = {i: p1_by_row[s * B + i] for i in M}
            R = {i for i in M if p[i] >= tau + TAU_BAND}
            A = {i for i in M if abs(p[i] - tau) < TAU_BAND}
            pmax = max(p.values())
            F = {i for i in M if p[i] >= pmax - TIE_BAND}
            ok_thr = bool(C) and R <= C <= (R | A)
            ok_fb = (not R) and len(C) == 1 and C <= F
            assert ok_thr or ok_fb, f"seq {s}: commits {sorted(C)} R={sorted(R)} A={sorted(A)} F={sorted(F)}"
            if A or len(F) > 1:
                exempt += 1
            for i in C:
                assert arg_ok(s * B + i, int(toks1[s, i])), f"seq {s} pos {i}: token {toks1[s, i]}"
        left = (toks1[s] == mask_id).sum()
        assert (state1[s] == oracle.SAVING) == (left == 0), f"seq {s}: state {state1[s]} with {left} masks"
    return exempt


class RoundState:
    """Device buffers of one workload's round state."""

    def __init__(self, w, fx):
        n = w.S * w.B
        self.bufs = api.RoundBuffers(
            row_index=torch.zeros(n, dtype=torch.int32, device="cuda"),
            num_rows=torch.zeros(1, dtype=torch.int32, device="cuda"),
            argmax_tok=torch.full((n,), -1, dtype=torch.int32, device="cuda"),
            conf=torch.full((n,), float("nan"), dtype=torch.float32, device="cuda"),
            block_tokens=dev_i32(fx.block_tokens0),
            seq_state=dev_u8(fx.seq_state0),
            num_committed=torch.zeros(w.S, dtype=torch.int32, device="cuda"),
            workspace=torch.empty(1, dtype=torch.uint8, device="cuda"))
        self.fixed = dict(k_cache=dev_bf16(fx.k_cache), v_cache=dev_bf16(fx.v_cache),
                          page_table=dev_i32(fx.page_table), prefix_len=dev_i32(fx.prefix_len),
                          w_vocab=dev_bf16(fx.w_vocab))
        self.w = w
        self.maxp = int(fx.page_table.shape[1])

    def init_rows(self):
        b = self.bufs
        api.dbd_remask_commit(b.block_tokens, b.seq_state, None, None, b.row_index, b.num_rows,
                              self.w.mask_id, self.w.tau, flags=api.DBD_COMPACT_ONLY)

    def args(self, rin_dev, attn_out):
        w = self.w
        a = api.make_round_args(
            S=w.S, B=w.B, Hq=w.Hq, Hkv=w.Hkv, D=w.D, page_size=w.P,
            max_pages_per_seq=self.maxp, Hd=w.Hd, V=w.V, mask_token_id=w.mask_id,
            dynamic_threshold=w.tau, attn_out=attn_out, bufs=self.bufs, **rin_dev, **self.fixed)
        need = api.dbd_round_workspace_size(a)
        if self.bufs.workspace.numel() < need:
            self.bufs.workspace = torch.empty(need, dtype=torch.uint8, device="cuda")
            a = api.make_round_args(
                S=w.S, B=w.B, Hq=w.Hq, Hkv=w.Hkv, D=w.D, page_size=w.P,
                max_pages_per_seq=self.maxp, Hd=w.Hd, V=w.V, mask_token_id=w.mask_id,
                dynamic_threshold=w.tau, attn_out=attn_out, bufs=self.bufs, **rin_dev,
                **self.fixed)
        # the args hold raw pointers: keep the round's input tensors alive
        # until the next round's args, so that no later allocation can take
        # their memory before the round has run
        self.inputs = (rin_dev, attn_out)
        return a


def round_inputs_dev(rin):
    return dict(q=dev_bf16(rin.q), k_blk=dev_bf16(rin.k_blk), v_blk=dev_bf16(rin.v_blk),
                hidden=dev_bf16(rin.hidden))


def check_filtered_rows(lg, rows, tok, conf, mask, T, k, p, seed, step):
    """Each listed row's token against the oracle's filtered draw on the
    kernel's own fp32 logits lg[j] (row id rows[j]); a different token is
    accepted only where float32 rounding could decide (two best blocks'
    Gumbel values within G_BAND, a draw within CDF_BAND of an inverse-CDF
    boundary, or a top-p boundary within P_BAND of the kept mass).  The
    confidence must be the token's probability at temperature 1.  Returns
    the number of rows accepted that way."""
    exempt = 0
    for j, r in enumerate(rows):
        l = lg[j].astype(np.float64)
        t_ref, c_ref, inf = oracle.sample_filtered(l, T, k, p, seed, int(r), step, mask_id=mask)
        t = int(tok[r])
        kept = inf["keep"]          # the kept set this row's token must belong to
        if t != t_ref:
            fi = inf["filter"]
            ok = (inf["g_gap"] < G_BAND and t == inf["runner_up"]) or \
                 (inf["cdf_margin"] < CDF_BAND and t in inf["block"])
            if not ok and fi["margin"] < P_BAND:
                # the top-p boundary one token shorter or longer: the token
                # is that kept set's draw and must lie in it
                for key in ("shorter", "longer"):
                    if oracle.sample_row(l, T, seed, int(r), step, fi[key], mask_id=mask)[0] == t:
                        ok, kept = True, fi[key]
                        break
            assert ok, f"row {r}: gpu {t} oracle {t_ref} info g_gap={inf['g_gap']:.3g} " \
                       f"cdf={inf['cdf_margin']:.3g} pmargin={fi['margin']:.3g}"
            exempt += 1
        assert 0 <= t < kept.size and kept[t], f"row {r}: token {t} outside the kept set"
        lse = l.max() + np.log(np.exp(l - l.max()).sum())
        assert abs(float(conf[r]) - np.exp(l[t] - lse)) <= 1e-5 + 1e-4 * np.exp(l[t] - lse)
    return exempt
