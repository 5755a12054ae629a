"""The device-side block loop through the C ABI: blocks of B gated rounds
followed by the SAVING step, run eagerly (each step checked against the CPU
oracle from the GPU's own state) and as one captured graph, which must give
the eager run's results bit for bit on every replay.

Rounds after a block is done must change nothing (gate_on_rows); the round
counter must count exactly the rounds that had rows to denoise.  Integer and
bit data are compared exactly; attention and confidences with the usual
tolerances."""
import numpy as np
import pytest
import torch

import oracle
from block_diffusion_amd import api, synth
from block_diffusion_amd.workloads import SDAR_1P7B, TINY, Workload
from gpu_util import (ATTN_MAX_ABS, ATTN_REL_L2, attn_errors, check_lm_rows, dev_bf16, dev_i32,
                      dev_u8, host_bits, round_inputs_dev, widen_bits)

pytestmark = pytest.mark.gpu

DEN, SAV, FIN = 2, 3, 4

# confident rows (large planted amplitude): blocks finish in one or two
# rounds, so most gated rounds find nothing to do
LOOP_FAST = Workload(name="loop_fast_b8", seed_id=50, S=4, B=8, Hq=8, Hkv=2, D=64, P=32,
                     Hd=256, V=1024, mask_id=1000, prefix_lo=0, prefix_hi=100, tau=0.9,
                     rounds=8, a_max=24.0)
# B = 16 with pre-committed positions in the first block and a 0.75 threshold
LOOP_MIX = Workload(name="loop_mix_b16", seed_id=51, S=12, B=16, Hq=16, Hkv=4, D=128, P=64,
                    Hd=512, V=2048, mask_id=5, prefix_lo=10, prefix_hi=300, tau=0.75,
                    rounds=16, a_max=16.0, init_committed_max=12)


class Loop:
    """Device buffers of a multi-block run and its schedule of steps."""

    def __init__(self, w, nb, rule=0, k=1):
        self.w, self.nb, self.rule, self.k = w, nb, rule, k
        self.fx = fx = synth.make_fixed(w, reserve_tokens=nb * w.B)
        self.L0 = fx.prefix_len.copy()
        self.end = (self.L0 + nb * w.B).astype(np.int32)
        self.cap = int(self.end.max())
        n = w.S * w.B
        d = dict(k_cache=dev_bf16(fx.k_cache), v_cache=dev_bf16(fx.v_cache),
                 page_table=dev_i32(fx.page_table), prefix_len=dev_i32(fx.prefix_len),
                 w_vocab=dev_bf16(fx.w_vocab))
        self.fixed = d
        self.bufs = api.RoundBuffers(
            row_index=torch.zeros(n, dtype=torch.int32, device="cuda"),
            num_rows=torch.zeros(1, dtype=torch.int32, device="cuda"),
            argmax_tok=torch.zeros(n, dtype=torch.int32, device="cuda"),
            conf=torch.zeros(n, dtype=torch.float32, device="cuda"),
            block_tokens=dev_i32(fx.block_tokens0), seq_state=dev_u8(fx.seq_state0),
            num_committed=torch.zeros(w.S, dtype=torch.int32, device="cuda"),
            workspace=torch.empty(1, dtype=torch.uint8, device="cuda"))
        self.ts = torch.zeros((w.S, self.cap), dtype=torch.int32, device="cuda")
        self.end_d = dev_i32(self.end)
        self.counter = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.attn_out = torch.zeros((w.S, w.B, w.Hq, w.D), dtype=torch.bfloat16, device="cuda")
        # schedule: per block, B gated rounds then the SAVING step
        self.steps = []
        k = 0
        for _ in range(nb):
            for r in range(w.B + 1):
                k += 1
                self.steps.append((k, r == w.B))
        self.rin = {k: synth.make_round(w, k, fx.w_vocab) for k, _ in self.steps}
        self.rin_dev = {k: round_inputs_dev(v) for k, v in self.rin.items()}
        self.args = [self._args(k, save) for k, save in self.steps]

    def _args(self, k, save):
        w = self.w
        kw = dict(S=w.S, B=w.B, Hq=w.Hq, Hkv=w.Hkv, D=w.D, page_size=w.P,
                  max_pages_per_seq=int(self.fx.page_table.shape[1]), Hd=w.Hd, V=w.V,
                  mask_token_id=w.mask_id, dynamic_threshold=w.tau, attn_out=self.attn_out,
                  bufs=self.bufs, save_kv=save, token_stream=self.ts, end_len=self.end_d,
                  **self.rin_dev[k], **self.fixed)
        a = api.make_round_args(**kw)
        need = api.dbd_round_workspace_size(a)
        if self.bufs.workspace.numel() < need:
            self.bufs.workspace = torch.empty(need, dtype=torch.uint8, device="cuda")
            a = api.make_round_args(**kw)
        a.gate_on_rows = 0 if save else 1
        a.round_counter = api._ptr(self.counter)
        a.rule, a.tokens_per_step = self.rule, self.k
        return a

    def reset(self):
        fx, b = self.fx, self.bufs
        self.fixed["k_cache"].copy_(dev_bf16(fx.k_cache))
        self.fixed["v_cache"].copy_(dev_bf16(fx.v_cache))
        self.fixed["prefix_len"].copy_(dev_i32(fx.prefix_len))
        b.block_tokens.copy_(dev_i32(fx.block_tokens0))
        b.seq_state.copy_(dev_u8(fx.seq_state0))
        for t, v in ((b.argmax_tok, -1), (b.conf, float("nan")), (self.ts, -1), (self.counter, 0),
                     (b.row_index, -1), (b.num_committed, -1)):
            t.fill_(v)
        self.attn_out.zero_()
        api.dbd_remask_commit(b.block_tokens, b.seq_state, None, None, b.row_index, b.num_rows,
                              self.w.mask_id, self.w.tau, flags=api.DBD_COMPACT_ONLY)
        torch.cuda.synchronize()

    def snapshot(self):
        b = self.bufs
        return dict(tokens=b.block_tokens.cpu().numpy(), state=b.seq_state.cpu().numpy(),
                    L=self.fixed["prefix_len"].cpu().numpy(), ts=self.ts.cpu().numpy(),
                    kc=host_bits(self.fixed["k_cache"]), vc=host_bits(self.fixed["v_cache"]),
                    counter=int(self.counter.item()), rows=b.row_index.cpu().numpy(),
                    nrows=int(b.num_rows.item()), arg=b.argmax_tok.cpu().numpy(),
                    conf=b.conf.cpu().numpy().view(np.uint32), attn=host_bits(self.attn_out))


def _run_eager_checked(lp):
    w, fx = lp.w, lp.fx
    g = np.random.default_rng(9)
    kc, vc = fx.k_cache.copy(), fx.v_cache.copy()
    toks, state, L = fx.block_tokens0.copy(), fx.seq_state0.copy(), lp.L0.copy()
    ts = np.full((w.S, lp.cap), -1, dtype=np.int64)
    active = 0
    prev = lp.snapshot()
    for (k, save), a in zip(lp.steps, lp.args):
        rin = lp.rin[k]
        rows0 = oracle.compact_rows(toks, state, w.mask_id)
        print(f"{w.name} step {k} save={save}: states {np.bincount(state, minlength=5).tolist()} "
              f"rows {rows0.size}", flush=True)
        api.dbd_round(a)
        torch.cuda.synchronize()
        now = lp.snapshot()
        if not save and rows0.size == 0:
            # a gated round after the block is done: nothing changes
            for key in ("tokens", "state", "L", "ts", "kc", "vc", "counter", "nrows", "attn"):
                assert np.array_equal(now[key], prev[key]), f"step {k}: gated round changed {key}"
            prev = now
            continue
        if save:
            kc, vc = oracle.kv_save(kc, vc, fx.page_table, L, state, rin.k_blk, rin.v_blk)
            assert np.array_equal(now["kc"], kc) and np.array_equal(now["vc"], vc), f"step {k}"
        else:
            assert np.array_equal(now["kc"], prev["kc"]) and np.array_equal(now["vc"], prev["vc"])
            active += 1
        assert now["counter"] == active, (k, now["counter"], active)
        groups = [(s, gk) for s in range(w.S) for gk in range(w.Hkv)]
        if len(groups) > 10:
            groups = [groups[i] for i in g.choice(len(groups), 10, replace=False)]
        got, ref = [], []
        for s, gk in groups:
            ref.append(oracle.attention_group(s, gk, rin.q, rin.k_blk, rin.v_blk, kc, vc,
                                              fx.page_table, L))
            got.append(widen_bits(now["attn"][s, :, gk * w.G:(gk + 1) * w.G, :]))
        mx, rl = attn_errors(np.stack(got), np.stack(ref))
        assert mx <= ATTN_MAX_ABS and rl <= ATTN_REL_L2, (k, mx, rl)
        conf = now["conf"].view(np.float32)
        if rows0.size:
            samp = rows0 if rows0.size <= 16 else rows0[:: rows0.size // 16]
            check_lm_rows(samp, now["arg"], conf, rin.hidden, fx.w_vocab, w.mask_id)
        if save:
            et, es, eL, ets, _, erows = oracle.step_commit(toks, state, L, conf, now["arg"],
                                                           w.mask_id, lp.rule, tau=np.float32(w.tau),
                                                           tokens_per_step=lp.k, token_stream=ts,
                                                           end_len=lp.end)
        else:
            et, es, _ = oracle.remask_rule(toks, state, conf, now["arg"], w.mask_id, lp.rule,
                                           tau=np.float32(w.tau), tokens_per_step=lp.k)
            eL, ets, erows = L, ts, oracle.compact_rows(et, es, w.mask_id)
        assert np.array_equal(now["tokens"], et) and np.array_equal(now["state"], es), f"step {k}"
        assert np.array_equal(now["L"], eL) and np.array_equal(now["ts"], ets), f"step {k}"
        assert now["nrows"] == erows.size and np.array_equal(now["rows"][:erows.size], erows)
        toks, state, L, ts = now["tokens"], now["state"], now["L"], ets
        prev = now
        if save:
            # the block loop is exact: B gated rounds finish every block
            assert not np.any(es == SAV)
    assert np.all(state == FIN) and np.array_equal(L, lp.end)
    return prev, active


@pytest.mark.parametrize("w,nb", [(LOOP_FAST, 3), (LOOP_MIX, 2), (TINY, 2), (SDAR_1P7B, 2)],
                         ids=lambda x: getattr(x, "name", str(x)))
def test_block_loop_graph(w, nb):
    lp = Loop(w, nb)
    lp.reset()
    eager, active = _run_eager_checked(lp)
    gated = sum(1 for _, s in lp.steps if not s) - active
    print(f"{w.name}: {len(lp.steps)} steps, {active} active rounds, {gated} gated off", flush=True)
    graph = api.dbd_graph_create(lp.args)
    try:
        for rep in range(3):
            lp.reset()
            graph.launch()
            torch.cuda.synchronize()
            got = lp.snapshot()
            for key, v in eager.items():
                assert np.array_equal(np.asarray(got[key]), np.asarray(v)), f"replay {rep}: {key}"
    finally:
        graph.close()


def test_block_loop_static_rule():
    """The static rule commits exactly k = 3 positions per round, so a block
    of 8 needs ceil(8/3) = 3 rounds and the other 5 gated rounds of each
    block change nothing; graph replays equal the eager run."""
    w = LOOP_FAST.with_(name="loop_static_b8")
    lp = Loop(w, 2, rule=1, k=3)
    lp.reset()
    eager, active = _run_eager_checked(lp)
    assert active == 2 * 3
    graph = api.dbd_graph_create(lp.args)
    try:
        lp.reset()
        graph.launch()
        torch.cuda.synchronize()
        got = lp.snapshot()
        for key, v in eager.items():
            assert np.array_equal(np.asarray(got[key]), np.asarray(v)), key
    finally:
        graph.close()


@pytest.mark.parametrize("w,nb", [(LOOP_FAST, 2), (TINY, 2)],
                         ids=lambda x: getattr(x, "name", str(x)))
def test_block_loop_filtered_graph(w, nb):
    """Blocks of gated rounds with temperature sampling and top-p filtering
    inside each round (stored logits, filtered draw), then the SAVING step:
    every sequence finishes its blocks with valid tokens, gated rounds
    change nothing (the round counter counts only rounds with rows), and
    three graph replays, with eager resets between them, equal the eager
    run bit for bit."""
    lp = Loop(w, nb)
    logits = torch.full((w.S * w.B, w.V), float("nan"), dtype=torch.float32, device="cuda")
    for i, a in enumerate(lp.args):
        a.sample, a.temperature, a.seed, a.step = 1, 0.8, 0xB10C, i + 1
        a.filter, a.top_k, a.top_p, a.logits = 1, 0, 0.9, logits.data_ptr()
    lp.reset()
    for a in lp.args:
        api.dbd_round(a)
    torch.cuda.synchronize()
    eager = lp.snapshot()
    assert np.all(eager["state"] == FIN) and np.array_equal(eager["L"], lp.end)
    ts = eager["ts"]
    for s in range(w.S):
        written = ts[s, int(lp.L0[s]):int(lp.end[s])]
        assert np.all((written >= 0) & (written < w.V) & (written != w.mask_id)), s
    assert 0 < eager["counter"] <= nb * w.B
    print(f"{w.name}: {eager['counter']} active rounds of {nb * w.B}", flush=True)
    graph = api.dbd_graph_create(lp.args)
    try:
        for rep in range(3):
            lp.reset()
            graph.launch()
            torch.cuda.synchronize()
            got = lp.snapshot()
            for key, v in eager.items():
                assert np.array_equal(np.asarray(got[key]), np.asarray(v)), f"replay {rep}: {key}"
    finally:
        graph.close()
