#!/usr/bin/env python3
"""Denoise-round throughput on one MI355X at SDAR-4B shapes (block_length 4,
batch 128, 32/8 heads, head dim 128, hidden 2560, vocab 151936, KV pages of
256, prefixes U[256,4096], threshold 0.9).

One step = one whole block: the initial all-masked state is restored and
the block's rounds (4) run as one captured graph, each round being paged
attention over every sequence, the selective fused LM head on the masked
rows and the threshold remask.  value = block-tokens per second =
batch * block_length * rounds * steps / elapsed.  All inputs (prefix cache,
LM-head weight, per-round queries/keys/values/hidden states) are seeded,
synthetic and resident in HBM before the timed region.

Prints one JSON line (rank 0).  Also times each entry point with HIP events
on the launch stream for the roofline object (the LM head between the
attention and the remask, as a round launches it; the others back to back),
and the CPU oracle on a bounded sample for the CPU baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="sdar4b_b4_bs128")
    ap.add_argument("--kernel-iters", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="the CPU oracle repeats whole blocks until this much time has passed")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-configuration entries (configs 0, 1, 3, 4)")
    ap.add_argument("--only", choices=["attention", "lmhead", "lmhead_round", "remask", "logits", "filtered",
                                       "prefill"],
                    help="launch only this entry point (warmup + steps times, round-1 inputs) and "
                         "print its mean launch time: the run that rocprofv3 counters are taken on; "
                         "lmhead_round runs attention, LM head and remask in turn and times the LM head")
    ap.add_argument("--copy-calibration", type=int, metavar="MIB",
                    help="copy MIB MiB device-to-device (warmup + steps times) and exit: the plain "
                         "copy kernel of known size that scales FETCH_SIZE / WRITE_SIZE")
    return ap.parse_args()


def traffic_table(workload, path=None):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE/WRITE_SIZE
    (scaled by the copy calibration), keyed by entry point and row count.
    An entry counts only while the kernel source it was taken on is
    unchanged (sha256 recorded beside it); otherwise the figure is None."""
    import hashlib
    import re
    if path is None:
        path = os.path.join(ROOT, "profiles", f"traffic_{workload}.md")
    table = {}
    if not os.path.exists(path):
        return table
    pat = re.compile(r"<!-- traffic (\S+) rows=(\d+) bytes=(\d+) src=(\S+) sha256=([0-9a-f]+) -->")
    for m in pat.finditer(open(path).read()):
        name, rows, nbytes, src, sha = m.groups()
        src_path = os.path.join(ROOT, "block_diffusion_amd", "csrc", src)
        ok = os.path.exists(src_path) and hashlib.sha256(open(src_path, "rb").read()).hexdigest() == sha
        table[(name, int(rows))] = int(nbytes) if ok else None
    return table


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the denoise round shards by sequence with no exchange, so one GPU's share is "
              "the measured unit", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from block_diffusion_amd import api, synth
    from block_diffusion_amd.workloads import BY_NAME

    api.lib()
    w = BY_NAME[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        nbytes = args.copy_calibration << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": nbytes, "launches": args.warmup + args.steps}))
        return

    def dbf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    t0 = time.time()
    # room for one more block per sequence, which the SAVING step writes
    fx = synth.make_fixed(w, reserve_tokens=w.B)
    rins = [synth.make_round(w, r, fx.w_vocab) for r in range(1, w.rounds + 1)]
    log(f"inputs generated in {time.time() - t0:.1f}s")

    n = w.S * w.B
    fixed = dict(k_cache=dbf(fx.k_cache), v_cache=dbf(fx.v_cache),
                 page_table=torch.from_numpy(fx.page_table).to(dev),
                 prefix_len=torch.from_numpy(fx.prefix_len).to(dev), w_vocab=dbf(fx.w_vocab))
    per_round = [dict(q=dbf(r.q), k_blk=dbf(r.k_blk), v_blk=dbf(r.v_blk), hidden=dbf(r.hidden))
                 for r in rins]
    tok0 = torch.from_numpy(fx.block_tokens0).to(dev)
    st0 = torch.from_numpy(fx.seq_state0).to(dev)
    bufs = api.RoundBuffers(
        row_index=torch.zeros(n, dtype=torch.int32, device=dev),
        num_rows=torch.zeros(1, dtype=torch.int32, device=dev),
        argmax_tok=torch.zeros(n, dtype=torch.int32, device=dev),
        conf=torch.zeros(n, dtype=torch.float32, device=dev),
        block_tokens=tok0.clone(), seq_state=st0.clone(),
        num_committed=torch.zeros(w.S, dtype=torch.int32, device=dev),
        workspace=torch.empty(1, dtype=torch.uint8, device=dev))
    attn_out = torch.empty((w.S, w.B, w.Hq, w.D), dtype=torch.bfloat16, device=dev)
    shape = dict(S=w.S, B=w.B, Hq=w.Hq, Hkv=w.Hkv, D=w.D, page_size=w.P,
                 max_pages_per_seq=int(fx.page_table.shape[1]), Hd=w.Hd, V=w.V, mask_token_id=w.mask_id,
                 dynamic_threshold=w.tau)

    def round_args():
        return [api.make_round_args(**shape, **pr, **fixed, attn_out=attn_out, bufs=bufs)
                for pr in per_round]

    need = api.dbd_round_workspace_size(round_args()[0])
    bufs.workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    graph = api.dbd_graph_create(round_args())

    def reset():
        bufs.block_tokens.copy_(tok0)
        bufs.seq_state.copy_(st0)
        api.dbd_remask_commit(bufs.block_tokens, bufs.seq_state, None, None, bufs.row_index,
                              bufs.num_rows, w.mask_id, w.tau, flags=api.DBD_COMPACT_ONLY)

    def step():
        reset()
        graph.launch()

    if args.only:
        only(args, w, api, fixed, per_round[0], attn_out, bufs, tok0, st0)
        graph.close()
        return

    # rows per round (for the LM-head breakdown), from one untimed block
    reset()
    rows_per_round = []
    for a in round_args():
        rows_per_round.append(int(bufs.num_rows.item()))
        api.dbd_round(a)
    torch.cuda.synchronize()
    saving = int((bufs.seq_state == 3).sum().item())
    log(f"rows per round {rows_per_round}, sequences SAVING after the block: {saving}/{w.S}")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    block_tokens = w.S * w.B * w.rounds * args.steps
    value = block_tokens / elapsed
    log(f"{args.steps} steps in {elapsed * 1e3:.2f} ms: {ms_per_step:.3f} ms/step, "
        f"{value:.0f} block-tokens/s")

    # ---- the same step with sampling as the pages benchmark it (temperature
    # 0.6, top_p 0.95): each round stores its rows' logits, draws the tokens
    # with the filter, then remasks; one graph of the four rounds
    lg_step = torch.empty((n, w.V), dtype=torch.float32, device=dev)
    targs = round_args()
    for i, a in enumerate(targs):
        a.sample, a.temperature, a.seed, a.step = 1, 0.6, 20240, i + 1
        a.filter, a.top_k, a.top_p, a.logits = 1, 0, 0.95, lg_step.data_ptr()
    tgraph = api.dbd_graph_create(targs)
    reset()
    rows_topp = []
    for a in targs:
        rows_topp.append(int(bufs.num_rows.item()))
        api.dbd_round(a)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        reset()
        tgraph.launch()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        reset()
        tgraph.launch()
    torch.cuda.synchronize()
    ms_topp = (time.perf_counter() - t0) * 1e3 / args.steps
    tgraph.close()
    del lg_step, targs
    log(f"step with temperature 0.6 / top_p 0.95 sampling (rows per round {rows_topp}): "
        f"{ms_topp:.3f} ms/step, {w.S * w.B * w.rounds / (ms_topp * 1e-3):.0f} block-tokens/s")

    # ---- per round (eager rounds, HIP events between them, median over
    # repetitions) and the same step with the 256 MB MALL flushed before it
    # (a 512 MB scratch write, untimed): the cold figure
    stream = torch.cuda.current_stream()
    ra = round_args()
    round_times = [[] for _ in ra]
    for _ in range(max(args.steps // 2, 5)):
        reset()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(ra) + 1)]
        evs[0].record(stream)
        for i, a in enumerate(ra):
            api.dbd_round(a)
            evs[i + 1].record(stream)
        evs[-1].synchronize()
        for i in range(len(ra)):
            round_times[i].append(evs[i].elapsed_time(evs[i + 1]) * 1e3)
    round_us = [float(np.median(x)) for x in round_times]
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = []
    for _ in range(max(args.steps // 2, 5)):
        flush.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        e1.synchronize()
        cold.append(e0.elapsed_time(e1))
    del flush
    cold_ms = float(np.median(cold))
    log("per round (eager, median): " + ", ".join(f"r{i + 1} {t:.1f} us ({w.S * w.B / t * 1e6:.0f} "
                                                  f"block-tokens/s)" for i, t in enumerate(round_us))
        + f"; cold step (MALL flushed) {cold_ms:.3f} ms")

    # ---- per entry point, HIP events on the launch stream
    it = args.kernel_iters

    def ev_time(fn):
        for _ in range(3):
            fn()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        for _ in range(it):
            fn()
        e.record(stream)
        e.synchronize()
        return s.elapsed_time(e) * 1e3 / it     # microseconds per launch

    r1 = per_round[0]
    t_attn = ev_time(lambda: api.dbd_attn_paged(r1["q"], r1["k_blk"], r1["v_blk"],
                                                fixed["k_cache"], fixed["v_cache"],
                                                fixed["page_table"], fixed["prefix_len"],
                                                attn_out, ws=bufs.workspace))
    lm_rows = torch.arange(n, dtype=torch.int32, device=dev)
    lm_times = {}
    for M in sorted(set(rows_per_round) | {n}, reverse=True):
        if M == 0:
            continue
        nr = torch.tensor([M], dtype=torch.int32, device=dev)
        lm_times[M] = ev_time(lambda: api.dbd_lmhead_conf(
            r1["hidden"], fixed["w_vocab"], nr, bufs.argmax_tok, bufs.conf, w.mask_id,
            row_index=lm_rows, max_rows=n, ws=bufs.workspace))
    nr1 = torch.tensor([rows_per_round[0]], dtype=torch.int32, device=dev)
    t_lm_sample = ev_time(lambda: api.dbd_lmhead_sample(
        r1["hidden"], fixed["w_vocab"], nr1, bufs.argmax_tok, bufs.conf, w.mask_id, 1.0, 1234, 1,
        row_index=lm_rows, max_rows=n, ws=bufs.workspace))
    # top-k / top-p: the logits stored, then the filtered draw (T 0.6, top_p 0.95)
    M1r = rows_per_round[0]
    lg_buf = torch.empty((n, w.V), dtype=torch.float32, device=dev)
    t_logits = ev_time(lambda: api.dbd_lmhead_logits(r1["hidden"], fixed["w_vocab"], nr1, lg_buf,
                                                     w.mask_id, row_index=lm_rows, max_rows=n))
    t_filter = ev_time(lambda: api.dbd_sample_filtered(lg_buf, nr1, bufs.argmax_tok, bufs.conf,
                                                       w.mask_id, 0.6, 0, 0.95, 1234, 1,
                                                       row_index=lm_rows, max_rows=n))
    del lg_buf
    conf_r = torch.rand(n, device=dev)
    arg_r = torch.zeros(n, dtype=torch.int32, device=dev)
    tk, ss = tok0.clone(), st0.clone()
    ri, nr2 = torch.zeros(n, dtype=torch.int32, device=dev), torch.zeros(1, dtype=torch.int32, device=dev)
    t_remask = ev_time(lambda: api.dbd_remask_commit(tk, ss, arg_r, conf_r, ri, nr2, w.mask_id,
                                                     2.0))   # tau > 1: one commit each, no state change until full
    # the LM head over the first round's rows inside a round's sequence
    # (attention, LM head, remask): the launch the roofline reports
    M1 = rows_per_round[0]
    nr_m1 = torch.tensor([M1], dtype=torch.int32, device=dev)
    t_lm_round = lm_in_round(
        lambda: api.dbd_attn_paged(r1["q"], r1["k_blk"], r1["v_blk"], fixed["k_cache"], fixed["v_cache"],
                                   fixed["page_table"], fixed["prefix_len"], attn_out, ws=bufs.workspace),
        lambda: api.dbd_lmhead_conf(r1["hidden"], fixed["w_vocab"], nr_m1, bufs.argmax_tok, bufs.conf,
                                    w.mask_id, row_index=lm_rows, max_rows=n, ws=bufs.workspace),
        lambda: api.dbd_remask_commit(tk, ss, arg_r, conf_r, ri, nr2, w.mask_id, 2.0),
        3, it)
    log(f"LM head at M={M1} in a round's sequence (attention, LM head, remask): {t_lm_round:.1f} us; "
        f"back to back alone: {lm_times[M1]:.1f} us")
    # the same two launches replayed from a captured graph (graph_time)
    tg_attn = graph_time(lambda: api.dbd_attn_paged(r1["q"], r1["k_blk"], r1["v_blk"],
                                                    fixed["k_cache"], fixed["v_cache"],
                                                    fixed["page_table"], fixed["prefix_len"],
                                                    attn_out, ws=bufs.workspace))
    tg_remask = graph_time(lambda: api.dbd_remask_commit(tk, ss, arg_r, conf_r, ri, nr2, w.mask_id, 2.0))
    log(f"attention {t_attn:.1f} us, LM head {', '.join(f'M={m}: {t:.1f} us' for m, t in lm_times.items())}, "
        f"remask {t_remask:.1f} us, LM head with temperature sampling M={rows_per_round[0]}: "
        f"{t_lm_sample:.1f} us; stored logits {t_logits:.1f} us + top-p draw {t_filter:.1f} us")

    # ---- a whole block on the device: B gated rounds, then the SAVING step
    # (attention with the K/V write, the block commit), one graph per block
    L0 = fixed["prefix_len"].clone()
    loop_args = []
    for i in range(w.B):
        a = api.make_round_args(**shape, **per_round[i % len(per_round)], **fixed,
                                attn_out=attn_out, bufs=bufs)
        a.gate_on_rows = 1
        loop_args.append(a)
    loop_args.append(api.make_round_args(**shape, **per_round[0], **fixed, attn_out=attn_out,
                                         bufs=bufs, save_kv=True))
    loop_graph = api.dbd_graph_create(loop_args)

    def loop_step():
        fixed["prefix_len"].copy_(L0)
        reset()
        loop_graph.launch()

    for _ in range(args.warmup):
        loop_step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        loop_step()
    torch.cuda.synchronize()
    t_block = (time.perf_counter() - t0) * 1e6 / args.steps
    fixed["prefix_len"].copy_(L0)
    loop_graph.close()
    ss_all = torch.full_like(st0, 3)
    t_save = ev_time(lambda: api.dbd_attn_paged_save(r1["q"], r1["k_blk"], r1["v_blk"],
                                                     fixed["k_cache"], fixed["v_cache"],
                                                     fixed["page_table"], fixed["prefix_len"],
                                                     ss_all, attn_out, ws=bufs.workspace))
    log(f"block on the device ({w.B} gated rounds + SAVING step): {t_block:.1f} us, "
        f"{w.S * w.B / t_block * 1e6:.0f} committed tokens/s; attention with the K/V write "
        f"(every sequence SAVING): {t_save:.1f} us")

    # ---- block-causal prefill of the same batch: every sequence's prefix as
    # one prompt (packed), the same heads and block length; inputs drawn on
    # the device (seeded), the prompt K/V stored into the paged cache
    Lp = fx.prefix_len.astype(np.int64)
    cu = np.concatenate([[0], np.cumsum(Lp)]).astype(np.int32)
    Tp = int(cu[-1])
    gen = torch.Generator(device=dev).manual_seed(4321)
    qp = torch.randn((Tp, w.Hq, w.D), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    kp = torch.randn((Tp, w.Hkv, w.D), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    vp = torch.randn((Tp, w.Hkv, w.D), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    op = torch.empty_like(qp)
    cu_d = torch.from_numpy(cu).to(dev)
    kc_p, vc_p = torch.empty_like(fixed["k_cache"]), torch.empty_like(fixed["v_cache"])
    pf_ws = api.workspace(api.lib().dbd_prefill_workspace_size(w.S), dev)
    t_prefill = ev_time(lambda: api.dbd_prefill_attn(qp, kp, vp, cu_d, op, w.B,
                                                     page_table=fixed["page_table"], k_cache=kc_p,
                                                     v_cache=vc_p, ws=pf_ws))
    # 2*D flops each for q.k and p.v per (row, visible key)
    vis = 0
    for Ls in Lp:
        i = np.arange(Ls)
        vis += int(np.minimum(Ls, (i // w.B + 1) * w.B).sum())
    pf_flops = 4.0 * w.D * w.Hq * vis
    pf_tflops = pf_flops / (t_prefill * 1e-6) / 1e12
    del qp, kp, vp, op, kc_p, vc_p
    log(f"block-causal prefill of the batch's prefixes ({Tp} tokens, block {w.B}): {t_prefill:.1f} us, "
        f"{pf_tflops:.0f} TFLOP/s ({pf_tflops / PEAK_BF16_TFLOPS:.1%} of bf16 peak)")

    # ---- practical ceilings on this machine: a streaming read of 4 GiB (the
    # library's measurement kernel) and a large bf16 GEMM (hipBLASLt through
    # torch.matmul)
    big = torch.ones((1 << 31,), dtype=torch.bfloat16, device=dev)
    sink = torch.empty(api.lib().dbd_stream_read_sink_words(), dtype=torch.int32, device=dev)
    t_read = ev_time(lambda: api.dbd_stream_read(big, sink))
    read_tbs = big.numel() * 2 / (t_read * 1e-6) / 1e12
    del big, sink
    ga = torch.randn((8192, 8192), device=dev, dtype=torch.float32).to(torch.bfloat16)
    gb = torch.randn((8192, 8192), device=dev, dtype=torch.float32).to(torch.bfloat16)
    t_gemm = ev_time(lambda: torch.matmul(ga, gb))
    gemm_tf = 2.0 * 8192 ** 3 / (t_gemm * 1e-6) / 1e12
    del ga, gb
    # register-resident bf16 MFMA loop on random operands (the library's
    # measurement kernel): the matrix cores' practical rate, power limit included
    mf_ops = torch.randn((api.lib().dbd_mfma_peak_operand_bytes() // 2,), generator=gen, device=dev,
                         dtype=torch.float32).to(torch.bfloat16)
    mf_sink = torch.empty((api.lib().dbd_mfma_peak_sink_floats(),), dtype=torch.float32, device=dev)
    mf_iters = 1024
    t_mfma = ev_time(lambda: api.dbd_mfma_peak(mf_ops, mf_iters, mf_sink))
    mfma_tf = api.lib().dbd_mfma_peak_flops(mf_iters) / (t_mfma * 1e-6) / 1e12
    del mf_ops, mf_sink
    # the LM head's own product as a plain library GEMM: bf16 logits of the
    # first round's rows (no argmax, no softmax), hipBLASLt through linear()
    M1g = rows_per_round[0]
    hg = r1["hidden"].view(-1, w.Hd)[:M1g]
    t_lmgemm = ev_time(lambda: torch.nn.functional.linear(hg, fixed["w_vocab"]))
    lmgemm_tf = 2.0 * M1g * w.Hd * w.V / (t_lmgemm * 1e-6) / 1e12
    log(f"practical ceilings: streaming read {read_tbs:.2f} TB/s, MFMA loop {mfma_tf:.0f} TFLOP/s, "
        f"bf16 GEMM 8192^3 {gemm_tf:.0f} TFLOP/s, "
        f"LM-head-shaped GEMM ({M1g} x {w.Hd} x {w.V}, bf16 logits out) {t_lmgemm:.1f} us = "
        f"{lmgemm_tf:.0f} TFLOP/s")

    # algorithmic work
    L = fx.prefix_len.astype(np.int64)
    npages = -(-L // w.P)
    attn_bytes = int(L.sum() * w.Hkv * w.D * 2 * 2                 # prefix K and V
                     + 2 * w.S * w.B * w.Hq * w.D * 2              # q in, out
                     + 2 * w.S * w.B * w.Hkv * w.D * 2             # block K and V
                     + w.S * 4 + npages.sum() * 4)                 # prefix lengths, page ids
    lm_flops = 2.0 * M1 * w.Hd * w.V
    t_lm1 = t_lm_round
    step_attn = t_attn * w.rounds
    step_lm = sum(lm_times.get(m, 0.0) for m in rows_per_round)
    attn_roof = dict(bound="hbm", achieved=attn_bytes / (t_attn * 1e-6) / 1e9, peak=PEAK_HBM_GBS,
                     unit="GB/s")
    lm_roof = dict(bound="mfma", achieved=lm_flops / (t_lm1 * 1e-6) / 1e12, peak=PEAK_BF16_TFLOPS,
                   unit="TFLOP/s")
    traffic = traffic_table(w.name)
    attn_roof["traffic"] = traffic.get(("dbd_attn_paged", n))
    lm_roof["traffic"] = traffic.get(("dbd_lmhead_conf", M1))
    for r in (attn_roof, lm_roof):
        r["frac"] = r["achieved"] / r["peak"]
    # attention + remask as one HBM figure: remask reads block tokens,
    # confidences and tokens (12 B per position) and writes block tokens and
    # the row list (8 B), plus the state byte read and written per sequence
    # (launch times from graph replays: the remask kernel runs for about 4 us,
    # less than the host needs to issue an eager launch)
    remask_bytes = 20 * w.S * w.B + 2 * w.S
    attn_remask = dict(bound="hbm", bytes=attn_bytes + remask_bytes,
                       us=round(tg_attn + tg_remask, 2), attention_us=round(tg_attn, 2),
                       remask_us=round(tg_remask, 2),
                       achieved=(attn_bytes + remask_bytes) / ((tg_attn + tg_remask) * 1e-6) / 1e9,
                       peak=PEAK_HBM_GBS, unit="GB/s")
    attn_remask["frac"] = attn_remask["achieved"] / PEAK_HBM_GBS
    eager_frac = (attn_bytes + remask_bytes) / ((t_attn + t_remask) * 1e-6) / 1e9 / PEAK_HBM_GBS
    attn_remask["frac_eager_launches"] = eager_frac
    log(f"attention + remask (graph replays): {tg_attn:.1f} + {tg_remask:.1f} us, "
        f"{attn_remask['achieved']:.0f} GB/s = {attn_remask['frac']:.1%} of HBM peak "
        f"({eager_frac:.1%} from eager launches)")
    dominant = "attention" if step_attn >= step_lm else "lmhead"
    roof = dict(attn_roof if dominant == "attention" else lm_roof)
    roof["kernel"] = "dbd_attn_paged" if dominant == "attention" else "dbd_lmhead_conf"

    out = {
        "metric": "denoise-round block-tokens/sec at SDAR-4B shapes, B=4, batch 128; % HBM/MFMA peak",
        "value": round(value, 1), "unit": "block-tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.S, "block_length": w.B, "rounds_per_step": w.rounds,
                   "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.D, "hidden": w.Hd,
                   "vocab": w.V, "page_size": w.P, "prefix": [w.prefix_lo, w.prefix_hi],
                   "threshold": w.tau, "rows_per_round": rows_per_round, "parallelism": "none"},
        "roofline": roof,
        "breakdown_us": {"attention": round(t_attn, 2),
                         "lmhead": {str(m): round(t, 2) for m, t in lm_times.items()},
                         "lmhead_in_round_M%d" % M1: round(t_lm_round, 2),
                         "remask": round(t_remask, 2),
                         "attention_kv_save": round(t_save, 2),
                         "per_round_eager_us": [round(t, 1) for t in round_us],
                         "per_round_block_tokens_per_s": [round(w.S * w.B / t * 1e6, 1) for t in round_us],
                         "cold_ms_per_step": round(cold_ms, 4),
                         "cold_block_tokens_per_s": round(w.S * w.B * w.rounds / (cold_ms * 1e-3), 1),
                         "practical_ceilings": {"stream_read_TBps": round(read_tbs, 3),
                                                "mfma_loop_TFLOPs": round(mfma_tf, 1),
                                                "bf16_gemm_8192_TFLOPs": round(gemm_tf, 1),
                                                "attention_frac_of_read": round(attn_roof["achieved"] / 1e3 / read_tbs, 4),
                                                "lmhead_frac_of_gemm": round(lm_roof["achieved"] / gemm_tf, 4),
                                                "lmhead_frac_of_mfma_loop": round(lm_roof["achieved"] / mfma_tf, 4),
                                                "lmhead_shape_gemm_us": round(t_lmgemm, 2),
                                                "lmhead_shape_gemm_TFLOPs": round(lmgemm_tf, 1)},
                         "lmhead_sample_T1_M%d" % rows_per_round[0]: round(t_lm_sample, 2),
                         "topp_step": {"ms_per_step": round(ms_topp, 4),
                                       "block_tokens_per_s": round(w.S * w.B * w.rounds / (ms_topp * 1e-3), 1),
                                       "rows_per_round": rows_topp, "temperature": 0.6, "top_p": 0.95},
                         "topp_M%d" % M1r: {"logits_us": round(t_logits, 2),
                                             "filtered_draw_us": round(t_filter, 2),
                                             "temperature": 0.6, "top_p": 0.95},
                         "prefill": {"tokens": Tp, "block_length": w.B, "us": round(t_prefill, 2),
                                     "tflops": round(pf_tflops, 1),
                                     "frac_bf16_peak": round(pf_tflops / PEAK_BF16_TFLOPS, 4),
                                     "kv_store": True},
                         "block_loop": {"rounds": w.B, "saving_step": True,
                                        "us_per_block": round(t_block, 2),
                                        "committed_tokens_per_s": round(w.S * w.B / t_block * 1e6, 1)},
                         "attention_roofline": {k: (round(v, 4) if isinstance(v, float) else v)
                                                for k, v in attn_roof.items()},
                         "attention_remask_frac": round(attn_remask["frac"], 4),
                         "attention_remask_roofline": {k: (round(v, 4) if isinstance(v, float) else v)
                                                       for k, v in attn_remask.items()},
                         "lmhead_roofline_M%d" % M1: {k: (round(v, 4) if isinstance(v, float) else v)
                                                      for k, v in lm_roof.items()}},
    }
    graph.close()

    if not args.no_configs:
        # the other configurations, each as whole blocks of its own rounds
        del fixed, per_round, bufs, attn_out
        torch.cuda.empty_cache()
        from block_diffusion_amd.workloads import LLADA_LONG, SDAR_1P7B, SDAR_8B, TINY
        out["breakdown_us"]["configs"] = {}
        for wc in (TINY, SDAR_1P7B, SDAR_8B, LLADA_LONG):
            out["breakdown_us"]["configs"][wc.name] = config_entry(api, synth, wc, dev, max(args.steps // 4, 3))
            torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, fx, rins, args.cpu_seconds)
        out["breakdown_us"]["cpu_oracle_1thread"] = cpu_single_thread(synth)
    print(json.dumps(out), flush=True)


def lm_in_round(attn_fn, lm_fn, remask_fn, warmup, reps):
    """The LM head's launch time in the setting of a round: each repetition
    launches the attention, the LM head between two HIP events, then the
    remask, in order on one stream.  Returns the mean over reps in
    microseconds.  Back-to-back launches of the LM head alone keep the matrix
    cores busy without the attention's pauses and run at a lower clock; the
    round is what the step runs."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        attn_fn()
        lm_fn()
        remask_fn()
    pairs = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        attn_fn()
        e0.record(stream)
        lm_fn()
        e1.record(stream)
        remask_fn()
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in pairs) * 1e3 / reps


def graph_time(fn, n=20):
    """Per-launch GPU time of fn, replayed n times from one captured graph:
    no host work between launches (as inside the round graph), inter-kernel
    gaps included.  Small kernels timed with eager launches are bound by the
    host's launch rate instead."""
    import numpy as np
    import torch
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            fn()
    g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(5):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        g.replay()
        e.record()
        e.synchronize()
        ts.append(s.elapsed_time(e) * 1e3 / n)
    del g
    return float(np.median(ts))


def attn_bytes_of(w, prefix_len):
    """Algorithmic bytes of one attention launch: prefix K and V, q in and
    out, the block's K and V, prefix lengths and page ids."""
    import numpy as np
    L = prefix_len.astype(np.int64)
    npages = -(-L // w.P)
    return int(L.sum() * w.Hkv * w.D * 2 * 2 + 2 * w.S * w.B * w.Hq * w.D * 2
               + 2 * w.S * w.B * w.Hkv * w.D * 2 + w.S * 4 + npages.sum() * 4)


def config_entry(api, synth, w, dev, steps):
    """Workload w as whole blocks: the rounds from the initial state until
    no masked row is left (each round's inputs drawn as for the parity
    tests), captured as one graph and replayed `steps` times after a
    warm-up, and again with the 256 MB MALL flushed before each replay (the
    cold figure); per-round eager times; attention, LM head (round-1 rows)
    and remask per launch with their roofline fractions."""
    import numpy as np
    import torch

    t0 = time.time()
    fx = synth.make_fixed(w)

    def dbf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    n = w.S * w.B
    fixed = dict(k_cache=dbf(fx.k_cache), v_cache=dbf(fx.v_cache),
                 page_table=torch.from_numpy(fx.page_table).to(dev),
                 prefix_len=torch.from_numpy(fx.prefix_len).to(dev), w_vocab=dbf(fx.w_vocab))
    tok0 = torch.from_numpy(fx.block_tokens0).to(dev)
    st0 = torch.from_numpy(fx.seq_state0).to(dev)
    bufs = api.RoundBuffers(
        row_index=torch.zeros(n, dtype=torch.int32, device=dev),
        num_rows=torch.zeros(1, dtype=torch.int32, device=dev),
        argmax_tok=torch.zeros(n, dtype=torch.int32, device=dev),
        conf=torch.zeros(n, dtype=torch.float32, device=dev),
        block_tokens=tok0.clone(), seq_state=st0.clone(),
        num_committed=torch.zeros(w.S, dtype=torch.int32, device=dev),
        workspace=torch.empty(1, dtype=torch.uint8, device=dev))
    attn_out = torch.empty((w.S, w.B, w.Hq, w.D), dtype=torch.bfloat16, device=dev)
    shape = dict(S=w.S, B=w.B, Hq=w.Hq, Hkv=w.Hkv, D=w.D, page_size=w.P,
                 max_pages_per_seq=int(fx.page_table.shape[1]), Hd=w.Hd, V=w.V, mask_token_id=w.mask_id,
                 dynamic_threshold=w.tau)

    def mk(pr):
        return api.make_round_args(**shape, **pr, **fixed, attn_out=attn_out, bufs=bufs)

    def reset():
        bufs.block_tokens.copy_(tok0)
        bufs.seq_state.copy_(st0)
        api.dbd_remask_commit(bufs.block_tokens, bufs.seq_state, None, None, bufs.row_index,
                              bufs.num_rows, w.mask_id, w.tau, flags=api.DBD_COMPACT_ONLY)

    # the block's rounds, found by running it once (untimed)
    reset()
    per_round, rows = [], []
    for r in range(1, w.rounds + 1):
        nr = int(bufs.num_rows.item())
        if nr == 0:
            break
        rin = synth.make_round(w, r, fx.w_vocab)
        per_round.append(dict(q=dbf(rin.q), k_blk=dbf(rin.k_blk), v_blk=dbf(rin.v_blk), hidden=dbf(rin.hidden)))
        rows.append(nr)
        if r == 1:
            bufs.workspace = torch.empty(api.dbd_round_workspace_size(mk(per_round[0])), dtype=torch.uint8,
                                         device=dev)
        api.dbd_round(mk(per_round[-1]))
    torch.cuda.synchronize()
    assert int(bufs.num_rows.item()) == 0, "block not finished within the round cap"
    R = len(per_round)
    graph = api.dbd_graph_create([mk(pr) for pr in per_round])
    for _ in range(2):
        reset()
        graph.launch()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(steps):
        reset()
        graph.launch()
    torch.cuda.synchronize()
    ms_block = (time.perf_counter() - t1) * 1e3 / steps
    # the same block with the 256 MB MALL flushed before it (a 512 MB scratch
    # write, untimed): the cold figure
    stream = torch.cuda.current_stream()
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = []
    for _ in range(max(steps // 2, 3)):
        reset()
        flush.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        graph.launch()
        e1.record(stream)
        e1.synchronize()
        cold.append(e0.elapsed_time(e1))
    del flush
    ms_cold = float(np.median(cold))
    graph.close()
    ra = [mk(pr) for pr in per_round]
    times = [[] for _ in ra]
    for _ in range(3):
        reset()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(R + 1)]
        evs[0].record(stream)
        for i, a in enumerate(ra):
            api.dbd_round(a)
            evs[i + 1].record(stream)
        evs[-1].synchronize()
        for i in range(R):
            times[i].append(evs[i].elapsed_time(evs[i + 1]) * 1e3)
    round_us = [float(np.median(x)) for x in times]

    def ev_time(fn, it=10):
        for _ in range(2):
            fn()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        for _ in range(it):
            fn()
        e.record(stream)
        e.synchronize()
        return s.elapsed_time(e) * 1e3 / it

    r1 = per_round[0]
    t_attn = ev_time(lambda: api.dbd_attn_paged(r1["q"], r1["k_blk"], r1["v_blk"], fixed["k_cache"],
                                                fixed["v_cache"], fixed["page_table"], fixed["prefix_len"],
                                                attn_out, ws=bufs.workspace))
    lm_rows = torch.arange(n, dtype=torch.int32, device=dev)
    nr1 = torch.tensor([rows[0]], dtype=torch.int32, device=dev)
    t_lm = ev_time(lambda: api.dbd_lmhead_conf(r1["hidden"], fixed["w_vocab"], nr1, bufs.argmax_tok, bufs.conf,
                                               w.mask_id, row_index=lm_rows, max_rows=n, ws=bufs.workspace))
    conf_r = torch.rand(n, device=dev)
    arg_r = torch.zeros(n, dtype=torch.int32, device=dev)
    tk, ss = tok0.clone(), st0.clone()
    ri, nr2 = torch.zeros(n, dtype=torch.int32, device=dev), torch.zeros(1, dtype=torch.int32, device=dev)
    t_remask = ev_time(lambda: api.dbd_remask_commit(tk, ss, arg_r, conf_r, ri, nr2, w.mask_id, 2.0))
    tg_attn = graph_time(lambda: api.dbd_attn_paged(r1["q"], r1["k_blk"], r1["v_blk"], fixed["k_cache"],
                                                    fixed["v_cache"], fixed["page_table"], fixed["prefix_len"],
                                                    attn_out, ws=bufs.workspace))
    tg_remask = graph_time(lambda: api.dbd_remask_commit(tk, ss, arg_r, conf_r, ri, nr2, w.mask_id, 2.0))
    a_bytes = attn_bytes_of(w, fx.prefix_len)
    r_bytes = 20 * w.S * w.B + 2 * w.S
    lm_flops = 2.0 * rows[0] * w.Hd * w.V
    w_bytes = 2.0 * w.V * w.Hd
    ent = {"rounds": R, "rows_per_round": rows, "ms_per_block": round(ms_block, 4),
           "block_tokens_per_s": round(w.S * w.B * R / (ms_block * 1e-3), 1),
           "cold_ms_per_block": round(ms_cold, 4),
           "cold_block_tokens_per_s": round(w.S * w.B * R / (ms_cold * 1e-3), 1),
           "per_round_eager_us": [round(t, 1) for t in round_us],
           "attention_us": round(t_attn, 2), "attention_bytes": a_bytes,
           "attention_frac_hbm": round(a_bytes / (t_attn * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
           "attention_remask_frac_hbm": round((a_bytes + r_bytes) / ((tg_attn + tg_remask) * 1e-6) / 1e9
                                              / PEAK_HBM_GBS, 4),
           "attention_remask_graph_us": [round(tg_attn, 2), round(tg_remask, 2)],
           "lmhead_us_round1": round(t_lm, 2), "lmhead_rows_round1": rows[0],
           "lmhead_frac_mfma": round(lm_flops / (t_lm * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "lmhead_w_frac_hbm": round(w_bytes / (t_lm * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
           "remask_us": round(t_remask, 2)}
    log(f"{w.name}: {R} rounds (rows {rows[0]} -> {rows[-1]}), {ms_block:.3f} ms per block = "
        f"{ent['block_tokens_per_s']:.0f} block-tokens/s (cold {ms_cold:.3f} ms); attention {t_attn:.1f} us "
        f"({ent['attention_frac_hbm']:.1%} of HBM), LM head {t_lm:.1f} us at {rows[0]} rows "
        f"({ent['lmhead_frac_mfma']:.1%} of bf16 MFMA), remask {t_remask:.1f} us "
        f"[{time.time() - t0:.1f} s]")
    return ent


def cpu_single_thread(synth):
    """The oracle with one BLAS thread on the two small configurations: the
    tiny one as whole blocks, the SDAR-1.7B one round by round, each for a
    bounded time (baseline only)."""
    import numpy as np

    import oracle
    from block_diffusion_amd.workloads import SDAR_1P7B, TINY
    try:
        from threadpoolctl import threadpool_limits
    except Exception:
        return None
    res = {}
    with threadpool_limits(1):
        for w, budget in ((TINY, 3.0), (SDAR_1P7B, 10.0)):
            fx = synth.make_fixed(w)
            rins = [synth.make_round(w, r, fx.w_vocab) for r in range(1, w.rounds + 1)]
            toks, state = fx.block_tokens0, fx.seq_state0
            rounds, t0 = 0, time.perf_counter()
            while True:
                rin = rins[rounds % len(rins)]
                if rounds % len(rins) == 0:
                    toks, state = fx.block_tokens0, fx.seq_state0
                r = oracle.denoise_round(rin, fx, w.mask_id, w.tau, block_tokens=toks, seq_state=state)
                toks, state = r["tokens"], r["state"]
                rounds += 1
                dt = time.perf_counter() - t0
                if dt >= budget and rounds % len(rins) == 0 or dt >= 4 * budget:
                    break
            res[w.name] = {"value": round(w.S * w.B * rounds / dt, 3), "unit": "block-tokens/s",
                           "threads": 1, "rounds": rounds, "seconds": round(dt, 2)}
    return res


def only(args, w, api, fixed, r1, attn_out, bufs, tok0, st0):
    """One entry point alone on the round-1 inputs (all S*B rows masked, so
    the LM head projects S*B rows), for counter runs."""
    import torch
    dev = attn_out.device
    n = w.S * w.B
    if args.only == "attention":
        fn = lambda: api.dbd_attn_paged(r1["q"], r1["k_blk"], r1["v_blk"], fixed["k_cache"],
                                        fixed["v_cache"], fixed["page_table"], fixed["prefix_len"],
                                        attn_out, ws=bufs.workspace)
    elif args.only == "lmhead":
        rows = torch.arange(n, dtype=torch.int32, device=dev)
        nr = torch.tensor([n], dtype=torch.int32, device=dev)
        fn = lambda: api.dbd_lmhead_conf(r1["hidden"], fixed["w_vocab"], nr, bufs.argmax_tok,
                                         bufs.conf, w.mask_id, row_index=rows, max_rows=n,
                                         ws=bufs.workspace)
    elif args.only == "lmhead_round":
        rows = torch.arange(n, dtype=torch.int32, device=dev)
        nr = torch.tensor([n], dtype=torch.int32, device=dev)
        conf_r = torch.rand(n, device=dev)
        arg_r = torch.zeros(n, dtype=torch.int32, device=dev)
        tk, ss = tok0.clone(), st0.clone()
        ri = torch.zeros(n, dtype=torch.int32, device=dev)
        nr2 = torch.zeros(1, dtype=torch.int32, device=dev)
        us = lm_in_round(
            lambda: api.dbd_attn_paged(r1["q"], r1["k_blk"], r1["v_blk"], fixed["k_cache"], fixed["v_cache"],
                                       fixed["page_table"], fixed["prefix_len"], attn_out, ws=bufs.workspace),
            lambda: api.dbd_lmhead_conf(r1["hidden"], fixed["w_vocab"], nr, bufs.argmax_tok, bufs.conf,
                                        w.mask_id, row_index=rows, max_rows=n, ws=bufs.workspace),
            lambda: api.dbd_remask_commit(tk, ss, arg_r, conf_r, ri, nr2, w.mask_id, 2.0),
            args.warmup, args.steps)
        print(json.dumps({"only": args.only, "workload": w.name, "rows": n, "launches": args.steps,
                          "us_per_launch": round(us, 2)}), flush=True)
        return
    elif args.only in ("logits", "filtered"):
        rows = torch.arange(n, dtype=torch.int32, device=dev)
        nr = torch.tensor([n], dtype=torch.int32, device=dev)
        lg = torch.empty((n, w.V), dtype=torch.float32, device=dev)
        api.dbd_lmhead_logits(r1["hidden"], fixed["w_vocab"], nr, lg, w.mask_id, row_index=rows, max_rows=n)
        if args.only == "logits":
            fn = lambda: api.dbd_lmhead_logits(r1["hidden"], fixed["w_vocab"], nr, lg, w.mask_id,
                                               row_index=rows, max_rows=n)
        else:
            fn = lambda: api.dbd_sample_filtered(lg, nr, bufs.argmax_tok, bufs.conf, w.mask_id, 0.6, 0,
                                                 0.95, 1234, 1, row_index=rows, max_rows=n)
    elif args.only == "prefill":
        import numpy as np
        Lp = fixed["prefix_len"].cpu().numpy().astype(np.int64)
        cu = torch.from_numpy(np.concatenate([[0], np.cumsum(Lp)]).astype(np.int32)).to(dev)
        Tp = int(Lp.sum())
        gen = torch.Generator(device=dev).manual_seed(4321)
        qp = torch.randn((Tp, w.Hq, w.D), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        kp = torch.randn((Tp, w.Hkv, w.D), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        vp = torch.randn((Tp, w.Hkv, w.D), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        op = torch.empty_like(qp)
        kc_p, vc_p = torch.empty_like(fixed["k_cache"]), torch.empty_like(fixed["v_cache"])
        pf_ws = api.workspace(api.lib().dbd_prefill_workspace_size(w.S), dev)
        fn = lambda: api.dbd_prefill_attn(qp, kp, vp, cu, op, w.B, page_table=fixed["page_table"],
                                          k_cache=kc_p, v_cache=vc_p, ws=pf_ws)
    else:
        conf_r = torch.rand(n, device=dev)
        arg_r = torch.zeros(n, dtype=torch.int32, device=dev)
        tk, ss = tok0.clone(), st0.clone()
        ri = torch.zeros(n, dtype=torch.int32, device=dev)
        nr2 = torch.zeros(1, dtype=torch.int32, device=dev)
        fn = lambda: api.dbd_remask_commit(tk, ss, arg_r, conf_r, ri, nr2, w.mask_id, 2.0)
    for _ in range(args.warmup):
        fn()
    stream = torch.cuda.current_stream()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record(stream)
    for _ in range(args.steps):
        fn()
    e.record(stream)
    e.synchronize()
    print(json.dumps({"only": args.only, "workload": w.name, "rows": n, "launches": args.steps,
                      "us_per_launch": round(s.elapsed_time(e) * 1e3 / args.steps, 2)}), flush=True)


def cpu_baseline(w, fx, rins, min_seconds):
    """The oracle, as it stands, on the same job: whole blocks (every round
    of every sequence: float64 attention over all heads, the full-vocabulary
    LM head on the masked rows, the remask), repeated until at least
    min_seconds have passed; value in the same unit as the GPU figure."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = None
    cores = len(os.sched_getaffinity(0))
    blocks = 0
    t0 = time.perf_counter()
    while True:
        toks, state = fx.block_tokens0, fx.seq_state0
        for rin in rins:
            r = oracle.denoise_round(rin, fx, w.mask_id, w.tau, block_tokens=toks, seq_state=state)
            toks, state = r["tokens"], r["state"]
        blocks += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    n_tok = w.S * w.B * len(rins) * blocks
    return {"value": round(n_tok / dt, 3), "unit": "block-tokens/s",
            "cores": blas_threads if blas_threads else cores, "kind": "oracle",
            "sample": f"{blocks} whole block(s) of the same workload ({len(rins)} rounds x {w.S} "
                      f"sequences x {w.B} positions = {n_tok} block tokens): float64 attention "
                      f"over every head, full-vocabulary LM head on the masked rows, remask; "
                      f"{dt:.1f} s on {cores} host cores (BLAS threads {blas_threads})"}


if __name__ == "__main__":
    main()
