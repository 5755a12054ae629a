"""dbd_round_noalloc (the round with the library's static scratch as its
workspace) against dbd_round with a caller workspace: bit-identical outputs
on two calls in a row, the second with a smaller input, greedy and with
top-p filtered sampling; and the host-side rejection of a round whose
workspace exceeds the scratch."""
import numpy as np
import pytest
import torch

from block_diffusion_amd import api, synth
from block_diffusion_amd.workloads import SDAR_1P7B, SDAR_8B, TINY
from gpu_util import RoundState, round_inputs_dev

pytestmark = pytest.mark.gpu


def _one(w, fx, rnd, noalloc, filtered=False):
    """One round of workload w from its initial state; returns every output.
    filtered: temperature 0.7, top_p 0.9 (stored logits, filtered draw)."""
    st = RoundState(w, fx)
    st.init_rows()
    attn_out = torch.full((w.S, w.B, w.Hq, w.D), float("nan"), dtype=torch.bfloat16, device="cuda")
    args = st.args(round_inputs_dev(synth.make_round(w, rnd, fx.w_vocab)), attn_out)
    logits = None
    if filtered:
        logits = torch.full((w.S * w.B, w.V), float("nan"), dtype=torch.float32, device="cuda")
        args.sample, args.temperature, args.seed, args.step = 1, 0.7, 0xA110C + rnd, rnd
        args.filter, args.top_k, args.top_p, args.logits = 1, 0, 0.9, logits.data_ptr()
    if noalloc:
        # the workspace fields must not be read: point them at nothing
        args.workspace = None
        args.workspace_bytes = 0
        api.dbd_round_noalloc(args)
    else:
        api.dbd_round(args)
    torch.cuda.synchronize()
    b = st.bufs
    n = int(b.num_rows.item())
    return dict(attn=attn_out.view(torch.int16).cpu().numpy(), tok=b.argmax_tok.cpu().numpy(),
                conf=b.conf.cpu().numpy(), block=b.block_tokens.cpu().numpy(),
                state=b.seq_state.cpu().numpy(), rows=b.row_index.cpu().numpy()[:n], n=n)


def _same(x, y):
    for k in x:
        assert np.array_equal(x[k], y[k], equal_nan=True), k


def test_noalloc_matches_round_twice():
    """The SDAR-1.7B shapes (17.0 MiB of workspace), then the tiny workload
    (8.3 MiB): each equal bit for bit to dbd_round on the same inputs; the
    second call finds the first call's data in the scratch."""
    for w, rnd in ((SDAR_1P7B, 1), (TINY, 2)):
        fx = synth.make_fixed(w)
        ref = _one(w, fx, rnd, noalloc=False)
        got = _one(w, fx, rnd, noalloc=True)
        _same(ref, got)
        assert got["n"] <= w.S * (w.B - 1)      # every sequence committed
        print(f"{w.name} round {rnd}: equal, {got['n']} rows left", flush=True)


def test_noalloc_filtered_matches_round():
    """Rounds with top-p filtered sampling (the LM head stores the logits and
    the filtered draw reads the row maxima it leaves in the workspace):
    the SDAR-1.7B shapes, then the tiny workload, each equal bit for bit to
    dbd_round."""
    for w, rnd in ((SDAR_1P7B, 2), (TINY, 1)):
        fx = synth.make_fixed(w)
        ref = _one(w, fx, rnd, noalloc=False, filtered=True)
        got = _one(w, fx, rnd, noalloc=True, filtered=True)
        _same(ref, got)
        assert got["n"] <= w.S * (w.B - 1)      # every sequence committed
        print(f"{w.name} round {rnd} filtered: equal, {got['n']} rows left", flush=True)


def test_noalloc_rejects_beyond_scratch():
    """The SDAR-8B shapes need 71.0 MiB of workspace: rejected with
    DBD_ERR_WORKSPACE before anything is enqueued."""
    w = SDAR_8B
    n = w.S * w.B
    d = lambda *shape, dt=torch.int32: torch.zeros(shape, dtype=dt, device="cuda")
    bufs = api.RoundBuffers(row_index=d(n), num_rows=d(1), argmax_tok=d(n),
                            conf=d(n, dt=torch.float32), block_tokens=d(w.S, w.B),
                            seq_state=d(w.S, dt=torch.uint8), num_committed=d(w.S),
                            workspace=d(1, dt=torch.uint8))
    bf = lambda *shape: torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    args = api.make_round_args(
        S=w.S, B=w.B, Hq=w.Hq, Hkv=w.Hkv, D=w.D, page_size=w.P, max_pages_per_seq=w.max_pages,
        Hd=w.Hd, V=w.V, mask_token_id=w.mask_id, dynamic_threshold=w.tau, bufs=bufs,
        q=bf(w.S, w.B, w.Hq, w.D), k_blk=bf(w.S, w.B, w.Hkv, w.D), v_blk=bf(w.S, w.B, w.Hkv, w.D),
        k_cache=bf(1, w.Hkv, w.P, w.D), v_cache=bf(1, w.Hkv, w.P, w.D), page_table=d(w.S, w.max_pages),
        prefix_len=d(w.S), attn_out=bf(w.S, w.B, w.Hq, w.D), hidden=bf(n, w.Hd), w_vocab=bf(8, w.Hd))
    assert api.dbd_round_workspace_size(args) > api.NOALLOC_SCRATCH_BYTES
    with pytest.raises(api.DbdError) as e:
        api.dbd_round_noalloc(args)
    assert e.value.status == api.DBD_ERR_WORKSPACE and "static scratch" in str(e.value)
