"""The CPU oracle against its pins (brute force, closed forms, library
special cases, invariants, hand-worked fixtures)."""
import pytest

import oracle
from pins import (ATTN_CHECKS, LM_CHECKS, REMASK_CHECKS, ROUND_CHECKS, RULE_CHECKS, SAVE_CHECKS, SAMPLE_CHECKS,
                  PREFILL_CHECKS)


@pytest.mark.parametrize("check", ATTN_CHECKS, ids=lambda f: f.__name__)
def test_attention_pins(check):
    check(oracle)


@pytest.mark.parametrize("check", LM_CHECKS, ids=lambda f: f.__name__)
def test_lmhead_pins(check):
    check(oracle)


@pytest.mark.parametrize("check", REMASK_CHECKS, ids=lambda f: f.__name__)
def test_remask_pins(check):
    check(oracle)


@pytest.mark.parametrize("check", RULE_CHECKS, ids=lambda f: f.__name__)
def test_rule_pins(check):
    check(oracle)


@pytest.mark.parametrize("check", ROUND_CHECKS, ids=lambda f: f.__name__)
def test_round_pins(check):
    check(oracle)


@pytest.mark.parametrize("check", SAVE_CHECKS, ids=lambda f: f.__name__)
def test_saving_step_pins(check):
    check(oracle)


@pytest.mark.parametrize("check", SAMPLE_CHECKS, ids=lambda f: f.__name__)
def test_sampling_pins(check):
    check(oracle)


@pytest.mark.parametrize("check", PREFILL_CHECKS, ids=lambda f: f.__name__)
def test_prefill_pins(check):
    check(oracle)


def test_round_on_tiny_workload():
    """Whole rounds of the tiny workload through the oracle: the block fills
    within its round cap; each round commits at least one masked position
    per DENOISING sequence, never re-masks a committed one, and moves a
    sequence to SAVING exactly when its block holds no mask."""
    import numpy as np
    from block_diffusion_amd import synth
    from block_diffusion_amd.workloads import TINY
    f = synth.make_fixed(TINY)
    toks, state = f.block_tokens0, f.seq_state0
    for r in range(1, TINY.rounds + 1):
        inp = synth.make_round(TINY, r, f.w_vocab)
        res = oracle.denoise_round(inp, f, TINY.mask_id, TINY.tau, block_tokens=toks, seq_state=state)
        assert np.all(np.isfinite(res["attn"]))
        masked_before = (toks == TINY.mask_id).sum(1)
        masked_after = (res["tokens"] == TINY.mask_id).sum(1)
        den = state == oracle.DENOISING
        assert np.all(masked_after[den & (masked_before > 0)] < masked_before[den & (masked_before > 0)])
        assert np.all(res["committed"].sum(1)[den & (masked_before > 0)] >= 1)
        kept = toks != TINY.mask_id                      # committed tokens are never re-masked or changed
        assert np.array_equal(res["tokens"][kept], toks[kept])
        assert np.array_equal(res["state"][den] == oracle.SAVING, masked_after[den] == 0)
        assert np.all(res["p1"][res["rows"]] > 0) and np.all(res["p1"][res["rows"]] <= 1)
        toks, state = res["tokens"], res["state"]
        if not np.any(state == oracle.DENOISING):
            break
    assert np.all(state == oracle.SAVING)
