"""CPU oracle for one denoise round of block-diffusion decoding.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import this package; the GPU product
path never calls it and has no fallback to it.

Plain, slow, float64 numpy written from the pages' description of the
round (JetEngine README: "Block Diffusion Decoding", "Selective Logits";
JetEngine developer notes (CLAUDE.md): "Remasking Strategies",
"Scheduler", "ModelRunner"; dlmrt README: "Highlights" on rounds run on
the device; developer notes, "Important Patterns" and "Sequence" on the
SAVING forward and the block commit).  It shares no code with the HIP path: it decodes bf16 bit
patterns itself and reads nothing from ``block_diffusion_amd``.

Every function is pinned by CPU tests against brute force, closed forms,
library special cases and invariants (tests/test_oracle_*.py); no function
here is "parity unpinned".
"""
from .bf16 import widen
from .attention import attention, attention_group
from .lmhead import lmhead_rows, lmhead_logits, lmhead_entropy
from .remask import (remask, remask_rule, compact_rows, DENOISING, SAVING,
                     RULE_DYNAMIC, RULE_STATIC, RULE_SEQUENTIAL, RULE_ENTROPY)
from .round import denoise_round
from .block_commit import kv_save, commit_block, step_commit, FINISHED
from .sampling import (philox4x32_10, uniform01, sample_row, lmhead_sample, topk_topp_keep,
                       sample_filtered)
from .prefill import prefill_attention, prefill_store

__all__ = ["widen", "attention", "attention_group", "lmhead_rows",
           "lmhead_logits", "lmhead_entropy", "remask", "remask_rule",
           "compact_rows", "denoise_round", "DENOISING", "SAVING",
           "RULE_DYNAMIC", "RULE_STATIC", "RULE_SEQUENTIAL", "RULE_ENTROPY",
           "kv_save", "commit_block", "step_commit", "FINISHED",
           "philox4x32_10", "uniform01", "sample_row", "lmhead_sample",
           "topk_topp_keep", "sample_filtered",
           "prefill_attention", "prefill_store"]
