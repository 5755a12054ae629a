"""Denoise-round workloads: the shapes of the block-diffusion models the
JetEngine README, the JetEngine developer notes (CLAUDE.md) and the SDAR
model page run, as frozen records.

Nothing here computes anything; it only names shapes.  Readings that the
pages leave open (mask id where unstated, amplitude range, round caps) are
fixed here: the mask id of the model family's tokenizer where a shape names
none, planted amplitudes up to 12 or 16 by shape (16 for the coverage
variants, so that confidences cross the threshold at full vocabulary), and
a round cap of one block's length.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

# Sequence states in the order the JetEngine developer notes give for the
# scheduler (Scheduler section: WAITING -> PREFILLING -> DENOISING -> SAVING
# -> FINISHED).  Only DENOISING and SAVING are touched by a denoise round.
WAITING, PREFILLING, DENOISING, SAVING, FINISHED = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class Workload:
    name: str
    seed_id: int          # seed component; keys every random stream
    S: int                # sequences in the batch
    B: int                # block_length
    Hq: int               # query heads
    Hkv: int              # key/value heads (GQA groups of Hq/Hkv)
    D: int                # head dim
    P: int                # KV page size (tokens per page)
    Hd: int               # hidden size
    V: int                # vocabulary size
    mask_id: int          # mask_token_id
    prefix_lo: int        # prefix lengths U{lo..hi}; lo == hi with
    prefix_hi: int        #   prefix_fixed set for the tiny case
    tau: float            # dynamic_threshold
    rounds: int           # round cap
    a_max: float          # planted-logit amplitude a ~ U[0, a_max]
    init_committed_max: int = 0   # >0: U{0..k} positions pre-committed
    prefix_fixed: tuple = ()      # explicit per-sequence prefix lengths

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def max_pages(self) -> int:
        hi = max(self.prefix_fixed) if self.prefix_fixed else self.prefix_hi
        return max(1, -(-hi // self.P))

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


TINY = Workload(
    name="tiny_s2_b4_h4x2_d64", seed_id=0, S=2, B=4, Hq=4, Hkv=2, D=64, P=16,
    Hd=256, V=1024, mask_id=1023, prefix_lo=16, prefix_hi=37, tau=0.9,
    rounds=4, a_max=12.0, prefix_fixed=(16, 37))

SDAR_1P7B = Workload(
    name="sdar1.7b_b4_bs32", seed_id=1, S=32, B=4, Hq=16, Hkv=8, D=128,
    P=256, Hd=2048, V=151936, mask_id=151669, prefix_lo=128, prefix_hi=2048,
    tau=0.9, rounds=4, a_max=16.0)

SDAR_4B = Workload(
    name="sdar4b_b4_bs128", seed_id=2, S=128, B=4, Hq=32, Hkv=8, D=128,
    P=256, Hd=2560, V=151936, mask_id=151669, prefix_lo=256, prefix_hi=4096,
    tau=0.9, rounds=4, a_max=12.0)

SDAR_8B = Workload(
    name="sdar8b_b16_bs64", seed_id=3, S=64, B=16, Hq=32, Hkv=8, D=128,
    P=256, Hd=4096, V=151936, mask_id=151669, prefix_lo=512, prefix_hi=8192,
    tau=0.75, rounds=16, a_max=12.0, init_committed_max=12)

LLADA_LONG = Workload(
    name="llada_b64_bs8_ctx32k", seed_id=4, S=8, B=64, Hq=32, Hkv=32, D=128,
    P=256, Hd=4096, V=126464, mask_id=126336, prefix_lo=16384,
    prefix_hi=32768, tau=0.9, rounds=64, a_max=16.0)

# Coverage variant of the SDAR-4B shapes with a ~ U[0,16]: at V=151936 the
# literal a <= 12 almost never reaches 0.9, so every commit is a fallback;
# this variant exercises the threshold branch at full vocabulary.
SDAR_4B_HIGHCONF = SDAR_4B.with_(name="sdar4b_b4_bs128_a16", a_max=16.0)

# The same coverage variant of the SDAR-8B shapes (block 16, threshold 0.75):
# with a <= 12 no position reaches 0.75 either.
SDAR_8B_HIGHCONF = SDAR_8B.with_(name="sdar8b_b16_bs64_a16", a_max=16.0)

ALL = (TINY, SDAR_1P7B, SDAR_4B, SDAR_8B, LLADA_LONG)
BY_NAME = {w.name: w for w in ALL + (SDAR_4B_HIGHCONF, SDAR_8B_HIGHCONF)}
