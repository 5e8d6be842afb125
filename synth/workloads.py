"""The synthetic workloads of the ReplaySSM decode path.

Shapes follow the pages' problem statement: a Mamba-2 layer whose FP32 state is
4 MiB per sequence (128 heads x 64 x 128 x 4 B; page "ReplaySSM caches SSM
inputs instead of state", section "What shipped"), a 16-record window (same
section), batch 256 for standard decode and batch 512 with T = 4 drafts for
speculative decoding (same page, evaluation paragraph), and a Gated DeltaNet
layer with two value heads per key/query head (same section, chunkwise-verify
paragraph).  The KDA layer (page 4 "Why it matters": the reframing carries over to
KDA's delta-rule update; not evaluated on the pages) takes the head shape of the
published Kimi Linear model: 32 heads of 128 x 128, one key/query head per value
head, with the Gated DeltaNet workload's batch, window and draft count.
"""
from __future__ import annotations

import dataclasses
from typing import Dict


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "mamba2", "gdn" or "kda"
    batch: int
    n_heads: int         # H, value heads
    n_qk_heads: int      # G, key/query heads (H % G == 0)
    dv: int              # P, rows of a state tile
    dk: int              # N, columns of a state tile (contiguous)
    in_dtype: str        # "fp32" or "bf16": alpha, beta, v, k, q and the ring
    L: int               # window (flush threshold)
    t_max: int           # max drafts per verify (1 = decode only)
    capacity: int        # ring slots C >= L + t_max - 1
    decode_steps: int
    verify_steps: int
    read_copy: str       # "none", "fp8", "mxfp4"
    seed: int
    s0: str = "normal"   # "normal": S0 ~ N(0, 0.1) (variance); "zero"

    @property
    def group(self) -> int:
        return self.n_heads // self.n_qk_heads

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


_BASE_SEED = 20261012

WORKLOADS: Dict[str, Workload] = {
    # tiny Mamba-2 replay decode: 64 steps = 4 flushes of a 16-record window
    "m2_tiny": Workload("m2_tiny", "mamba2", batch=2, n_heads=4, n_qk_heads=4,
                        dv=16, dk=32, in_dtype="fp32", L=16, t_max=1, capacity=16,
                        decode_steps=64, verify_steps=0, read_copy="none",
                        seed=_BASE_SEED + 0),
    # Mamba-2 standard decode at serving shape, 4 MiB fp32 state per sequence
    "m2_decode_b256": Workload("m2_decode_b256", "mamba2", batch=256, n_heads=128,
                               n_qk_heads=128, dv=64, dk=128, in_dtype="bf16", L=16,
                               t_max=1, capacity=16, decode_steps=256, verify_steps=0,
                               read_copy="none", seed=_BASE_SEED + 1),
    # Mamba-2 speculative verify: T = 4 drafts per step, accepted prefix ~ U{0..4}
    "m2_verify_b512": Workload("m2_verify_b512", "mamba2", batch=512, n_heads=128,
                               n_qk_heads=128, dv=64, dk=128, in_dtype="bf16", L=16,
                               t_max=4, capacity=19, decode_steps=0, verify_steps=128,
                               read_copy="none", seed=_BASE_SEED + 2),
    # Gated DeltaNet decode then verify: 32 value heads sharing 16 key/query heads
    "gdn_b256": Workload("gdn_b256", "gdn", batch=256, n_heads=32, n_qk_heads=16,
                         dv=128, dk=128, in_dtype="bf16", L=16, t_max=4, capacity=19,
                         decode_steps=256, verify_steps=256, read_copy="none",
                         seed=_BASE_SEED + 3),
    # Kimi Delta Attention: per-key-channel gates, 32 heads of 128 x 128, decode then verify
    "kda_b256": Workload("kda_b256", "kda", batch=256, n_heads=32, n_qk_heads=32,
                         dv=128, dk=128, in_dtype="bf16", L=16, t_max=4, capacity=19,
                         decode_steps=256, verify_steps=256, read_copy="none",
                         seed=_BASE_SEED + 5),
    # low-precision read copy of the fp32 checkpoint (fp8 e4m3; MXFP4 variant)
    "m2_readcopy_b256": Workload("m2_readcopy_b256", "mamba2", batch=256, n_heads=128,
                                 n_qk_heads=128, dv=64, dk=128, in_dtype="bf16", L=16,
                                 t_max=1, capacity=16, decode_steps=4096, verify_steps=0,
                                 read_copy="fp8", seed=_BASE_SEED + 4),
}


def get_workload(name: str, **overrides) -> Workload:
    wl = WORKLOADS[name]
    return wl.replace(**overrides) if overrides else wl
