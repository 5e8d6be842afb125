"""ReplaySSM decode hot path for AMD MI355X (gfx950): C ABI ``librssm.so`` over
hand-written HIP kernels, with a ctypes binding of the same names.

Checkpoint + ring representation of Mamba-2 and Gated DeltaNet state: replay
decode with a fused flush, standalone flush, output-only speculative verify,
pointer commit, a low-precision read copy, and a conventional
read-modify-write comparator.
"""
from . import rssm
from .rssm import (
    rssm_config, rssm_state, rssm_buffer_sizes, RssmError,
    rssm_check_config, rssm_sizes, rssm_ring_offsets, rssm_init_state, rssm_decode_step,
    rssm_flush, rssm_verify, rssm_commit, rssm_decode_step_conventional, rssm_get_error,
    rssm_verify_snapshot, rssm_commit_snapshot, rssm_verify_tree, rssm_commit_tree, rssm_verify_fold,
    rssm_stream_copy, rssm_strerror, rssm_version,
)

__all__ = [
    "rssm", "rssm_config", "rssm_state", "rssm_buffer_sizes", "RssmError",
    "rssm_check_config", "rssm_sizes", "rssm_ring_offsets", "rssm_init_state", "rssm_decode_step",
    "rssm_flush", "rssm_verify", "rssm_commit", "rssm_decode_step_conventional", "rssm_get_error",
    "rssm_verify_snapshot", "rssm_commit_snapshot", "rssm_verify_tree", "rssm_commit_tree", "rssm_verify_fold",
    "rssm_stream_copy", "rssm_strerror", "rssm_version",
]
