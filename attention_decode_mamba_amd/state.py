"""Device buffers of an ``rssm_state``, allocated with torch (memory plumbing only)."""
from __future__ import annotations

from typing import Optional

import torch

from . import rssm as R

_KIND = {"mamba2": R.RSSM_KIND_MAMBA2, "gdn": R.RSSM_KIND_GDN, "kda": R.RSSM_KIND_KDA}
_DTYPE = {"fp32": R.RSSM_DTYPE_F32, "bf16": R.RSSM_DTYPE_BF16}
_READ = {"none": R.RSSM_READ_NONE, "fp8": R.RSSM_READ_FP8, "mxfp4": R.RSSM_READ_MXFP4}


def make_config(kind: str, batch: int, n_heads: int, n_qk_heads: int, dv: int, dk: int, L: int,
                t_max: int, capacity: int, in_dtype: str, read_copy: str = "none") -> R.rssm_config:
    return R.rssm_config(_KIND[kind], batch, n_heads, n_qk_heads, dv, dk, L, t_max, capacity,
                         _DTYPE[in_dtype], _READ[read_copy])


def config_of(obj) -> R.rssm_config:
    """Config from any object with the config's field names (kind/in_dtype/read_copy as strings)."""
    return make_config(obj.kind, obj.batch, obj.n_heads, obj.n_qk_heads, obj.dv, obj.dk, obj.L,
                       obj.t_max, obj.capacity, obj.in_dtype, obj.read_copy)


class DeviceState:
    """Caller-owned buffers of one state, sized by ``rssm_sizes``."""

    def __init__(self, cfg: R.rssm_config, device: str = "cuda"):
        self.cfg = cfg
        sz = R.rssm_sizes(cfg)
        self.sizes = sz
        dev = torch.device(device)
        tiles = cfg.batch * cfg.n_heads
        self.s_ckpt = torch.empty(max(sz.s_ckpt // 4, 1), dtype=torch.float32, device=dev)
        self.s_read = torch.empty(sz.s_read, dtype=torch.uint8, device=dev) if sz.s_read else None
        self.s_read_scale = (torch.empty(sz.s_read_scale, dtype=torch.uint8, device=dev)
                             if sz.s_read_scale else None)
        self.ring = torch.zeros(max(sz.ring, 256), dtype=torch.uint8, device=dev)
        self.n_committed = torch.zeros(max(tiles, 1), dtype=torch.int64, device=dev)
        self.n_ckpt = torch.zeros(max(tiles, 1), dtype=torch.int64, device=dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        self.st = R.rssm_state(
            self.s_ckpt.data_ptr(),
            self.s_read.data_ptr() if self.s_read is not None else None,
            self.s_read_scale.data_ptr() if self.s_read_scale is not None else None,
            self.ring.data_ptr(), self.n_committed.data_ptr(), self.n_ckpt.data_ptr(),
            self.err.data_ptr())

    def tiles(self):
        c = self.cfg
        return c.batch, c.n_heads

    def ckpt(self) -> torch.Tensor:
        c = self.cfg
        return self.s_ckpt[: c.batch * c.n_heads * c.dv * c.dk].view(c.batch, c.n_heads, c.dv, c.dk)

    def counters(self):
        B, H = self.tiles()
        return (self.n_committed[: B * H].view(B, H), self.n_ckpt[: B * H].view(B, H))

    def ring_arrays(self):
        """Typed views of the ring regions, indexed [b, head, slot, ...]: alpha [B,H,C] (KDA
        [B,H,C,N]), beta (GDN, KDA) [B,H,C], v [B,H,C,P], k, q [B,G,C,N].  The ring stores
        every region slot-major ([C][B][H]...), so these are permuted views of it."""
        c = self.cfg
        off = R.rssm_ring_offsets(c)
        es = 2 if c.in_dtype == R.RSSM_DTYPE_BF16 else 4
        dt = torch.int16 if es == 2 else torch.float32
        B, H, G, C, P, N = c.batch, c.n_heads, c.n_qk_heads, c.capacity, c.dv, c.dk

        def view(o, shape):
            n = 1
            for d in shape:
                n *= d
            t = self.ring[o: o + n * es].view(dt).view(*shape)          # [C][rows][...]
            return t.permute(1, 2, 0, *range(3, len(shape)))
        kda = c.kind == R.RSSM_KIND_KDA
        out = {"alpha": view(off[0], (C, B, H, N)) if kda else view(off[0], (C, B, H)),
               "v": view(off[2], (C, B, H, P)),
               "k": view(off[3], (C, B, G, N)),
               "q": view(off[4], (C, B, G, N))}
        out["beta"] = view(off[1], (C, B, H)) if c.kind != R.RSSM_KIND_MAMBA2 else None
        return out

    def read_copy(self):
        c = self.cfg
        B, H, P, N = c.batch, c.n_heads, c.dv, c.dk
        if c.read_copy == R.RSSM_READ_FP8:
            return (self.s_read.view(B, H, P, N),
                    self.s_read_scale.view(torch.float32).view(B, H, P, N // 32))
        if c.read_copy == R.RSSM_READ_MXFP4:
            return self.s_read.view(B, H, P, N // 2), self.s_read_scale.view(B, H, P, N // 32)
        return None

    def init(self, s0: Optional[torch.Tensor] = None, stream=0):
        R.rssm_init_state(self.cfg, self.st, s0.data_ptr() if s0 is not None else None, stream)

    def error(self, stream=0) -> int:
        return R.rssm_get_error(self.st, stream)
