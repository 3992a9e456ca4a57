"""Seeded normal draws and their encoding into storage dtypes."""
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
import os

import numpy as np

from .formats import DT_F32, DT_BF16, DT_E4M3, bf16_bits, e4m3_encode, e4m3_scale

CHUNK = 1 << 22          # elements per independently seeded chunk


def _draw_chunk(config_id, seed, tensor_id, c, n, std):
    rng = np.random.default_rng(np.random.SeedSequence([config_id, seed, tensor_id, c]))
    out = rng.standard_normal(n, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def normal(config_id, seed, tensor_id, shape, std=1.0, threads=None):
    """fp32 draws ~ N(0, std^2) of the given shape (chunked, seeded)."""
    total = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(total, dtype=np.float32)
    nchunks = (total + CHUNK - 1) // CHUNK

    def work(c):
        lo = c * CHUNK
        n = min(CHUNK, total - lo)
        out[lo:lo + n] = _draw_chunk(config_id, seed, tensor_id, c, n, std)

    if nchunks <= 1:
        for c in range(nchunks):
            work(c)
    else:
        nt = threads or min(16, len(os.sched_getaffinity(0)))
        with ThreadPoolExecutor(max_workers=nt) as ex:
            list(ex.map(work, range(nchunks)))
    return out.reshape(shape)


@dataclass
class Tensor:
    """A stored input: raw bytes in `dt` (uint16 bits for bf16, uint8 codes
    for e4m3, float32 for fp32) plus the per-tensor scale for e4m3."""
    raw: np.ndarray
    dt: int
    scale: float = 1.0

    @property
    def shape(self):
        return self.raw.shape


def encode(values, dt):
    """fp32 values -> Tensor in storage dtype `dt`."""
    if dt == DT_F32:
        return Tensor(np.ascontiguousarray(values, dtype=np.float32), dt)
    if dt == DT_BF16:
        return Tensor(bf16_bits(values), dt)
    if dt == DT_E4M3:
        s = e4m3_scale(values)
        return Tensor(e4m3_encode(values, s), dt, s)
    raise ValueError(f"unknown dtype code {dt}")
