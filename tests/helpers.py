"""Shared helpers for the GPU parity tests (device transfers, tolerances)."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

# Max-abs-error bounds against the fp64 oracle: fp16 2e-3 and bf16 1e-2 are
# the stated targets; fp32 1e-5 is derived (fp32 accumulation over at most a
# few hundred positions of N(0,1) data stays below 1e-6).
TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 1e-2}
TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
# spacing of representable numbers just above 1.0
EPS = {"f32": 2.0 ** -23, "f16": 2.0 ** -10, "bf16": 2.0 ** -7}


def note(msg: str) -> None:
    """Name the case about to run on the GPU (flushed, so a crash shows it)."""
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def to_dev(arr: np.ndarray, dtype: str | None = None) -> torch.Tensor:
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16))
        return t.view(torch.bfloat16).to("cuda")
    return torch.from_numpy(np.ascontiguousarray(arr)).to("cuda")


def from_dev(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def as_f64(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> exact float64 values."""
    if t.dtype == torch.bfloat16:
        return oracle.to_f64(from_dev(t), "bf16")
    return from_dev(t).astype(np.float64)


def rounding_bound(ref: np.ndarray, dtype: str) -> np.ndarray:
    """Half a unit in the last place of ``dtype`` at each reference value:
    the error the final round-to-nearest alone may add."""
    mag = np.maximum(np.abs(ref), np.finfo(np.float32).tiny)
    return 0.5 * EPS[dtype] * 2.0 ** np.floor(np.log2(mag))


class DeviceBatch:
    """A generated workload uploaded to the GPU."""

    def __init__(self, w, *, written: bool = False):
        c = w.cfg
        self.w = w
        self.dtype = c.dtype
        self.q = to_dev(w.q, c.dtype)
        self.k_pool = to_dev(w.k_pool, c.dtype)
        self.v_pool = to_dev(w.v_pool, c.dtype)
        self.key_new = to_dev(w.key_new, c.dtype)
        self.value_new = to_dev(w.value_new, c.dtype)
        self.block_table = to_dev(w.block_table)
        self.context_lens = to_dev(w.context_lens)
        self.slot_mapping = to_dev(w.slot_mapping)
        self.scale = w.scale
        self.partition_size = c.partition_size
        self.max_partitions = c.max_partitions

    def empty_out(self):
        return torch.full_like(self.q, float("nan"))


def oracle_pools_after_write(w):
    return oracle.oracle_cache_write(w.k_pool, w.v_pool, w.key_new,
                                     w.value_new, w.slot_mapping,
                                     w.cfg.block_size)


def oracle_out(w, k_pool, v_pool, rows=None):
    c = w.cfg
    return oracle.oracle_decode(w.q, k_pool, v_pool, w.block_table,
                                w.context_lens, w.scale, c.gqa_group,
                                c.block_size, c.dtype, rows=rows)
