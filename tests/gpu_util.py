"""GPU-side test helpers: build the device pools of a workload through the
library's own scatter and copy entry points, and compare with the oracle."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

import paged_kv_cache_342_amd as pa
from workloads.device import DeviceBatch as GpuBatch, POISON_BITS, TORCH_DT, new_pool, storage_to_torch, torch_to_bytes  # noqa: F401


def log(msg: str):
    print(msg, file=sys.stderr, flush=True)


def errors(gpu: np.ndarray, ref: np.ndarray):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    max_abs = float(np.max(np.abs(gpu - ref))) if gpu.size else 0.0
    den = float(np.sqrt((ref * ref).sum()))
    rel = float(np.sqrt(((gpu - ref) ** 2).sum())) / den if den else max_abs
    return max_abs, rel


def tolerance(cache_dtype: str):
    """Bounds of the decode parity gate: fp16/bf16 caches max-abs 2e-3 and
    relative L2 1e-3; fp8 caches max-abs 3e-2 (fp32 output against the fp64
    oracle over the same dequantised cache)."""
    return (3e-2, None) if cache_dtype == "fp8" else (2e-3, 1e-3)


def set_variant(v):
    if v is None:
        os.environ.pop("PA_DECODE_VARIANT", None)
    else:
        os.environ["PA_DECODE_VARIANT"] = v
