"""Helpers for the GPU parity tests (host <-> device marshalling, error metric)."""
from __future__ import annotations

import numpy as np
import torch

from looped_transformer_latent_amd import gen, lla
from looped_transformer_latent_amd.workloads import to_device, to_host  # noqa: F401


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per output row (last axis): ||got - ref||_inf / max(||ref||_inf, 1e-6)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.abs(got - ref).max(axis=-1)
    den = np.maximum(np.abs(ref).max(axis=-1), 1e-6)
    return num / den


def out_to_f64(t: torch.Tensor) -> np.ndarray:
    return gen.storage_to_f64(to_host(t))


def device_codec(codec_host: dict, device="cuda"):
    d = {k: to_device(v, device) for k, v in codec_host.items()}
    c = lla.make_codec(d["mu_k"], d["mu_v"], d["w_down_k"], d["w_down_v"], d["w_up_k"], d["w_up_v"])
    return c, d  # keep the tensors alive alongside the struct
