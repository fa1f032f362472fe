"""Host-side input recipes for the tests (seeded; numpy only).

The SVD codec below is the initialisation recipe of the close reading
(cc.laoqi.cc, 方法 item 4): collect loop-concatenated activations, centre them,
take the top-r right singular vectors as W_down, and use its loop slices as the
initial W_up,t.  It builds *inputs*; it is not part of the attention path.
"""
from __future__ import annotations

import numpy as np

from looped_transformer_latent_amd import gen

F32, BF16 = 0, 1
PER_HEAD, TWO_D = 0, 1


def dims(T, D, H, d_head, r_k, r_v, variant=PER_HEAD, dtype=BF16, page_size=16, rope_base=10000.0):
    return dict(T=T, D=D, H=H, d_head=d_head, r_k=r_k, r_v=r_v, variant=variant, dtype=dtype,
                page_size=page_size, rope_base=rope_base)


def store(x: np.ndarray, dtype: int) -> np.ndarray:
    """float array -> storage array (fp32 values, or bf16 bits with RNE)."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    return x32 if dtype == F32 else gen.f32_to_bf16_bits(x32)


def f64(a: np.ndarray) -> np.ndarray:
    return gen.storage_to_f64(a)


def param_shapes(m: dict) -> dict:
    T, D, H, d, rk, rv = m["T"], m["D"], m["H"], m["d_head"], m["r_k"], m["r_v"]
    if m["variant"] == PER_HEAD:
        return dict(mu_k=(D, H, T, d), mu_v=(D, H, T, d), w_down_k=(D, H, T * d, rk),
                    w_down_v=(D, H, T * d, rv), w_up_k=(D, H, T, d, rk), w_up_v=(D, H, T, d, rv))
    return dict(mu_k=(D, T, H, d), mu_v=(D, T, H, d), w_down_k=(D, T * H * d, rk),
                w_down_v=(D, T * H * d, rv), w_up_k=(D, T, H, d, rk), w_up_v=(D, T, H, d, rv))


def pool_shape(m: dict, num_pages: int, kv: str) -> tuple:
    r = m["r_k"] if kv == "k" else m["r_v"]
    if m["variant"] == PER_HEAD:
        return (m["D"], num_pages, m["H"], m["page_size"], r)
    return (m["D"], num_pages, m["page_size"], r)


def random_codec(m: dict, seed: int, ortho_down: bool = True) -> dict:
    """mu_t, W_up,t ~ N(0,1)/sqrt(r) (r of the K or V side); W_down orthonormal
    columns (QR of a seeded Gaussian) or Gaussian / sqrt(width)."""
    dt = "bf16" if m["dtype"] == BF16 else "f32"
    sh = param_shapes(m)
    out = {}
    for i, name in enumerate(["mu_k", "mu_v", "w_up_k", "w_up_v"]):
        r = m["r_k"] if name.endswith("k") else m["r_v"]
        out[name] = gen.normal(seed, 101 + i, sh[name], scale=1.0 / np.sqrt(r), dtype=dt)
    for i, name in enumerate(["w_down_k", "w_down_v"]):
        shape = sh[name]
        g = gen.normal_f32(seed, 111 + i, int(np.prod(shape))).reshape(shape).astype(np.float64)
        if ortho_down and shape[-2] >= shape[-1]:
            flat = g.reshape(-1, shape[-2], shape[-1])
            qs = np.stack([np.linalg.qr(x)[0] for x in flat])
            g = qs.reshape(shape)
        else:
            g = g / np.sqrt(shape[-2])
        out[name] = store(g, m["dtype"])
    return out


def random_pools(m: dict, num_pages: int, seed: int, scale: float = 1.0):
    dt = "bf16" if m["dtype"] == BF16 else "f32"
    k = gen.normal(seed, 201, pool_shape(m, num_pages, "k"), scale=scale, dtype=dt)
    v = gen.normal(seed, 202, pool_shape(m, num_pages, "v"), scale=scale, dtype=dt)
    return k, v


def rank8_activations(seed: int, stream: int, n_tok: int, width: int, rank: int = 8,
                      noise: float = 0.05, offset_scale: float = 0.5, draw: int = 0) -> np.ndarray:
    """x = z A + noise * eps + offset: a rank-`rank` Gaussian signal plus noise
    (the tiny fp32 workload), with a fixed non-zero mean so that mu matters.
    A and the offset depend on (seed, stream) only; `draw` selects fresh z and eps
    (draw 0 = calibration set, draw 1 = fresh tokens)."""
    A = gen.normal_f32(seed, stream, rank * width).reshape(rank, width).astype(np.float64) / np.sqrt(rank)
    off = offset_scale * gen.normal_f32(seed, stream + 1, width).astype(np.float64)
    base = np.uint64(draw) << np.uint64(40)
    z = gen.normal_f32(seed, stream + 2, base + np.arange(n_tok * rank, dtype=np.uint64))
    eps = gen.normal_f32(seed, stream + 3, base + np.arange(n_tok * width, dtype=np.uint64))
    z = z.reshape(n_tok, rank).astype(np.float64)
    eps = eps.reshape(n_tok, width).astype(np.float64)
    return z @ A + noise * eps + off


def svd_codec_one(calib: np.ndarray, r: int, T: int, d: int):
    """SVD initialisation for one (layer, head, K|V): returns
    mu [T*d], W_down [T*d][r], W_up [T][d][r] (float64)."""
    mu = calib.mean(axis=0)
    _, _, vt = np.linalg.svd(calib - mu, full_matrices=False)
    w_down = vt[:r].T.copy()                      # top-r right singular vectors
    w_up = w_down.reshape(T, d, r).copy()         # loop slices: rows [t*d, (t+1)*d)
    return mu, w_down, w_up
