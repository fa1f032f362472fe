"""CPU oracle for Looped Latent Attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and it shares no code with
them: the arithmetic lives in ``lla_oracle.c`` (plain C, IEEE double), built
here with gcc, and this module only marshals numpy arrays into it.

What it computes is documented at the top of ``lla_oracle.c``: the plain
definition of LLA decode -- rebuild every cached token's full loop-t K and V
from its latents (encoder eq. (2), loop decoder eq. (3) of the cc.laoqi.cc close
reading, 方法 item 1), apply RoPE after reconstruction (方法 item 3), and run
textbook softmax attention.  Nothing is absorbed or fused.

Pins (tests/test_oracle_pins.py) tie it to facts fixed by the pages and by
mathematics; every function below is pinned there.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lla_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liblla_oracle.so")

F32, BF16 = 0, 1
PER_HEAD, TWO_D = 0, 1


def build(force: bool = False) -> str:
    """Compile lla_oracle.c with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wno-unknown-pragmas", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        _i, _p, _d = ctypes.c_int, ctypes.c_void_p, ctypes.c_double
        _lib.lla_oracle_bf16_rne.restype = ctypes.c_uint16
        _lib.lla_oracle_bf16_rne.argtypes = [_d]
        _lib.lla_oracle_slot.restype = ctypes.c_int64
        _lib.lla_oracle_slot.argtypes = [_p, _i, _i, _i, _i, ctypes.c_int64]
        _lib.lla_oracle_rope.restype = None
        _lib.lla_oracle_rope.argtypes = [_p, _i, _d, _d, _p]
        _lib.lla_oracle_cache_scalars.restype = None
        _lib.lla_oracle_cache_scalars.argtypes = [_i, _i, _i, _i, _i, _i, _p, _p]
        _lib.lla_oracle_encode.restype = _i
        _lib.lla_oracle_encode.argtypes = [_i] * 9 + [_p] * 7 + [_i] * 3 + [_p, _p, _p, _i, _i, _i]
        _lib.lla_oracle_decode.restype = _i
        _lib.lla_oracle_decode.argtypes = ([_i] * 9 + [_d] + [_p] * 7 + [_i] * 5 +
                                           [_p, _p, _p, _d, _p, _i])
        _lib.lla_oracle_decode_window.restype = _i
        _lib.lla_oracle_decode_window.argtypes = ([_i] * 9 + [_d] + [_p] * 7 + [_i] * 5 +
                                                  [_p, _p, _p, _i, _i, _d, _p, _i])
        _lib.lla_oracle_prefill.restype = _i
        _lib.lla_oracle_prefill.argtypes = ([_i] * 9 + [_d] + [_p] * 7 + [_i] * 6 +
                                            [_p, _p, _d, _p, _i])
        _lib.lla_oracle_rope_key_append.restype = _i
        _lib.lla_oracle_rope_key_append.argtypes = [_i, _i, _i, _d, _i, _p, _p, _i, _i, _i, _p, _p,
                                                    _i, _i, _i]
        _lib.lla_oracle_decoupled_decode.restype = _i
        _lib.lla_oracle_decoupled_decode.argtypes = ([_i] * 9 + [_d] + [_p] * 8 + [_i] * 5 +
                                                     [_p, _p, _p, _d, _p, _i])
        _lib.lla_oracle_max_threads.restype = _i
        _lib.lla_oracle_max_threads.argtypes = [_i]
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _stored(a: np.ndarray, dtype: int) -> np.ndarray:
    want = np.float32 if dtype == F32 else np.uint16
    if a.dtype != want:
        raise TypeError(f"expected {want} storage, got {a.dtype}")
    return np.ascontiguousarray(a)


def bf16_rne(x: float) -> int:
    """bf16 bit pattern nearest to the double x (ties to even)."""
    return int(lib().lla_oracle_bf16_rne(float(x)))


def slot(page_table: np.ndarray, num_pages: int, page_size: int, b: int, j: int) -> int:
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    return int(lib().lla_oracle_slot(_ptr(pt), pt.shape[1], num_pages, page_size, b, j))


def rope(x: np.ndarray, pos: float, base: float = 10000.0) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty_like(x)
    lib().lla_oracle_rope(_ptr(x), x.shape[0], float(pos), float(base), _ptr(out))
    return out


def cache_scalars(T: int, H: int, d: int, r_k: int, r_v: int, variant: int) -> tuple[int, int]:
    """(teacher scalars, latent scalars) per token and layer, eq. (4)."""
    t, l = ctypes.c_int64(), ctypes.c_int64()
    lib().lla_oracle_cache_scalars(T, H, d, r_k, r_v, variant, ctypes.byref(t), ctypes.byref(l))
    return t.value, l.value


def encode(dims: dict, codec: dict, k_pool: np.ndarray, v_pool: np.ndarray,
           page_table: np.ndarray, x_k: np.ndarray, x_v: np.ndarray, pos0: np.ndarray,
           n_new: int, layer0: int, n_layers: int) -> int:
    """Encode + append in place into k_pool / v_pool (storage arrays)."""
    dt = dims["dtype"]
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    p0 = np.ascontiguousarray(pos0, dtype=np.int32)
    assert k_pool.flags["C_CONTIGUOUS"] and v_pool.flags["C_CONTIGUOUS"]
    args = [_stored(codec[k], dt) for k in ("mu_k", "mu_v", "w_down_k", "w_down_v")]
    xk, xv = _stored(x_k, dt), _stored(x_v, dt)
    return lib().lla_oracle_encode(
        dims["T"], dims["D"], dims["H"], dims["d_head"], dims["r_k"], dims["r_v"],
        dims["variant"], dt, dims["page_size"],
        *[_ptr(a) for a in args], _ptr(k_pool), _ptr(v_pool), _ptr(pt),
        pt.shape[0], pt.shape[1], k_pool.shape[1],
        _ptr(xk), _ptr(xv), _ptr(p0), n_new, layer0, n_layers)


def _attn_common(dims, codec, k_pool, v_pool, page_table):
    dt = dims["dtype"]
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    params = [_stored(codec[k], dt) for k in ("mu_k", "mu_v", "w_up_k", "w_up_v")]
    pools = [_stored(k_pool, dt), _stored(v_pool, dt)]
    head = (dims["T"], dims["D"], dims["H"], dims["d_head"], dims["r_k"], dims["r_v"],
            dims["variant"], dt, dims["page_size"], float(dims.get("rope_base", 10000.0)))
    return head, params, pools, pt


def decode(dims: dict, codec: dict, k_pool, v_pool, page_table, layer: int, loop: int,
           q: np.ndarray, q_pos: np.ndarray, ctx_len: np.ndarray, scale: float | None = None,
           threads: int = 0) -> tuple[np.ndarray, int]:
    """Decode attention, one query per sequence.  Returns (out [B][H][d] float64, status)."""
    head, params, pools, pt = _attn_common(dims, codec, k_pool, v_pool, page_table)
    B, H, d = pt.shape[0], dims["H"], dims["d_head"]
    qs = _stored(q, dims["dtype"])
    assert qs.size == B * H * d
    qp = np.ascontiguousarray(q_pos, dtype=np.int32)
    cl = np.ascontiguousarray(ctx_len, dtype=np.int32)
    out = np.empty((B, H, d), dtype=np.float64)
    scale = (1.0 / np.sqrt(d)) if scale is None else float(scale)
    rc = lib().lla_oracle_decode(*head, *[_ptr(a) for a in params], *[_ptr(a) for a in pools],
                                 _ptr(pt), B, pt.shape[1], pools[0].shape[1], layer, loop,
                                 _ptr(qs), _ptr(qp), _ptr(cl), scale, _ptr(out), threads)
    return out, rc


def decode_window(dims: dict, codec: dict, k_pool, v_pool, page_table, layer: int, loop: int,
                  q: np.ndarray, q_pos: np.ndarray, ctx_len: np.ndarray, n_sink: int, window: int,
                  scale: float | None = None, threads: int = 0) -> tuple[np.ndarray, int]:
    """Decode over the sink + window retained set: tokens j < n_sink and
    j >= ctx_len - window of each sequence (original positions).  Returns
    (out [B][H][d] float64, status)."""
    head, params, pools, pt = _attn_common(dims, codec, k_pool, v_pool, page_table)
    B, H, d = pt.shape[0], dims["H"], dims["d_head"]
    qs = _stored(q, dims["dtype"])
    assert qs.size == B * H * d
    qp = np.ascontiguousarray(q_pos, dtype=np.int32)
    cl = np.ascontiguousarray(ctx_len, dtype=np.int32)
    out = np.empty((B, H, d), dtype=np.float64)
    scale = (1.0 / np.sqrt(d)) if scale is None else float(scale)
    rc = lib().lla_oracle_decode_window(*head, *[_ptr(a) for a in params], *[_ptr(a) for a in pools],
                                        _ptr(pt), B, pt.shape[1], pools[0].shape[1], layer, loop,
                                        _ptr(qs), _ptr(qp), _ptr(cl), n_sink, window, scale, _ptr(out),
                                        threads)
    return out, rc


def prefill(dims: dict, codec: dict, k_pool, v_pool, page_table, layer: int, loop: int,
            n_q: int, q: np.ndarray, p0: np.ndarray, scale: float | None = None,
            threads: int = 0) -> tuple[np.ndarray, int]:
    """Causal prefill.  Returns (out [B][n_q][H][d] float64, status)."""
    head, params, pools, pt = _attn_common(dims, codec, k_pool, v_pool, page_table)
    B, H, d = pt.shape[0], dims["H"], dims["d_head"]
    qs = _stored(q, dims["dtype"])
    assert qs.size == B * n_q * H * d
    pp = np.ascontiguousarray(p0, dtype=np.int32)
    out = np.empty((B, n_q, H, d), dtype=np.float64)
    scale = (1.0 / np.sqrt(d)) if scale is None else float(scale)
    rc = lib().lla_oracle_prefill(*head, *[_ptr(a) for a in params], *[_ptr(a) for a in pools],
                                  _ptr(pt), B, pt.shape[1], pools[0].shape[1], layer, loop,
                                  n_q, _ptr(qs), _ptr(pp), scale, _ptr(out), threads)
    return out, rc


def rope_key_append(dims: dict, d_rope: int, kr_pool: np.ndarray, page_table: np.ndarray,
                    kr_new: np.ndarray, pos0: np.ndarray, layer0: int) -> int:
    """Decoupled-RoPE rotary keys: rotate kr_new [n_layers][B][n_new][d_rope] at
    positions pos0[b] + n and store them in kr_pool [D][num_pages][P][d_rope]
    (in place, storage arrays)."""
    dt = dims["dtype"]
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    p0 = np.ascontiguousarray(pos0, dtype=np.int32)
    assert kr_pool.flags["C_CONTIGUOUS"] and kr_pool.shape[-1] == d_rope
    kn = _stored(kr_new, dt)
    n_layers, B, n_new = kn.shape[0], kn.shape[1], kn.shape[2]
    assert B == pt.shape[0]
    return lib().lla_oracle_rope_key_append(
        dims["D"], dims["page_size"], d_rope, float(dims.get("rope_base", 10000.0)), dt,
        _ptr(kr_pool), _ptr(pt), B, pt.shape[1], kr_pool.shape[1], _ptr(kn), _ptr(p0),
        n_new, layer0, n_layers)


def decoupled_decode(dims: dict, codec: dict, k_pool, v_pool, kr_pool, page_table, layer: int,
                     loop: int, q: np.ndarray, q_pos: np.ndarray, ctx_len: np.ndarray,
                     d_rope: int, scale: float | None = None,
                     threads: int = 0) -> tuple[np.ndarray, int]:
    """Decode with a NoPE content path and a rotary branch of width d_rope.
    q [B][H][d + d_rope].  Returns (out [B][H][d] float64, status)."""
    head, params, pools, pt = _attn_common(dims, codec, k_pool, v_pool, page_table)
    assert dims["variant"] == PER_HEAD
    B, H, d = pt.shape[0], dims["H"], dims["d_head"]
    qs = _stored(q, dims["dtype"])
    krs = _stored(kr_pool, dims["dtype"])
    assert qs.size == B * H * (d + d_rope) and krs.shape[1] == pools[0].shape[1]
    qp = np.ascontiguousarray(q_pos, dtype=np.int32)
    cl = np.ascontiguousarray(ctx_len, dtype=np.int32)
    out = np.empty((B, H, d), dtype=np.float64)
    scale = (1.0 / np.sqrt(d + d_rope)) if scale is None else float(scale)
    T, D, H_, d_, r_k, r_v, _variant, dt, P, base = head
    rc = lib().lla_oracle_decoupled_decode(
        T, D, H_, d_, r_k, r_v, d_rope, dt, P, base, *[_ptr(a) for a in params],
        *[_ptr(a) for a in pools], _ptr(krs), _ptr(pt), B, pt.shape[1], pools[0].shape[1],
        layer, loop, _ptr(qs), _ptr(qp), _ptr(cl), scale, _ptr(out), threads)
    return out, rc


def max_threads(threads: int = 0) -> int:
    return int(lib().lla_oracle_max_threads(threads))
