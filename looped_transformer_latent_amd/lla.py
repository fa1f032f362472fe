"""Thin ctypes binding of the LLA C ABI (include/lla.h).

Argument marshalling only: every step of the attention, encode and RoPE-table
work runs in the HIP kernels of ``liblla.so``.  torch supplies device memory
(``tensor.data_ptr()``) and the current HIP stream.  If the library is not
built, every call raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblla.so")
GEN_LIB_PATH = os.path.join(_PKG, "liblla_gen.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_LAUNCH = 0, -1, -2, -3, -4
PER_HEAD, TWO_D = 0, 1
F32, BF16 = 0, 1
OP_ENCODE, OP_DECODE, OP_PREFILL, OP_RECONSTRUCT, OP_FULL_DECODE = 0, 1, 2, 3, 4
OP_ROPE_KEY_APPEND, OP_DECOUPLED_DECODE, OP_WINDOW_DECODE = 5, 6, 7
DEVERR_CTX, DEVERR_PAGE, DEVERR_APPEND = 1, 2, 4

EXPORTS = ["lla_rope_table", "lla_workspace_bytes", "lla_encode_append", "lla_decode_attn",
           "lla_prefill_attn", "lla_reconstruct_kv", "lla_full_decode_attn", "lla_rope_key_append",
           "lla_decoupled_decode_attn", "lla_decode_window_attn", "lla_cache_scalars", "lla_supported", "lla_status_string",
           "lla_last_error", "lla_attn_plan", "lla_window_pages", "lla_decode_attn_noalloc"]


class LlaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"LLA status {status}: {msg}")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("D", ctypes.c_int32), ("H", ctypes.c_int32),
                ("d_head", ctypes.c_int32), ("r_k", ctypes.c_int32), ("r_v", ctypes.c_int32),
                ("variant", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("rope_base", ctypes.c_float)]


class Codec(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("mu_k", "mu_v", "w_down_k", "w_down_v", "w_up_k", "w_up_v")]


class Cache(ctypes.Structure):
    _fields_ = [("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("page_table", ctypes.c_void_p), ("batch", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32), ("num_pages", ctypes.c_int32)]


_lib = None
_gen = None


def load() -> ctypes.CDLL:
    """Load liblla.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m looped_transformer_latent_amd.build` (no CPU fallback exists)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, S, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    pd, pc, pk = ctypes.POINTER(Dims), ctypes.POINTER(Codec), ctypes.POINTER(Cache)
    lib.lla_rope_table.argtypes = [pd, I, P, P]
    lib.lla_workspace_bytes.argtypes = [pd, I, I, I, I]
    lib.lla_workspace_bytes.restype = S
    lib.lla_encode_append.argtypes = [pd, pc, pk, P, P, P, I, I, I, P, S, P]
    lib.lla_decode_attn.argtypes = [pd, pc, pk, P, I, I, I, P, P, P, I, F, P, P, S, P]
    lib.lla_prefill_attn.argtypes = [pd, pc, pk, P, I, I, I, I, P, P, I, F, P, P, S, P]
    lib.lla_reconstruct_kv.argtypes = [pd, pc, pk, P, I, I, I, P, I, P, P, P, S, P]
    lib.lla_full_decode_attn.argtypes = [pd, pk, P, P, P, I, P, P, P, I, F, P, P, S, P]
    lib.lla_rope_key_append.argtypes = [pd, pk, I, P, P, I, P, P, I, I, I, P, S, P]
    lib.lla_decoupled_decode_attn.argtypes = [pd, pc, pk, I, P, P, I, I, I, P, P, P, I, F, P, P, S, P]
    lib.lla_decode_attn_noalloc.argtypes = [pd, pc, pk, P, I, I, I, P, P, P, I, F, P, P, P]
    lib.lla_decode_window_attn.argtypes = [pd, pc, pk, P, I, I, I, P, P, P, I, I, I, F, P, P, S, P]
    lib.lla_cache_scalars.argtypes = [pd, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]
    lib.lla_supported.argtypes = [pd, I]
    pi = ctypes.POINTER(I)
    lib.lla_attn_plan.argtypes = [pd, I, I, I, I, pi, pi]
    lib.lla_window_pages.argtypes = [I, I, I, pi, pi]
    lib.lla_status_string.argtypes = [I]
    lib.lla_status_string.restype = ctypes.c_char_p
    lib.lla_last_error.argtypes = []
    lib.lla_last_error.restype = ctypes.c_char_p
    for name in ("lla_rope_table", "lla_encode_append", "lla_decode_attn", "lla_prefill_attn",
                 "lla_reconstruct_kv", "lla_full_decode_attn",
                 "lla_cache_scalars", "lla_supported", "lla_attn_plan", "lla_window_pages"):
        getattr(lib, name).restype = I
    _lib = lib
    return lib


def load_gen() -> ctypes.CDLL:
    global _gen
    if _gen is None:
        if not os.path.exists(GEN_LIB_PATH):
            raise RuntimeError(f"{GEN_LIB_PATH} is missing: build it first")
        g = ctypes.CDLL(GEN_LIB_PATH)
        g.llagen_normal.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64,
                                    ctypes.c_uint64, ctypes.c_float, ctypes.c_void_p]
        g.llagen_normal.restype = ctypes.c_int
        _gen = g
    return _gen


def _check(status: int) -> None:
    if status != OK:
        raise LlaError(status, load().lla_last_error().decode())


def make_dims(T, D, H, d_head, r_k, r_v, variant=PER_HEAD, dtype=BF16, page_size=16,
              rope_base=10000.0) -> Dims:
    return Dims(T, D, H, d_head, r_k, r_v, variant, dtype, page_size, rope_base)


def dims_from_dict(m: dict) -> Dims:
    return make_dims(m["T"], m["D"], m["H"], m["d_head"], m["r_k"], m["r_v"], m["variant"],
                     m["dtype"], m.get("page_size", 16), m.get("rope_base", 10000.0))


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("LLA tensors must be contiguous device tensors")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def make_codec(mu_k, mu_v, w_down_k, w_down_v, w_up_k, w_up_v) -> Codec:
    ts = (mu_k, mu_v, w_down_k, w_down_v, w_up_k, w_up_v)
    c = Codec(*[(t.data_ptr() if t is not None else None) for t in ts])
    c._tensors = ts  # the struct holds raw pointers: keep the storage alive with it
    return c


def make_cache(k_pool: torch.Tensor, v_pool: torch.Tensor, page_table: torch.Tensor,
               num_pages: int) -> Cache:
    assert page_table.dtype == torch.int32 and page_table.dim() == 2
    c = Cache(k_pool.data_ptr(), v_pool.data_ptr(), page_table.data_ptr(),
              page_table.shape[0], page_table.shape[1], num_pages)
    c._tensors = (k_pool, v_pool, page_table)  # keep the storage alive with the pointers
    return c


def cache_scalars(dims: Dims) -> tuple[int, int]:
    t, l = ctypes.c_int64(), ctypes.c_int64()
    _check(load().lla_cache_scalars(ctypes.byref(dims), ctypes.byref(t), ctypes.byref(l)))
    return t.value, l.value


def supported(dims: Dims, op: int) -> bool:
    return bool(load().lla_supported(ctypes.byref(dims), op))


def workspace_bytes(dims: Dims, op: int, batch: int, max_ctx: int, n: int = 0) -> int:
    return int(load().lla_workspace_bytes(ctypes.byref(dims), op, batch, max_ctx, n))


def attn_plan(dims: Dims, op: int, batch: int, max_ctx: int, n: int = 0) -> tuple[int, int]:
    """(splits, pages per split) of an attention call (lla_attn_plan)."""
    s, p = ctypes.c_int32(), ctypes.c_int32()
    _check(load().lla_attn_plan(ctypes.byref(dims), op, batch, max_ctx, n, ctypes.byref(s), ctypes.byref(p)))
    return s.value, p.value


def window_pages(ctx: int, n_sink: int, window: int) -> tuple[int, int]:
    """(sink pages, first window page) that a windowed decode reads (lla_window_pages)."""
    a, b = ctypes.c_int32(), ctypes.c_int32()
    _check(load().lla_window_pages(ctx, n_sink, window, ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def workspace(dims: Dims, op: int, batch: int, max_ctx: int, n: int = 0, device="cuda") -> torch.Tensor:
    """A zeroed workspace of the size lla_workspace_bytes() asks for."""
    nbytes = workspace_bytes(dims, op, batch, max_ctx, n)
    if nbytes == 0:
        raise LlaError(ERR_INVALID_ARG, "lla_workspace_bytes returned 0 (invalid or unsupported)")
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def device_error_word(ws: torch.Tensor) -> int:
    return int(ws[:4].view(torch.int32).item())


def rope_table(dims: Dims, n_pos: int, device="cuda", stream=None) -> torch.Tensor:
    t = torch.empty((n_pos, dims.d_head // 2, 2), dtype=torch.float32, device=device)
    _check(load().lla_rope_table(ctypes.byref(dims), n_pos, _ptr(t), _stream(stream)))
    return t


def encode_append(dims: Dims, codec: Codec, cache: Cache, x_k, x_v, pos0, n_new: int,
                  layer0: int, n_layers: int, ws: torch.Tensor, stream=None) -> None:
    _check(load().lla_encode_append(ctypes.byref(dims), ctypes.byref(codec), ctypes.byref(cache),
                                    _ptr(x_k), _ptr(x_v), _ptr(pos0), n_new, layer0, n_layers,
                                    _ptr(ws), ws.numel(), _stream(stream)))


def decode_attn(dims: Dims, codec: Codec, cache: Cache, rope: torch.Tensor, layer: int, loop: int,
                q, q_pos, ctx_len, max_ctx: int, out, ws: torch.Tensor, scale: float = 0.0,
                stream=None) -> None:
    _check(load().lla_decode_attn(ctypes.byref(dims), ctypes.byref(codec), ctypes.byref(cache),
                                  _ptr(rope), rope.shape[0], layer, loop, _ptr(q), _ptr(q_pos),
                                  _ptr(ctx_len), max_ctx, scale, _ptr(out), _ptr(ws), ws.numel(),
                                  _stream(stream)))


def decode_attn_noalloc(dims: Dims, codec: Codec, cache: Cache, rope: torch.Tensor, layer: int, loop: int,
                        q, q_pos, ctx_len, max_ctx: int, out, err: torch.Tensor, scale: float = 0.0,
                        stream=None) -> None:
    """lla_decode_attn_noalloc: no workspace; err is a device int32 error word."""
    if err.dtype != torch.int32 or err.numel() < 1:
        raise ValueError("err must be a device int32 tensor")
    _check(load().lla_decode_attn_noalloc(ctypes.byref(dims), ctypes.byref(codec), ctypes.byref(cache),
                                          _ptr(rope), rope.shape[0], layer, loop, _ptr(q), _ptr(q_pos),
                                          _ptr(ctx_len), max_ctx, scale, _ptr(out), _ptr(err),
                                          _stream(stream)))


def decode_window_attn(dims: Dims, codec: Codec, cache: Cache, rope: torch.Tensor, layer: int, loop: int,
                       q, q_pos, ctx_len, n_sink: int, window: int, max_ctx: int, out, ws: torch.Tensor,
                       scale: float = 0.0, stream=None) -> None:
    """Decode over the retained tokens j < n_sink and j >= ctx_len - window."""
    _check(load().lla_decode_window_attn(ctypes.byref(dims), ctypes.byref(codec), ctypes.byref(cache),
                                         _ptr(rope), rope.shape[0], layer, loop, _ptr(q), _ptr(q_pos),
                                         _ptr(ctx_len), n_sink, window, max_ctx, scale, _ptr(out), _ptr(ws),
                                         ws.numel(), _stream(stream)))


def reconstruct_kv(dims: Dims, codec: Codec, cache: Cache, rope: torch.Tensor, layer: int, loop: int,
                   ctx_len, max_ctx: int, k_full, v_full, ws: torch.Tensor, stream=None) -> None:
    """Rebuild the full (rotated K, V) cache of (layer, loop) from the latents."""
    _check(load().lla_reconstruct_kv(ctypes.byref(dims), ctypes.byref(codec), ctypes.byref(cache),
                                     _ptr(rope), rope.shape[0], layer, loop, _ptr(ctx_len), max_ctx,
                                     _ptr(k_full), _ptr(v_full), _ptr(ws), ws.numel(), _stream(stream)))


def full_decode_attn(dims: Dims, cache: Cache, k_full, v_full, rope: torch.Tensor, q, q_pos, ctx_len,
                     max_ctx: int, out, ws: torch.Tensor, scale: float = 0.0, stream=None) -> None:
    """Decode attention over a full K/V cache (the cache's page table)."""
    _check(load().lla_full_decode_attn(ctypes.byref(dims), ctypes.byref(cache), _ptr(k_full), _ptr(v_full),
                                       _ptr(rope), rope.shape[0], _ptr(q), _ptr(q_pos), _ptr(ctx_len),
                                       max_ctx, scale, _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))


def rope_key_append(dims: Dims, cache: Cache, kr_pool, rope_r: torch.Tensor, kr_new, pos0, n_new: int,
                    layer0: int, n_layers: int, ws: torch.Tensor, stream=None) -> None:
    """Rotate the rotary-branch keys kr_new [n_layers][B][n_new][d_rope] at
    positions pos0[b] + n and write them into kr_pool [D][num_pages][16][d_rope]."""
    d_rope = kr_pool.shape[-1]
    _check(load().lla_rope_key_append(ctypes.byref(dims), ctypes.byref(cache), d_rope, _ptr(kr_pool),
                                      _ptr(rope_r), rope_r.shape[0], _ptr(kr_new), _ptr(pos0), n_new,
                                      layer0, n_layers, _ptr(ws), ws.numel(), _stream(stream)))


def decoupled_decode_attn(dims: Dims, codec: Codec, cache: Cache, kr_pool, rope_r: torch.Tensor, layer: int,
                          loop: int, q, q_pos, ctx_len, max_ctx: int, out, ws: torch.Tensor,
                          scale: float = 0.0, stream=None) -> None:
    """Decode with a NoPE content path absorbed into q plus a rotary branch;
    q [B][H][d_head + d_rope], out [B][H][d_head]."""
    d_rope = kr_pool.shape[-1]
    _check(load().lla_decoupled_decode_attn(ctypes.byref(dims), ctypes.byref(codec), ctypes.byref(cache),
                                            d_rope, _ptr(kr_pool), _ptr(rope_r), rope_r.shape[0], layer, loop,
                                            _ptr(q), _ptr(q_pos), _ptr(ctx_len), max_ctx, scale, _ptr(out),
                                            _ptr(ws), ws.numel(), _stream(stream)))


def prefill_attn(dims: Dims, codec: Codec, cache: Cache, rope: torch.Tensor, layer: int, loop: int,
                 n_q: int, q, p0, max_ctx: int, out, ws: torch.Tensor, scale: float = 0.0,
                 stream=None) -> None:
    _check(load().lla_prefill_attn(ctypes.byref(dims), ctypes.byref(codec), ctypes.byref(cache),
                                   _ptr(rope), rope.shape[0], layer, loop, n_q, _ptr(q), _ptr(p0),
                                   max_ctx, scale, _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))


def gen_normal_(t: torch.Tensor, seed: int, stream_id: int, scale: float = 1.0, offset: int = 0,
                stream=None) -> torch.Tensor:
    """Fill a device tensor (fp32, or bf16 storage) with the seeded generator of gen.py."""
    from . import gen
    if t.dtype not in (torch.float32, torch.bfloat16, torch.int16):
        raise TypeError("gen_normal_ fills fp32 or bf16 tensors")
    bf = 0 if t.dtype == torch.float32 else 1
    rc = load_gen().llagen_normal(_ptr(t), bf, t.numel(), gen.key(seed, stream_id), offset,
                                  float(gen.mult_for(scale)), _stream(stream))
    if rc != 0:
        raise RuntimeError(f"llagen_normal failed ({rc})")
    return t
