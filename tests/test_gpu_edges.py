"""GPU edge cases: empty calls leave every output untouched, and the latent
decode (full context and sink + window) over one 262144-token sequence, the
longest context of the benchmark configurations, matches the CPU oracle over
the whole context (all 16 heads)."""
from __future__ import annotations

import gc

import numpy as np
import pytest
import torch

import oracle
from gpu_util import device_codec, out_to_f64, row_rel_err, to_device, to_host
from looped_transformer_latent_amd import gen, lla
from looped_transformer_latent_amd import workloads as wl

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]
TOL = 2e-2


def small_setup(batch):
    w = wl.WORKLOADS["ouro1.4b-21x-b32"].replace(D=2, batch=max(batch, 1), ctx=64)
    D = lla.dims_from_dict(w.dims)
    codec, keep = device_codec(wl.codec_host(w))
    k = wl.device_pool(w, "k")
    v = wl.device_pool(w, "v")
    pt = wl.to_device(wl.page_table_host(w))
    cache = lla.make_cache(k, v, pt, w.num_pages)
    if batch == 0:  # the same storage, zero sequences
        cache = lla.Cache(k.data_ptr(), v.data_ptr(), pt.data_ptr(), 0, pt.shape[1], w.num_pages)
        cache._tensors = (k, v, pt)
    return w, D, codec, keep, k, v, pt, cache


def test_empty_calls_touch_nothing():
    """batch 0 decode / windowed / decoupled / full-cache decode, n_q = 0
    prefill and n_new = 0 or n_layers = 0 encode all return LLA_OK and write
    nothing (outputs and pools keep their bits, the error word stays 0)."""
    w, D, codec, keep, k, v, pt, cache0 = small_setup(0)
    rope = lla.rope_table(D, w.ctx)
    k0, v0 = k.clone(), v.clone()
    q = torch.zeros((1, w.H, w.d_head), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, 3.0)
    pos = torch.full((1,), 10, dtype=torch.int32, device="cuda")
    ws = lla.workspace(D, lla.OP_DECODE, 1, w.ctx)
    lla.decode_attn(D, codec, cache0, rope, 0, 0, q, pos, pos, w.ctx, out, ws)
    lla.decode_window_attn(D, codec, cache0, rope, 0, 0, q, pos, pos, 4, 16, w.ctx, out,
                           lla.workspace(D, lla.OP_WINDOW_DECODE, 1, w.ctx, 20))
    kf = torch.zeros((w.num_pages, w.H, 16, w.d_head), dtype=torch.bfloat16, device="cuda")
    lla.full_decode_attn(D, cache0, kf, kf, rope, q, pos, pos, w.ctx, out, lla.workspace(D, lla.OP_FULL_DECODE, 1, w.ctx))
    lla.reconstruct_kv(D, codec, cache0, rope, 0, 0, pos, w.ctx, kf, kf, lla.workspace(D, lla.OP_RECONSTRUCT, 1, w.ctx))
    kr = torch.zeros((w.D, w.num_pages, 16, 64), dtype=torch.bfloat16, device="cuda")
    rope_r = lla.rope_table(lla.dims_from_dict(dict(w.dims, d_head=64)), w.ctx)
    qd = torch.zeros((1, w.H, w.d_head + 64), dtype=torch.bfloat16, device="cuda")
    lla.decoupled_decode_attn(D, codec, cache0, kr, rope_r, 0, 0, qd, pos, pos, w.ctx, out,
                              lla.workspace(D, lla.OP_DECOUPLED_DECODE, 1, w.ctx, 64))
    # a non-empty cache with nothing to do
    cache1 = lla.make_cache(k, v, pt, w.num_pages)
    qp = torch.zeros((1, 1, w.H, w.d_head), dtype=torch.bfloat16, device="cuda")
    lla.prefill_attn(D, codec, cache1, rope, 0, 0, 0, qp, pos, w.ctx, qp, lla.workspace(D, lla.OP_PREFILL, 1, w.ctx, 0))
    wse = lla.workspace(D, lla.OP_ENCODE, 1, 0, w.D)
    x = torch.ones((w.D, 1, 1, w.H, w.T, w.d_head), dtype=torch.bfloat16, device="cuda")
    lla.encode_append(D, codec, cache1, x, x, pos, 0, 0, w.D, wse)
    lla.encode_append(D, codec, cache1, x, x, pos, 1, 0, 0, wse)
    lla.rope_key_append(D, cache1, kr, rope_r, qd, pos, 0, 0, 1, wse)
    torch.cuda.synchronize()
    assert (out.float() == 3.0).all()
    assert torch.equal(k.view(torch.int16), k0.view(torch.int16)) and torch.equal(v.view(torch.int16), v0.view(torch.int16))
    assert (kf.float() == 0).all() and (kr.float() == 0).all()
    assert lla.device_error_word(ws) == 0 and lla.device_error_word(wse) == 0


@pytest.fixture
def release():
    yield
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_latent_decode_over_262144_tokens(release):
    """Full context and sink 4 + window 256 over one 262144-token sequence: the
    split / merge configuration of the long-context runs, every head against the
    oracle."""
    w = wl.WORKLOADS["ouro1.4b-21x-ctx256k-decoupled"]
    D = lla.dims_from_dict(w.dims)
    codec_h = wl.codec_host(w)
    codec, keep = device_codec(codec_h)
    pt_h = wl.page_table_host(w)
    cache = lla.make_cache(wl.device_pool(w, "k"), wl.device_pool(w, "v"), wl.to_device(pt_h), w.num_pages)
    rope = lla.rope_table(D, w.ctx)
    ctx = torch.full((1,), w.ctx, dtype=torch.int32, device="cuda")
    q = torch.empty((1, w.H, w.d_head), dtype=torch.bfloat16, device="cuda")
    lla.gen_normal_(q, w.seed, wl.STREAMS["q"], offset=77)
    layer, loop = 17, 2
    m1 = dict(w.dims, D=1)
    codec1 = {k_: np.ascontiguousarray(v_[layer:layer + 1]) for k_, v_ in codec_h.items()}
    kp = wl.pool_pages_host(w, "k", layer, pt_h[0])[None]
    vp = wl.pool_pages_host(w, "v", layer, pt_h[0])[None]
    local = np.arange(pt_h.shape[1], dtype=np.int32)[None]
    c = np.full(1, w.ctx, np.int32)
    for name, n_sink, window in (("full", 0, 0), ("sink 4 + window 256", 4, 256)):
        out = torch.empty_like(q)
        if window:
            ws = lla.workspace(D, lla.OP_WINDOW_DECODE, 1, w.ctx, n_sink + window)
            lla.decode_window_attn(D, codec, cache, rope, layer, loop, q, ctx - 1, ctx, n_sink, window, w.ctx, out, ws)
            ref, rc = oracle.decode_window(m1, codec1, kp, vp, local, 0, loop, to_host(q), c - 1, c, n_sink, window)
        else:
            ws = lla.workspace(D, lla.OP_DECODE, 1, w.ctx)
            lla.decode_attn(D, codec, cache, rope, layer, loop, q, ctx - 1, ctx, w.ctx, out, ws)
            ref, rc = oracle.decode(m1, codec1, kp, vp, local, 0, loop, to_host(q), c - 1, c)
        torch.cuda.synchronize()
        assert rc == 0 and lla.device_error_word(ws) == 0
        err = row_rel_err(out_to_f64(out), ref)
        print(f"262144 tokens, {name}: max row rel err {err.max():.3e}", flush=True)
        assert err.max() <= TOL
