"""lla_decode_attn_noalloc: the decode without a workspace (split partials in
the library's per-device scratch array, the error word a caller-owned device
int32).  Its output must be the output of lla_decode_attn on the same inputs,
bit for bit (same kernels, same split plan), and both within the bf16 bar of
the oracle; two calls in a row, the second smaller, so the second reads only
what it wrote over the first call's partials."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle
from fixtures import BF16, PER_HEAD, dims, random_codec, random_pools
from gpu_util import device_codec, out_to_f64, row_rel_err, to_device
from looped_transformer_latent_amd import gen, lla

TOL = 2e-2


def test_noalloc_rejects_calls_beyond_the_scratch_and_null_error_word():
    """Host-side checks only (nothing is enqueued): 768 sequences at a 2^20
    context need 32 splits, 53 MB of partials, above the 16 MiB scratch."""
    lib = lla.load()
    d = lla.make_dims(4, 24, 16, 128, 16, 32)
    codec = lla.Codec(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000)
    fake = ctypes.c_void_p(0x1000)

    def call(batch, max_ctx, err):
        cache = lla.Cache(0x1000, 0x1000, 0x1000, batch, (max_ctx + 15) // 16, 1 << 24)
        return lib.lla_decode_attn_noalloc(ctypes.byref(d), ctypes.byref(codec), ctypes.byref(cache), fake,
                                           max_ctx, 0, 0, fake, fake, fake, max_ctx, 0.0, fake, err, None)
    assert call(768, 1 << 20, fake) == lla.ERR_WORKSPACE
    assert b"scratch" in lib.lla_last_error()
    assert call(4, 4096, None) == lla.ERR_INVALID_ARG
    assert lla.workspace_bytes(d, lla.OP_DECODE, 768, 1 << 20) - 256 > 16 << 20


def _problem(B, ctx, seed):
    m = dims(4, 2, 16, 128, 16, 32, PER_HEAD, BF16)
    pps = (int(ctx.max()) + 15) // 16
    codec = random_codec(m, seed=seed, ortho_down=False)
    kp, vp = random_pools(m, B * pps, seed=seed + 1)
    pt = gen.shuffled_page_table(seed + 2, B, pps)
    q = gen.normal(seed + 3, 1, (B, 16, 128))
    return m, codec, kp, vp, pt, q


def _both(m, codec, kp, vp, pt, q, ctx, layer, loop, bad_page=None):
    D = lla.dims_from_dict(m)
    c, keep = device_codec(codec)
    pt_dev = pt.copy()
    if bad_page is not None:
        pt_dev[bad_page] = kp.shape[1] + 5
    cache = lla.make_cache(to_device(kp), to_device(vp), to_device(np.ascontiguousarray(pt_dev, np.int32)),
                           kp.shape[1])
    max_ctx = int(ctx.max())
    rope = lla.rope_table(D, max_ctx)
    q_d = to_device(q)
    qp, cl = to_device(np.int32(ctx - 1)), to_device(np.int32(ctx))
    out_ws = torch.empty_like(q_d)
    ws = lla.workspace(D, lla.OP_DECODE, len(ctx), max_ctx)
    lla.decode_attn(D, c, cache, rope, layer, loop, q_d, qp, cl, max_ctx, out_ws, ws)
    out_na = torch.full_like(q_d, float("nan"))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    lla.decode_attn_noalloc(D, c, cache, rope, layer, loop, q_d, qp, cl, max_ctx, out_na, err)
    torch.cuda.synchronize()
    splits, _ = lla.attn_plan(D, lla.OP_DECODE, len(ctx), max_ctx)
    return out_ws, out_na, lla.device_error_word(ws), int(err.item()), splits


@pytest.mark.gpu
def test_noalloc_matches_workspace_decode_two_calls():
    # call 1: 4 sequences, contexts 1 .. 3000, many splits per row
    ctx1 = np.array([1, 17, 1000, 3000])
    m, codec, kp, vp, pt, q = _problem(4, ctx1, seed=7100)
    print(f"no-alloc call 1: batch 4, contexts {ctx1.tolist()}", flush=True)
    o_ws, o_na, e_ws, e_na, splits1 = _both(m, codec, kp, vp, pt, q, ctx1, 1, 2)
    assert splits1 > 1 and e_ws == 0 and e_na == 0
    assert torch.equal(o_ws.view(torch.int16), o_na.view(torch.int16))
    ref, rc = oracle.decode(m, codec, kp, vp, pt, 1, 2, q, np.int32(ctx1 - 1), np.int32(ctx1))
    assert rc == 0 and row_rel_err(out_to_f64(o_na), ref).max() <= TOL

    # call 2: smaller (2 sequences, shorter contexts, other codec and pools)
    ctx2 = np.array([300, 65])
    m, codec, kp, vp, pt, q = _problem(2, ctx2, seed=7200)
    print(f"no-alloc call 2: batch 2, contexts {ctx2.tolist()}", flush=True)
    o_ws, o_na, e_ws, e_na, splits2 = _both(m, codec, kp, vp, pt, q, ctx2, 0, 0)
    assert splits2 > 1 and e_ws == 0 and e_na == 0
    assert torch.equal(o_ws.view(torch.int16), o_na.view(torch.int16))
    ref, rc = oracle.decode(m, codec, kp, vp, pt, 0, 0, q, np.int32(ctx2 - 1), np.int32(ctx2))
    assert rc == 0 and row_rel_err(out_to_f64(o_na), ref).max() <= TOL


@pytest.mark.gpu
def test_noalloc_reports_device_errors_in_the_callers_word():
    ctx = np.array([200, 200, 200])
    m, codec, kp, vp, pt, q = _problem(3, ctx, seed=7300)
    print("no-alloc: bad page entry of sequence 1", flush=True)
    o_ws, o_na, e_ws, e_na, _ = _both(m, codec, kp, vp, pt, q, ctx, 0, 1, bad_page=(1, 4))
    assert e_ws == lla.DEVERR_PAGE and e_na == lla.DEVERR_PAGE
    g = out_to_f64(o_na)
    assert np.isnan(g[1]).all() and np.isfinite(g[[0, 2]]).all()
    assert torch.equal(o_ws.view(torch.int16), o_na.view(torch.int16))
