"""GPU parity: LLA-2D decode / prefill (HIP) against the CPU oracle.

LLA-2D keeps one K latent and one V latent per (token, layer), shared by all
heads; head h of loop t decodes it with its own mu_t,h and W_up,t,h.  The
oracle reconstructs every head's loop-t K and V from the shared latent in fp64
and runs textbook attention.  Tolerance: 2e-2 per output row (bf16).
"""
from __future__ import annotations

import gc

import numpy as np
import pytest
import torch

import oracle
from fixtures import BF16, TWO_D, dims, random_codec, random_pools
from gpu_util import device_codec, out_to_f64, row_rel_err, to_device, to_host
from looped_transformer_latent_amd import gen, lla
from looped_transformer_latent_amd import workloads as wl

pytestmark = pytest.mark.gpu
TOL = 2e-2


def gpu_decode(m, codec_h, kp, vp, pt, q, q_pos, ctx, layer, loop, max_ctx=None):
    D = lla.dims_from_dict(m)
    assert lla.supported(D, lla.OP_DECODE)
    c, keep = device_codec(codec_h)
    kp_d, vp_d = to_device(kp), to_device(vp)
    pt_d = to_device(np.ascontiguousarray(pt, dtype=np.int32))
    cache = lla.make_cache(kp_d, vp_d, pt_d, kp.shape[1])
    max_ctx = int(np.max(ctx)) if max_ctx is None else max_ctx
    rope = lla.rope_table(D, max(max_ctx, int(np.max(q_pos)) + 1))
    q_d = to_device(q)
    out = torch.empty_like(q_d)
    ws = lla.workspace(D, lla.OP_DECODE, pt.shape[0], max_ctx)
    lla.decode_attn(D, c, cache, rope, layer, loop, q_d, to_device(np.int32(q_pos)),
                    to_device(np.int32(ctx)), max_ctx, out, ws)
    torch.cuda.synchronize()
    return out_to_f64(out), ws


def check(m, codec, kp, vp, pt, q, ctx, layer, loop, label):
    got, ws = gpu_decode(m, codec, kp, vp, pt, q, ctx - 1, ctx, layer, loop)
    ref, rc = oracle.decode(m, codec, kp, vp, pt, layer, loop, q, np.int32(ctx - 1), np.int32(ctx))
    assert rc == 0
    err = row_rel_err(got, ref)
    print(f"{label} layer={layer} loop={loop}: max row rel err {err.max():.3e}", flush=True)
    assert np.isfinite(got).all()
    assert err.max() <= TOL
    assert lla.device_error_word(ws) == 0
    return got


@pytest.mark.parametrize("shape", [(8, 64, 128, 256), (32, 128, 256, 256)])
def test_lla2d_ragged_contexts_shuffled_pages(shape):
    """Contexts 1, 31, 33 (partial 32-token blocks), 300 and 1000 (several splits)."""
    H, d, rk, rv = shape
    m = dims(3, 2, H, d, rk, rv, TWO_D, BF16)
    ctx = np.array([1, 31, 33, 300, 1000])
    B, pps = len(ctx), 64
    codec = random_codec(m, seed=5002, ortho_down=False)
    kp, vp = random_pools(m, B * pps, seed=5003)
    pt = gen.shuffled_page_table(5004, B, pps)
    q = gen.normal(5005, 1, (B, H, d))
    for layer, loop in ((0, 0), (1, 2)):
        check(m, codec, kp, vp, pt, q, ctx, layer, loop, f"2D H={H} d={d} r={rk}/{rv}")


def test_lla2d_context_beyond_one_split_stage():
    """One row of 20000 tokens (1250 pages): more pages than a workgroup stages
    (1024), so the row is cut into several splits of whole 32-token blocks and
    merged; plus a short second row.  The oracle runs the whole context."""
    H, d, rk, rv = 8, 64, 128, 256
    m = dims(2, 1, H, d, rk, rv, TWO_D, BF16)
    ctx = np.array([20000, 77])
    B, pps = len(ctx), 1250
    codec = random_codec(m, seed=5102, ortho_down=False)
    kp, vp = random_pools(m, B * pps, seed=5103)
    pt = gen.shuffled_page_table(5104, B, pps)
    q = gen.normal(5105, 1, (B, H, d))
    D = lla.dims_from_dict(m)
    splits, per = lla.attn_plan(D, lla.OP_DECODE, B, int(ctx.max()))
    assert splits >= 2 and per <= 1024 and per % 2 == 0
    check(m, codec, kp, vp, pt, q, ctx, 0, 1, "2D 20000 tokens")


def test_lla2d_unused_slots_may_hold_nan_and_page_table_invariance():
    m = dims(2, 1, 8, 64, 128, 256, TWO_D, BF16)
    ctx = np.array([45, 70])
    B, pps = 2, 6
    codec = random_codec(m, seed=5102, ortho_down=False)
    kp, vp = random_pools(m, B * pps, seed=5103)
    pt = gen.identity_page_table(B, pps)
    # slots past ctx in the last page, and whole unused pages, hold NaN / -inf
    kp[:, 2, 13:] = 0x7FC1
    vp[:, 2, 13:] = 0x7FC1
    kp[:, 3:6] = 0xFF80
    vp[:, 3:6] = 0x7FC1
    kp[:, 6 + 4, 6:] = 0x7FC1
    vp[:, 6 + 4, 6:] = 0x7FC1
    q = gen.normal(5104, 1, (B, 8, 64))
    a = check(m, codec, kp, vp, pt, q, ctx, 0, 1, "2D nan-tail")
    pt_sh = gen.shuffled_page_table(5105, B, pps)
    kp_sh, vp_sh = np.empty_like(kp), np.empty_like(vp)
    kp_sh[:, pt_sh.reshape(-1)] = kp[:, pt.reshape(-1)]
    vp_sh[:, pt_sh.reshape(-1)] = vp[:, pt.reshape(-1)]
    b2, _ = gpu_decode(m, codec, kp_sh, vp_sh, pt_sh, q, ctx - 1, ctx, 0, 1)
    assert np.array_equal(a, b2)


def test_lla2d_device_errors():
    m = dims(2, 1, 8, 64, 128, 256, TWO_D, BF16)
    B, pps = 3, 4
    codec = random_codec(m, seed=5202, ortho_down=False)
    kp, vp = random_pools(m, B * pps, seed=5203)
    pt = gen.identity_page_table(B, pps)
    pt[1, 2] = 1000
    ctx = np.array([60, 60, 65])   # row 2 exceeds max_ctx = 64
    q = gen.normal(5204, 1, (B, 8, 64))
    got, ws = gpu_decode(m, codec, kp, vp, pt, q, np.array([59, 59, 59]), ctx, 0, 0, max_ctx=64)
    assert np.isnan(got[1]).all() and np.isnan(got[2]).all()
    word = lla.device_error_word(ws)
    assert word & lla.DEVERR_PAGE and word & lla.DEVERR_CTX
    ref, _ = oracle.decode(m, codec, kp, vp, pt, 0, 0, q, np.int32([59] * 3), np.int32(ctx))
    assert row_rel_err(got[0], ref[0]).max() <= TOL


def test_lla2d_prefill():
    m = dims(2, 1, 8, 64, 128, 256, TWO_D, BF16)
    B, pps, n_q = 2, 6, 19
    p0 = np.array([0, 70])
    codec = random_codec(m, seed=5302, ortho_down=False)
    kp, vp = random_pools(m, B * pps, seed=5303)
    pt = gen.shuffled_page_table(5304, B, pps)
    q = gen.normal(5305, 1, (B, n_q, 8, 64))
    D = lla.dims_from_dict(m)
    c, keep = device_codec(codec)
    kp_d, vp_d, pt_d = to_device(kp), to_device(vp), to_device(pt)
    cache = lla.make_cache(kp_d, vp_d, pt_d, kp.shape[1])
    max_ctx = int(p0.max()) + n_q
    rope = lla.rope_table(D, max_ctx)
    q_d = to_device(q)
    out = torch.empty_like(q_d)
    ws = lla.workspace(D, lla.OP_PREFILL, B, max_ctx, n_q)
    lla.prefill_attn(D, c, cache, rope, 0, 1, n_q, q_d, to_device(np.int32(p0)), max_ctx, out, ws)
    torch.cuda.synchronize()
    ref, rc = oracle.prefill(m, codec, kp, vp, pt, 0, 1, n_q, q, np.int32(p0))
    assert rc == 0
    err = row_rel_err(out_to_f64(out), ref)
    print(f"2D prefill: max row rel err {err.max():.3e}", flush=True)
    assert err.max() <= TOL


@pytest.mark.timeout(600)
def test_lla2d_full_size_sampled():
    """T=8, D=4, H=32, d=128, r_k=r_v=256, batch 128, context 16384, shuffled pages,
    in the benchmark's launch configuration; a few rows recomputed by the oracle."""
    w = wl.WORKLOADS["lla2d-t8-h32-b128"]
    D = lla.dims_from_dict(w.dims)
    codec_h = wl.codec_host(w)
    c, keep = device_codec(codec_h)
    pt_h = wl.page_table_host(w)
    pt = wl.to_device(pt_h)
    k_pool, v_pool = wl.device_pool(w, "k"), wl.device_pool(w, "v")
    cache = lla.make_cache(k_pool, v_pool, pt, w.num_pages)
    rope = lla.rope_table(D, w.ctx)
    layer, loop = w.D - 1, w.T - 1
    q = torch.empty((w.batch, w.H, w.d_head), dtype=torch.bfloat16, device="cuda")
    lla.gen_normal_(q, w.seed, wl.STREAMS["q"], offset=(loop * w.D + layer) * q.numel())
    ctx = torch.full((w.batch,), w.ctx, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    ws = lla.workspace(D, lla.OP_DECODE, w.batch, w.ctx)
    lla.decode_attn(D, c, cache, rope, layer, loop, q, ctx - 1, ctx, w.ctx, out, ws)
    torch.cuda.synchronize()
    assert lla.device_error_word(ws) == 0
    got = out_to_f64(out)
    assert np.isfinite(got).all()
    rows = np.array([0, 77, 127])
    pages = pt_h[rows].reshape(-1)
    kp = wl.pool_pages_host(w, "k", layer, pages)[None]
    vp = wl.pool_pages_host(w, "v", layer, pages)[None]
    local = np.arange(len(pages), dtype=np.int32).reshape(len(rows), -1)
    m1 = dict(w.dims, D=1)
    codec1 = {k: np.ascontiguousarray(v[layer:layer + 1]) for k, v in codec_h.items()}
    cl = np.full(len(rows), w.ctx, np.int32)
    ref, rc = oracle.decode(m1, codec1, np.ascontiguousarray(kp), np.ascontiguousarray(vp), local, 0,
                            loop, np.ascontiguousarray(to_host(q)[rows]), cl - 1, cl)
    assert rc == 0
    err = row_rel_err(got[rows], ref)
    print(f"2D full size rows {list(rows)}: max row rel err {err.max():.3e}", flush=True)
    assert err.max() <= TOL
    del k_pool, v_pool, cache
    gc.collect()
    torch.cuda.empty_cache()
