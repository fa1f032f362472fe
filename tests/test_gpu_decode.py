"""GPU parity: lla_decode_attn / lla_prefill_attn (HIP) against the CPU oracle.

Both sides read the same seeded inputs; the oracle decompresses every latent to
full loop-t K/V in fp64 and runs textbook attention.  Tolerances (per output
row, ||gpu - ref||_inf / ||ref||_inf): 1e-4 for fp32 storage, 2e-2 for bf16.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from fixtures import (BF16, F32, PER_HEAD, dims, param_shapes, pool_shape, random_codec,
                      random_pools, rank8_activations, store, svd_codec_one)
from gpu_util import device_codec, out_to_f64, row_rel_err, to_device
from looped_transformer_latent_amd import gen, lla

pytestmark = pytest.mark.gpu
TOL = {F32: 1e-4, BF16: 2e-2}


def gpu_decode(m, codec_h, kp, vp, pt, q, q_pos, ctx, layer, loop, max_ctx=None, scale=0.0,
               ws=None, rope_len=None):
    D = lla.dims_from_dict(m)
    c, keep = device_codec(codec_h)
    kp_d, vp_d = to_device(kp), to_device(vp)
    pt_d = to_device(np.ascontiguousarray(pt, dtype=np.int32))
    cache = lla.make_cache(kp_d, vp_d, pt_d, kp.shape[1])
    max_ctx = int(np.max(ctx)) if max_ctx is None else max_ctx
    rope = lla.rope_table(D, rope_len or max(max_ctx, int(np.max(q_pos)) + 1))
    q_d = to_device(q)
    out = torch.empty_like(q_d)
    ws = lla.workspace(D, lla.OP_DECODE, pt.shape[0], max_ctx) if ws is None else ws
    lla.decode_attn(D, c, cache, rope, layer, loop, q_d, to_device(np.int32(q_pos)),
                    to_device(np.int32(ctx)), max_ctx, out, ws, scale=scale)
    torch.cuda.synchronize()
    return out_to_f64(out), ws


def check(m, codec_h, kp, vp, pt, q, q_pos, ctx, layer, loop, label=""):
    got, ws = gpu_decode(m, codec_h, kp, vp, pt, q, q_pos, ctx, layer, loop)
    ref, rc = oracle.decode(m, codec_h, kp, vp, pt, layer, loop, q, np.int32(q_pos), np.int32(ctx))
    assert rc == 0
    err = row_rel_err(got, ref)
    print(f"{label} layer={layer} loop={loop}: max row rel err {err.max():.3e}", flush=True)
    assert np.isfinite(got).all()
    assert err.max() <= TOL[m["dtype"]], err.max()
    assert lla.device_error_word(ws) == 0
    return got


# ---------------------------------------------------------------- tiny fp32 (SVD codec)

def test_tiny_fp32_svd_codec_all_loops():
    """T=4, D=1, H=2, d=64, r_k=16, r_v=32, batch 1, context 256: rank-8 signal plus
    0.05 N(0,1) noise; codec from the SVD of a 4096-token calibration draw; the
    cache holds 256 fresh tokens encoded by the oracle; q ~ N(0,1) at position 255."""
    T, H, d, L, rk, rv = 4, 2, 64, 256, 16, 32
    m = dims(T, 1, H, d, rk, rv, PER_HEAD, F32)
    sh = param_shapes(m)
    codec = {k: np.zeros(v) for k, v in sh.items()}
    xs = {}
    for h in range(H):
        for kv, r in (("k", rk), ("v", rv)):
            stream = 5000 + 10 * h + (0 if kv == "k" else 5)
            mu, wd, wu = svd_codec_one(rank8_activations(1001, stream, 4096, T * d), r, T, d)
            codec["mu_" + kv][0, h] = mu.reshape(T, d)
            codec["w_down_" + kv][0, h] = wd
            codec["w_up_" + kv][0, h] = wu
            xs[kv + str(h)] = rank8_activations(1001, stream, L, T * d, draw=1)
    codec = {k: store(v, F32) for k, v in codec.items()}
    npages = L // 16
    pt = gen.identity_page_table(1, npages)
    kp = np.zeros(pool_shape(m, npages, "k"), np.float32)
    vp = np.zeros(pool_shape(m, npages, "v"), np.float32)
    xk = store(np.stack([xs["k%d" % h] for h in range(H)], 1).reshape(1, 1, L, H, T, d), F32)
    xv = store(np.stack([xs["v%d" % h] for h in range(H)], 1).reshape(1, 1, L, H, T, d), F32)
    assert oracle.encode(m, codec, kp, vp, pt, xk, xv, np.array([0]), L, 0, 1) == 0
    q = gen.normal(1001, 301, (1, H, d), dtype="f32")
    for t in range(T):
        check(m, codec, kp, vp, pt, q, [L - 1], [L], 0, t, "tiny-fp32")


def test_tiny_fp32_gpu_encode_then_gpu_decode():
    """The tiny fp32 workload end to end on the GPU: the 256 fresh tokens are
    appended by lla_encode_append into an empty pool (checked against the
    oracle's encode at 1e-4 per latent row), then every loop's decode reads the
    GPU-written cache; the reference is the oracle's decode over the oracle's
    own cache."""
    T, H, d, L, rk, rv = 4, 2, 64, 256, 16, 32
    m = dims(T, 1, H, d, rk, rv, PER_HEAD, F32)
    sh = param_shapes(m)
    codec = {k: np.zeros(v) for k, v in sh.items()}
    xs = {}
    for h in range(H):
        for kv, r in (("k", rk), ("v", rv)):
            stream = 5000 + 10 * h + (0 if kv == "k" else 5)
            mu, wd, wu = svd_codec_one(rank8_activations(1001, stream, 4096, T * d), r, T, d)
            codec["mu_" + kv][0, h] = mu.reshape(T, d)
            codec["w_down_" + kv][0, h] = wd
            codec["w_up_" + kv][0, h] = wu
            xs[kv + str(h)] = rank8_activations(1001, stream, L, T * d, draw=1)
    codec = {k: store(v, F32) for k, v in codec.items()}
    npages = L // 16
    pt = gen.identity_page_table(1, npages)
    xk = store(np.stack([xs["k%d" % h] for h in range(H)], 1).reshape(1, 1, L, H, T, d), F32)
    xv = store(np.stack([xs["v%d" % h] for h in range(H)], 1).reshape(1, 1, L, H, T, d), F32)
    kp_ref = np.zeros(pool_shape(m, npages, "k"), np.float32)
    vp_ref = np.zeros(pool_shape(m, npages, "v"), np.float32)
    assert oracle.encode(m, codec, kp_ref, vp_ref, pt, xk, xv, np.array([0]), L, 0, 1) == 0

    D = lla.dims_from_dict(m)
    c, keep = device_codec(codec)
    kp_d = torch.full(pool_shape(m, npages, "k"), float("nan"), dtype=torch.float32, device="cuda")
    vp_d = torch.full(pool_shape(m, npages, "v"), float("nan"), dtype=torch.float32, device="cuda")
    pt_d = to_device(pt)
    cache = lla.make_cache(kp_d, vp_d, pt_d, npages)
    ws = lla.workspace(D, lla.OP_ENCODE, 1, 0, 1)
    lla.encode_append(D, c, cache, to_device(xk), to_device(xv), to_device(np.int32([0])), L, 0, 1, ws)
    torch.cuda.synchronize()
    assert lla.device_error_word(ws) == 0
    for g, r in ((kp_d, kp_ref), (vp_d, vp_ref)):
        gh = g.cpu().numpy().astype(np.float64).reshape(-1, g.shape[-1])
        err = row_rel_err(gh, r.astype(np.float64).reshape(-1, r.shape[-1]))
        assert np.isfinite(gh).all() and err.max() <= 1e-4, err.max()

    rope = lla.rope_table(D, L)
    q = gen.normal(1001, 301, (1, H, d), dtype="f32")
    q_d = to_device(q)
    wsd = lla.workspace(D, lla.OP_DECODE, 1, L)
    for t in range(T):
        out = torch.empty_like(q_d)
        lla.decode_attn(D, c, cache, rope, 0, t, q_d, to_device(np.int32([L - 1])), to_device(np.int32([L])),
                        L, out, wsd)
        torch.cuda.synchronize()
        ref, rc = oracle.decode(m, codec, kp_ref, vp_ref, pt, 0, t, q, np.int32([L - 1]), np.int32([L]))
        assert rc == 0
        err = row_rel_err(out_to_f64(out), ref)
        print(f"tiny fp32 GPU encode -> GPU decode, loop {t}: max row rel err {err.max():.3e}", flush=True)
        assert err.max() <= 1e-4
    assert lla.device_error_word(wsd) == 0


# ---------------------------------------------------------------- Ouro-shaped, reduced sizes

@pytest.mark.parametrize("dtype", [BF16, F32])
def test_ouro_shapes_ragged_contexts_shuffled_pages(dtype):
    """H=16, d=128, r_k=16, r_v=32 (21.3x); contexts 1, 17, 300, 1000 (ragged last
    pages, several splits); shuffled page table; N(0,1) latents."""
    m = dims(4, 2, 16, 128, 16, 32, PER_HEAD, dtype)
    ctx = np.array([1, 17, 300, 1000])
    B, pps = len(ctx), 64
    codec = random_codec(m, seed=2002, ortho_down=False)
    kp, vp = random_pools(m, B * pps, seed=2003)
    pt = gen.shuffled_page_table(2004, B, pps)
    q = gen.normal(2005, 1, (B, 16, 128), dtype="bf16" if dtype == BF16 else "f32")
    for layer, loop in ((0, 0), (1, 3)):
        check(m, codec, kp, vp, pt, q, ctx - 1, ctx, layer, loop, f"ouro-small dt={dtype}")


def test_q_position_independent_of_context_and_custom_scale():
    m = dims(2, 1, 16, 128, 16, 32, PER_HEAD, BF16)
    ctx = np.array([64, 200])
    codec = random_codec(m, seed=2102, ortho_down=False)
    kp, vp = random_pools(m, 2 * 13, seed=2103)
    pt = gen.shuffled_page_table(2104, 2, 13)
    q = gen.normal(2105, 1, (2, 16, 128))
    q_pos = np.array([1000, 7])
    got, _ = gpu_decode(m, codec, kp, vp, pt, q, q_pos, ctx, 0, 1, max_ctx=208, scale=0.05,
                        rope_len=1001)
    ref, _ = oracle.decode(m, codec, kp, vp, pt, 0, 1, q, np.int32(q_pos), np.int32(ctx), scale=0.05)
    assert row_rel_err(got, ref).max() <= 2e-2


def test_mild_compression_r96_r160():
    """The 4x point (r_k=96, r_v=160) at a reduced batch and context."""
    m = dims(4, 1, 16, 128, 96, 160, PER_HEAD, BF16)
    ctx = np.array([513, 90])
    codec = random_codec(m, seed=2202, ortho_down=False)
    kp, vp = random_pools(m, 2 * 33, seed=2203)
    pt = gen.shuffled_page_table(2204, 2, 33)
    q = gen.normal(2205, 1, (2, 16, 128))
    check(m, codec, kp, vp, pt, q, ctx - 1, ctx, 0, 2, "r96")


def _scaled(bits: np.ndarray, k: int) -> np.ndarray:
    """bf16 storage array times 2^k (exact: only the exponent changes)."""
    return store(gen.storage_to_f64(bits) * 2.0 ** k, BF16)


@pytest.mark.parametrize("shape", [(128, 16, 32), (128, 96, 160)])
@pytest.mark.parametrize("a,b", [(10, 10), (-10, -6), (-14, 0)])
def test_decoder_fold_range(shape, a, b):
    """Magnitudes far from N(0,1): q x 2^a, W_up,k x 2^b, mu_k x 2^-a and c_k x
    2^-(a+b) leave every score unchanged in exact arithmetic, while the folded
    decoder q' W_up,k grows by 2^(a+b) (2^20: beyond fp16's 65504) or shrinks
    (2^-16: below fp16's normal range).  The result must still match the oracle
    on the scaled inputs within the bf16 bar."""
    d, rk, rv = shape
    m = dims(4, 1, 16, d, rk, rv, PER_HEAD, BF16)
    ctx = np.array([300, 1000])
    codec = random_codec(m, seed=2152, ortho_down=False)
    kp, vp = random_pools(m, 2 * 64, seed=2153)
    pt = gen.shuffled_page_table(2154, 2, 64)
    q = gen.normal(2155, 1, (2, 16, d))
    codec = dict(codec, w_up_k=_scaled(codec["w_up_k"], b), mu_k=_scaled(codec["mu_k"], -a))
    check(m, codec, _scaled(kp, -(a + b)), vp, pt, _scaled(q, a), ctx - 1, ctx, 0, 1, f"range a={a} b={b} {shape}")


# ---------------------------------------------------------------- bitwise properties

def test_deterministic_and_page_table_invariant_bitwise():
    m = dims(4, 1, 16, 128, 16, 32, PER_HEAD, BF16)
    ctx = np.array([1000, 777, 5])
    B, pps = 3, 64
    codec = random_codec(m, seed=2302, ortho_down=False)
    kp, vp = random_pools(m, B * pps, seed=2303)
    pt_id = gen.identity_page_table(B, pps)
    pt_sh = gen.shuffled_page_table(2304, B, pps)
    kp_sh, vp_sh = np.empty_like(kp), np.empty_like(vp)
    kp_sh[:, pt_sh.reshape(-1)] = kp[:, pt_id.reshape(-1)]
    vp_sh[:, pt_sh.reshape(-1)] = vp[:, pt_id.reshape(-1)]
    q = gen.normal(2305, 1, (B, 16, 128))
    a, _ = gpu_decode(m, codec, kp, vp, pt_id, q, ctx - 1, ctx, 0, 1)
    b, _ = gpu_decode(m, codec, kp, vp, pt_id, q, ctx - 1, ctx, 0, 1)
    c, _ = gpu_decode(m, codec, kp_sh, vp_sh, pt_sh, q, ctx - 1, ctx, 0, 1)
    assert np.array_equal(a, b)
    assert np.array_equal(a, c)


def test_split_merges_share_one_workspace_across_shapes():
    """Several context splits per row, merged by the merge launch: one
    workspace serves calls of 4, 48, 49 and again 4 rows (different split
    layouts over the same scratch); every result matches the oracle and the
    header beyond the error word stays zero."""
    m = dims(4, 1, 16, 128, 16, 32, PER_HEAD, BF16)
    D = lla.dims_from_dict(m)
    codec = random_codec(m, seed=2402, ortho_down=False)
    pps = 16
    ws = lla.workspace(D, lla.OP_DECODE, 64, pps * 16)
    for B, seed in ((4, 2410), (48, 2420), (49, 2430), (4, 2440)):
        ctx = 256 - (np.arange(B) * 37) % 200
        kp, vp = random_pools(m, B * pps, seed=seed)
        pt = gen.shuffled_page_table(seed + 1, B, pps)
        q = gen.normal(seed + 2, 1, (B, 16, 128))
        splits, _ = lla.attn_plan(D, lla.OP_DECODE, B, int(ctx.max()))
        assert splits > 1
        got, _ = gpu_decode(m, codec, kp, vp, pt, q, ctx - 1, ctx, 0, 2, max_ctx=int(ctx.max()), ws=ws)
        ref, rc = oracle.decode(m, codec, kp, vp, pt, 0, 2, q, np.int32(ctx - 1), np.int32(ctx))
        assert rc == 0
        err = row_rel_err(got, ref)
        print(f"B={B} splits={splits}: max row rel err {err.max():.3e}", flush=True)
        assert np.isfinite(got).all() and err.max() <= TOL[BF16]
        assert (ws[:256].cpu().numpy() == 0).all()


@pytest.mark.parametrize("dtype", [BF16, F32])
def test_one_long_row_many_splits(dtype):
    """One sequence of 8000 tokens (500 pages): the context is cut into more
    than 64 splits, which a workgroup per (row, head) merges (one split per
    thread), for both storage types."""
    m = dims(4, 1, 16, 128, 16, 32, PER_HEAD, dtype)
    D = lla.dims_from_dict(m)
    ctx = np.array([8000])
    pps = 500
    codec = random_codec(m, seed=2502, ortho_down=False)
    kp, vp = random_pools(m, pps, seed=2503)
    pt = gen.shuffled_page_table(2504, 1, pps)
    q = gen.normal(2505, 1, (1, 16, 128), dtype="bf16" if dtype == BF16 else "f32")
    splits, _ = lla.attn_plan(D, lla.OP_DECODE, 1, int(ctx[0]))
    assert 64 < splits <= 256, splits
    check(m, codec, kp, vp, pt, q, ctx - 1, ctx, 0, 3, f"one long row, {splits} splits, dt={dtype}")


def test_unused_slots_may_hold_nan():
    """Slots past ctx_len inside the last page (and whole unused pages) are never
    read into the result, even when they hold NaN."""
    m = dims(4, 1, 16, 128, 16, 32, PER_HEAD, BF16)
    ctx = np.array([37])
    codec = random_codec(m, seed=2402, ortho_down=False)
    kp, vp = random_pools(m, 4, seed=2403)
    pt = gen.identity_page_table(1, 4)
    kp[:, 2, :, 5:] = 0x7FC1
    vp[:, 2, :, 5:] = 0x7FC1
    kp[:, 3] = 0xFF80
    vp[:, 3] = 0x7FC1
    q = gen.normal(2404, 1, (1, 16, 128))
    check(m, codec, kp, vp, pt, q, ctx - 1, ctx, 0, 0, "nan-tail")


def test_device_side_errors_poison_only_their_rows():
    m = dims(4, 1, 16, 128, 16, 32, PER_HEAD, BF16)
    B, pps = 4, 8
    codec = random_codec(m, seed=2502, ortho_down=False)
    kp, vp = random_pools(m, B * pps, seed=2503)
    pt = gen.identity_page_table(B, pps)
    pt[1, 3] = B * pps + 7                  # page entry out of range
    ctx = np.array([100, 100, 129, 100])     # row 2 exceeds max_ctx=128
    q = gen.normal(2504, 1, (B, 16, 128))
    got, ws = gpu_decode(m, codec, kp, vp, pt, q, np.array([99, 99, 99, 99]), ctx, 0, 0, max_ctx=128)
    assert np.isnan(got[1]).all() and np.isnan(got[2]).all()
    assert np.isfinite(got[0]).all() and np.isfinite(got[3]).all()
    word = lla.device_error_word(ws)
    assert word & lla.DEVERR_PAGE and word & lla.DEVERR_CTX
    ref, _ = oracle.decode(m, codec, kp, vp, pt, 0, 0, q, np.int32([99] * 4), np.int32(ctx))
    assert row_rel_err(got[[0, 3]], ref[[0, 3]]).max() <= 2e-2


# ---------------------------------------------------------------- prefill

@pytest.mark.parametrize("dtype", [BF16, F32])
def test_prefill_matches_oracle(dtype):
    m = dims(4, 1, 16, 128, 16, 32, PER_HEAD, dtype)
    B, pps, n_q = 2, 8, 21
    p0 = np.array([0, 90])
    codec = random_codec(m, seed=2602, ortho_down=False)
    kp, vp = random_pools(m, B * pps, seed=2603)
    pt = gen.shuffled_page_table(2604, B, pps)
    q = gen.normal(2605, 1, (B, n_q, 16, 128), dtype="bf16" if dtype == BF16 else "f32")
    D = lla.dims_from_dict(m)
    c, keep = device_codec(codec)
    kp_d, vp_d, pt_d = to_device(kp), to_device(vp), to_device(pt)
    cache = lla.make_cache(kp_d, vp_d, pt_d, kp.shape[1])
    max_ctx = int(p0.max()) + n_q
    rope = lla.rope_table(D, max_ctx)
    q_d = to_device(q)
    out = torch.empty_like(q_d)
    ws = lla.workspace(D, lla.OP_PREFILL, B, max_ctx, n_q)
    lla.prefill_attn(D, c, cache, rope, 0, 2, n_q, q_d, to_device(np.int32(p0)), max_ctx, out, ws)
    torch.cuda.synchronize()
    got = out_to_f64(out)
    ref, rc = oracle.prefill(m, codec, kp, vp, pt, 0, 2, n_q, q, np.int32(p0))
    assert rc == 0
    err = row_rel_err(got, ref)
    print(f"prefill dt={dtype}: max row rel err {err.max():.3e}")
    assert err.max() <= TOL[dtype]
