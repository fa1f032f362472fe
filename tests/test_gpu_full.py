"""GPU parity: the full ("teacher") K/V cache path -- lla_reconstruct_kv followed
by lla_full_decode_attn -- against the CPU oracle's LLA decode of the same
latents.

Rebuilding K/V exactly (eq. (3), RoPE after reconstruction) and attending over
them is the textbook definition the oracle computes, so the chained result must
match it within the bf16 tolerance (per row ||gpu - ref||_inf / ||ref||_inf <=
2e-2; the full cache adds one rounding of K and V to bf16).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from fixtures import BF16, PER_HEAD, dims, random_codec, random_pools
from gpu_util import device_codec, out_to_f64, row_rel_err, to_device, to_host
from looped_transformer_latent_amd import gen, lla

pytestmark = pytest.mark.gpu
TOL = 2e-2
SENTINEL = 0x7F7F  # finite bf16 bits: slots the rebuild must not touch keep them


def run_full(m, codec, kp, vp, pt, q, q_pos, ctx, layer, loop, max_ctx):
    D = lla.dims_from_dict(m)
    c, keep = device_codec(codec)
    kp_d, vp_d, pt_d = to_device(kp), to_device(vp), to_device(np.ascontiguousarray(pt, np.int32))
    cache = lla.make_cache(kp_d, vp_d, pt_d, kp.shape[1])
    rope = lla.rope_table(D, max_ctx)
    shape = (kp.shape[1], m["H"], 16, m["d_head"])
    k_full = torch.full(shape, SENTINEL, dtype=torch.int16, device="cuda")
    v_full = torch.full(shape, SENTINEL, dtype=torch.int16, device="cuda")
    ctx_d = to_device(np.int32(ctx))
    ws_r = lla.workspace(D, lla.OP_RECONSTRUCT, pt.shape[0], max_ctx)
    lla.reconstruct_kv(D, c, cache, rope, layer, loop, ctx_d, max_ctx, k_full, v_full, ws_r)
    q_d = to_device(q)
    out = torch.empty_like(q_d)
    ws_d = lla.workspace(D, lla.OP_FULL_DECODE, pt.shape[0], max_ctx)
    lla.full_decode_attn(D, cache, k_full, v_full, rope, q_d, to_device(np.int32(q_pos)), ctx_d, max_ctx,
                         out, ws_d)
    torch.cuda.synchronize()
    return (out_to_f64(out), lla.device_error_word(ws_r), lla.device_error_word(ws_d),
            to_host(k_full), to_host(v_full), out)


def problem(shape, B, H, ctx, seed, extra_pages=1):
    d, rk, rv = shape
    m = dims(4, 2, H, d, rk, rv, PER_HEAD, BF16)
    pps = (int(np.max(ctx)) + 15) // 16 + extra_pages
    codec = random_codec(m, seed=seed, ortho_down=False)
    kp, vp = random_pools(m, B * pps, seed=seed + 1)
    pt = gen.shuffled_page_table(seed + 2, B, pps)
    q = gen.normal(seed + 3, 1, (B, H, d), dtype="bf16")
    return m, codec, kp, vp, pt, q


@pytest.mark.parametrize("shape", [(128, 16, 32), (64, 16, 32), (128, 32, 64), (128, 64, 64), (128, 96, 160)],
                         ids=lambda s: "d%d_rk%d_rv%d" % s)
def test_full_cache_decode_matches_oracle(shape):
    """Rebuilt full cache + full-cache decode against the oracle's LLA decode:
    contexts 1, 37, 300 and 4000 (one page, a ragged page, many splits), shuffled
    pages, layer 1 and loop 3 of 2 x 4, query at the last position and at 0."""
    B, H = 4, 4
    ctx = np.array([1, 37, 300, 4000])
    q_pos = np.array([0, 36, 5, 3999])
    m, codec, kp, vp, pt, q = problem(shape, B, H, ctx, seed=4100 + shape[1] + shape[2])
    max_ctx = int(ctx.max())
    got, e_r, e_d, kf, vf, _ = run_full(m, codec, kp, vp, pt, q, q_pos, ctx, 1, 3, max_ctx)
    ref, rc = oracle.decode(m, codec, kp, vp, pt, 1, 3, q, np.int32(q_pos), np.int32(ctx))
    assert rc == 0 and e_r == 0 and e_d == 0
    err = row_rel_err(got, ref)
    print(f"full cache {shape}: max row rel err {err.max():.3e}", flush=True)
    assert np.isfinite(got).all()
    assert err.max() <= TOL, err.max()

    # the rebuild wrote exactly the slots of tokens [0, ctx_len) of each sequence
    written = np.zeros(kp.shape[1] * 16, bool)
    for b in range(B):
        for j in range(int(ctx[b])):
            written[int(pt[b, j // 16]) * 16 + j % 16] = True
    kf2 = kf.reshape(kp.shape[1], H, 16, -1).transpose(0, 2, 1, 3).reshape(kp.shape[1] * 16, -1)
    vf2 = vf.reshape(kp.shape[1], H, 16, -1).transpose(0, 2, 1, 3).reshape(kp.shape[1] * 16, -1)
    assert (kf2[~written] == SENTINEL).all() and (vf2[~written] == SENTINEL).all()
    assert not (kf2[written] == SENTINEL).all(axis=1).any()


def test_full_cache_page_table_invariance_and_errors():
    """Identity vs shuffled page table: bit-identical outputs.  A page-table
    entry out of range sets LLA_DEVERR_PAGE in both calls and poisons its row;
    ctx_len beyond max_ctx sets LLA_DEVERR_CTX."""
    shape = (128, 16, 32)
    B, H = 2, 4
    ctx = np.array([700, 333])
    q_pos = ctx - 1
    m, codec, kp, vp, _, q = problem(shape, B, H, ctx, seed=4200)
    pps = kp.shape[1] // B
    pt_id = gen.identity_page_table(B, pps)
    pt_sh = gen.shuffled_page_table(4201, B, pps)
    kp_sh, vp_sh = np.empty_like(kp), np.empty_like(vp)
    kp_sh[:, pt_sh.reshape(-1)] = kp[:, pt_id.reshape(-1)]
    vp_sh[:, pt_sh.reshape(-1)] = vp[:, pt_id.reshape(-1)]
    max_ctx = int(ctx.max())
    *_, o1 = run_full(m, codec, kp, vp, pt_id, q, q_pos, ctx, 0, 1, max_ctx)
    *_, o2 = run_full(m, codec, kp_sh, vp_sh, pt_sh, q, q_pos, ctx, 0, 1, max_ctx)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))

    bad = pt_id.copy()
    bad[1, 3] = kp.shape[1] + 9
    got, e_r, e_d, *_ = run_full(m, codec, kp, vp, bad, q, q_pos, ctx, 0, 1, max_ctx)
    assert e_r & lla.DEVERR_PAGE and e_d & lla.DEVERR_PAGE
    assert np.isnan(got[1]).all() and np.isfinite(got[0]).all()

    got, e_r, e_d, *_ = run_full(m, codec, kp, vp, pt_id, q, np.array([699, 332]), np.array([700, 800]), 0, 1,
                                 max_ctx)
    assert e_r & lla.DEVERR_CTX and e_d & lla.DEVERR_CTX
    assert np.isnan(got[1]).all()
