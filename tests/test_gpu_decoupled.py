"""GPU parity: decoupled-RoPE decode with the K decoder absorbed into the query
(lla_decoupled_decode_attn) and the rotary-key append (lla_rope_key_append),
against the CPU oracle's plain definition (the content key rebuilt by eq. (3),
not rotated; the rotary branch as stored keys dotted with the rotated query;
textbook softmax; V rebuilt per token).

Bars: per output row ||gpu - ref||_inf / ||ref||_inf <= 2e-2 (bf16 storage);
appended rotary keys within one bf16 rounding of the oracle's (both round once,
from fp32 table angles on the GPU and double angles in the oracle); the set of
slots the append writes is exact.
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
SENTINEL = 0x7F7F

SHAPES = [(128, 16, 32, 16, 64), (128, 16, 32, 16, 32), (128, 96, 160, 4, 64), (128, 96, 160, 4, 32)]


def rope_r_table(m, d_rope, n_pos):
    return lla.rope_table(lla.dims_from_dict(dict(m, d_head=d_rope)), n_pos)


def problem(shape, B, ctx_max, seed, extra_pages=1):
    d, rk, rv, H, d_rope = shape
    m = dims(4, 2, H, d, rk, rv, PER_HEAD, BF16)
    pps = (ctx_max + 15) // 16 + extra_pages
    codec = random_codec(m, seed=seed, ortho_down=False)
    kp, vp = random_pools(m, B * pps, seed=seed + 1)
    kr = gen.normal(seed + 2, 1, (m["D"], B * pps, 16, d_rope), dtype="bf16")  # stored (rotated) keys
    pt = gen.shuffled_page_table(seed + 3, B, pps)
    q = gen.normal(seed + 4, 1, (B, H, d + d_rope), dtype="bf16")
    return m, codec, kp, vp, kr, pt, q


def run_decoupled(m, codec, kp, vp, kr, pt, q, q_pos, ctx, layer, loop, max_ctx, rope_len=None, scale=0.0):
    D = lla.dims_from_dict(m)
    d_rope = kr.shape[-1]
    c, keep = device_codec(codec)
    kp_d, vp_d, kr_d = to_device(kp), to_device(vp), to_device(kr)
    pt_d = to_device(np.ascontiguousarray(pt, np.int32))
    cache = lla.make_cache(kp_d, vp_d, pt_d, kp.shape[1])
    rope_r = rope_r_table(m, d_rope, rope_len or max_ctx)
    q_d = to_device(q)
    out = torch.full((q.shape[0], m["H"], m["d_head"]), SENTINEL, dtype=torch.int16, device="cuda")
    out = out.view(torch.bfloat16)
    ws = lla.workspace(D, lla.OP_DECOUPLED_DECODE, pt.shape[0], max_ctx, d_rope)
    lla.decoupled_decode_attn(D, c, cache, kr_d, rope_r, layer, loop, q_d, to_device(np.int32(q_pos)),
                              to_device(np.int32(ctx)), max_ctx, out, ws, scale=scale)
    torch.cuda.synchronize()
    return out_to_f64(out), lla.device_error_word(ws), out


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "d%d_rk%d_rv%d_H%d_dr%d" % s)
def test_decoupled_decode_matches_oracle(shape):
    """Contexts 1, 37, 300 and 4000 (one page, a ragged page, several ring trips,
    several splits), shuffled pages, layer 1 and loop 3 of 2 x 4, queries at the
    last position, at 0 and beyond the context."""
    B = 4
    ctx = np.array([1, 37, 300, 4000])
    q_pos = np.array([0, 36, 5, 4100])
    m, codec, kp, vp, kr, pt, q = problem(shape, B, int(ctx.max()), seed=5100 + shape[1] + shape[4])
    got, errw, _ = run_decoupled(m, codec, kp, vp, kr, pt, q, q_pos, ctx, 1, 3, int(ctx.max()), rope_len=4200)
    ref, rc = oracle.decoupled_decode(m, codec, kp, vp, kr, pt, 1, 3, q, q_pos, ctx, shape[4])
    assert rc == 0 and errw == 0
    err = row_rel_err(got, ref)
    print(f"decoupled {shape}: max row rel err {err.max():.3e}", flush=True)
    assert np.isfinite(got).all()
    assert err.max() <= TOL, err.max()


def test_decoupled_decode_scale_and_page_table_invariance():
    """An explicit scale; the same logical cache behind identity and shuffled
    page tables gives bit-identical outputs."""
    shape = (128, 16, 32, 16, 64)
    B = 2
    ctx = np.array([700, 333])
    q_pos = ctx - 1
    m, codec, kp, vp, kr, _, q = problem(shape, B, int(ctx.max()), seed=5200)
    pps = kp.shape[1] // B
    pt_id = gen.identity_page_table(B, pps)
    pt_sh = gen.shuffled_page_table(5201, B, pps)
    kp_sh, vp_sh, kr_sh = np.empty_like(kp), np.empty_like(vp), np.empty_like(kr)
    for src, dst in ((kp, kp_sh), (vp, vp_sh), (kr, kr_sh)):
        dst[:, pt_sh.reshape(-1)] = src[:, pt_id.reshape(-1)]
    g1, e1, o1 = run_decoupled(m, codec, kp, vp, kr, pt_id, q, q_pos, ctx, 0, 1, 700, scale=0.05)
    g2, e2, o2 = run_decoupled(m, codec, kp_sh, vp_sh, kr_sh, pt_sh, q, q_pos, ctx, 0, 1, 700, scale=0.05)
    assert e1 == 0 and e2 == 0
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    ref, _ = oracle.decoupled_decode(m, codec, kp, vp, kr, pt_id, 0, 1, q, q_pos, ctx, 64, scale=0.05)
    assert row_rel_err(g1, ref).max() <= TOL


def test_decoupled_decode_device_errors():
    """Sequence 0: an out-of-range page-table entry (rows poisoned, PAGE);
    sequence 1: ctx_len beyond max_ctx (CTX); sequence 2: q_pos past the
    rotary table (CTX); sequence 3 is exact."""
    shape = (128, 16, 32, 16, 64)
    B = 4
    ctx = np.array([300, 900, 200, 250])
    m, codec, kp, vp, kr, pt, q = problem(shape, B, 900, seed=5300)
    bad = pt.copy()
    bad[0, 5] = kp.shape[1] + 3
    q_pos = np.array([299, 10, 600, 249])
    got, errw, _ = run_decoupled(m, codec, kp, vp, kr, bad, q, q_pos, ctx, 0, 0, 400, rope_len=512)
    assert errw == (lla.DEVERR_PAGE | lla.DEVERR_CTX), errw
    assert np.isnan(got[:3]).all() and np.isfinite(got[3]).all()
    ref, _ = oracle.decoupled_decode(m, codec, kp, vp, kr, pt, 0, 0, q, q_pos, ctx, 64)
    assert row_rel_err(got[3], ref[3]).max() <= TOL


@pytest.mark.parametrize("d_rope", [64, 32])
def test_rope_key_append_matches_oracle(d_rope):
    """Two layers of a 4-layer pool, 3 sequences x 40 tokens at positions 0,
    9 and 30 (page boundaries inside the chunk), shuffled pages."""
    m = dims(4, 4, 16, 128, 16, 32, PER_HEAD, BF16)
    B, n_new, pps = 3, 40, 5
    pt = gen.shuffled_page_table(5400, B, pps)
    npages = B * pps
    pool0 = np.full((m["D"], npages, 16, d_rope), SENTINEL, np.uint16)
    kr_new = gen.normal(5401, 1, (2, B, n_new, d_rope), dtype="bf16")
    pos0 = np.array([0, 9, 30], np.int32)
    want = pool0.copy()
    assert oracle.rope_key_append(m, d_rope, want, pt, kr_new, pos0, 1) == 0

    D = lla.dims_from_dict(m)
    kp_dummy = torch.zeros(1, dtype=torch.int16, device="cuda")
    cache = lla.make_cache(kp_dummy, kp_dummy, to_device(pt), npages)
    pool_d = to_device(pool0)
    ws = lla.workspace(D, lla.OP_ROPE_KEY_APPEND, B, 0)
    lla.rope_key_append(D, cache, pool_d, rope_r_table(m, d_rope, 128), to_device(kr_new),
                        to_device(pos0), n_new, 1, 2, ws)
    torch.cuda.synchronize()
    assert lla.device_error_word(ws) == 0
    got = to_host(pool_d)
    written = want != SENTINEL
    assert np.array_equal(got != SENTINEL, written)             # exactly the oracle's slots
    g = gen.storage_to_f64(got[written])
    w = gen.storage_to_f64(want[written])
    assert (np.abs(g - w) <= np.abs(w) * 2.0 ** -8 + 1e-30).all()   # within one bf16 rounding


def test_rope_key_append_device_errors():
    """Positions outside the page-table row (APPEND), past the rotary table
    (CTX) and on an invalid page (PAGE) are not written."""
    m = dims(4, 1, 16, 128, 16, 32, PER_HEAD, BF16)
    pt = np.array([[0, 1], [2, 99]], np.int32)
    pool0 = np.full((1, 3, 16, 64), SENTINEL, np.uint16)
    D = lla.dims_from_dict(m)
    dummy = torch.zeros(1, dtype=torch.int16, device="cuda")
    cache = lla.make_cache(dummy, dummy, to_device(pt), 3)
    kr_new = to_device(gen.normal(5500, 1, (1, 2, 8, 64), dtype="bf16"))

    def run(pos0, rope_len):
        pool = to_device(pool0)
        ws = lla.workspace(D, lla.OP_ROPE_KEY_APPEND, 2, 0)
        lla.rope_key_append(D, cache, pool, rope_r_table(m, 64, rope_len), kr_new,
                            to_device(np.array(pos0, np.int32)), 8, 0, 1, ws)
        torch.cuda.synchronize()
        return lla.device_error_word(ws), to_host(pool)

    e, pool = run([28, 4], 64)       # seq 0: positions 32.. beyond its 2 pages
    assert e == lla.DEVERR_APPEND and (pool[0, 1, 12:] != SENTINEL).all() and (pool[0, 1, :12] == SENTINEL).all()
    e, pool = run([0, 10], 12)       # positions 12.. past a 12-row table
    assert e == lla.DEVERR_CTX and (pool[0, 0, :8] != SENTINEL).all() and (pool[0, 2, 12:] == SENTINEL).all()
    e, pool = run([0, 12], 64)       # seq 1 crosses into page entry 99
    assert e == lla.DEVERR_PAGE and (pool[0, 2, 12:] != SENTINEL).all()
