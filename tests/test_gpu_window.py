"""GPU parity: decode with token eviction (lla_decode_window_attn: a sink of
n_sink tokens plus the last `window` tokens, at their own positions) against
the CPU oracle's retained-set decode.

Bars: per output row ||gpu - ref||_inf / ||ref||_inf <= 2e-2 (bf16 storage);
page-table entries of pages with no retained token are never read (set to -1
they change nothing and raise no error).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from fixtures import BF16, PER_HEAD, dims, random_codec, random_pools
from gpu_util import device_codec, out_to_f64, row_rel_err, to_device
from looped_transformer_latent_amd import gen, lla

pytestmark = pytest.mark.gpu
TOL = 2e-2


def run_window(m, codec, kp, vp, pt, q, q_pos, ctx, n_sink, window, layer, loop, max_ctx):
    D = lla.dims_from_dict(m)
    c, keep = device_codec(codec)
    cache = lla.make_cache(to_device(kp), to_device(vp), to_device(np.ascontiguousarray(pt, np.int32)),
                           kp.shape[1])
    rope = lla.rope_table(D, max(max_ctx, int(np.max(q_pos)) + 1))
    q_d = to_device(q)
    out = torch.full(q_d.shape, 0x7F7F, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    ws = lla.workspace(D, lla.OP_WINDOW_DECODE, pt.shape[0], max_ctx, n_sink + window)
    lla.decode_window_attn(D, c, cache, rope, layer, loop, q_d, to_device(np.int32(q_pos)),
                           to_device(np.int32(ctx)), n_sink, window, max_ctx, out, ws)
    torch.cuda.synchronize()
    return out_to_f64(out), lla.device_error_word(ws), out


def problem(shape, B, ctx_max, seed):
    d, rk, rv, H = shape
    m = dims(4, 2, H, d, rk, rv, PER_HEAD, BF16)
    pps = (ctx_max + 15) // 16 + 1
    codec = random_codec(m, seed=seed, ortho_down=False)
    kp, vp = random_pools(m, B * pps, seed=seed + 1)
    pt = gen.shuffled_page_table(seed + 2, B, pps)
    q = gen.normal(seed + 3, 1, (B, H, d), dtype="bf16")
    return m, codec, kp, vp, pt, q


CASES = [((128, 16, 32, 16), 4, 256), ((128, 16, 32, 16), 0, 16), ((128, 16, 32, 16), 20, 37),
         ((128, 96, 160, 16), 4, 256), ((64, 16, 32, 16), 4, 256), ((128, 32, 64, 8), 4, 1024),
         ((128, 16, 32, 16), 4, 8000),  # a budget above max_ctx keeps every token
         ((128, 16, 32, 16), 225, 0), ((128, 16, 32, 16), 4, 0), ((128, 96, 160, 16), 20, 0)]  # sink only


@pytest.mark.parametrize("shape,n_sink,window", CASES, ids=lambda v: str(v))
def test_window_decode_matches_oracle(shape, n_sink, window):
    """Contexts 3 (inside the sink), 100 (nothing evicted yet), 301 (window
    from a mid-page row), 4000 and 4001 (page-aligned and ragged window edge),
    shuffled pages, layer 1 and loop 2."""
    B = 5
    ctx = np.array([3, 100, 301, 4000, 4001])
    q_pos = ctx - 1
    m, codec, kp, vp, pt, q = problem(shape, B, int(ctx.max()), seed=6100 + n_sink + window + shape[1])
    got, errw, _ = run_window(m, codec, kp, vp, pt, q, q_pos, ctx, n_sink, window, 1, 2, int(ctx.max()))
    ref, rc = oracle.decode_window(m, codec, kp, vp, pt, 1, 2, q, q_pos, ctx, n_sink, window)
    assert rc == 0 and errw == 0
    err = row_rel_err(got, ref)
    print(f"window {shape} sink {n_sink} window {window}: max row rel err {err.max():.3e}", flush=True)
    assert np.isfinite(got).all()
    assert err.max() <= TOL, err.max()


def test_evicted_pages_are_never_read():
    """Entries of pages that hold no retained token set to -1 (released): the
    same bits out, no device error; a bad entry on a retained page still
    poisons its row."""
    shape, n_sink, window = (128, 16, 32, 16), 4, 256
    B = 3
    ctx = np.array([4000, 1000, 700])
    q_pos = ctx - 1
    m, codec, kp, vp, pt, q = problem(shape, B, 4000, seed=6200)
    _, e1, o1 = run_window(m, codec, kp, vp, pt, q, q_pos, ctx, n_sink, window, 0, 0, 4000)
    released = pt.copy()
    for b in range(B):
        first_window_page = (ctx[b] - window) // 16
        released[b, 1:first_window_page] = -1
        released[b, (ctx[b] + 15) // 16:] = -1
    g2, e2, o2 = run_window(m, codec, kp, vp, released, q, q_pos, ctx, n_sink, window, 0, 0, 4000)
    assert e1 == 0 and e2 == 0
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    bad = released.copy()
    bad[1, (ctx[1] - 1) // 16] = kp.shape[1] + 7       # the window's last page
    g3, e3, _ = run_window(m, codec, kp, vp, bad, q, q_pos, ctx, n_sink, window, 0, 0, 4000)
    assert e3 == lla.DEVERR_PAGE
    assert np.isnan(g3[1]).all() and np.isfinite(g3[[0, 2]]).all()
    assert np.array_equal(g3[[0, 2]], g2[[0, 2]])


def test_window_decode_with_small_retained_set_at_long_context():
    """Batch 2 at 16384 tokens with a 260-token budget: the plan sizes splits to
    the retained pages (one page-table read per retained page)."""
    shape, n_sink, window = (128, 16, 32, 16), 4, 256
    ctx = np.array([16384, 9000])
    m, codec, kp, vp, pt, q = problem(shape, 2, 16384, seed=6300)
    got, errw, _ = run_window(m, codec, kp, vp, pt, q, ctx - 1, ctx, n_sink, window, 1, 3, 16384)
    ref, rc = oracle.decode_window(m, codec, kp, vp, pt, 1, 3, q, ctx - 1, ctx, n_sink, window)
    assert rc == 0 and errw == 0
    assert row_rel_err(got, ref).max() <= TOL


@pytest.mark.parametrize("n_sink,ctx", [(225, 1000), (4, 1000), (4, 37)])
def test_sink_only_ragged_context(n_sink, ctx):
    """No window (window = 0) at a ragged context: batch 1, 16 heads, context =
    max_ctx.  With sink 225 and ctx 1000 the plan has 4 splits of 5 pages over
    the 15 sink pages, so the last split holds no page; the page of tokens
    992..999 (all evicted) must not become a split of its own.  Entries of every
    page past the sink are released (-1): none of them is read."""
    shape = (128, 16, 32, 16)
    m, codec, kp, vp, pt, q = problem(shape, 1, ctx, seed=6400 + n_sink + ctx)
    c = np.array([ctx])
    released = pt.copy()
    released[0, (n_sink + 15) // 16:] = -1
    got, errw, _ = run_window(m, codec, kp, vp, released, q, c - 1, c, n_sink, 0, 0, 1, ctx)
    ref, rc = oracle.decode_window(m, codec, kp, vp, pt, 0, 1, q, c - 1, c, n_sink, 0)
    assert rc == 0 and errw == 0
    assert np.isfinite(got).all()
    err = row_rel_err(got, ref)
    print(f"sink-only {n_sink} ctx {ctx}: max row rel err {err.max():.3e}", flush=True)
    assert err.max() <= TOL
