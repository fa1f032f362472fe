"""Pins for the oracle's decode over a sink + window retained set (token
eviction composed with LLA: the close reading, 四:结果 items 9-10, Table 9 keeps
a 4-token sink and a 256-token window).

Reading: of ctx_len tokens, the first n_sink and the last `window` take part;
retained tokens keep their logical positions for RoPE; evicted tokens are never
looked up.  References: the already pinned full-context oracle decode, torch's
float64 SDPA with RoPE as complex rotation, and closed forms.  A slip (an
off-by-one window edge, positions renumbered inside the cache, an evicted page
read, the sink dropped) fails at least one test here.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from fixtures import F32, BF16, PER_HEAD, dims, f64, random_codec, random_pools
from looped_transformer_latent_amd import gen
from test_oracle_pins import gather_latents, rope_complex, sdpa
from test_oracle_pins_decoupled import identity_codec

P = 16


def test_window_covering_the_context_is_plain_decode():
    m = dims(2, 1, 2, 8, 3, 5, PER_HEAD, BF16)
    codec = random_codec(m, seed=400)
    kp, vp = random_pools(m, 4, seed=401)
    pt = gen.shuffled_page_table(402, 2, 2)
    q = gen.normal(403, 1, (2, 2, 8))
    ctx = np.array([29, 7])
    qp = ctx - 1
    want, _ = oracle.decode(m, codec, kp, vp, pt, 0, 1, q, qp, ctx)
    for n_sink, window in ((0, 29), (4, 25), (29, 0), (40, 3), (2, 100)):
        got, rc = oracle.decode_window(m, codec, kp, vp, pt, 0, 1, q, qp, ctx, n_sink, window)
        assert rc == 0 and np.array_equal(got, want), (n_sink, window)


@pytest.mark.parametrize("ctx,window", [(100, 37), (64, 16), (50, 49)])
def test_window_alone_is_decode_of_the_window_at_relative_positions(ctx, window):
    """n_sink = 0: attending over [ctx - W, ctx) at their positions equals the
    plain decode of a sequence holding only those tokens at 0 .. W-1 with the
    query moved by the same offset (RoPE depends on position differences)."""
    m = dims(2, 1, 2, 8, 4, 6, PER_HEAD, F32)
    codec = random_codec(m, seed=410)
    npages = (ctx + P - 1) // P
    kp, vp = random_pools(m, npages, seed=411)
    pt = gen.identity_page_table(1, npages)
    q = gen.normal(412, 1, (1, 2, 8), dtype="f32")
    got, rc = oracle.decode_window(m, codec, kp, vp, pt, 0, 0, q, np.array([ctx - 1]), np.array([ctx]), 0, window)
    assert rc == 0
    # the window's tokens re-packed from position 0
    j0 = ctx - window
    npw = (window + P - 1) // P
    kw = np.zeros((1, npw, 2, P, 4), np.float32)
    vw = np.zeros((1, npw, 2, P, 6), np.float32)
    for i in range(window):
        kw[0, i // P, :, i % P] = kp[0, (j0 + i) // P, :, (j0 + i) % P]
        vw[0, i // P, :, i % P] = vp[0, (j0 + i) // P, :, (j0 + i) % P]
    want, _ = oracle.decode(m, codec, kw, vw, gen.identity_page_table(1, npw), 0, 0, q,
                            np.array([window - 1]), np.array([window]))
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_sink_plus_window_is_rope_attention_over_the_retained_tokens():
    """Identity decoder: keys and values are the latents; reference = torch SDPA
    over the retained tokens rotated at their own positions."""
    T, D, H, d = 2, 1, 2, 16
    ctx, n_sink, window = 90, 4, 37
    m = dims(T, D, H, d, d, d, PER_HEAD, F32)
    codec = identity_codec(m)
    npages = 6
    kp, vp = random_pools(m, npages, seed=420)
    pt = gen.shuffled_page_table(421, 1, npages)
    q = gen.normal(422, 1, (1, H, d), dtype="f32")
    qpos = 95
    got, rc = oracle.decode_window(m, codec, kp, vp, pt, 0, 1, q, np.array([qpos]), np.array([ctx]),
                                   n_sink, window)
    assert rc == 0
    keep = np.r_[np.arange(n_sink), np.arange(ctx - window, ctx)]
    for h in range(H):
        K = gather_latents(kp, pt, 0, ctx, P, h)[0][keep]
        V = gather_latents(vp, pt, 0, ctx, P, h)[0][keep]
        want = sdpa(rope_complex(f64(q)[0, h], qpos), rope_complex(K, keep), V, 1 / math.sqrt(d))
        np.testing.assert_allclose(got[0, h], want, rtol=0, atol=1e-12)


def test_evicted_tokens_are_never_read_and_zero_query_averages_the_retained_set():
    T, D, H, d, r_k, r_v = 2, 1, 2, 8, 3, 5
    ctx, n_sink, window = 150, 4, 40          # retained: 0..3 and 110..149
    m = dims(T, D, H, d, r_k, r_v, PER_HEAD, F32)
    codec = random_codec(m, seed=430, ortho_down=False)
    npages = 10
    kp, vp = random_pools(m, npages, seed=431)
    pt = gen.shuffled_page_table(432, 1, npages)
    q = gen.normal(433, 1, (1, H, d), dtype="f32")
    a, rc = oracle.decode_window(m, codec, kp, vp, pt, 0, 0, q, np.array([149]), np.array([ctx]), n_sink, window)
    assert rc == 0
    # scramble every evicted token's latents and drop the entries of wholly evicted pages
    kp2, vp2, pt2 = kp.copy(), vp.copy(), pt.copy()
    for j in range(n_sink, ctx - window):
        kp2[0, pt[0, j // P], :, j % P] = 1e6
        vp2[0, pt[0, j // P], :, j % P] = -1e6
    for lp in range(1, (ctx - window) // P):    # pages 1 .. 5 hold no retained token
        pt2[0, lp] = -1
    b, rc = oracle.decode_window(m, codec, kp2, vp2, pt2, 0, 0, q, np.array([149]), np.array([ctx]), n_sink, window)
    assert rc == 0 and np.array_equal(a, b)
    # q = 0: the mean of v_hat over exactly the retained tokens
    z, _ = oracle.decode_window(m, codec, kp, vp, pt, 0, 1, np.zeros_like(q), np.array([3]), np.array([ctx]),
                                n_sink, window)
    keep = np.r_[np.arange(n_sink), np.arange(ctx - window, ctx)]
    for h in range(H):
        cv = gather_latents(vp, pt, 0, ctx, P, h)[0][keep]
        wv, muv = f64(codec["w_up_v"])[0, h, 1], f64(codec["mu_v"])[0, h, 1]
        np.testing.assert_allclose(z[0, h], muv + wv @ cv.mean(axis=0), atol=1e-12)
