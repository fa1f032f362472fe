"""GPU parity at the benchmark sizes, on sampled outputs.

The whole workload is built on the device exactly as the benchmark builds it
(the seeded generator fills the pools and q in place; codec parameters come
from the host generator), the call runs in the benchmark's launch
configuration, and a few output rows are recomputed by the CPU oracle from
host-regenerated inputs: the pages of those sequences only, re-indexed through
a local page table.
"""
from __future__ import annotations

import gc

import numpy as np
import pytest
import torch

import oracle
from gpu_util import device_codec, out_to_f64, row_rel_err, to_host
from looped_transformer_latent_amd import gen, lla
from looped_transformer_latent_amd import workloads as wl

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]
TOL = {wl.F32: 1e-4, wl.BF16: 2e-2}


@pytest.fixture
def release():
    yield
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


class Built:
    """Device-resident workload: codec, full pools, page table, RoPE table."""

    def __init__(self, w: wl.Workload):
        self.w = w
        self.D = lla.dims_from_dict(w.dims)
        self.codec_h = wl.codec_host(w)
        self.codec, self._keep = device_codec(self.codec_h)
        self.pt_h = wl.page_table_host(w)
        self.pt = wl.to_device(self.pt_h)
        print(f"[{w.name}] filling pools on the device", flush=True)
        self.k_pool = wl.device_pool(w, "k")
        self.v_pool = wl.device_pool(w, "v")
        self.cache = lla.make_cache(self.k_pool, self.v_pool, self.pt, w.num_pages)
        self.rope = lla.rope_table(self.D, w.ctx)
        torch.cuda.synchronize()

    def decode(self, layer, loop, q_stream_offset=0):
        w = self.w
        dt = torch.bfloat16 if w.dtype == wl.BF16 else torch.float32
        q = torch.empty((w.batch, w.H, w.d_head), dtype=dt, device="cuda")
        lla.gen_normal_(q, w.seed, wl.STREAMS["q"], offset=q_stream_offset)
        ctx = torch.full((w.batch,), w.ctx, dtype=torch.int32, device="cuda")
        out = torch.empty_like(q)
        ws = lla.workspace(self.D, lla.OP_DECODE, w.batch, w.ctx)
        lla.decode_attn(self.D, self.codec, self.cache, self.rope, layer, loop, q, ctx - 1, ctx,
                        w.ctx, out, ws)
        torch.cuda.synchronize()
        assert lla.device_error_word(ws) == 0
        return to_host(q), out_to_f64(out)

    def oracle_rows(self, rows, layer, loop, q_h, from_device=False):
        """Oracle decode of the given sequences at full context."""
        w = self.w
        m1 = dict(w.dims, D=1)
        codec1 = {k: np.ascontiguousarray(v[layer:layer + 1]) for k, v in self.codec_h.items()}
        pages = self.pt_h[rows].reshape(-1)
        if from_device:
            idx = torch.from_numpy(pages.astype(np.int64)).cuda()
            kp = to_host(self.k_pool[layer].index_select(0, idx))[None]
            vp = to_host(self.v_pool[layer].index_select(0, idx))[None]
        else:
            kp = wl.pool_pages_host(w, "k", layer, pages)[None]
            vp = wl.pool_pages_host(w, "v", layer, pages)[None]
        local = np.arange(len(pages), dtype=np.int32).reshape(len(rows), -1)
        ctx = np.full(len(rows), w.ctx, np.int32)
        ref, rc = oracle.decode(m1, codec1, np.ascontiguousarray(kp), np.ascontiguousarray(vp),
                                local, 0, loop, np.ascontiguousarray(q_h[rows]), ctx - 1, ctx)
        assert rc == 0
        return ref


def check_rows(b: Built, rows, layer, loop, from_device=False):
    q_h, got = b.decode(layer, loop, q_stream_offset=(loop * b.w.D + layer) * q_elems(b.w))
    ref = b.oracle_rows(rows, layer, loop, q_h, from_device)
    err = row_rel_err(got[rows], ref)
    print(f"[{b.w.name}] layer {layer} loop {loop} rows {list(rows)}: "
          f"max row rel err {err.max():.3e}", flush=True)
    assert np.isfinite(got).all()
    assert err.max() <= TOL[b.w.dtype]


def q_elems(w):
    return w.batch * w.H * w.d_head


def test_ouro_b32_ctx4096_full(release):
    """Batch 32, context 4096, all 24 layers resident; every row of two calls."""
    b = Built(wl.WORKLOADS["ouro1.4b-21x-b32"])
    check_rows(b, np.arange(32), 23, 3)
    check_rows(b, np.arange(0, 32, 4), 0, 0)


def test_ouro_b768_ctx4096_shuffled_sampled(release):
    """The high-capacity point: batch 768, 4k context, 116 GB shuffled pool; then
    the same calls with a 4-token sink and a 256-token window, as the benchmark
    runs them."""
    b = Built(wl.WORKLOADS["ouro1.4b-21x-b768-paged"])
    check_rows(b, np.array([0, 1, 383, 500, 766, 767]), 23, 3)
    check_rows(b, np.array([2, 640]), 11, 0)
    w = b.w
    layer, loop, rows = 23, 3, np.array([0, 383, 767])
    q = torch.empty((w.batch, w.H, w.d_head), dtype=torch.bfloat16, device="cuda")
    lla.gen_normal_(q, w.seed, wl.STREAMS["q"], offset=12345)
    ctx = torch.full((w.batch,), w.ctx, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    ws = lla.workspace(b.D, lla.OP_WINDOW_DECODE, w.batch, w.ctx, 260)
    lla.decode_window_attn(b.D, b.codec, b.cache, b.rope, layer, loop, q, ctx - 1, ctx, 4, 256, w.ctx, out, ws)
    torch.cuda.synchronize()
    assert lla.device_error_word(ws) == 0
    got = out_to_f64(out)
    m1 = dict(w.dims, D=1)
    codec1 = {k: np.ascontiguousarray(v[layer:layer + 1]) for k, v in b.codec_h.items()}
    pages = b.pt_h[rows].reshape(-1)
    kp = wl.pool_pages_host(w, "k", layer, pages)[None]
    vp = wl.pool_pages_host(w, "v", layer, pages)[None]
    local = np.arange(len(pages), dtype=np.int32).reshape(len(rows), -1)
    c = np.full(len(rows), w.ctx, np.int32)
    ref, rc = oracle.decode_window(m1, codec1, kp, vp, local, 0, loop, np.ascontiguousarray(to_host(q)[rows]),
                                   c - 1, c, 4, 256)
    assert rc == 0
    err = row_rel_err(got[rows], ref)
    print(f"[{w.name}] sink 4 + window 256, rows {list(rows)}: max row rel err {err.max():.3e}", flush=True)
    assert err.max() <= TOL[w.dtype]


def test_ouro_4x_encode_then_decode_sampled(release):
    """4x compression, batch 64: 7680 cached tokens, append 512 per sequence into all
    24 layers with one lla_encode_append call, then decode at context 8192.
    Sampled appended latents are checked against the oracle's encode; the decode
    check reads the GPU-written cache back into the oracle."""
    w = wl.WORKLOADS["ouro1.4b-4x-b64-encode"]
    b = Built(w)
    n_new = w.n_new
    xs = (w.D, w.batch, n_new, w.H, w.T, w.d_head)
    x_k = torch.empty(xs, dtype=torch.bfloat16, device="cuda")
    x_v = torch.empty(xs, dtype=torch.bfloat16, device="cuda")
    lla.gen_normal_(x_k, w.seed, wl.STREAMS["x_k"])
    lla.gen_normal_(x_v, w.seed, wl.STREAMS["x_v"])
    pos0 = torch.full((w.batch,), w.ctx - n_new, dtype=torch.int32, device="cuda")
    ws = lla.workspace(b.D, lla.OP_ENCODE, w.batch, 0, w.D)
    before = to_host(b.k_pool[5, int(b.pt_h[7, (w.ctx - n_new - 1) // 16])])
    lla.encode_append(b.D, b.codec, b.cache, x_k, x_v, pos0, n_new, 0, w.D, ws)
    torch.cuda.synchronize()
    assert lla.device_error_word(ws) == 0
    del x_k, x_v
    # untouched: the page holding position 7679 keeps its generator bits
    after = to_host(b.k_pool[5, int(b.pt_h[7, (w.ctx - n_new - 1) // 16])])
    assert np.array_equal(before, after)

    # sampled appended latents against the oracle's encode of the same x rows
    rng = np.random.default_rng(4001)
    width = w.T * w.d_head
    worst = 0.0
    for _ in range(24):
        layer, bb, n, h = (int(rng.integers(w.D)), int(rng.integers(w.batch)),
                           int(rng.integers(n_new)), int(rng.integers(w.H)))
        flat = (((layer * w.batch + bb) * n_new + n) * w.H + h) * width
        m1 = dict(w.dims, D=1, H=1)
        codec1 = {k: np.ascontiguousarray(v[layer:layer + 1, h:h + 1]) for k, v in b.codec_h.items()}
        xk = gen.normal(w.seed, wl.STREAMS["x_k"], (1, 1, 1, 1, w.T, w.d_head), offset=flat)
        xv = gen.normal(w.seed, wl.STREAMS["x_v"], (1, 1, 1, 1, w.T, w.d_head), offset=flat)
        pos = w.ctx - n_new + n
        kp = np.zeros((1, 1, 1, 16, w.r_k), np.uint16)
        vp = np.zeros((1, 1, 1, 16, w.r_v), np.uint16)
        assert oracle.encode(m1, codec1, kp, vp, np.zeros((1, 1), np.int32), xk, xv,
                             np.array([pos % 16]), 1, 0, 1) == 0
        page = int(b.pt_h[bb, pos // 16])
        gk = to_host(b.k_pool[layer, page, h, pos % 16])
        gv = to_host(b.v_pool[layer, page, h, pos % 16])
        for g, r in ((gk, kp[0, 0, 0, pos % 16]), (gv, vp[0, 0, 0, pos % 16])):
            e = row_rel_err(gen.storage_to_f64(g), gen.storage_to_f64(r))
            worst = max(worst, float(e))
    print(f"[{w.name}] encode: 24 sampled (layer, token, head) rows, max row rel err {worst:.3e}",
          flush=True)
    assert worst <= 2e-2

    check_rows(b, np.array([0, 37, 63]), 23, 3, from_device=True)

    # chunked prefill of the appended chunk: query i of every sequence sits at
    # position 7680 + i; sampled rows against the oracle's decode at that
    # position (causal context 7681 + i), read from the GPU-written cache
    layer, loop = 23, 3
    q = torch.empty((w.batch, n_new, w.H, w.d_head), dtype=torch.bfloat16, device="cuda")
    lla.gen_normal_(q, w.seed, wl.STREAMS["q"], offset=1 << 40)
    out = torch.empty_like(q)
    wsp = lla.workspace(b.D, lla.OP_PREFILL, w.batch, w.ctx, n_new)
    lla.prefill_attn(b.D, b.codec, b.cache, b.rope, layer, loop, n_new, q, pos0, w.ctx, out, wsp)
    torch.cuda.synchronize()
    assert lla.device_error_word(wsp) == 0
    got_all = out_to_f64(out)
    assert np.isfinite(got_all).all()
    q_h = to_host(q)
    m1 = dict(w.dims, D=1)
    codec1 = {k: np.ascontiguousarray(v[layer:layer + 1]) for k, v in b.codec_h.items()}
    worst = 0.0
    for bb, i in ((0, 0), (0, 511), (37, 255), (37, 256), (63, 100)):
        pages = b.pt_h[bb]
        idx = torch.from_numpy(pages.astype(np.int64)).cuda()
        kp = to_host(b.k_pool[layer].index_select(0, idx))[None]
        vp = to_host(b.v_pool[layer].index_select(0, idx))[None]
        local = np.arange(len(pages), dtype=np.int32)[None]
        pos = w.ctx - n_new + i
        ref, rc = oracle.decode(m1, codec1, np.ascontiguousarray(kp), np.ascontiguousarray(vp), local, 0,
                                loop, np.ascontiguousarray(q_h[bb:bb + 1, i]), np.int32([pos]),
                                np.int32([pos + 1]))
        assert rc == 0
        worst = max(worst, float(row_rel_err(got_all[bb, i], ref[0]).max()))
    print(f"[{w.name}] prefill of the 512-token chunk: 5 sampled (sequence, query) rows, "
          f"max row rel err {worst:.3e}", flush=True)
    assert worst <= TOL[w.dtype]


def test_decoupled_ctx256k_in_the_benchmark_configuration(release):
    """Decoupled RoPE at the pages' micro-benchmark context: one sequence of
    262144 tokens, 24 layers of latents and rotary keys resident, the split and
    merge configuration the benchmark times (about a thousand splits).  Both
    calls (two (layer, loop) pairs) against the oracle's plain definition over
    the whole context, all 16 heads."""
    w = wl.WORKLOADS["ouro1.4b-21x-ctx256k-decoupled"]
    b = Built(w)
    kr_pool = wl.device_pool(w, "kr")
    rope_r = lla.rope_table(lla.dims_from_dict(dict(w.dims, d_head=w.d_rope)), w.ctx)
    ctx = torch.full((w.batch,), w.ctx, dtype=torch.int32, device="cuda")
    ws = lla.workspace(b.D, lla.OP_DECOUPLED_DECODE, w.batch, w.ctx, w.d_rope)
    m1 = dict(w.dims, D=1)
    pages = b.pt_h[0]
    for layer, loop in ((23, 3), (4, 0)):
        q = torch.empty((w.batch, w.H, w.q_width), dtype=torch.bfloat16, device="cuda")
        lla.gen_normal_(q, w.seed, wl.STREAMS["q"], offset=layer * 7919 + loop)
        out = torch.empty((w.batch, w.H, w.d_head), dtype=torch.bfloat16, device="cuda")
        lla.decoupled_decode_attn(b.D, b.codec, b.cache, kr_pool, rope_r, layer, loop, q, ctx - 1, ctx, w.ctx,
                                  out, ws)
        torch.cuda.synchronize()
        assert lla.device_error_word(ws) == 0
        got = out_to_f64(out)
        codec1 = {k: np.ascontiguousarray(v[layer:layer + 1]) for k, v in b.codec_h.items()}
        kp = wl.pool_pages_host(w, "k", layer, pages)[None]
        vp = wl.pool_pages_host(w, "v", layer, pages)[None]
        kr = wl.pool_pages_host(w, "kr", layer, pages)[None]
        local = np.arange(len(pages), dtype=np.int32)[None]
        c = np.full(1, w.ctx, np.int32)
        ref, rc = oracle.decoupled_decode(m1, codec1, kp, vp, kr, local, 0, loop, to_host(q), c - 1, c, w.d_rope)
        assert rc == 0
        err = row_rel_err(got, ref)
        print(f"[{w.name}] layer {layer} loop {loop}: all 16 heads over 262144 tokens, "
              f"max row rel err {err.max():.3e}", flush=True)
        assert err.max() <= TOL[w.dtype]
