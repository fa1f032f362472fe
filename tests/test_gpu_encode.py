"""GPU parity: lla_encode_append (HIP) against the CPU oracle.

Encode is eq. (2) of the LLA pages (c = (x - mu) W_down over the loop-concatenated
pre-RoPE vector), appended at slot(b, pos0[b] + n) of the paged pool.  Checks:
  * placement is bit-exact: every slot the oracle writes is written, every
    other slot keeps its sentinel bits;
  * values: bf16 storage within 2e-2 per latent row (||.||_inf relative) and at
    most one bf16 ulp apart elementwise for nearly all elements (the GPU sums
    x W_down - mu W_down in fp32; the oracle sums (x - mu) W_down in fp64, and
    both round once to bf16); fp32 storage within 1e-4 per row.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from fixtures import BF16, F32, PER_HEAD, TWO_D, dims, pool_shape, random_codec, store
from gpu_util import device_codec, row_rel_err, to_device, to_host
from looped_transformer_latent_amd import gen, lla

pytestmark = pytest.mark.gpu
SENT = {BF16: np.uint16(0x7FC1), F32: np.float32(np.nan)}


def x_shape(m, n_layers, B, n_new):
    if m["variant"] == PER_HEAD:
        return (n_layers, B, n_new, m["H"], m["T"], m["d_head"])
    return (n_layers, B, n_new, m["T"], m["H"], m["d_head"])


def run_both(m, codec, pt, num_pages, pos0, n_new, layer0, n_layers, seed):
    B = pt.shape[0]
    dt = "bf16" if m["dtype"] == BF16 else "f32"
    xk = gen.normal(seed, 401, x_shape(m, n_layers, B, n_new), dtype=dt)
    xv = gen.normal(seed, 402, x_shape(m, n_layers, B, n_new), dtype=dt)
    sent = SENT[m["dtype"]]
    kp = np.full(pool_shape(m, num_pages, "k"), sent)
    vp = np.full(pool_shape(m, num_pages, "v"), sent)
    kp_ref, vp_ref = kp.copy(), vp.copy()
    assert oracle.encode(m, codec, kp_ref, vp_ref, pt, xk, xv, pos0, n_new, layer0, n_layers) == 0

    D = lla.dims_from_dict(m)
    c, keep = device_codec(codec)
    kp_d, vp_d = to_device(kp), to_device(vp)
    cache = lla.make_cache(kp_d, vp_d, to_device(np.ascontiguousarray(pt, np.int32)), num_pages)
    ws = lla.workspace(D, lla.OP_ENCODE, B, 0, n_layers)
    lla.encode_append(D, c, cache, to_device(xk), to_device(xv), to_device(np.int32(pos0)),
                      n_new, layer0, n_layers, ws)
    torch.cuda.synchronize()
    assert lla.device_error_word(ws) == 0
    return (to_host(kp_d), to_host(vp_d)), (kp_ref, vp_ref), (kp, vp)


def placement_report(g_written, r_written):
    """Readable summary of where the written-slot masks differ."""
    diff = np.argwhere(g_written != r_written)
    return (f"written: gpu {int(g_written.sum())}, oracle {int(r_written.sum())}; "
            f"{len(diff)} elements differ, first (layer, page, [head,] row, r): "
            f"{[tuple(int(v) for v in x) for x in diff[:6]]}")


def compare(m, got, ref, init, label):
    for g, r, i in zip(got, ref, init):
        if m["dtype"] == BF16:
            written = r != i
            # placement: bit-exact (a written latent is never the sentinel NaN pattern)
            assert np.array_equal(g != i, written), f"{label}: " + placement_report(g != i, written)
            assert np.array_equal(g[~written], i[~written])
            gv = gen.storage_to_f64(g[written]).reshape(-1, g.shape[-1])
            rv = gen.storage_to_f64(r[written]).reshape(-1, r.shape[-1])
            err = row_rel_err(gv, rv)
            # ulp distance on the bf16 lattice (same-sign values)
            ud = np.abs(g[written].astype(np.int64) - r[written].astype(np.int64))
            same_sign = (g[written] >> 15) == (r[written] >> 15)
            frac_1ulp = np.mean((ud <= 1) & same_sign | (np.abs(gv.reshape(-1) - rv.reshape(-1)) == 0))
            print(f"{label}: rows {gv.shape[0]}, max row rel err {err.max():.3e}, "
                  f"elements within 1 ulp {frac_1ulp:.5f}", flush=True)
            assert err.max() <= 2e-2
            assert frac_1ulp >= 0.995
        else:
            written = ~np.isnan(r)
            assert np.array_equal(~np.isnan(g), written), f"{label}: " + placement_report(~np.isnan(g), written)
            gv = g[written].astype(np.float64).reshape(-1, g.shape[-1])
            rv = r[written].astype(np.float64).reshape(-1, r.shape[-1])
            err = row_rel_err(gv, rv)
            print(f"{label}: rows {gv.shape[0]}, max row rel err {err.max():.3e}", flush=True)
            assert err.max() <= 1e-4


@pytest.mark.parametrize("dtype", [BF16, F32])
def test_encode_per_head_ragged_positions(dtype):
    """4x-compression shapes (r_k=96, r_v=160), 3 sequences appending 37 tokens each
    at positions that start mid-page, cross page boundaries and end mid-page; a
    shuffled page table with pages that no sequence owns; two of three layers."""
    m = dims(4, 3, 16, 128, 96, 160, PER_HEAD, dtype)
    B, pps = 3, 6
    num_pages = B * pps + 5
    pt = gen.shuffled_page_table(3001, B, pps, num_pages)
    codec = random_codec(m, seed=3002, ortho_down=True)
    pos0 = np.array([0, 13, 55])
    got, ref, init = run_both(m, codec, pt, num_pages, pos0, 37, 1, 2, seed=3003)
    compare(m, got, ref, init, f"encode per-head dt={dtype}")


@pytest.mark.parametrize("ranks", [(32, 48), (64, 128), (16, 256), (256, 160)])
def test_encode_rank_tilings(ranks):
    """Every instantiated rank pairing of K and V: the encoder's column tiles and
    its mu W_down tiles are spread over the waves differently for each."""
    rk, rv = ranks
    m = dims(4, 2, 4, 128, rk, rv, PER_HEAD, BF16)
    B, pps = 2, 3
    pt = gen.shuffled_page_table(3401 + rk, B, pps)
    codec = random_codec(m, seed=3402 + rv, ortho_down=True)
    pos0 = np.array([5, 16])
    got, ref, init = run_both(m, codec, pt, B * pps, pos0, 29, 0, 2, seed=3403)
    compare(m, got, ref, init, f"encode r_k={rk} r_v={rv}")


@pytest.mark.parametrize("T", [1, 3, 5])
def test_encode_many_tiles_and_chunk_counts(T):
    """600 tokens per layer (several 256-token workgroups and a ragged last
    one) at widths T x 64 = 64, 192 and 320: one chunk of W_down rows, a whole
    number of three-chunk rounds, and a round with two chunks left over."""
    m = dims(T, 2, 2, 64, 96, 160, PER_HEAD, BF16)
    B, n_new, pps = 3, 200, 14
    pt = gen.shuffled_page_table(3501 + T, B, pps)
    codec = random_codec(m, seed=3502 + T, ortho_down=False)
    pos0 = np.array([0, 9, 21])
    got, ref, init = run_both(m, codec, pt, B * pps, pos0, n_new, 0, 2, seed=3503 + T)
    compare(m, got, ref, init, f"encode T={T} width={64 * T} tokens={B * n_new}")


def test_encode_more_tiles_than_workgroups():
    """288 (token tile, head, layer) tiles for 256 persistent workgroups: some
    workgroups run two tiles, so a tile's output drains while the next one's
    first chunks load (32 heads, 3 layers, 600 tokens, width 64)."""
    m = dims(1, 3, 32, 64, 96, 160, PER_HEAD, BF16)
    B, n_new, pps = 3, 200, 14
    pt = gen.shuffled_page_table(3601, B, pps)
    codec = random_codec(m, seed=3602, ortho_down=False)
    pos0 = np.array([3, 0, 17])
    got, ref, init = run_both(m, codec, pt, B * pps, pos0, n_new, 0, 3, seed=3603)
    compare(m, got, ref, init, "encode 288 tiles")


def test_encode_21x_single_token_all_layers():
    """The decode-step append: one token per sequence into every layer (r_k=16, r_v=32)."""
    m = dims(4, 24, 16, 128, 16, 32, PER_HEAD, BF16)
    B, pps = 5, 2
    pt = gen.shuffled_page_table(3101, B, pps)
    codec = random_codec(m, seed=3102, ortho_down=True)
    pos0 = np.array([0, 15, 16, 31, 7])
    got, ref, init = run_both(m, codec, pt, B * pps, pos0, 1, 0, 24, seed=3103)
    compare(m, got, ref, init, "encode 21x n_new=1")


@pytest.mark.parametrize("dtype", [BF16, F32])
def test_encode_lla2d(dtype):
    """LLA-2D: one latent per token and layer from the [t][h][d] concatenation."""
    m = dims(2, 2, 4, 64, 32, 48, TWO_D, dtype)
    B, pps = 2, 3
    pt = gen.shuffled_page_table(3201, B, pps)
    codec = random_codec(m, seed=3202, ortho_down=True)
    pos0 = np.array([3, 20])
    got, ref, init = run_both(m, codec, pt, B * pps, pos0, 21, 0, 2, seed=3203)
    compare(m, got, ref, init, f"encode 2D dt={dtype}")


@pytest.mark.parametrize("case", ["per-head", "2D"])
def test_encode_split_over_the_width(case):
    """Few tiles over a wide input: the width is cut into ranges whose fp32
    products are added in a second launch (per-head: 4 heads, width 1024, 3
    sequences x 37 tokens -> 4 tiles, 4 ranges; LLA-2D: width 4096, 2 layers,
    16 ranges), ragged positions, shuffled pages."""
    if case == "per-head":
        m = dims(8, 1, 4, 128, 96, 160, PER_HEAD, BF16)
        B, pps, n_new, n_layers = 3, 6, 37, 1
    else:
        m = dims(8, 2, 8, 64, 32, 48, TWO_D, BF16)
        B, pps, n_new, n_layers = 4, 3, 21, 2
    pt = gen.shuffled_page_table(3701, B, pps)
    codec = random_codec(m, seed=3702, ortho_down=False)
    pos0 = np.arange(B) * 7 % 16
    D = lla.dims_from_dict(m)
    assert lla.workspace_bytes(D, lla.OP_ENCODE, B, 0, n_layers) > lla.workspace_bytes(
        lla.dims_from_dict(dict(m, T=1)), lla.OP_ENCODE, B, 0, n_layers)  # the products region
    got, ref, init = run_both(m, codec, pt, B * pps, pos0, n_new, 0, n_layers, seed=3703)
    compare(m, got, ref, init, f"encode split width {case}")


@pytest.mark.timeout(600)
def test_encode_lla2d_benchmark_shape():
    """The LLA-2D decode step's append in the benchmark's launch configuration:
    one token per sequence for 128 sequences into all 4 layers, width
    T H d = 8 x 32 x 128 = 32768, r_k = r_v = 256, seeded x as the benchmark
    draws it, pos0 = 16383.  The pool holds one page per sequence (the token's
    page, shuffled; the launch does not depend on the pool size).  Placement is
    checked bit-exact over every layer; the latents of 8 sequences in layers 0
    and 3 against the oracle's encode."""
    from looped_transformer_latent_amd import workloads as wl
    w = wl.WORKLOADS["lla2d-t8-h32-b128"]
    m = w.dims
    codec_h = wl.codec_host(w)
    B, pos = w.batch, w.ctx - 1
    perm = gen.shuffled_page_table(w.seed, 1, B)[0]
    pt = np.full((B, w.pages_per_seq), -1, np.int32)  # entries never read stay -1
    pt[:, pos // 16] = perm
    sent = SENT[BF16]
    kp = np.full(pool_shape(m, B, "k"), sent)
    vp = np.full(pool_shape(m, B, "v"), sent)
    D = lla.dims_from_dict(m)
    c, keep = device_codec(codec_h)
    kp_d, vp_d = to_device(kp), to_device(vp)
    cache = lla.make_cache(kp_d, vp_d, to_device(pt), B)
    xs = (w.D, B, 1, w.T, w.H, w.d_head)
    x_k = torch.empty(xs, dtype=torch.bfloat16, device="cuda")
    x_v = torch.empty(xs, dtype=torch.bfloat16, device="cuda")
    lla.gen_normal_(x_k, w.seed, wl.STREAMS["x_k"])
    lla.gen_normal_(x_v, w.seed, wl.STREAMS["x_v"])
    ws = lla.workspace(D, lla.OP_ENCODE, B, 0, w.D)
    lla.encode_append(D, c, cache, x_k, x_v, to_device(np.full(B, pos, np.int32)), 1, 0, w.D, ws)
    torch.cuda.synchronize()
    assert lla.device_error_word(ws) == 0
    gk, gv = to_host(kp_d), to_host(vp_d)
    for g, init in ((gk, kp), (gv, vp)):          # placement: row 15 of each token's page only
        written = np.zeros(g.shape[:3], bool)
        written[:, perm, pos % 16] = True
        assert ((g != init).any(axis=-1) == written).all()
        assert (g[:, perm, pos % 16] != sent).all()
    width = w.T * w.H * w.d_head
    rows = np.array([0, 1, 37, 63, 64, 100, 126, 127])
    for layer in (0, w.D - 1):
        m1 = dict(m, D=1)
        codec1 = {k: np.ascontiguousarray(v[layer:layer + 1]) for k, v in codec_h.items()}
        xk = np.concatenate([gen.normal(w.seed, wl.STREAMS["x_k"], (1, 1, 1, w.T, w.H, w.d_head),
                                        offset=(layer * B + b) * width) for b in rows], axis=1)
        xv = np.concatenate([gen.normal(w.seed, wl.STREAMS["x_v"], (1, 1, 1, w.T, w.H, w.d_head),
                                        offset=(layer * B + b) * width) for b in rows], axis=1)
        local = np.arange(len(rows), dtype=np.int32)[:, None]
        kr = np.full((1, len(rows), 16, w.r_k), sent)
        vr = np.full((1, len(rows), 16, w.r_v), sent)
        assert oracle.encode(m1, codec1, kr, vr, local, xk, xv, np.zeros(len(rows), np.int32) + pos % 16,
                             1, 0, 1) == 0
        got = (gk[layer:layer + 1, perm[rows]], gv[layer:layer + 1, perm[rows]])
        init = (np.full_like(kr, sent), np.full_like(vr, sent))
        compare(m1, got, (kr, vr), init, f"encode 2D benchmark shape, layer {layer}")


@pytest.mark.timeout(600)
def test_encode_4x_benchmark_shape():
    """The 4x append in the benchmark's launch configuration: 512 tokens for
    each of 64 sequences into all 24 layers (r_k = 96, r_v = 160, width
    T d = 512 per head), seeded x as the benchmark draws it, pos0 = 7680, so
    every workgroup runs many tiles (both tile parities, several groups and
    layers).  The pool holds the 32 pages each sequence's new tokens land in,
    shuffled among 512 pages that no sequence owns.  Placement is checked
    bit-exact over the whole pool (owned pages fully written, the others
    untouched); the latents of 16 tokens in layers 0, 11 and 23 against the
    oracle's encode."""
    from looped_transformer_latent_amd import workloads as wl
    w = wl.WORKLOADS["ouro1.4b-4x-b64-encode"]
    m = w.dims
    B, n_new = w.batch, w.n_new
    pos0 = w.ctx - n_new
    first, owned = pos0 // 16, n_new // 16
    spare = 512
    perm = np.random.default_rng(w.seed + 7).permutation(B * owned + spare).astype(np.int32)
    pt = np.full((B, w.pages_per_seq), -1, np.int32)  # entries never read stay -1
    pt[:, first:first + owned] = perm[:B * owned].reshape(B, owned)
    num_pages = B * owned + spare
    sent = int(SENT[BF16])
    pools = {kv: torch.full(pool_shape(m, num_pages, kv), sent, dtype=torch.int16, device="cuda")
             for kv in ("k", "v")}
    codec_h = wl.codec_host(w)
    D = lla.dims_from_dict(m)
    c, keep = device_codec(codec_h)
    cache = lla.make_cache(pools["k"].view(torch.bfloat16), pools["v"].view(torch.bfloat16),
                           to_device(pt), num_pages)
    xs = (w.D, B, n_new, w.H, w.T, w.d_head)
    x_k = torch.empty(xs, dtype=torch.bfloat16, device="cuda")
    x_v = torch.empty(xs, dtype=torch.bfloat16, device="cuda")
    lla.gen_normal_(x_k, w.seed, wl.STREAMS["x_k"])
    lla.gen_normal_(x_v, w.seed, wl.STREAMS["x_v"])
    ws = lla.workspace(D, lla.OP_ENCODE, B, 0, w.D)
    lla.encode_append(D, c, cache, x_k, x_v, to_device(np.full(B, pos0, np.int32)), n_new, 0, w.D, ws)
    torch.cuda.synchronize()
    assert lla.device_error_word(ws) == 0
    del x_k, x_v
    used = torch.from_numpy(perm[:B * owned].astype(np.int64)).cuda()
    unused = torch.from_numpy(perm[B * owned:].astype(np.int64)).cuda()
    for kv, t in pools.items():
        for layer in range(w.D):
            assert not (t[layer].index_select(0, used) == sent).any(), f"{kv} layer {layer}: slot left unwritten"
            assert (t[layer].index_select(0, unused) == sent).all(), f"{kv} layer {layer}: page not owned was written"
    width = w.H * w.T * w.d_head
    toks = [(0, 0), (0, 511), (1, 17), (5, 255), (9, 256), (13, 100), (20, 301), (31, 15),
            (32, 16), (40, 479), (47, 480), (50, 7), (55, 333), (60, 128), (62, 500), (63, 511)]
    for layer in (0, 11, w.D - 1):
        m1 = dict(m, D=1)
        codec1 = {k: np.ascontiguousarray(v[layer:layer + 1]) for k, v in codec_h.items()}
        xk = np.concatenate([gen.normal(w.seed, wl.STREAMS["x_k"], (1, 1, 1, w.H, w.T, w.d_head),
                                        offset=((layer * B + b) * n_new + n) * width) for b, n in toks], axis=1)
        xv = np.concatenate([gen.normal(w.seed, wl.STREAMS["x_v"], (1, 1, 1, w.H, w.T, w.d_head),
                                        offset=((layer * B + b) * n_new + n) * width) for b, n in toks], axis=1)
        local = np.arange(len(toks), dtype=np.int32)[:, None]
        slots = np.int32([(pos0 + n) % 16 for _, n in toks])
        kr = np.full((1, len(toks), w.H, 16, w.r_k), SENT[BF16])
        vr = np.full((1, len(toks), w.H, 16, w.r_v), SENT[BF16])
        assert oracle.encode(m1, codec1, kr, vr, local, xk, xv, slots, 1, 0, 1) == 0
        got = (np.full_like(kr, SENT[BF16]), np.full_like(vr, SENT[BF16]))
        for i, (b, n) in enumerate(toks):
            page = int(pt[b, (pos0 + n) // 16])
            for g, t in zip(got, (pools["k"], pools["v"])):
                g[0, i, :, slots[i]] = t[layer, page, :, slots[i]].cpu().numpy().view(np.uint16)
        init = (np.full_like(kr, SENT[BF16]), np.full_like(vr, SENT[BF16]))
        compare(m1, got, (kr, vr), init, f"encode 4x benchmark shape, layer {layer}")


def test_encode_device_errors():
    """A position past the page-table row, or a page entry out of range, is
    flagged in the workspace error word and the slot is not written."""
    m = dims(2, 1, 2, 64, 16, 16, PER_HEAD, BF16)
    B, pps = 2, 2
    pt = gen.identity_page_table(B, pps)
    pt[1, 1] = 999
    codec = random_codec(m, seed=3302, ortho_down=True)
    D = lla.dims_from_dict(m)
    c, keep = device_codec(codec)
    kp = np.full(pool_shape(m, B * pps, "k"), SENT[BF16])
    vp = np.full(pool_shape(m, B * pps, "v"), SENT[BF16])
    kp_d, vp_d = to_device(kp), to_device(vp)
    cache = lla.make_cache(kp_d, vp_d, to_device(pt), B * pps)
    xk = to_device(gen.normal(3303, 401, x_shape(m, 1, B, 4)))
    xv = to_device(gen.normal(3303, 402, x_shape(m, 1, B, 4)))
    ws = lla.workspace(D, lla.OP_ENCODE, B, 0, 1)
    lla.encode_append(D, c, cache, xk, xv, to_device(np.int32([30, 14])), 4, 0, 1, ws)
    torch.cuda.synchronize()
    word = lla.device_error_word(ws)
    assert word & lla.DEVERR_APPEND and word & lla.DEVERR_PAGE
    k_after = to_host(kp_d)
    # sequence 0: positions 30, 31 land in its page 1; 32, 33 are past its row
    assert (k_after[0, 1, :, 14:16] != SENT[BF16]).all()
    # sequence 1: positions 14, 15 in page 2; 16, 17 hit the bad entry and are dropped
    assert (k_after[0, 2, :, 14:16] != SENT[BF16]).all()
    assert (k_after[0, 3] == SENT[BF16]).all()
    assert (k_after[0, 0] == SENT[BF16]).all()
