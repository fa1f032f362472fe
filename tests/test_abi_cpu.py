"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
its host-side logic (validation, workspace planning, eq. (4)) behaves.  No call
here reaches a kernel launch."""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest

from looped_transformer_latent_amd import lla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NULL = ctypes.c_void_p(0)
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def declared_functions():
    names = set()
    for hdr in os.listdir(os.path.join(ROOT, "include")):
        if hdr.endswith(".h"):
            text = open(os.path.join(ROOT, "include", hdr)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(lla_\w+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    lib = lla.load()
    names = declared_functions()
    assert len(names) >= 9
    for name in names:
        assert hasattr(lib, name), name
    assert set(lla.EXPORTS) <= set(names)


def _dims(**kw):
    base = dict(T=4, D=24, H=16, d_head=128, r_k=16, r_v=32)
    base.update(kw)
    return lla.make_dims(**base)


@pytest.mark.parametrize("rk,rv,teacher_kib,latent_kib", [(96, 160, 768, 192), (16, 32, 768, 36)])
def test_cache_scalars_table5(rk, rv, teacher_kib, latent_kib):
    # Table 5 (cc.laoqi.cc close reading, 四:结果 item 9): KV bytes per token of Ouro-1.4B in bf16
    t, l = lla.cache_scalars(_dims(r_k=rk, r_v=rv))
    assert t * 24 * 2 == teacher_kib * 1024 and l * 24 * 2 == latent_kib * 1024
    t2, l2 = lla.cache_scalars(_dims(r_k=rk, r_v=rv, variant=lla.TWO_D))
    assert t2 == t and l2 * 16 == l


def test_supported_shapes():
    assert lla.supported(_dims(), lla.OP_DECODE)
    assert lla.supported(_dims(dtype=lla.F32, T=4, D=1, H=2, d_head=64), lla.OP_DECODE)
    assert lla.supported(_dims(r_k=96, r_v=160), lla.OP_DECODE)
    assert not lla.supported(_dims(d_head=96), lla.OP_DECODE)
    assert not lla.supported(_dims(r_k=24), lla.OP_DECODE)
    assert lla.supported(_dims(), lla.OP_ENCODE)
    assert not lla.supported(_dims(page_size=32), lla.OP_DECODE)


def test_workspace_bytes_planning():
    d = _dims()
    small = lla.workspace_bytes(d, lla.OP_DECODE, 32, 4096)
    big = lla.workspace_bytes(d, lla.OP_DECODE, 768, 4096)
    assert small >= 256 and big >= 256
    assert lla.workspace_bytes(d, lla.OP_DECODE, 1, 16) == 256          # one split: header only
    assert lla.workspace_bytes(d, lla.OP_DECODE, 32, 0) == 0            # invalid max_ctx
    assert lla.workspace_bytes(_dims(d_head=96), lla.OP_DECODE, 32, 4096) == 0
    # bf16 per-head shapes with a chunked prefill kernel need only the header;
    # other shapes run prefill as decode rows and plan like them (4 x 8 rows)
    assert lla.workspace_bytes(d, lla.OP_PREFILL, 4, 4096, 8) == 256
    assert lla.supported(_dims(H=2), lla.OP_PREFILL)                    # no decode grid needed
    assert lla.workspace_bytes(_dims(H=2), lla.OP_PREFILL, 4, 4096, 300) == 256
    df = _dims(dtype=lla.F32, d_head=64)
    pre = lla.workspace_bytes(df, lla.OP_PREFILL, 4, 4096, 8)
    assert pre == lla.workspace_bytes(df, lla.OP_DECODE, 32, 4096)
    enc = lla.workspace_bytes(d, lla.OP_ENCODE, 64, 0, 24)
    assert enc >= 256 + 4 * 24 * 16 * 48


def _decode(d, cache=None, codec=None, rope=FAKE, rope_len=4096, layer=0, loop=0, q=FAKE,
            q_pos=FAKE, ctx=FAKE, max_ctx=4096, scale=0.0, out=FAKE, ws=FAKE, ws_bytes=1 << 30):
    lib = lla.load()
    codec = codec or lla.Codec(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000)
    cache = cache or lla.Cache(0x1000, 0x1000, 0x1000, 32, 256, 8192)
    return lib.lla_decode_attn(ctypes.byref(d) if d is not None else None, ctypes.byref(codec),
                               ctypes.byref(cache), rope, rope_len, layer, loop, q, q_pos, ctx,
                               max_ctx, scale, out, ws, ws_bytes, NULL)


def test_decode_validation_errors():
    d = _dims()
    E = lla.ERR_INVALID_ARG
    assert _decode(None) == E
    assert _decode(d, layer=24) == E and _decode(d, layer=-1) == E
    assert _decode(d, loop=4) == E
    assert _decode(d, rope=NULL) == E
    assert _decode(d, max_ctx=4097) == E                                 # beyond the RoPE table
    assert _decode(d, max_ctx=0) == E
    assert _decode(d, rope_len=1 << 20, max_ctx=256 * 16 + 1) == E       # beyond the page table
    assert _decode(d, q=NULL) == E and _decode(d, out=NULL) == E and _decode(d, ctx=NULL) == E
    assert _decode(d, scale=-1.0) == E or _decode(d, scale=float("nan")) == E
    assert _decode(d, codec=lla.Codec(0x1000, 0, 0x1000, 0x1000, 0x1000, 0x1000)) == E
    assert _decode(d, cache=lla.Cache(0x1000, 0x1000, 0, 32, 256, 8192)) == E
    assert _decode(_dims(d_head=96)) == lla.ERR_UNSUPPORTED
    assert _decode(_dims(page_size=8)) == E
    assert _decode(d, ws_bytes=16) == lla.ERR_WORKSPACE
    assert _decode(d, ws=NULL) == lla.ERR_WORKSPACE
    assert b"workspace" in lla.load().lla_last_error()


def test_encode_and_prefill_validation_errors():
    lib = lla.load()
    d = _dims()
    codec = lla.Codec(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000)
    cache = lla.Cache(0x1000, 0x1000, 0x1000, 64, 512, 32768)
    enc = lambda **kw: lib.lla_encode_append(
        ctypes.byref(d), ctypes.byref(kw.get("codec", codec)), ctypes.byref(cache), FAKE, FAKE,
        kw.get("pos0", FAKE), kw.get("n_new", 512), kw.get("layer0", 0), kw.get("n_layers", 24),
        kw.get("ws", FAKE), kw.get("ws_bytes", 16), NULL)
    assert enc(layer0=1) == lla.ERR_INVALID_ARG                         # 1 + 24 > D
    assert enc(n_new=-1) == lla.ERR_INVALID_ARG
    assert enc(pos0=NULL) == lla.ERR_INVALID_ARG
    assert enc(codec=lla.Codec(0x1000, 0x1000, 0, 0x1000, 0x1000, 0x1000)) == lla.ERR_INVALID_ARG
    assert enc() == lla.ERR_WORKSPACE
    pre = lib.lla_prefill_attn(ctypes.byref(d), ctypes.byref(codec), ctypes.byref(cache), FAKE,
                               8192, 0, 0, -1, FAKE, FAKE, 8192, 0.0, FAKE, FAKE, 1 << 30, NULL)
    assert pre == lla.ERR_INVALID_ARG
    assert lib.lla_rope_table(ctypes.byref(d), -1, FAKE, NULL) == lla.ERR_INVALID_ARG
    assert lla.load().lla_status_string(lla.ERR_WORKSPACE) == b"workspace missing or too small"


def test_full_cache_validation_and_planning():
    """Host-side checks of lla_reconstruct_kv / lla_full_decode_attn (no launch)."""
    lib = lla.load()
    d = _dims()
    codec = lla.Codec(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000)
    cache = lla.Cache(0x1000, 0x1000, 0x1000, 32, 256, 8192)
    E = lla.ERR_INVALID_ARG
    rec = lambda **kw: lib.lla_reconstruct_kv(
        ctypes.byref(kw.get("dims", d)), ctypes.byref(codec), ctypes.byref(cache), kw.get("rope", FAKE), 4096,
        kw.get("layer", 0), kw.get("loop", 0), kw.get("ctx", FAKE), kw.get("max_ctx", 4096),
        kw.get("kf", FAKE), FAKE, kw.get("ws", FAKE), kw.get("ws_bytes", 16), NULL)
    assert rec(layer=24) == E and rec(loop=4) == E
    assert rec(rope=NULL) == E and rec(max_ctx=4097) == E and rec(ctx=NULL) == E and rec(kf=NULL) == E
    assert rec(dims=_dims(dtype=lla.F32, d_head=64)) == lla.ERR_UNSUPPORTED
    assert rec() == lla.ERR_WORKSPACE
    full = lambda **kw: lib.lla_full_decode_attn(
        ctypes.byref(kw.get("dims", d)), ctypes.byref(cache), FAKE, FAKE, FAKE, 4096, kw.get("q", FAKE),
        FAKE, FAKE, kw.get("max_ctx", 4096), 0.0, FAKE, FAKE, kw.get("ws_bytes", 16), NULL)
    assert full(q=NULL) == E and full(max_ctx=0) == E
    assert full(dims=_dims(H=6)) == lla.ERR_UNSUPPORTED
    assert full() == lla.ERR_WORKSPACE
    # workspace: header only for the rebuild; split partials (d_head + 2 floats) for the decode
    assert lla.workspace_bytes(d, lla.OP_RECONSTRUCT, 32, 4096) == 256
    big = lla.workspace_bytes(d, lla.OP_FULL_DECODE, 32, 4096)
    assert big > 256 and (big - 256) % (32 * 16 * (128 + 2) * 4) < 256
    assert lla.workspace_bytes(d, lla.OP_FULL_DECODE, 1024, 4096) == 256   # one split at large batch
    assert lla.supported(d, lla.OP_RECONSTRUCT) and lla.supported(d, lla.OP_FULL_DECODE)
    assert lla.supported(_dims(r_k=96, r_v=160), lla.OP_RECONSTRUCT)
    assert not lla.supported(_dims(r_k=48, r_v=96), lla.OP_RECONSTRUCT)


def test_decoupled_validation_and_planning():
    """Host-side checks of lla_rope_key_append / lla_decoupled_decode_attn (no launch)."""
    lib = lla.load()
    d = _dims()
    codec = lla.Codec(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000)
    cache = lla.Cache(0x1000, 0x1000, 0x1000, 32, 256, 8192)
    E = lla.ERR_INVALID_ARG
    app = lambda **kw: lib.lla_rope_key_append(
        ctypes.byref(kw.get("dims", d)), ctypes.byref(cache), kw.get("d_rope", 64), kw.get("pool", FAKE), FAKE,
        kw.get("rope_len", 4096), FAKE, FAKE, kw.get("n_new", 1), kw.get("layer0", 0), kw.get("n_layers", 1),
        kw.get("ws", FAKE), kw.get("ws_bytes", 16), NULL)
    assert app(d_rope=63) == E and app(d_rope=0) == E and app(pool=NULL) == E and app(rope_len=0) == E
    assert app(layer0=24) == E and app(n_new=-1) == E
    assert app(dims=_dims(dtype=lla.F32, d_head=64)) == lla.ERR_UNSUPPORTED
    assert app() == lla.ERR_WORKSPACE
    dec = lambda **kw: lib.lla_decoupled_decode_attn(
        ctypes.byref(kw.get("dims", d)), ctypes.byref(codec), ctypes.byref(cache), kw.get("d_rope", 64),
        kw.get("kr", FAKE), FAKE, 4096, kw.get("layer", 0), 0, kw.get("q", FAKE), FAKE, FAKE,
        kw.get("max_ctx", 4096), 0.0, FAKE, FAKE, kw.get("ws_bytes", 16), NULL)
    assert dec(kr=NULL) == E and dec(q=NULL) == E and dec(layer=24) == E and dec(max_ctx=0) == E
    assert dec(max_ctx=256 * 16 + 1) == E
    assert dec(d_rope=48) == lla.ERR_UNSUPPORTED and dec(dims=_dims(H=8)) == lla.ERR_UNSUPPORTED
    assert dec() == lla.ERR_WORKSPACE
    # planning: as the latent decode (16 heads per workgroup), partials r_v + 2 when split
    assert lla.workspace_bytes(d, lla.OP_ROPE_KEY_APPEND, 32, 0) == 256
    big = lla.workspace_bytes(d, lla.OP_DECOUPLED_DECODE, 1, 262144, 64)
    assert big > 256 and (big - 256) % (16 * 34 * 4) < 256
    assert lla.workspace_bytes(d, lla.OP_DECOUPLED_DECODE, 1024, 4096, 64) == 256
    assert lla.workspace_bytes(d, lla.OP_DECOUPLED_DECODE, 1, 4096, 48) == 0
    assert lla.supported(d, lla.OP_DECOUPLED_DECODE) and lla.supported(_dims(r_k=96, r_v=160, H=4),
                                                                       lla.OP_DECOUPLED_DECODE)
    assert not lla.supported(_dims(r_k=32, r_v=64), lla.OP_DECOUPLED_DECODE)


def test_window_validation_and_planning():
    """Host-side checks of lla_decode_window_attn (no launch)."""
    lib = lla.load()
    d = _dims()
    codec = lla.Codec(0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000)
    cache = lla.Cache(0x1000, 0x1000, 0x1000, 32, 256, 8192)
    E = lla.ERR_INVALID_ARG
    win = lambda **kw: lib.lla_decode_window_attn(
        ctypes.byref(kw.get("dims", d)), ctypes.byref(codec), ctypes.byref(cache), FAKE, 4096, 0, 0, FAKE, FAKE,
        FAKE, kw.get("n_sink", 4), kw.get("window", 256), kw.get("max_ctx", 4096), 0.0, FAKE, FAKE,
        kw.get("ws_bytes", 16), NULL)
    assert win(n_sink=-1) == E and win(window=-2) == E and win(n_sink=0, window=0) == E
    assert win(n_sink=1 << 29, window=(1 << 29) + 1) == E                # budget beyond 2^30
    assert win(n_sink=100, window=5000) == lla.ERR_WORKSPACE             # a budget above max_ctx is valid
    assert win(dims=_dims(dtype=lla.F32, d_head=64)) == lla.ERR_UNSUPPORTED
    assert win() == lla.ERR_WORKSPACE
    # a 260-token budget plans like a 260 + 2 page context, not like 4096
    assert lla.workspace_bytes(d, lla.OP_WINDOW_DECODE, 1, 4096, 260) == \
        lla.workspace_bytes(d, lla.OP_DECODE, 1, 16 * (17 + 2))
    assert lla.workspace_bytes(d, lla.OP_WINDOW_DECODE, 1, 4096, 0) == 0
    assert lla.supported(d, lla.OP_WINDOW_DECODE) and not lla.supported(_dims(dtype=lla.F32, d_head=64),
                                                                         lla.OP_WINDOW_DECODE)


def test_m0_check_of_the_build():
    """The build's scan of device assembly for M0 uses outside the LDS copy
    blocks (the copies set M0 themselves from inline assembly)."""
    from looped_transformer_latent_amd import build
    ok = "\ts_mov_b32 m0, s4\n\tglobal_load_lds_dwordx4 v[2:3], off\n\tv_mov_b32 v1, v2 ; m0 in a comment\n"
    assert build.m0_misuse(ok) is None
    assert build.m0_misuse(ok + "\ts_mov_b32 m0, -1\n\tds_read_b32 v1, v2\n") == "s_mov_b32 m0, -1"
    assert build.m0_misuse("\tv_movrels_b32 v1, v2\n\ts_add_i32 s5, m0, 4\n") == "s_add_i32 s5, m0, 4"
    built = os.path.join(ROOT, "_build", "lla_encode.hip.s")
    if os.path.exists(built):  # written by the last build
        assert build.m0_misuse(open(built).read()) is None


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: asked for more it prints one JSON line saying
    so and exits non-zero, before touching a device."""
    import json
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_profiled_traffic_needs_matching_sources(tmp_path, monkeypatch):
    """The bench reports a kernel's profiled HBM traffic only while the digest
    in its profile matches the current sources."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    (tmp_path / "profiles").mkdir()
    good = bench.kernel_source_digest(bench.DECODE_SOURCES)
    (tmp_path / "profiles" / "decode_g_kernel_w1.md").write_text(
        f"# x\nkernel_source_sha256: {good}\ntraffic_bytes_per_launch: 1234\n")
    (tmp_path / "profiles" / "decode_g_kernel_w2.md").write_text(
        "# x\nkernel_source_sha256: 00\ntraffic_bytes_per_launch: 1234\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    # the sources are still those of the repository
    monkeypatch.setattr(bench, "kernel_source_digest", lambda names=bench.DECODE_SOURCES: good)
    assert bench.profiled_traffic("w1") == 1234
    assert bench.profiled_traffic("w2") is None
    assert bench.profiled_traffic("w3") is None


def _retained_pages_brute(ctx, n_sink, window):
    """Pages holding at least one retained token, from the definition: token j of
    [0, ctx) is kept when j < n_sink or j >= ctx - window."""
    return sorted({j // 16 for j in range(ctx) if j < n_sink or j >= ctx - window})


@pytest.mark.parametrize("batch,max_ctx,n_sink,window", [
    (1, 1000, 225, 0), (1, 1000, 4, 0), (5, 4001, 225, 0), (768, 4096, 4, 256), (1, 4096, 4, 256),
    (3, 16384, 4, 256), (2, 300, 20, 37), (1, 4000, 0, 16), (1, 4000, 17, 1), (64, 8192, 1024, 1024),
    (1, 257, 300, 0), (1, 5000, 0, 4999)])
def test_window_plan_reads_only_retained_pages(batch, max_ctx, n_sink, window):
    """The windowed decode's splits run over exactly the pages that hold a
    retained token (lla_window_pages, the rule the kernel itself evaluates),
    every such page lies in some split, so no split can see only evicted
    tokens; a split past the last such page is empty and merges with weight 0."""
    d = _dims()
    splits, pps = lla.attn_plan(d, lla.OP_WINDOW_DECODE, batch, max_ctx, n_sink + window)
    rng = np.random.default_rng(max_ctx + n_sink + window)
    ctxs = sorted(set(range(1, min(max_ctx, 70) + 1)) | set(rng.integers(1, max_ctx + 1, 60).tolist()) |
                  {max_ctx, max(1, max_ctx - 1)})
    for ctx in ctxs:
        n_a, p_b = lla.window_pages(ctx, n_sink, window)
        npages = (ctx + 15) // 16
        virtual = list(range(n_a)) + list(range(p_b, npages))
        assert virtual == _retained_pages_brute(ctx, n_sink, window), (ctx, n_a, p_b)
        assert len(virtual) <= splits * pps, (ctx, splits, pps)


def test_window_plan_sink_only_case_has_an_empty_split():
    """Batch 1, 16 heads, sink 225, no window, ctx = max_ctx = 1000: 4 splits of 5
    pages over 15 sink pages; the last split holds no page at all (the page of
    tokens 992..999, all evicted, is not one of them)."""
    d = _dims()
    assert lla.attn_plan(d, lla.OP_WINDOW_DECODE, 1, 1000, 225) == (4, 5)
    assert lla.window_pages(1000, 225, 0) == (15, 63)
    assert lla.window_pages(1000, 4, 256) == (1, 46)
    with pytest.raises(lla.LlaError):
        lla.window_pages(10, 0, 0)
    with pytest.raises(lla.LlaError):
        lla.attn_plan(_dims(d_head=96), lla.OP_DECODE, 1, 100)


def test_lla2d_plan_stays_within_the_staged_page_table():
    """LLA-2D workgroups stage at most 1024 page-table entries: long contexts at
    large batch get several splits of whole 32-token blocks (even page counts)."""
    d = _dims(T=8, D=4, H=32, d_head=128, r_k=256, r_v=256, variant=lla.TWO_D)
    for batch, ctx in ((128, 16384), (128, 40000), (1, 1 << 20), (512, 2049)):
        splits, pps = lla.attn_plan(d, lla.OP_DECODE, batch, ctx)
        assert pps <= 1024 and pps % 2 == 0 and splits * pps * 16 >= ctx, (batch, ctx, splits, pps)
    assert lla.attn_plan(d, lla.OP_DECODE, 128, 40000)[0] >= 3
