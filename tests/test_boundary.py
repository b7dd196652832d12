"""Host-side checks of the C ABI (no GPU needed).

The library loads without a GPU; every argument check runs before any HIP
call, so each error code can be provoked here with placeholder pointers.  No
call in this file reaches a kernel launch.
"""
import ctypes
import os
import re

import pytest

from diffusion_self_conditioning_amd import _binding as b

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "softembed.h")
lib = b.lib

# 16-byte aligned placeholder addresses: never dereferenced (calls below fail validation)
P1, P2, P3, P4, P5 = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(se_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) == set(b.EXPORTS)
    raw = ctypes.CDLL(b.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_every_entry_point_has_declared_argument_types():
    """Undeclared ctypes argument types would pass int64 sizes as 32-bit ints."""
    for n in b.EXPORTS:
        fn = getattr(lib, n)
        assert fn.argtypes is not None, n
        decl = re.search(r"(?:se_status|size_t|int32_t|int64_t|const char\*)\s+" + n + r"\s*\(([^)]*)\)",
                         open(HEADER).read())
        params = [x for x in decl.group(1).split(",") if x.strip() not in ("", "void")]
        assert len(fn.argtypes) == len(params), n


def test_status_strings():
    for code, name in enumerate(b.STATUS_NAMES):
        assert b.se_status_string(code).startswith(name)
    assert "gfx950" in b.se_version()


def fused(**kw):
    a = dict(logits=P1, ld=262144, lse=P2, n=256, vocab=262144, s=65536, e=131072, w=P3,
             w_rows=65536, ldw=2816, d=2816, gamma=53.0, out=P4, ldo=2816, ws=P5,
             ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return lib.se_soft_embed_fused(a["logits"], a["ld"], a["lse"], a["n"], a["vocab"], a["s"],
                                   a["e"], a["w"], a["w_rows"], a["ldw"], a["d"], a["gamma"],
                                   a["out"], a["ldo"], a["ws"], a["ws_bytes"], a["stream"])


def unfused(**kw):
    a = dict(probs=P1, ld=262144, n=256, vocab=262144, s=65536, e=131072, w=P3, w_rows=65536,
             ldw=2816, d=2816, gamma=53.0, out=P4, ldo=2816, ws=P5, ws_bytes=1 << 40,
             stream=None)
    a.update(kw)
    return lib.se_soft_embed(a["probs"], a["ld"], a["n"], a["vocab"], a["s"], a["e"], a["w"],
                             a["w_rows"], a["ldw"], a["d"], a["gamma"], a["out"], a["ldo"],
                             a["ws"], a["ws_bytes"], a["stream"])


def test_the_pages_failure_is_an_error_code():
    """Full-width probabilities against a 65,536-row shard (calvarado04.com, 'The symptom')."""
    assert fused(s=0, e=262144) == b.SE_ERR_SLICE
    assert unfused(s=0, e=262144) == b.SE_ERR_SLICE


@pytest.mark.parametrize("call", [fused, unfused])
@pytest.mark.parametrize("kw,code", [
    (dict(w=None), b.SE_ERR_NULL),
    (dict(out=None), b.SE_ERR_NULL),
    (dict(n=-1), b.SE_ERR_SHAPE),
    (dict(d=0), b.SE_ERR_SHAPE),
    (dict(vocab=0), b.SE_ERR_SHAPE),
    (dict(vocab=1 << 31), b.SE_ERR_SHAPE),
    (dict(ld=262143), b.SE_ERR_SHAPE),
    (dict(ldw=2815), b.SE_ERR_SHAPE),
    (dict(ldo=2808), b.SE_ERR_SHAPE),
    (dict(s=-8), b.SE_ERR_SLICE),
    (dict(s=131072, e=65536), b.SE_ERR_SLICE),
    (dict(e=262152), b.SE_ERR_SLICE),
    (dict(w_rows=65535), b.SE_ERR_SLICE),
    (dict(s=65540, e=131072, w_rows=70000), b.SE_ERR_ALIGN),
    (dict(d=2812, ldw=2816, ldo=2816), b.SE_ERR_ALIGN),
    (dict(ldw=2820), b.SE_ERR_ALIGN),
    (dict(ldo=2818), b.SE_ERR_ALIGN),
    (dict(w=P3 + 8), b.SE_ERR_ALIGN),
    (dict(out=P4 + 4), b.SE_ERR_ALIGN),
    (dict(ws_bytes=1024), b.SE_ERR_WORKSPACE),
    (dict(ws=None), b.SE_ERR_NULL),
])
def test_argument_errors(call, kw, code):
    assert call(**kw) == code


def test_input_specific_errors():
    assert fused(lse=None) == b.SE_ERR_NULL
    assert fused(logits=P1 + 4) == b.SE_ERR_ALIGN
    assert fused(ld=262146) == b.SE_ERR_ALIGN
    assert unfused(probs=None) == b.SE_ERR_NULL
    assert unfused(ld=262148) == b.SE_ERR_ALIGN
    assert unfused(probs=P1 + 2) == b.SE_ERR_ALIGN


def test_empty_rows_is_a_noop():
    assert fused(n=0, ws=None, ws_bytes=0) == b.SE_OK
    assert unfused(n=0, ws=None, ws_bytes=0) == b.SE_OK
    assert lib.se_row_stats(P1, 64, 0, 64, P2, P3, P4, P5, None) == b.SE_OK
    assert lib.se_probs_bf16(P1, 64, P2, 0, 64, 0, 64, P3, 64, None) == b.SE_OK
    assert lib.se_probs_bf16(P1, 64, P2, 4, 64, 8, 8, P3, 64, None) == b.SE_OK   # empty slice
    # with no rows, no buffer is touched: NULL pointers are accepted
    assert fused(n=0, logits=None, lse=None, w=None, out=None, ws=None, ws_bytes=0) == b.SE_OK
    assert unfused(n=0, probs=None, w=None, out=None, ws=None, ws_bytes=0) == b.SE_OK
    assert lib.se_row_stats(None, 64, 0, 64, None, None, None, None, None) == b.SE_OK
    # ... but sizes are still checked
    assert fused(n=0, s=0, e=262144, logits=None) == b.SE_ERR_SLICE


def test_row_stats_errors():
    rs = lib.se_row_stats
    assert rs(None, 64, 4, 64, P2, P3, P4, P5, None) == b.SE_ERR_NULL
    assert rs(P1, 64, 4, 64, P2, None, P4, P5, None) == b.SE_ERR_NULL
    assert rs(P1, 60, 4, 64, P2, P3, P4, P5, None) == b.SE_ERR_SHAPE
    assert rs(P1, 64, 4, 0, P2, P3, P4, P5, None) == b.SE_ERR_SHAPE
    assert rs(P1, 66, 4, 64, P2, P3, P4, P5, None) == b.SE_ERR_ALIGN
    assert rs(P1 + 4, 64, 4, 64, P2, P3, P4, P5, None) == b.SE_ERR_ALIGN
    assert rs(P1, 64, 4, 64, P2 + 1, P3, P4, P5, None) == b.SE_ERR_ALIGN


def test_probs_errors():
    pb = lib.se_probs_bf16
    assert pb(P1, 64, P2, 4, 64, 8, 72, P3, 64, None) == b.SE_ERR_SLICE
    assert pb(P1, 64, P2, 4, 64, 4, 8, P3, 64, None) == b.SE_ERR_ALIGN
    assert pb(P1, 64, P2, 4, 64, 8, 16, P3, 60, None) == b.SE_ERR_SHAPE
    assert pb(P1, 64, P2, 4, 64, 8, 16, P3, 68, None) == b.SE_ERR_ALIGN


def test_workspace_plan():
    """256 x 256 output tiles, vocab split in blocks of 128 positions; the split count
    minimises the library's makespan model (waves of workgroups x blocks per workgroup,
    plus the fp32 partials' round trip), at least 2 blocks per split, and is the same on
    a host without a GPU (the MI355X count of 256 CUs).  Partial tiles are fp32."""
    tile = 256 * 256 * 4
    ws = b.se_soft_embed_workspace_bytes
    assert ws(256, 65536, 131072, 2816) == 23 * 11 * tile        # one rank: 11 tiles x 23 splits
    assert ws(256, 0, 262144, 2816) == 23 * 11 * tile
    assert ws(1024, 0, 65536, 2816) == 11 * 44 * tile            # 44 tiles x 11 splits
    assert ws(16, 0, 4096, 256) == 16 * 1 * tile                 # 32 blocks -> 16 splits
    assert ws(16, 0, 64, 256) == 0                               # one block: no split
    assert ws(16, 8, 8, 256) == 0                                # empty slice
    assert ws(0, 0, 4096, 256) == 0


def test_workspace_plan_large_m():
    """Many row tiles: more splits than fit one wave of workgroups can still win, because
    every CU then works (88 tiles x 2 splits would leave 80 of 256 CUs idle)."""
    tile = 256 * 256 * 4
    assert b.se_soft_embed_workspace_bytes(2048, 0, 262144, 2816) == 17 * 88 * tile
    assert b.se_soft_embed_workspace_bytes(4096, 0, 262144, 2816) == 10 * 176 * tile
    assert b.se_soft_embed_workspace_bytes(8192, 0, 262144, 2816) == 8 * 352 * tile


def accept(**kw):
    a = dict(ent=P1, am=P2, n=8, L=256, budget=1.0, k=2, tau=0.5, limit=16, acc=P3, prev=P4,
             sc=P5, stc=P5 + 64, newly=P5 + 128, conv=P5 + 192, stream=None)
    a.update(kw)
    return lib.se_accept_converge(a["ent"], a["am"], a["n"], a["L"], a["budget"], a["k"],
                                  a["tau"], a["limit"], a["acc"], a["prev"], a["sc"], a["stc"],
                                  a["newly"], a["conv"], a["stream"])


def test_accept_converge_errors():
    assert accept(n=-1) == b.SE_ERR_SHAPE
    assert accept(L=0) == b.SE_ERR_SHAPE
    assert accept(L=1025) == b.SE_ERR_SHAPE
    assert accept(k=0) == b.SE_ERR_SHAPE
    assert accept(limit=0) == b.SE_ERR_SHAPE
    assert accept(budget=float("nan")) == b.SE_ERR_SHAPE
    assert accept(tau=float("nan")) == b.SE_ERR_SHAPE
    assert accept(ent=None) == b.SE_ERR_NULL
    assert accept(conv=None) == b.SE_ERR_NULL
    assert accept(am=P2 + 2) == b.SE_ERR_ALIGN
    assert accept(sc=P5 + 1) == b.SE_ERR_ALIGN
    # bytes (accepted, newly, converged) need no alignment; no canvases is a no-op
    assert accept(n=0, ent=None, am=None, acc=None, prev=None, sc=None, stc=None, newly=None,
                  conv=None) == b.SE_OK


def test_reduce_partials_errors():
    rp = lib.se_reduce_partials
    ok = dict(parts=P1, t=4, stride=256 * 2816, n=256, d=2816, ldp=2816, out=P2, ldo=2816,
              ob=P3, ldb=2816)

    def call(**kw):
        a = dict(ok); a.update(kw)
        return rp(a["parts"], a["t"], a["stride"], a["n"], a["d"], a["ldp"], a["out"], a["ldo"],
                  a["ob"], a["ldb"], None)
    assert call(t=0) == b.SE_ERR_SHAPE
    assert call(ldp=2812) == b.SE_ERR_SHAPE
    assert call(stride=100) == b.SE_ERR_SHAPE
    assert call(ldo=2000) == b.SE_ERR_SHAPE
    assert call(parts=None) == b.SE_ERR_NULL
    assert call(out=None, ob=None) == b.SE_ERR_NULL
    assert call(d=2814, ldp=2816, ldo=2816, ldb=2816) == b.SE_ERR_ALIGN
    assert call(out=P2 + 8) == b.SE_ERR_ALIGN
    assert call(ob=P3 + 4) == b.SE_ERR_ALIGN
    assert call(n=0, parts=None, out=None, ob=None) == b.SE_OK


def fp8_call(fused_call, **kw):
    a = dict(a=P1, ld=262144, lse=P2, n=256, vocab=262144, s=65536, e=131072, w=P3, sc=P5 + 256,
             w_rows=65536, ldw=2816, d=2816, gamma=53.0, out=P4, ldo=2816, ws=P5,
             ws_bytes=1 << 40, stream=None)
    a.update(kw)
    if fused_call:
        return lib.se_soft_embed_fp8_fused(a["a"], a["ld"], a["lse"], a["n"], a["vocab"], a["s"],
                                           a["e"], a["w"], a["sc"], a["w_rows"], a["ldw"], a["d"],
                                           a["gamma"], a["out"], a["ldo"], a["ws"], a["ws_bytes"],
                                           a["stream"])
    return lib.se_soft_embed_fp8(a["a"], a["ld"], a["n"], a["vocab"], a["s"], a["e"], a["w"],
                                 a["sc"], a["w_rows"], a["ldw"], a["d"], a["gamma"], a["out"],
                                 a["ldo"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("fused_call", [True, False])
@pytest.mark.parametrize("kw,code", [
    (dict(sc=None), b.SE_ERR_NULL),
    (dict(w=None), b.SE_ERR_NULL),
    (dict(sc=P5 + 2), b.SE_ERR_ALIGN),
    (dict(d=2808, ldw=2816, ldo=2816), b.SE_ERR_ALIGN),      # d % 16
    (dict(ldw=2824), b.SE_ERR_ALIGN),                         # ld_w % 16
    (dict(w=P3 + 8), b.SE_ERR_ALIGN),
    (dict(s=0, e=262144), b.SE_ERR_SLICE),
    (dict(w_rows=65535), b.SE_ERR_SLICE),
    (dict(ws_bytes=1024), b.SE_ERR_WORKSPACE),
    (dict(n=0, a=None, lse=None, w=None, sc=None, out=None, ws=None, ws_bytes=0), b.SE_OK),
])
def test_fp8_soft_embed_errors(fused_call, kw, code):
    assert fp8_call(fused_call, **kw) == code


def test_quantize_table_fp8_errors():
    q = lib.se_quantize_table_fp8
    assert q(P1, 2816, -1, 2816, P2, 2816, P3, None) == b.SE_ERR_SHAPE
    assert q(P1, 2816, 16, 0, P2, 2816, P3, None) == b.SE_ERR_SHAPE
    assert q(P1, 2808, 16, 2816, P2, 2816, P3, None) == b.SE_ERR_SHAPE
    assert q(P1, 2816, 16, 2816, P2, 2800, P3, None) == b.SE_ERR_SHAPE
    assert q(None, 2816, 16, 2816, P2, 2816, P3, None) == b.SE_ERR_NULL
    assert q(P1, 2816, 16, 2816, P2, 2816, None, None) == b.SE_ERR_NULL
    assert q(P1, 2816, 16, 2808, P2, 2816, P3, None) == b.SE_ERR_ALIGN    # d % 16
    assert q(P1, 2820, 16, 2816, P2, 2816, P3, None) == b.SE_ERR_ALIGN    # ld_w % 8
    assert q(P1, 2816, 16, 2816, P2, 2824, P3, None) == b.SE_ERR_ALIGN    # ld_codes % 16
    assert q(P1 + 2, 2816, 16, 2816, P2, 2816, P3, None) == b.SE_ERR_ALIGN
    assert q(P1, 2816, 16, 2816, P2 + 8, 2816, P3, None) == b.SE_ERR_ALIGN
    assert q(P1, 2816, 16, 2816, P2, 2816, P3 + 1, None) == b.SE_ERR_ALIGN
    assert q(None, 2816, 0, 2816, None, 2816, None, None) == b.SE_OK


def onepass_call(**kw):
    a = dict(x=P1, ld=262144, n=256, vocab=262144, s=0, e=262144, w=P3, w_rows=262144, ldw=2816,
             d=2816, gamma=53.0, out=P4, ldo=2816, mx=P5, lse=P5 + 1024, ent=P5 + 2048,
             am=P5 + 4096, ws=P2, ws_bytes=1 << 40, stream=None)
    a.update(kw)
    return lib.se_soft_embed_onepass(a["x"], a["ld"], a["n"], a["vocab"], a["s"], a["e"], a["w"],
                                     a["w_rows"], a["ldw"], a["d"], a["gamma"], a["out"],
                                     a["ldo"], a["mx"], a["lse"], a["ent"], a["am"], a["ws"],
                                     a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(s=8, e=8), b.SE_ERR_SLICE),                  # empty slice: no softmax
    (dict(e=262152), b.SE_ERR_SLICE),
    (dict(w_rows=1000), b.SE_ERR_SLICE),
    (dict(n=-1), b.SE_ERR_SHAPE),
    (dict(ld=100), b.SE_ERR_SHAPE),
    (dict(mx=None), b.SE_ERR_NULL),
    (dict(am=None), b.SE_ERR_NULL),
    (dict(ws=None), b.SE_ERR_NULL),
    (dict(ws_bytes=4096), b.SE_ERR_WORKSPACE),
    (dict(lse=P5 + 1026), b.SE_ERR_ALIGN),
    (dict(x=P1 + 4), b.SE_ERR_ALIGN),
    (dict(ws=P2 + 8), b.SE_ERR_ALIGN),
    (dict(s=4, e=1000), b.SE_ERR_ALIGN),
    (dict(n=0, x=None, w=None, out=None, mx=None, lse=None, ent=None, am=None, ws=None,
          ws_bytes=0), b.SE_OK),
])
def test_onepass_errors(kw, code):
    assert onepass_call(**kw) == code


def test_onepass_workspace_plan():
    """bf16 probabilities of the slice in super-steps of 128 positions, partials of every split
    (kept even for one split), 20 bytes of statistics and a 4-byte factor per (split, row)."""
    ws = b.se_soft_embed_onepass_workspace_bytes
    up = lambda x: (x + 255) // 256 * 256
    tile = 256 * 256 * 4
    assert ws(256, 0, 262144, 2816) == up(256 * 262144 * 2) + up(23 * 11 * tile) + \
        up(23 * 256 * 16) + up(23 * 256 * 4) + up(23 * 256 * 4)
    assert ws(5, 16, 17, 16) == up(5 * 128 * 2) + up(tile) + up(256 * 16) + up(256 * 4) + \
        up(256 * 4)
    assert ws(5, 16, 16, 16) == 0 and ws(0, 0, 64, 16) == 0


def test_merge_slices_errors():
    m = lib.se_merge_slices

    def call(**kw):
        a = dict(outs=P1, t=4, stride=256 * 2816, n=256, d=2816, ldp=2816, mx=P2, lse=P2 + 64,
                 ent=P2 + 128, am=P2 + 192, out=P3, ldo=2816, rmx=P4, rlse=P4 + 64, rent=P4 + 128,
                 ram=P4 + 192)
        a.update(kw)
        return m(a["outs"], a["t"], a["stride"], a["n"], a["d"], a["ldp"], a["mx"], a["lse"],
                 a["ent"], a["am"], a["out"], a["ldo"], a["rmx"], a["rlse"], a["rent"], a["ram"],
                 None)
    assert call(t=0) == b.SE_ERR_SHAPE
    assert call(n=70000) == b.SE_ERR_SHAPE
    assert call(stride=100) == b.SE_ERR_SHAPE
    assert call(ldo=100) == b.SE_ERR_SHAPE
    assert call(outs=None) == b.SE_ERR_NULL
    assert call(ram=None) == b.SE_ERR_NULL
    assert call(d=2814) == b.SE_ERR_ALIGN
    assert call(out=P3 + 8) == b.SE_ERR_ALIGN
    assert call(ent=P2 + 130) == b.SE_ERR_ALIGN
    assert call(n=0, outs=None, out=None) == b.SE_OK


def test_staged_workspace_plan_and_errors():
    """Tiled bf16 probabilities (super-steps of 128 positions) plus the split partials."""
    ws = b.se_soft_embed_staged_workspace_bytes
    up = lambda x: (x + 255) // 256 * 256
    assert ws(256, 65536, 131072, 2816) == up(256 * 65536 * 2) + 23 * 11 * 256 * 256 * 4
    assert ws(16, 0, 64, 256) == up(16 * 128 * 2)                     # one split: no partials
    assert ws(16, 8, 8, 256) == 0
    st = lib.se_soft_embed_staged

    def call(**kw):
        a = dict(x=P1, ld=262144, lse=P2, n=256, vocab=262144, s=65536, e=131072, w=P3,
                 w_rows=65536, ldw=2816, d=2816, gamma=53.0, out=P4, ldo=2816, ws=P5,
                 ws_bytes=1 << 40)
        a.update(kw)
        return st(a["x"], a["ld"], a["lse"], a["n"], a["vocab"], a["s"], a["e"], a["w"],
                  a["w_rows"], a["ldw"], a["d"], a["gamma"], a["out"], a["ldo"], a["ws"],
                  a["ws_bytes"], None)
    assert call(s=0, e=262144) == b.SE_ERR_SLICE          # the pages' failure, as an error code
    assert call(lse=None) == b.SE_ERR_NULL
    assert call(ws=None) == b.SE_ERR_NULL
    assert call(ws_bytes=1024) == b.SE_ERR_WORKSPACE
    assert call(ws=P5 + 8) == b.SE_ERR_ALIGN
    assert call(x=P1 + 4) == b.SE_ERR_ALIGN
    assert call(d=2812, ldw=2816, ldo=2816) == b.SE_ERR_ALIGN
    assert call(n=0, x=None, lse=None, w=None, out=None, ws=None, ws_bytes=0) == b.SE_OK


def test_step_onepass_workspace_plan_and_errors():
    """Tiled bf16 slice, partials of every split (kept even for one split), 20 bytes of
    statistics per (range, row) and a factor per (split, row).  At the one-rank shape the
    row is 22 chunks of 3072 positions before the slice, 23 split ranges, 43 chunks after.
    An empty slice or split ranges too long for the sweep take the two-pass step and its
    workspace."""
    ws = b.se_soft_embed_step_onepass_workspace_bytes
    staged = b.se_soft_embed_staged_workspace_bytes
    up = lambda x: (x + 255) // 256 * 256
    tile = 256 * 256 * 4
    n_r = 22 + 23 + 43
    assert ws(256, 262144, 65536, 131072, 2816) == up(256 * 65536 * 2) + up(23 * 11 * tile) + \
        up(n_r * 256 * 16) + up(n_r * 256 * 4) + up(23 * 256 * 4)
    # slice [16, 17) of 1000 columns, one split: 1 chunk before, 1 range, 1 chunk after
    assert ws(5, 1000, 16, 17, 16) == up(5 * 128 * 2) + up(tile) + up(3 * 5 * 16) + \
        up(3 * 5 * 4) + up(5 * 4)
    assert ws(8, 512, 16, 16, 16) == staged(8, 16, 16, 16) == 0
    assert ws(4096, 110000, 0, 110000, 1024) == staged(4096, 0, 110000, 1024) > 0
    assert ws(4096, 50000, 0, 50000, 1024) != staged(4096, 0, 50000, 1024)   # 8-wave sweep
    assert ws(0, 1000, 0, 64, 16) == 0 and ws(4, 100, 0, 200, 16) == 0
    st = lib.se_soft_embed_step_onepass

    def call(**kw):
        a = dict(x=P1, ld=262144, n=256, vocab=262144, s=65536, e=131072, w=P3, w_rows=65536,
                 ldw=2816, d=2816, gamma=53.0, out=P4, ldo=2816, mx=P2, lse=P2 + 1024,
                 ent=P2 + 2048, am=P2 + 3072, ws=P5, ws_bytes=1 << 40)
        a.update(kw)
        return st(a["x"], a["ld"], a["n"], a["vocab"], a["s"], a["e"], a["w"], a["w_rows"],
                  a["ldw"], a["d"], a["gamma"], a["out"], a["ldo"], a["mx"], a["lse"], a["ent"],
                  a["am"], a["ws"], a["ws_bytes"], None)
    assert call(w_rows=1000) == b.SE_ERR_SLICE
    assert call(ld=1000) == b.SE_ERR_SHAPE
    assert call(x=None) == b.SE_ERR_NULL
    assert call(am=None) == b.SE_ERR_NULL
    assert call(ws=None) == b.SE_ERR_NULL
    assert call(ws_bytes=1024) == b.SE_ERR_WORKSPACE
    assert call(ws=P5 + 8) == b.SE_ERR_ALIGN
    assert call(x=P1 + 4) == b.SE_ERR_ALIGN
    assert call(ent=P2 + 2050) == b.SE_ERR_ALIGN
    assert call(s=65540) == b.SE_ERR_ALIGN
    assert call(n=0, x=None, w=None, out=None, mx=None, lse=None, ent=None, am=None, ws=None,
                ws_bytes=0) == b.SE_OK


def test_workspace_queries_are_thread_safe():
    """The plan reads the per-device compute-unit count once (std::call_once) and is
    otherwise pure: concurrent queries from many threads agree with a serial one."""
    import threading
    shapes = [(256, 65536, 131072, 2816), (2048, 0, 262144, 2816), (16, 0, 4096, 256),
              (1024, 0, 65536, 2816)]
    want = [b.se_soft_embed_workspace_bytes(*sh) for sh in shapes]
    want1 = b.se_soft_embed_step_onepass_workspace_bytes(256, 262144, 65536, 131072, 2816)
    bad = []

    def worker():
        for _ in range(200):
            got = [b.se_soft_embed_workspace_bytes(*sh) for sh in shapes]
            got1 = b.se_soft_embed_step_onepass_workspace_bytes(256, 262144, 65536, 131072, 2816)
            if got != want or got1 != want1:
                bad.append((got, got1))
    ts = [threading.Thread(target=worker) for _ in range(16)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not bad


def test_step_fp8_errors():
    st = lib.se_soft_embed_step_fp8

    def call(**kw):
        a = dict(x=P1, ld=262144, n=256, vocab=262144, s=65536, e=131072, w=P3, sc=P2 + 4096,
                 w_rows=65536, ldw=2816, d=2816, gamma=53.0, out=P4, ldo=2816, mx=P2, lse=P2 + 1024,
                 ent=P2 + 2048, am=P2 + 3072, ws=P5, ws_bytes=1 << 40)
        a.update(kw)
        return st(a["x"], a["ld"], a["n"], a["vocab"], a["s"], a["e"], a["w"], a["sc"],
                  a["w_rows"], a["ldw"], a["d"], a["gamma"], a["out"], a["ldo"], a["mx"], a["lse"],
                  a["ent"], a["am"], a["ws"], a["ws_bytes"], None)
    assert call(w_rows=1000) == b.SE_ERR_SLICE
    assert call(sc=None) == b.SE_ERR_NULL
    assert call(x=None) == b.SE_ERR_NULL
    assert call(d=2808, ldw=2816, ldo=2816) == b.SE_ERR_ALIGN     # d % 16 != 0
    assert call(ldw=2824) == b.SE_ERR_ALIGN                      # ld_w % 16 != 0
    assert call(sc=P2 + 4098) == b.SE_ERR_ALIGN
    assert call(ws_bytes=1024) == b.SE_ERR_WORKSPACE
    assert call(n=0, x=None, w=None, sc=None, out=None, mx=None, lse=None, ent=None, am=None,
                ws=None, ws_bytes=0) == b.SE_OK


def test_step_onepass_fp8_errors():
    """The one-read e4m3 step: the e4m3 table checks, a scale array that must be 16-byte
    aligned (the sweep reads four scales at a time), the one-read workspace; the empty
    slice goes to the two-pass e4m3 step (its own checks)."""
    st = lib.se_soft_embed_step_onepass_fp8

    def call(**kw):
        a = dict(x=P1, ld=262144, n=256, vocab=262144, s=65536, e=131072, w=P3, sc=P2 + 4096,
                 w_rows=65536, ldw=2816, d=2816, gamma=53.0, out=P4, ldo=2816, mx=P2, lse=P2 + 1024,
                 ent=P2 + 2048, am=P2 + 3072, ws=P5, ws_bytes=1 << 40)
        a.update(kw)
        return st(a["x"], a["ld"], a["n"], a["vocab"], a["s"], a["e"], a["w"], a["sc"],
                  a["w_rows"], a["ldw"], a["d"], a["gamma"], a["out"], a["ldo"], a["mx"], a["lse"],
                  a["ent"], a["am"], a["ws"], a["ws_bytes"], None)
    assert call(w_rows=1000) == b.SE_ERR_SLICE
    assert call(ld=1000) == b.SE_ERR_SHAPE
    assert call(sc=None) == b.SE_ERR_NULL
    assert call(x=None) == b.SE_ERR_NULL
    assert call(d=2808, ldw=2816, ldo=2816) == b.SE_ERR_ALIGN     # d % 16 != 0
    assert call(ldw=2824) == b.SE_ERR_ALIGN                      # ld_w % 16 != 0
    assert call(sc=P2 + 4100) == b.SE_ERR_ALIGN                  # 4-byte, not 16-byte aligned
    assert call(s=65540) == b.SE_ERR_ALIGN
    assert call(ws_bytes=1024) == b.SE_ERR_WORKSPACE
    assert call(ws=None) == b.SE_ERR_NULL
    assert call(n=0, x=None, w=None, sc=None, out=None, mx=None, lse=None, ent=None, am=None,
                ws=None, ws_bytes=0) == b.SE_OK
    # empty slice: the two-pass e4m3 step, with the same scale checks
    assert call(s=16, e=16, sc=None) == b.SE_ERR_NULL
    assert call(s=16, e=16, sc=P2 + 4100) == b.SE_ERR_ALIGN


def test_32bit_offset_limits_both_sides():
    """The kernels address staged probabilities, a split's shard rows and a 256-row tile of the
    probability operand with 32-bit byte offsets, so each must stay below 4 GiB; at the limit the
    calls return SE_ERR_SHAPE, just below it they pass the check and stop at the (empty)
    workspace."""
    step = lib.se_soft_embed_step

    def call_step(n=256, s=0, e=262144, ldw=2816, d=2816):
        return step(P1, 262144, n, 262144, s, e, P3, e - s, ldw, d, 53.0, P4, 2816, P2,
                    P2 + 1024, P2 + 2048, P2 + 3072, P5, 0, None)
    # staged bf16 probabilities: n_rows x 262144 positions x 2 bytes
    assert call_step(n=8191) == b.SE_ERR_WORKSPACE           # 4 GiB - 512 KiB
    assert call_step(n=8192) == b.SE_ERR_SHAPE               # 4 GiB exactly
    # the shard slice: (e - s) x ld_w x 2 bytes
    assert call_step(ldw=8184) == b.SE_ERR_WORKSPACE         # 262144 x 8184 x 2 < 2^32
    assert call_step(ldw=8192) == b.SE_ERR_SHAPE             # = 2^32
    fused = lib.se_soft_embed_fused

    def call_fused(ld, ldw=2816, s=65536, e=131072):
        return fused(P1, ld, P2, 256, 262144, s, e, P3, e - s, ldw, 2816, 53.0, P4, 2816, P5, 0,
                     None)
    # one 256-row tile of fp32 logits: 255 x ld x 4 + (e - s) x 4 bytes
    assert call_fused(4210492) == b.SE_ERR_WORKSPACE
    assert call_fused(4210496) == b.SE_ERR_SHAPE
    assert call_fused(262144, ldw=32768) == b.SE_ERR_SHAPE   # 65536 x 32768 x 2 = 2^32
    assert call_fused(262144, ldw=32760) == b.SE_ERR_WORKSPACE


def test_launch_markers_and_split_query():
    assert lib.se_set_launch_events(None, -1) == b.SE_ERR_SHAPE
    assert lib.se_set_launch_events(None, 2) == b.SE_ERR_NULL
    assert lib.se_set_launch_events(None, 0) == b.SE_OK
    assert b.se_launch_events_used() == 0
    b.se_set_launch_events([])
    # the contraction's split ranges (the header's rule); without a device 256 CUs are assumed
    S = b.se_soft_embed_splits(256, 65536, 131072, 2816)
    assert S == 23
    r = b.se_soft_embed_ranges(256, 65536, 131072, 2816)
    assert len(r) == S + 1 and r[0] == 65536 and r[-1] == 131072
    assert all(128 * 22 <= y - x <= 128 * 23 for x, y in zip(r, r[1:]))
    assert all((x - 65536) % 128 == 0 for x in r[:-1])
    assert b.se_soft_embed_splits(16, 0, 64, 256) == 1
    assert b.se_soft_embed_ranges(16, 0, 100, 256) == [0, 100]
    assert b.se_soft_embed_splits(0, 0, 64, 256) == 0 and b.se_soft_embed_splits(4, 8, 8, 16) == 0


def test_mfma_loop_errors():
    assert lib.se_mfma_loop(P1, 0, 10, 1.0, None) == b.SE_ERR_SHAPE
    assert lib.se_mfma_loop(P1, 65537, 10, 1.0, None) == b.SE_ERR_SHAPE
    assert lib.se_mfma_loop(P1, 1, 0, 1.0, None) == b.SE_ERR_SHAPE
    assert lib.se_mfma_loop(P1, 1, (1 << 24) + 1, 1.0, None) == b.SE_ERR_SHAPE
    assert lib.se_mfma_loop(None, 1, 1, 1.0, None) == b.SE_ERR_NULL
    assert lib.se_mfma_loop(P1 + 2, 1, 1, 1.0, None) == b.SE_ERR_ALIGN
