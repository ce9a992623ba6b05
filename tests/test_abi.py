"""The C ABI on the CPU: the library loads without a GPU, exports exactly what
include/zl_attn.h declares, sizes workspaces, and rejects every bad argument
with the documented status before making any HIP call."""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zl_attn.h")


@pytest.fixture(scope="module")
def zl():
    import mla_attention_amd
    if not os.path.exists(mla_attention_amd.LIB_PATH):
        from mla_attention_amd import build
        build.build()
    mla_attention_amd.library()
    return mla_attention_amd


def declared_symbols():
    text = open(HEADER).read()
    return set(re.findall(r"^ZL_API [^;(]*?\b(zl_\w+)\s*\(", text, flags=re.M))


def test_header_declares_the_boundary():
    names = declared_symbols()
    for required in ("zl_decode_attn_gqa", "zl_decode_attn_mla", "zl_attn_combine",
                     "zl_decode_attn_workspace_size", "zl_status_string"):
        assert required in names


def test_library_exports_every_declared_symbol(zl):
    lib = zl.library()
    for name in declared_symbols():
        assert hasattr(lib, name), name
    assert declared_symbols() == set(zl.SIGNATURES), "binding signatures out of step with the header"
    nm = os.popen(f"nm -D --defined-only {zl.LIB_PATH}").read()
    exported = set(re.findall(r" T (zl_\w+)", nm))
    assert exported == declared_symbols()


def test_status_strings(zl):
    for code, name in [(0, "ZL_OK"), (1, "ZL_ERR_INVALID_ARGUMENT"), (2, "ZL_ERR_UNSUPPORTED"),
                       (3, "ZL_ERR_WORKSPACE_TOO_SMALL"), (4, "ZL_ERR_HIP")]:
        assert zl.zl_status_string(code) == name
    assert "unknown" in zl.zl_status_string(99)


def test_workspace_sizes(zl):
    lib = zl.library()
    s = lib.zl_decode_attn_workspace_size(32, 32, 8, 128, 4096, 0)
    assert s > 0 and s % 4 == 0
    # two partial slots per worker: independent of the batch, grows with workers and head dim
    assert lib.zl_decode_attn_workspace_size(64, 32, 8, 128, 4096, 0) == s
    assert lib.zl_decode_attn_workspace_size_ex(32, 32, 8, 128, 4096, 0, 4096) > s
    assert lib.zl_decode_attn_workspace_size_ex(32, 32, 8, 64, 4096, 0, 768) < s
    assert lib.zl_decode_attn_mla_workspace_size(32, 16, 512, 64, 8192, 1) > 0
    # invalid shapes -> 0
    for args in [(32, 32, 8, 96, 4096, 0), (32, 30, 8, 128, 4096, 0), (-1, 32, 8, 128, 4096, 0),
                 (32, 32, 8, 128, -5, 0), (32, 32, 8, 128, 4096, 7), (32, 40, 2, 128, 64, 0)]:
        assert lib.zl_decode_attn_workspace_size(*args) == 0, args
    assert lib.zl_decode_attn_workspace_size_ex(32, 32, 8, 128, 4096, 0, 12) == 0   # not a multiple of 8
    assert lib.zl_decode_attn_mla_workspace_size(32, 16, 256, 64, 8192, 1) == 0


BIG = 1 << 20
A = 0x100000  # a 256-byte aligned fake address: never dereferenced (validation fails first)


def gqa(lib, **kw):
    args = dict(q=A, k=A, v=A, cu=A, B=4, Hq=8, Hkv=2, D=128, maxL=128, scale=0.125, dt=0, out=A,
                lse=None, workers=0, phases=3, ws=A, wsb=BIG, stream=None)
    args.update(kw)
    return lib.zl_decode_attn_gqa_ex(args["q"], args["k"], args["v"], args["cu"], args["B"], args["Hq"],
                                     args["Hkv"], args["D"], args["maxL"], args["scale"], args["dt"],
                                     args["out"], args["lse"], args["workers"], args["phases"], args["ws"],
                                     args["wsb"], args["stream"])


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), 1), (dict(cu=None), 1), (dict(out=None), 1), (dict(ws=None), 1),
    (dict(q=A + 2), 1), (dict(out=A + 8), 1), (dict(k=A + 4), 1), (dict(lse=A + 2), 1),
    (dict(ws=A + 16), 1), (dict(cu=A + 2), 1),
    (dict(B=-1), 1), (dict(Hq=0), 1), (dict(Hkv=0), 1), (dict(Hq=6, Hkv=4), 1),
    (dict(maxL=-1), 1), (dict(scale=float("inf")), 1), (dict(scale=float("nan")), 1),
    (dict(dt=2), 1), (dict(workers=12), 1), (dict(workers=-8), 1), (dict(phases=0), 1), (dict(phases=4), 1),
    (dict(D=96), 2), (dict(D=256), 2), (dict(D=0), 1), (dict(Hq=40, Hkv=2), 2),
    (dict(wsb=16), 3),
    (dict(B=0, q=None, k=None, v=None, cu=None, out=None, ws=None), 0),   # empty batch: no-op
])
def test_gqa_rejects_bad_arguments_before_any_hip_call(zl, kw, expect):
    assert gqa(zl.library(), **kw) == expect


def test_mla_and_combine_reject_bad_arguments(zl):
    lib = zl.library()

    def mla(**kw):
        a = dict(q=A, c=A, cu=A, B=2, H=16, r=512, rope=64, maxL=10, scale=0.07, dt=1, out=A, lse=None,
                 workers=0, phases=3, ws=A, wsb=BIG, stream=None)
        a.update(kw)
        return lib.zl_decode_attn_mla_ex(a["q"], a["c"], a["cu"], a["B"], a["H"], a["r"], a["rope"],
                                         a["maxL"], a["scale"], a["dt"], a["out"], a["lse"], a["workers"],
                                         a["phases"], a["ws"], a["wsb"], a["stream"])
    assert mla(r=256) == 2 and mla(rope=32) == 2 and mla(r=0) == 1
    assert mla(H=0) == 1 and mla(H=24) == 2 and mla(q=None) == 1 and mla(wsb=8) == 3 and mla(phases=7) == 1
    assert mla(B=0, q=None, c=None, cu=None, out=None, ws=None) == 0

    def comb(**kw):
        a = dict(po=A, pl=A, S=4, B=2, H=8, Dv=128, dt=0, out=A, lse=None, stream=None)
        a.update(kw)
        return lib.zl_attn_combine(a["po"], a["pl"], a["S"], a["B"], a["H"], a["Dv"], a["dt"], a["out"],
                                   a["lse"], a["stream"])
    assert comb(S=0) == 1 and comb(S=1025) == 1 and comb(Dv=6) == 1 and comb(H=0) == 1
    assert comb(po=None) == 1 and comb(po=A + 4) == 1 and comb(dt=5) == 1
    assert comb(B=0, po=None, pl=None, out=None) == 0


def test_paged_entry_points_reject_bad_arguments(zl):
    lib = zl.library()

    def gqa_paged(**kw):
        a = dict(q=A, k=A, v=A, table=A, maxp=8, ps=16, cu=A, B=4, Hq=8, Hkv=2, D=128, maxL=128, scale=0.125,
                 dt=0, out=A, lse=None, workers=0, phases=3, ws=A, wsb=BIG, stream=None)
        a.update(kw)
        return lib.zl_decode_attn_gqa_paged_ex(a["q"], a["k"], a["v"], a["table"], a["maxp"], a["ps"], a["cu"],
                                               a["B"], a["Hq"], a["Hkv"], a["D"], a["maxL"], a["scale"], a["dt"],
                                               a["out"], a["lse"], a["workers"], a["phases"], a["ws"], a["wsb"],
                                               a["stream"])

    def mla_paged(**kw):
        a = dict(q=A, c=A, table=A, maxp=4, ps=64, cu=A, B=2, H=16, r=512, rope=64, maxL=200, scale=0.07,
                 dt=1, out=A, lse=None, workers=0, phases=3, ws=A, wsb=BIG, stream=None)
        a.update(kw)
        return lib.zl_decode_attn_mla_paged_ex(a["q"], a["c"], a["table"], a["maxp"], a["ps"], a["cu"], a["B"],
                                               a["H"], a["r"], a["rope"], a["maxL"], a["scale"], a["dt"],
                                               a["out"], a["lse"], a["workers"], a["phases"], a["ws"],
                                               a["wsb"], a["stream"])
    # page size: a power of two in 16 .. 256
    for ps, expect in [(8, 2), (24, 2), (512, 2), (0, 2), (16, 0), (256, 0)]:
        got = gqa_paged(ps=ps, maxp=64, B=0, q=None, k=None, v=None, cu=None, out=None, ws=None)
        assert got == expect, (ps, got)
    assert gqa_paged(table=None) == 1 and gqa_paged(table=A + 2) == 1
    assert gqa_paged(maxp=0) == 1
    assert gqa_paged(maxL=129) == 1          # longer than 8 pages of 16
    assert gqa_paged(D=96) == 2 and gqa_paged(q=None) == 1 and gqa_paged(wsb=16) == 3
    assert mla_paged(ps=48) == 2 and mla_paged(table=None) == 1 and mla_paged(maxL=257) == 1
    assert mla_paged(r=256) == 2 and mla_paged(wsb=8) == 3
    assert mla_paged(B=0, q=None, c=None, cu=None, out=None, ws=None) == 0


def test_varlen_entry_points_reject_bad_arguments(zl):
    lib = zl.library()

    def gqa(**kw):
        a = dict(q=A, k=A, v=A, cq=A, ck=A, B=4, Tq=16, Hq=8, Hkv=2, D=128, maxL=128, scale=0.125, causal=1,
                 dt=0, out=A, lse=None, workers=0, phases=3, ws=A, wsb=BIG, stream=None)
        a.update(kw)
        return lib.zl_attn_varlen_gqa_ex(a["q"], a["k"], a["v"], a["cq"], a["ck"], a["B"], a["Tq"], a["Hq"],
                                         a["Hkv"], a["D"], a["maxL"], a["scale"], a["causal"], a["dt"], a["out"],
                                         a["lse"], a["workers"], a["phases"], a["ws"], a["wsb"], a["stream"])

    def mla(**kw):
        a = dict(q=A, c=A, cq=A, ck=A, B=2, Tq=4, H=16, r=512, rope=64, maxL=200, scale=0.07, causal=1, dt=1,
                 out=A, lse=None, workers=0, phases=3, ws=A, wsb=BIG, stream=None)
        a.update(kw)
        return lib.zl_attn_varlen_mla_ex(a["q"], a["c"], a["cq"], a["ck"], a["B"], a["Tq"], a["H"], a["r"],
                                         a["rope"], a["maxL"], a["scale"], a["causal"], a["dt"], a["out"],
                                         a["lse"], a["workers"], a["phases"], a["ws"], a["wsb"], a["stream"])
    assert gqa(cq=None) == 1 and gqa(cq=A + 2) == 1
    assert gqa(Tq=-1) == 1 and gqa(causal=2) == 1
    assert gqa(D=96) == 2 and gqa(q=None) == 1 and gqa(wsb=16) == 3 and gqa(Hq=7) == 1
    # nothing to compute: no rows of q, or no sequences
    assert gqa(Tq=0, q=None, k=None, v=None, ck=None, out=None, ws=None) == 0
    assert gqa(B=0, Tq=0, q=None, k=None, v=None, ck=None, out=None, ws=None) == 0
    # work-line positions beyond 32 bits
    assert gqa(Tq=1 << 20, maxL=1 << 20) == 2
    assert mla(cq=None) == 1 and mla(r=256) == 2 and mla(wsb=8) == 3 and mla(causal=-1) == 1
    assert mla(Tq=1 << 16, maxL=1 << 16) == 2
    assert mla(Tq=0, q=None, c=None, ck=None, out=None, ws=None) == 0


def test_paged_varlen_entry_points_reject_bad_arguments(zl):
    lib = zl.library()

    def gqa(**kw):
        a = dict(q=A, k=A, v=A, table=A, maxp=8, ps=16, cq=A, ck=A, B=4, Tq=16, Hq=8, Hkv=2, D=128, maxL=128,
                 scale=0.125, causal=1, dt=0, out=A, lse=None, workers=0, phases=3, ws=A, wsb=BIG, stream=None)
        a.update(kw)
        return lib.zl_attn_varlen_gqa_paged_ex(a["q"], a["k"], a["v"], a["table"], a["maxp"], a["ps"], a["cq"],
                                               a["ck"], a["B"], a["Tq"], a["Hq"], a["Hkv"], a["D"], a["maxL"],
                                               a["scale"], a["causal"], a["dt"], a["out"], a["lse"], a["workers"],
                                               a["phases"], a["ws"], a["wsb"], a["stream"])

    def mla(**kw):
        a = dict(q=A, c=A, table=A, maxp=4, ps=64, cq=A, ck=A, B=2, Tq=4, H=16, r=512, rope=64, maxL=200,
                 scale=0.07, causal=1, dt=1, out=A, lse=None, workers=0, phases=3, ws=A, wsb=BIG, stream=None)
        a.update(kw)
        return lib.zl_attn_varlen_mla_paged_ex(a["q"], a["c"], a["table"], a["maxp"], a["ps"], a["cq"], a["ck"],
                                               a["B"], a["Tq"], a["H"], a["r"], a["rope"], a["maxL"], a["scale"],
                                               a["causal"], a["dt"], a["out"], a["lse"], a["workers"],
                                               a["phases"], a["ws"], a["wsb"], a["stream"])
    # both a query prefix and a page table are required
    assert gqa(cq=None) == 1 and gqa(table=None) == 1 and mla(cq=None) == 1 and mla(table=None) == 1
    assert gqa(ps=24) == 2 and gqa(maxp=0) == 1 and gqa(maxL=129) == 1 and gqa(causal=3) == 1
    assert gqa(D=96) == 2 and gqa(wsb=16) == 3 and gqa(table=A + 2) == 1 and gqa(Tq=-1) == 1
    assert mla(ps=512) == 2 and mla(maxL=257) == 1 and mla(r=256) == 2 and mla(wsb=8) == 3
    assert gqa(Tq=0, q=None, k=None, v=None, ck=None, out=None, ws=None) == 0
    assert mla(B=0, Tq=0, q=None, c=None, ck=None, out=None, ws=None) == 0


def test_codec_entry_points_reject_bad_arguments(zl):
    lib = zl.library()
    q = lambda **kw: lib.zl_int8_quantize(kw.get("x", A), kw.get("dt", 0), kw.get("n", 1000), kw.get("chunk", 512),
                                          kw.get("codes", A), kw.get("scales", A), None)
    d = lambda **kw: lib.zl_int8_dequantize(kw.get("codes", A), kw.get("scales", A), kw.get("n", 1000),
                                            kw.get("chunk", 512), kw.get("dt", 1), kw.get("out", A), None)

    def r(**kw):
        return lib.zl_int8_reduce_step(kw.get("codes", A), kw.get("scales", A), kw.get("local", A), kw.get("dt", 0),
                                       kw.get("n", 1000), kw.get("chunk", 256), kw.get("codes_out", A),
                                       kw.get("scales_out", A), kw.get("sum_out", A), None)
    for f in (q, d, r):
        assert f(chunk=128) == 2 and f(chunk=2048) == 2 and f(chunk=300) == 2
        assert f(dt=5) == 1 and f(n=-1) == 1 and f(n=1 << 41) == 1
    assert q(x=None) == 1 and q(codes=A + 4) == 1 and q(scales=A + 2) == 1 and q(x=A + 8) == 1
    assert q(n=0, x=None, codes=None, scales=None) == 0
    assert d(out=None) == 1 and d(codes=A + 8) == 1
    assert r(codes_out=None) == 1                      # codes without scales
    assert r(codes_out=None, scales_out=None, sum_out=None) == 1
    assert r(local=None) == 1 and r(sum_out=A + 2) == 1
    assert r(n=0, codes=None, scales=None, local=None, codes_out=None, scales_out=None) == 0


def test_prefill_entry_point_rejects_bad_arguments(zl):
    lib = zl.library()

    def pf(**kw):
        a = dict(q=A, k=A, v=A, cq=A, ck=A, B=2, Tq=300, Hq=8, Hkv=2, D=128, maxL=300, scale=0.1, causal=1, dt=1,
                 out=A, lse=None, stream=None)
        a.update(kw)
        return lib.zl_attn_prefill_gqa(a["q"], a["k"], a["v"], a["cq"], a["ck"], a["B"], a["Tq"], a["Hq"], a["Hkv"],
                                       a["D"], a["maxL"], a["scale"], a["causal"], a["dt"], a["out"], a["lse"],
                                       a["stream"])
    assert pf(cq=None) == 1 and pf(ck=None) == 1 and pf(q=None) == 1 and pf(out=A + 2) == 1
    assert pf(D=96) == 2 and pf(D=0) == 1 and pf(Hq=7) == 1 and pf(causal=3) == 1 and pf(dt=4) == 1
    assert pf(scale=float("inf")) == 1 and pf(Tq=-1) == 1
    assert pf(Tq=0, q=None, k=None, v=None, cq=None, ck=None, out=None) == 0
    assert pf(Tq=1 << 30, Hq=1024, Hkv=1024) == 2   # 2^22 blocks x 1024 heads


def test_paged_prefill_entry_point_rejects_bad_arguments(zl):
    lib = zl.library()

    def pp(**kw):
        a = dict(q=A, k=A, v=A, bt=A, mp=8, ps=64, cq=A, ck=A, B=2, Tq=300, Hq=8, Hkv=2, D=128, maxL=300, scale=0.1,
                 causal=1, dt=1, out=A, lse=None, stream=None)
        a.update(kw)
        return lib.zl_attn_prefill_gqa_paged(a["q"], a["k"], a["v"], a["bt"], a["mp"], a["ps"], a["cq"], a["ck"],
                                             a["B"], a["Tq"], a["Hq"], a["Hkv"], a["D"], a["maxL"], a["scale"],
                                             a["causal"], a["dt"], a["out"], a["lse"], a["stream"])
    assert pp(bt=None) == 1 and pp(bt=A + 2) == 1 and pp(mp=0) == 1 and pp(maxL=513) == 1   # 513 > 8 x 64
    assert pp(ps=8) == 2 and pp(ps=48) == 2 and pp(ps=512) == 2
    # every check of the packed prefill call holds here too
    assert pp(cq=None) == 1 and pp(q=None) == 1 and pp(D=96) == 2 and pp(causal=3) == 1 and pp(dt=4) == 1
    assert pp(Tq=0, q=None, k=None, v=None, cq=None, ck=None, out=None) == 0


def test_read_probe_rejects_bad_arguments(zl):
    lib = zl.library()

    def rp(**kw):
        a = dict(src=A, nbytes=1 << 20, D=128, wg=0, sink=A)
        a.update(kw)
        return lib.zl_hbm_read_probe(a["src"], a["nbytes"], a["D"], a["wg"], a["sink"], None)
    assert rp(D=96) == 2 and rp(D=0) == 2
    assert rp(wg=12) == 1 and rp(wg=-8) == 1 and rp(wg=1 << 17) == 1
    assert rp(src=None) == 1 and rp(sink=None) == 1 and rp(src=A + 8) == 1 and rp(sink=A + 2) == 1
    assert rp(nbytes=1000, src=None, sink=None) == 0   # under one block: no-op


def test_no_alloc_entry_point_rejects_bad_sizes_before_any_hip_call(zl):
    lib = zl.library()

    def na(**kw):
        a = dict(q=A, k=A, v=A, cu=A, B=2, Hq=8, Hkv=2, D=128, maxL=100, scale=0.1, dt=0, out=A, lse=None)
        a.update(kw)
        return lib.zl_decode_attn_gqa_no_alloc(a["q"], a["k"], a["v"], a["cu"], a["B"], a["Hq"], a["Hkv"], a["D"],
                                               a["maxL"], a["scale"], a["dt"], a["out"], a["lse"], None)
    # invalid sizes take the plain call's status, with no HIP call (no GPU here)
    assert na(D=96) == 2 and na(D=0) == 1 and na(Hq=7) == 1 and na(B=-1) == 1 and na(dt=3) == 1
    assert na(Hq=40, Hkv=2) == 2   # a group of 20 heads
