"""C-ABI checks that need no GPU: the library loads and exports every symbol
the header declares, and every launch entry point rejects bad arguments
before any HIP call (the error path makes no HIP call, so it runs here)."""

import ctypes
import os
import re

import numpy as np
import pytest

import transformer_attention_05_amd as mi
from transformer_attention_05_amd import (ATTN_BF16, ATTN_E_INVALID, ATTN_E_NOMEM, ATTN_E_UNSUPPORTED,
                                          ATTN_F32)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mi_attn.h")


@pytest.fixture(scope="module")
def lib():
    return mi.load()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"ATTN_API\s+[\w\s\*]*?\b(attn_\w+)\s*\(", text)))


def test_header_declares_entry_points():
    syms = declared_symbols()
    for name in ("attn_prefill", "attn_prefill_paged", "attn_prefill_workspace_size", "attn_decode_paged_plan",
                 "attn_prefill_paged_workspace_size", "attn_decode_paged", "attn_decode_paged_workspace_size",
                 "attn_decode_paged_rope", "attn_prefill_masked", "attn_seq_fork", "attn_seq_reserve_cow",
                 "attn_copy_blocks", "attn_residual_rms_norm", "attn_prefill_paged_ex",
                 "attn_kv_cache_write_rope", "attn_pool_create", "attn_pool_alloc", "attn_pool_free",
                 "attn_pool_retain", "attn_seq_reserve", "attn_last_error"):
        assert name in syms


def declared_arg_counts():
    """{name: number of parameters} from the header's prototypes."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for m in re.finditer(r"ATTN_API\s+[\w\s\*]*?\b(attn_\w+)\s*\(([^)]*)\)\s*;", text):
        params = m.group(2).strip()
        out[m.group(1)] = 0 if params in ("", "void") else len(params.split(","))
    return out


def test_binding_signatures_match_header():
    """Every ctypes prototype of the binding has as many arguments as the
    header's declaration, and every declared symbol has a prototype."""
    counts = declared_arg_counts()
    assert set(counts) == set(declared_symbols())
    for name, n in counts.items():
        assert name in mi._SIGNATURES, f"{name} has no ctypes prototype"
        assert len(mi._SIGNATURES[name][1]) == n, (name, len(mi._SIGNATURES[name][1]), n)


@pytest.mark.parametrize("debug", [False, True], ids=["release", "debug"])
def test_library_exports_every_declared_symbol(debug):
    lib = mi.load(debug=debug)
    for name in declared_symbols():
        assert hasattr(lib, name), name
    # and nothing else: the build hides internal symbols
    out = os.popen(f"nm -D --defined-only {mi.lib_path(debug)}").read()
    exported = sorted(set(re.findall(r" T (attn_\w+)", out)))
    assert exported == declared_symbols()


def test_debug_flags_entry_point():
    """The release library has no debug record (UNSUPPORTED, flags 0); both
    reject a NULL output before any HIP call."""
    rel, dbg = mi.load(debug=False), mi.load(debug=True)
    out = ctypes.c_uint32(123)
    assert rel.attn_debug_flags(ctypes.byref(out), 1) == ATTN_E_UNSUPPORTED and out.value == 0
    assert "release library" in rel.attn_last_error().decode()
    for lib in (rel, dbg):
        assert lib.attn_debug_flags(None, 0) == ATTN_E_INVALID


def test_library_selection(monkeypatch):
    """MI_ATTN_DEBUG=1 selects the debug library; debug_library() overrides
    the variable for a block and restores the previous choice."""
    monkeypatch.delenv("MI_ATTN_DEBUG", raising=False)
    assert mi.lib_path().endswith("libmi_attn.so")
    monkeypatch.setenv("MI_ATTN_DEBUG", "1")
    assert mi.lib_path().endswith("libmi_attn_debug.so")
    with mi.debug_library(False) as lib:
        assert mi.lib_path().endswith("libmi_attn.so") and lib is mi.load(debug=False)
        with mi.debug_library() as dlib:
            assert dlib is mi.load(debug=True) and mi.load() is dlib
        assert mi.load() is lib
    assert mi.lib_path().endswith("libmi_attn_debug.so")
    monkeypatch.setenv("MI_ATTN_DEBUG", "0")
    assert mi.lib_path().endswith("libmi_attn.so")
    with pytest.raises(mi.AttnError, match="release library"):
        mi.attn_debug_flags()


# fake, aligned device addresses: never dereferenced on the error path
P = 0x100000
S3 = (ctypes.c_int64 * 3)(8 * 128, 128, 128)


def prefill(lib, **kw):
    args = dict(q=P, k=P, v=P, o=P, lse=None, batch=1, tq=64, tk=64, hq=1, hkv=1, d=64,
                qs=S3, ks=S3, vs=S3, os_=S3, scale=0.0, causal=1, dtype=ATTN_F32, ws=None, wsb=0)
    args.update(kw)
    return lib.attn_prefill(args["q"], args["k"], args["v"], args["o"], args["lse"], args["batch"], args["tq"],
                            args["tk"], args["hq"], args["hkv"], args["d"], args["qs"], args["ks"], args["vs"],
                            args["os_"], args["scale"], args["causal"], args["dtype"], args["ws"], args["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), ATTN_E_INVALID),
    (dict(o=None), ATTN_E_INVALID),
    (dict(qs=None), ATTN_E_INVALID),
    (dict(batch=-1), ATTN_E_INVALID),
    (dict(tq=-5), ATTN_E_INVALID),
    (dict(hq=12, hkv=5), ATTN_E_INVALID),
    (dict(hq=0), ATTN_E_INVALID),
    (dict(d=96), ATTN_E_UNSUPPORTED),
    (dict(d=256), ATTN_E_UNSUPPORTED),
    (dict(dtype=7), ATTN_E_UNSUPPORTED),
    (dict(tq=65, tk=64), ATTN_E_INVALID),      # causal needs tk >= tq
    (dict(scale=-1.0), ATTN_E_INVALID),
    (dict(scale=float("nan")), ATTN_E_INVALID),
    (dict(q=P + 2), ATTN_E_INVALID),            # misaligned
    (dict(qs=(ctypes.c_int64 * 3)(8 * 128, 130, 128)), ATTN_E_INVALID),  # stride not a multiple of 4
    (dict(dtype=ATTN_BF16, ks=(ctypes.c_int64 * 3)(1024, 132, 128)), ATTN_E_INVALID),
    (dict(dtype=ATTN_BF16, vs=(ctypes.c_int64 * 3)(1 << 30, 1 << 28, 128)), ATTN_E_UNSUPPORTED),
])
def test_prefill_rejects(lib, kw, status):
    assert prefill(lib, **kw) == status
    assert lib.attn_last_error().decode().startswith("attn_prefill")


M3 = (ctypes.c_int64 * 3)(0, 0, 64)


def prefill_masked(lib, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, mask=P, ms=M3, batch=1, tq=64, tk=64, hq=1, hkv=1, d=64,
             qs=S3, ks=S3, vs=S3, os_=S3, scale=0.0, causal=0, dtype=ATTN_F32)
    a.update(kw)
    return lib.attn_prefill_masked(a["q"], a["k"], a["v"], a["o"], a["lse"], a["mask"], a["ms"], a["batch"],
                                   a["tq"], a["tk"], a["hq"], a["hkv"], a["d"], a["qs"], a["ks"], a["vs"],
                                   a["os_"], a["scale"], a["causal"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(mask=None), ATTN_E_INVALID),
    (dict(ms=None), ATTN_E_INVALID),
    (dict(mask=P + 4), ATTN_E_INVALID),                               # not 16-byte aligned
    (dict(ms=(ctypes.c_int64 * 3)(0, 0, 66)), ATTN_E_INVALID),        # row stride not a multiple of 4
    (dict(ms=(ctypes.c_int64 * 3)(-64, 0, 64)), ATTN_E_INVALID),
    (dict(d=96), ATTN_E_UNSUPPORTED),                                 # the prefill's own checks
    (dict(q=None), ATTN_E_INVALID),
    (dict(tq=65, tk=64, causal=1), ATTN_E_INVALID),
])
def test_prefill_masked_rejects(lib, kw, status):
    assert prefill_masked(lib, **kw) == status
    assert lib.attn_last_error().decode().startswith("attn_prefill_masked")


def test_prefill_masked_empty_is_ok_without_launch(lib):
    assert prefill_masked(lib, batch=0) == 0


# batch 1, T 2048, 12/2 heads, D 128: too few query tiles to fill the GPU, so
# the plan splits each query tile's keys and needs a workspace
SPLIT = dict(dtype=ATTN_BF16, batch=1, tq=2048, tk=2048, hq=12, hkv=2, d=128,
             qs=(ctypes.c_int64 * 3)(2048 * 12 * 128, 12 * 128, 128),
             ks=(ctypes.c_int64 * 3)(2048 * 2 * 128, 2 * 128, 128),
             vs=(ctypes.c_int64 * 3)(2048 * 2 * 128, 2 * 128, 128),
             os_=(ctypes.c_int64 * 3)(2048 * 12 * 128, 12 * 128, 128))


def test_prefill_workspace_size(lib):
    rows = 2048 * 12
    n = lib.attn_prefill_workspace_size(1, 2048, 2048, 12, 2, 128, ATTN_BF16)
    # whole shares of (D floats of output + max + sum) per (query row, head)
    assert n > 0 and n % (rows * (128 * 4 + 8)) == 0 and 2 <= n // (rows * (128 * 4 + 8)) <= 64
    # enough query tiles to fill the GPU, the f32 kernel and degenerate sizes: no split
    assert lib.attn_prefill_workspace_size(1, 16384, 16384, 12, 2, 128, ATTN_BF16) == 0
    assert lib.attn_prefill_workspace_size(1, 2048, 2048, 12, 2, 128, ATTN_F32) == 0
    assert lib.attn_prefill_workspace_size(1, 0, 2048, 12, 2, 128, ATTN_BF16) == 0
    assert lib.attn_prefill_workspace_size(1, 64, 64, 12, 2, 128, ATTN_BF16) == 0
    # two chunks (200 + 50 new tokens) over up to 3200 keys: few query tiles, long rows
    m = lib.attn_prefill_paged_workspace_size(2, 250, 200, 3200, 12, 2, 128)
    assert m > 0 and m % (250 * 12 * (128 * 4 + 8)) == 0
    assert lib.attn_prefill_paged_workspace_size(2, 250, 200, 0, 12, 2, 128) == 0
    # eight 512-token chunks fill the GPU without splitting
    assert lib.attn_prefill_paged_workspace_size(8, 4096, 512, 2560, 12, 2, 128) == 0


def test_prefill_workspace_rejects(lib):
    need = lib.attn_prefill_workspace_size(1, 2048, 2048, 12, 2, 128, ATTN_BF16)
    assert prefill(lib, **SPLIT, ws=P, wsb=need - 1) == ATTN_E_NOMEM
    assert prefill(lib, **SPLIT, ws=P + 16, wsb=need) == ATTN_E_INVALID   # not 256-byte aligned
    assert lib.attn_last_error().decode().startswith("attn_prefill")


def test_prefill_empty_is_ok_without_launch(lib):
    assert prefill(lib, batch=0) == 0
    assert prefill(lib, tq=0, tk=0) == 0


def decode(lib, **kw):
    a = dict(q=P, kc=P, vc=P, bt=P, cl=P, o=P, S=4, hq=12, hkv=2, d=128, bs=16, nb=100, maxb=8, maxctx=128,
             part=0, scale=0.0, dtype=ATTN_BF16, plan=None, nplan=0, ws=P, wsb=1 << 30)
    a.update(kw)
    return lib.attn_decode_paged(a["q"], a["kc"], a["vc"], a["bt"], a["cl"], a["o"], a["S"], a["hq"], a["hkv"],
                                 a["d"], a["bs"], a["nb"], a["maxb"], a["maxctx"], a["part"], a["scale"],
                                 a["dtype"], a["plan"], a["nplan"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), ATTN_E_INVALID),
    (dict(bt=None), ATTN_E_INVALID),
    (dict(bs=32), ATTN_E_UNSUPPORTED),
    (dict(dtype=7), ATTN_E_UNSUPPORTED),
    (dict(maxb=7), ATTN_E_INVALID),             # 128 tokens need 8 blocks
    (dict(part=100), ATTN_E_INVALID),
    (dict(part=40), ATTN_E_INVALID),            # partitions: multiples of 16
    (dict(part=1024 + 16), ATTN_E_INVALID),     # bf16 partitions: at most 1024
    (dict(part=40, dtype=ATTN_F32), ATTN_E_INVALID),      # fp32 partitions: multiples of 16
    (dict(part=65536 + 16, dtype=ATTN_F32), ATTN_E_INVALID),
    (dict(part=-128), ATTN_E_INVALID),
    (dict(part=2048), ATTN_E_INVALID),
    (dict(maxctx=0), ATTN_E_INVALID),
    (dict(maxctx=4096, maxb=256, part=128, ws=None), ATTN_E_INVALID),
    (dict(maxctx=4096, maxb=256, part=128, wsb=16), ATTN_E_NOMEM),
    (dict(maxctx=4096, maxb=256, part=128, ws=P + 16), ATTN_E_INVALID),
    (dict(hq=12, hkv=5), ATTN_E_INVALID),
    (dict(plan=None, nplan=3), ATTN_E_INVALID),       # items without a plan
    (dict(plan=P, nplan=-1), ATTN_E_INVALID),
    (dict(plan=P + 2, nplan=1), ATTN_E_INVALID),      # misaligned
    (dict(plan=P, nplan=4 * 1 + 1), ATTN_E_INVALID),  # more items than sequences x partitions
])
def test_decode_rejects(lib, kw, status):
    assert decode(lib, **kw) == status


def test_decode_f32_partition_sizes_accepted_by_the_plan():
    """Decodes take any multiple of 16 as partition size (bf16 up to 1024);
    the host plan lists their partitions."""
    lens = np.array([1, 16, 17, 100], np.int32)
    items = mi.attn_decode_paged_plan(lens, 2, 100, 16)
    assert len(items) == 1 + 1 + 2 + 7
    with pytest.raises(mi.AttnError):
        mi.attn_decode_paged_plan(lens, 2, 100, 24)


def decode_rope(lib, **kw):
    a = dict(qr=None, q=P, kn=P, vn=P, pos=P, slots=P, base=10000.0, kc=P, vc=P, bt=P, cl=P, o=P, S=4, hq=12,
             hkv=2, d=128, bs=16, nb=100, maxb=8, maxctx=128, part=0, scale=0.0, dtype=ATTN_BF16, plan=None,
             nplan=0, ws=P, wsb=1 << 30)
    a.update(kw)
    return lib.attn_decode_paged_rope(a["qr"], a["q"], a["kn"], a["vn"], a["pos"], a["slots"], a["base"], a["kc"],
                                      a["vc"], a["bt"], a["cl"], a["o"], a["S"], a["hq"], a["hkv"], a["d"], a["bs"],
                                      a["nb"], a["maxb"], a["maxctx"], a["part"], a["scale"], a["dtype"], a["plan"],
                                      a["nplan"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(kn=None), ATTN_E_INVALID),
    (dict(vn=None), ATTN_E_INVALID),
    (dict(pos=None), ATTN_E_INVALID),
    (dict(slots=None), ATTN_E_INVALID),
    (dict(base=1.0), ATTN_E_INVALID),
    (dict(base=-2.0), ATTN_E_INVALID),
    (dict(base=float("inf")), ATTN_E_INVALID),
    (dict(kn=P + 2), ATTN_E_INVALID),           # misaligned
    (dict(pos=P + 2), ATTN_E_INVALID),
    (dict(qr=P), ATTN_E_INVALID),               # rotated queries may not overwrite q
    (dict(q=None), ATTN_E_INVALID),             # and the decode's own checks still apply
    (dict(dtype=ATTN_F32), ATTN_E_UNSUPPORTED),
    (dict(maxb=7), ATTN_E_INVALID),
    (dict(maxctx=4096, maxb=256, part=128, wsb=16), ATTN_E_NOMEM),
])
def test_decode_rope_rejects(lib, kw, status):
    assert decode_rope(lib, **kw) == status
    assert "attn_decode_paged_rope" in mi.attn_last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(kc=None), ATTN_E_INVALID),
    (dict(pairs=None), ATTN_E_INVALID),
    (dict(n=-1), ATTN_E_INVALID),
    (dict(nb=0), ATTN_E_INVALID),
    (dict(d=96), ATTN_E_UNSUPPORTED),
    (dict(bs=32), ATTN_E_UNSUPPORTED),
    (dict(dtype=7), ATTN_E_UNSUPPORTED),
    (dict(vc=P + 8), ATTN_E_INVALID),
    (dict(pairs=P + 2), ATTN_E_INVALID),
])
def test_copy_blocks_rejects(lib, kw, status):
    a = dict(kc=P, vc=P, pairs=P, n=4, hkv=2, d=128, bs=16, nb=100, dtype=ATTN_BF16)
    a.update(kw)
    assert lib.attn_copy_blocks(a["kc"], a["vc"], a["pairs"], a["n"], a["hkv"], a["d"], a["bs"], a["nb"],
                                a["dtype"], None) == status
    assert lib.attn_last_error().decode().startswith("attn_copy_blocks")


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), ATTN_E_INVALID),
    (dict(rows=-1), ATTN_E_INVALID),
    (dict(hidden=12), ATTN_E_UNSUPPORTED),
    (dict(hidden=8200), ATTN_E_UNSUPPORTED),
    (dict(hidden=0), ATTN_E_UNSUPPORTED),
    (dict(eps=-1.0), ATTN_E_INVALID),
    (dict(eps=float("nan")), ATTN_E_INVALID),
    (dict(dtype=7), ATTN_E_UNSUPPORTED),
    (dict(w=P + 8), ATTN_E_INVALID),
    (dict(y=P), ATTN_E_INVALID),                 # y aliases x
])
def test_residual_rms_norm_rejects(lib, kw, status):
    a = dict(x=P, r=P + 4096, w=P + 8192, y=P + 12288, h=P + 4096, rows=4, hidden=1536, eps=1e-6, dtype=ATTN_BF16)
    a.update(kw)
    assert lib.attn_residual_rms_norm(a["x"], a["r"], a["w"], a["y"], a["h"], a["rows"], a["hidden"], a["eps"],
                                      a["dtype"], None) == status
    assert lib.attn_last_error().decode().startswith("attn_residual_rms_norm")


def test_decode_workspace_size(lib):
    # one partition: no workspace; several: an arrival counter per (seq, kv
    # head slice) for the most sequences a call may have (65535), whatever
    # this call's count, then (D + 2) floats per (seq, head, partition)
    assert lib.attn_decode_paged_workspace_size(4, 12, 2, 128, 128, 128) == 0
    n = lib.attn_decode_paged_workspace_size(4, 12, 2, 128, 1024, 128)
    rows = 4 * 12 * 8
    cnt = ((65535 * 2 * 4 + 255) // 256) * 256
    assert n == cnt + ((rows * 128 * 4 + 255) // 256) * 256 + rows * 8
    # the counter block is the same for 4 and for 1000 sequences of the same heads
    n2 = lib.attn_decode_paged_workspace_size(1000, 12, 2, 128, 1024, 128)
    assert n2 == cnt + ((1000 * 12 * 8 * 128 * 4 + 255) // 256) * 256 + 1000 * 12 * 8 * 8
    # 40 query heads on 2 kv heads (groups of 20): two slices (16 + 4 heads) per kv head
    n = lib.attn_decode_paged_workspace_size(100, 40, 2, 64, 1024, 128)
    rows = 100 * 40 * 8
    assert n == ((65535 * 2 * 2 * 4 + 255) // 256) * 256 + ((rows * 64 * 4 + 255) // 256) * 256 + rows * 8
    p = lib.attn_decode_paged_auto_partition(64, 2, 4096)
    assert p % 128 == 0 and 128 <= p <= 1024


def test_decode_plan():
    """The plan lists each sequence's ceil(ctx / P) partitions, longest
    sequences first, partitions in order, P as the decode launch picks it."""
    lens = np.array([1000, 5, 0, 3000, 1000, 769], dtype=np.int32)
    P = 256
    items = mi.attn_decode_paged_plan(lens, 2, 3000, P)
    counts = -(-lens // P)
    assert items.shape == (counts.sum(), 2)
    order = sorted(range(len(lens)), key=lambda s: -counts[s])   # stable: ties keep their order
    expect = [(s, p) for s in order for p in range(counts[s])]
    assert [tuple(x) for x in items] == expect
    # automatic partition size: the decode's choice for the same arguments
    auto = mi.attn_decode_paged_auto_partition(len(lens), 2, 3000)
    assert len(mi.attn_decode_paged_plan(lens, 2, 3000)) == int((-(-lens // auto)).sum())
    # lengths beyond max_context_len are clamped, as the kernel clamps them
    assert len(mi.attn_decode_paged_plan(np.array([5000], np.int32), 2, 1024, 512)) == 2
    with pytest.raises(mi.AttnError):
        mi.attn_decode_paged_plan(lens, 2, 3000, 100)   # not a multiple of 16


def test_paged_prefill_and_write_reject(lib):
    def paged(**kw):
        a = dict(bt=P, tot=100, maxq=60, maxctx=0, dtype=ATTN_BF16, ws=None, wsb=0)
        a.update(kw)
        return lib.attn_prefill_paged(P, P, P, a["bt"], 8, P, P, P, 2, a["tot"], a["maxq"], a["maxctx"], 12, 2,
                                      128, 16, 100, 0.0, 1, a["dtype"], a["ws"], a["wsb"], None)
    assert paged(dtype=7) == ATTN_E_UNSUPPORTED
    assert paged(bt=None) == ATTN_E_INVALID
    assert paged(tot=50) == ATTN_E_INVALID       # max_seqlen_q > total_q
    assert paged(maxctx=-1) == ATTN_E_INVALID
    # two chunks over up to 3200 keys: the plan splits
    need = lib.attn_prefill_paged_workspace_size(2, 250, 200, 3200, 12, 2, 128)
    assert need > 0
    st = lib.attn_prefill_paged(P, P, P, P, 200, P, P, P, 2, 250, 200, 3200, 12, 2, 128, 16, 100, 0.0, 1,
                                ATTN_BF16, P, need - 256, None)
    assert st == ATTN_E_NOMEM

    # the flagged form: same checks, plus unknown flag bits
    def paged_ex(flags, **kw):
        a = dict(dtype=ATTN_BF16, ws=None, wsb=0)
        a.update(kw)
        return lib.attn_prefill_paged_ex(P, P, P, P, 200, P, P, P, 2, 250, 200, 3200, 12, 2, 128, 16, 100, 0.0, 1,
                                         a["dtype"], flags, a["ws"], a["wsb"], None)
    assert paged_ex(2) == ATTN_E_INVALID
    assert paged_ex(-1) == ATTN_E_INVALID
    assert paged_ex(mi.ATTN_PREFILL_SHARE_CU, dtype=7) == ATTN_E_UNSUPPORTED
    # (the flagged plan fits one workgroup per CU, so it splits into no more
    # shares than the default: a workspace far below either is refused)
    assert paged_ex(mi.ATTN_PREFILL_SHARE_CU, ws=P, wsb=256) == ATTN_E_NOMEM
    st = lib.attn_kv_cache_write_rope(P, P, P, P, P, P, P, 10, 12, 2, 128, 8, 100, 10000.0, ATTN_BF16, None)
    assert st == ATTN_E_UNSUPPORTED
    st = lib.attn_kv_cache_write_rope(P, None, P, P, P, P, P, 10, 12, 2, 128, 16, 100, 10000.0, ATTN_BF16, None)
    assert st == ATTN_E_INVALID
    st = lib.attn_kv_cache_write_rope(P, P, P, P, P, P, P, 10, 12, 2, 128, 16, 100, 0.5, ATTN_BF16, None)
    assert st == ATTN_E_INVALID
    st = lib.attn_kv_cache_write_rope(None, P, P, P, P, P, P, 0, 12, 2, 128, 16, 100, 10000.0, ATTN_BF16, None)
    assert st == 0  # nothing to do


def test_decode_noalloc_rejects_before_any_hip_call(lib):
    """The no-allocation decode validates like attn_decode_paged, and a call
    whose scratch need exceeds the fixed 32 MiB is refused with NOMEM before
    any HIP call (these run without a GPU)."""
    def na(**kw):
        a = dict(q=P, s=64, hq=12, hkv=2, d=128, bs=16, mb=256, mctx=4096, part=0, dtype=ATTN_BF16)
        a.update(kw)
        return lib.attn_decode_paged_noalloc(a["q"], P, P, P, P, P, a["s"], a["hq"], a["hkv"], a["d"], a["bs"], 1000,
                                             a["mb"], a["mctx"], a["part"], 0.0, a["dtype"], None, 0, None)
    assert na(q=None) == ATTN_E_INVALID
    assert na(d=96) == ATTN_E_UNSUPPORTED
    assert na(part=100) == ATTN_E_INVALID
    assert na(mb=10) == ATTN_E_INVALID
    # 4096 sequences x 12 heads x 32 partitions of 1024 tokens: ~200 MiB of partials
    need = lib.attn_decode_paged_workspace_size(4096, 12, 2, 128, 32768, 1024)
    assert need > (32 << 20)
    assert na(s=4096, mb=2048, mctx=32768, part=1024) == ATTN_E_NOMEM
    assert "32" in mi.attn_last_error() or "scratch" in mi.attn_last_error()
    # the scratch's fixed counter block holds 16 kv head slices: 17 kv heads
    # (one slice each) are refused, 16 fit (small partials)
    assert na(s=4, hq=17, hkv=17, mctx=2048, part=1024) == ATTN_E_NOMEM
    assert "16" in mi.attn_last_error()


def test_paged_masked_rejects(lib):
    ms = (ctypes.c_int64 * 2)(12 * 304, 304)

    def pm(**kw):
        a = dict(mask=P, ms=ms, mk=300, dtype=ATTN_BF16, d=128, bs=16)
        a.update(kw)
        return lib.attn_prefill_paged_masked(P, P, P, P, 20, P, P, a["mask"], a["ms"], a["mk"], P, 2, 250, 200,
                                             300, 12, 2, a["d"], a["bs"], 100, 0.0, 1, a["dtype"], None)
    assert pm(mask=None) == ATTN_E_INVALID
    assert pm(ms=None) == ATTN_E_INVALID
    assert pm(mask=P + 4) == ATTN_E_INVALID                                   # not 16-byte aligned
    assert pm(ms=(ctypes.c_int64 * 2)(12 * 302, 302)) == ATTN_E_INVALID      # stride not a multiple of 4
    assert pm(ms=(ctypes.c_int64 * 2)(-4, 0)) == ATTN_E_INVALID
    assert pm(mk=-1) == ATTN_E_INVALID
    assert pm(d=96) == ATTN_E_UNSUPPORTED
    assert pm(bs=8) == ATTN_E_UNSUPPORTED
    assert pm(dtype=7) == ATTN_E_UNSUPPORTED


def test_bindings_validate_tensors():
    """The binding refuses malformed tensors before taking any pointer: wrong
    integer dtypes, non-contiguous or wrongly shaped caches and queries."""
    import torch
    bf = torch.bfloat16
    q = torch.zeros(3, 12, 128, dtype=bf)
    kc = torch.zeros(10, 2, 16, 128, dtype=bf)
    vc = torch.zeros(10, 2, 128, 16, dtype=bf)
    bt = torch.zeros(3, 4, dtype=torch.int32)
    cl = torch.full((3,), 20, dtype=torch.int32)
    cu = torch.tensor([0, 1, 2, 3], dtype=torch.int32)
    dec = lambda **kw: mi.attn_decode_paged(**{**dict(q=q, k_cache=kc, v_cache=vc, block_table=bt,
                                                      context_lens=cl, max_context_len=64), **kw})
    with pytest.raises(ValueError, match="block_table must be int32"):
        dec(block_table=bt.long())
    with pytest.raises(ValueError, match="context_lens must be int32"):
        dec(context_lens=cl.long())
    with pytest.raises(ValueError, match="context_lens must have shape"):
        dec(context_lens=cl[:2])
    with pytest.raises(ValueError, match="v_cache"):
        dec(v_cache=torch.zeros(10, 2, 16, 128, dtype=bf))           # token-major values
    with pytest.raises(ValueError, match="v_cache"):
        dec(v_cache=vc.transpose(2, 3).contiguous().transpose(2, 3))  # right shape, not contiguous
    with pytest.raises(ValueError, match="k_cache"):
        dec(k_cache=kc.float())
    with pytest.raises(ValueError, match="q must"):
        dec(q=torch.zeros(3, 128, 12, dtype=bf).transpose(1, 2))
    with pytest.raises(ValueError, match="block_table has"):
        dec(block_table=bt[:2], context_lens=cl[:2])
    with pytest.raises(ValueError, match="plan must be int32"):
        dec(plan=torch.zeros(4, 2, dtype=torch.int64))
    with pytest.raises(ValueError, match="o must"):
        dec(o=torch.zeros(3, 12, 64, dtype=bf))
    pf = lambda **kw: mi.attn_prefill_paged(**{**dict(q=q, k_cache=kc, v_cache=vc, block_table=bt,
                                                      cu_seqlens_q=cu, context_lens=cl, max_seqlen_q=1), **kw})
    with pytest.raises(ValueError, match="cu_seqlens_q must be int32"):
        pf(cu_seqlens_q=cu.long())
    with pytest.raises(ValueError, match="cu_seqlens_q must have shape"):
        pf(cu_seqlens_q=cu[:3])
    mask = torch.zeros(3, 12, 64)
    with pytest.raises(ValueError, match="mask must be float32"):
        mi.attn_prefill_paged_masked(q, kc, vc, bt, cu, cl, 1, mask.double())
    with pytest.raises(ValueError, match="mask must be"):
        mi.attn_prefill_paged_masked(q, kc, vc, bt, cu, cl, 1, torch.zeros(2, 64))
    rw = lambda **kw: mi.attn_kv_cache_write_rope(**{**dict(q=q, k=torch.zeros(3, 2, 128, dtype=bf),
                                                            v=torch.zeros(3, 2, 128, dtype=bf),
                                                            positions=cl, slot_mapping=cl, k_cache=kc,
                                                            v_cache=vc), **kw})
    with pytest.raises(ValueError, match="slot_mapping must be int32"):
        rw(slot_mapping=cl.long())
    with pytest.raises(ValueError, match="positions must have shape"):
        rw(positions=cl[:1])
    with pytest.raises(ValueError, match="v must"):
        rw(v=torch.zeros(3, 2, 128, dtype=torch.float32))
    with pytest.raises(ValueError, match="v_cache"):
        rw(v_cache=torch.zeros(10, 2, 16, 128, dtype=bf))
    dr = lambda **kw: mi.attn_decode_paged_rope(**{**dict(q=q, k_new=torch.zeros(3, 2, 128, dtype=bf),
                                                          v_new=torch.zeros(3, 2, 128, dtype=bf), positions=cl,
                                                          slot_mapping=cl, k_cache=kc, v_cache=vc, block_table=bt,
                                                          context_lens=cl, max_context_len=64), **kw})
    with pytest.raises(ValueError, match="slot_mapping must be int32"):
        dr(slot_mapping=cl.long())
    with pytest.raises(ValueError, match="k_new must have shape"):
        dr(k_new=torch.zeros(3, 12, 128, dtype=bf))
    with pytest.raises(ValueError, match="pairs must be int32"):
        mi.attn_copy_blocks(kc, vc, torch.zeros(2, 2, dtype=torch.int64))
    x = torch.zeros(4, 64, dtype=bf)
    with pytest.raises(ValueError, match="residual"):
        mi.attn_residual_rms_norm(x, torch.zeros(4, 64, dtype=torch.float32), torch.zeros(64, dtype=bf))
    k4 = torch.zeros(1, 64, 1, 64)
    with pytest.raises(ValueError, match="lse must have shape"):
        mi.attn_prefill(k4, k4, k4, lse=torch.zeros(1, 1, 63))
    with pytest.raises(ValueError, match="share one dtype"):
        mi.attn_prefill(k4, k4.to(bf), k4)


def test_wrappers_refuse_cpu_tensors():
    import torch
    q = torch.zeros(1, 64, 1, 64)
    with pytest.raises(ValueError, match="GPU"):
        mi.attn_prefill(q, q, q)


def test_partition_for_lengths():
    """attn_decode_paged_partition_for: the shortest multiple of 128 (up to
    1024) whose items x kv heads x 16-head slices fit in 256 CUs x 2 (D 128)
    or x 4 (D 64) workgroups; 1024 when none does (host logic, no GPU)."""
    def brute(lengths, hq, hkv, d):
        slots = 256 * (2 if d == 128 else 4)
        per = hkv * ((hq // hkv + 15) // 16)
        for p in range(128, 1025, 128):
            if sum((max(int(L), 0) + p - 1) // p for L in lengths) * per <= slots:
                return p
        return 1024
    g = np.random.default_rng(5)
    cases = [
        (g.integers(128, 4097, 64), 12, 2, 128),
        (np.full(256, 1024), 12, 2, 128),
        (np.full(257, 1024), 12, 2, 128),
        (np.full(64, 100), 12, 2, 128),
        (np.exp(g.uniform(np.log(16), np.log(32768), 128)).astype(int), 12, 2, 128),
        (g.integers(1, 3000, 40), 12, 12, 128),
        (g.integers(1, 3000, 40), 32, 1, 64),
        (np.array([0, -5, 7]), 12, 2, 128),
        (np.zeros(0), 12, 2, 128),
    ]
    for lengths, hq, hkv, d in cases:
        assert mi.attn_decode_paged_partition_for(lengths, hq, hkv, d) == brute(lengths, hq, hkv, d), (len(lengths), hq, hkv, d)
    # the uniform-context decode batch of 64 sequences, U[128, 4096] (seed 1002)
    from workloads import decode_case
    dc = decode_case(1002, 64, 128, 4096)
    assert mi.attn_decode_paged_partition_for(dc.lengths, 12, 2, 128) == 640
    assert mi.attn_decode_paged_partition_for(np.full(256, 1024), 12, 2, 128) == 1024
    lib = mi.load()
    assert lib.attn_decode_paged_partition_for(None, 3, 12, 2, 128) == ATTN_E_INVALID
    arr = (ctypes.c_int32 * 2)(5, 6)
    for hq, hkv, d in ((12, 2, 96), (12, 5, 128), (1, 2, 128), (12, 0, 128)):
        assert lib.attn_decode_paged_partition_for(arr, 2, hq, hkv, d) == ATTN_E_INVALID


def mixed_parts(**kw):
    """Valid-looking parts for attn_prefill_decode_paged (fake device
    pointers: only calls that fail validation or have nothing to launch are
    made on the CPU)."""
    pre = mi._PrefillPart(q=P, block_table=P, max_blocks_per_seq=8, cu_seqlens_q=P, context_lens=P, o=P,
                          num_seqs=2, total_q=100, max_seqlen_q=50, max_context_len=128, causal=1)
    dec = mi._DecodePart(q=P, block_table=P, max_blocks_per_seq=8, context_lens=P, o=P, num_seqs=4,
                         max_context_len=128, partition_size=0, plan=None, plan_items=0, workspace=P,
                         workspace_bytes=1 << 30)
    for k, v in kw.items():
        part, field = k.split("__")
        setattr(pre if part == "pre" else dec, field, v)
    return pre, dec


@pytest.mark.parametrize("kw,status", [
    (dict(pre__num_seqs=-1), ATTN_E_INVALID),
    (dict(pre__max_seqlen_q=101), ATTN_E_INVALID),          # longer than total_q
    (dict(dec__partition_size=40), ATTN_E_INVALID),
    (dict(dec__q_rot_out=P), ATTN_E_INVALID),               # rotated queries without the token write
    (dict(dec__k_new=P), ATTN_E_INVALID),                   # an incomplete token write
    (dict(dec__max_blocks_per_seq=7), ATTN_E_INVALID),      # 128 tokens need 8 blocks
    (dict(dec__plan=P, dec__plan_items=-1), ATTN_E_INVALID),
])
def test_prefill_decode_rejects(lib, kw, status):
    pre, dec = mixed_parts(**kw)
    st = lib.attn_prefill_decode_paged(ctypes.byref(pre), ctypes.byref(dec), P, P, 12, 2, 128, 16, 100, 0.0,
                                       ATTN_BF16, None)
    assert st == status
    assert lib.attn_last_error().decode().startswith("attn_prefill_decode_paged")


def test_prefill_decode_argument_rules(lib):
    pre, dec = mixed_parts()
    args = (P, P, 12, 2, 128, 16, 100, 0.0)
    assert lib.attn_prefill_decode_paged(None, ctypes.byref(dec), *args, ATTN_BF16, None) == ATTN_E_INVALID
    assert lib.attn_prefill_decode_paged(ctypes.byref(pre), ctypes.byref(dec), *args, ATTN_F32, None) == \
        ATTN_E_UNSUPPORTED
    # both parts empty: nothing to launch, success
    pre, dec = mixed_parts(pre__num_seqs=0, pre__total_q=0, pre__max_seqlen_q=0, dec__num_seqs=0)
    assert lib.attn_prefill_decode_paged(ctypes.byref(pre), ctypes.byref(dec), *args, ATTN_BF16, None) == 0
