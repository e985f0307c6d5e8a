"""Host-side checks of the C-ABI library (no GPU needed): exported symbols, struct
layout against the header, plan refusals, chunking and the workspace contract."""
import ctypes
import math
import os
import re
import subprocess

import numpy as np
import pytest

import paged_split_kv_02_amd as K
from tests.golden.read import load as load_golden

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_decode.h")


def declared_functions():
    text = "".join(open(os.path.join(ROOT, "include", f)).read()
                   for f in sorted(os.listdir(os.path.join(ROOT, "include"))) if f.endswith(".h"))
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(attn_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(K.SYMBOLS), names
    lib = ctypes.CDLL(K.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", K.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(attn_\w+)$", out, re.M))
    assert set(names) <= exported


def test_struct_layout_matches_header(tmp_path):
    fields = [f for f, _ in K.AttnDecodeDesc._fields_]
    pfields = [f for f, _ in K.AttnDecodePlan._fields_]
    src = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', "int main(void){",
           'printf("%zu %zu\\n", sizeof(attn_decode_desc), sizeof(attn_decode_plan_t));']
    src += [f'printf("%zu\\n", offsetof(attn_decode_desc, {f}));' for f in fields]
    src += [f'printf("%zu\\n", offsetof(attn_decode_plan_t, {f}));' for f in pfields]
    src += ["return 0;}"]
    c = tmp_path / "layout.c"
    c.write_text("\n".join(src))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-o", str(exe), str(c)], check=True)
    vals = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()
    assert int(vals[0]) == ctypes.sizeof(K.AttnDecodeDesc)
    assert int(vals[1]) == ctypes.sizeof(K.AttnDecodePlan)
    offs = [int(v) for v in vals[2:]]
    assert offs[:len(fields)] == [getattr(K.AttnDecodeDesc, f).offset for f in fields]
    assert offs[len(fields):] == [getattr(K.AttnDecodePlan, f).offset for f in pfields]


def global_desc(L=1024, **kw):
    ps, hkv, cols = 256, 4, 1024
    pages = (L + ps - 1) // ps
    f = dict(batch=1, num_q_heads=32, num_kv_heads=hkv, head_dim=512, format=0, rot_cols=0,
             page_size=ps, max_pages_per_seq=pages, window=0, num_chunks=0, merge_group=0,
             scale=1 / math.sqrt(512), num_pages=pages + 4, page_stride=hkv * ps * cols,
             head_stride=ps * cols, row_stride=cols, k_offset=0, v_offset=512)
    f.update(kw)
    return f


def plan_status(lens, **fields):
    d = K.make_desc(**fields)
    p = K.AttnDecodePlan()
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    return K._lib.attn_decode_plan(ctypes.byref(d), lens.ctypes.data, ctypes.byref(p)), p


S = K.STATUS


@pytest.mark.parametrize("lens,fields,status", [
    ([1024], dict(batch=0), "ATTN_E_INVALID_ARG"),
    ([1024], dict(num_kv_heads=5), "ATTN_E_UNSUPPORTED"),
    ([1024], dict(num_kv_heads=8), "ATTN_E_UNSUPPORTED"),          # GQA 4 at D=512
    ([1024], dict(head_dim=128), "ATTN_E_UNSUPPORTED"),
    ([1024], dict(format=1, rot_cols=64, v_offset=64), "ATTN_E_UNSUPPORTED"),
    ([1024], dict(format=2), "ATTN_E_INVALID_ARG"),
    ([1024], dict(page_size=8, max_pages_per_seq=128), "ATTN_E_UNSUPPORTED"),
    ([1024], dict(row_stride=1020), "ATTN_E_INVALID_ARG"),
    ([1024], dict(v_offset=516), "ATTN_E_INVALID_ARG"),
    ([1024], dict(page_stride=4 * 256 * 1024 - 8), "ATTN_E_INVALID_ARG"),  # last row overruns the page
    ([1024], dict(scale=float("nan")), "ATTN_E_INVALID_ARG"),
    ([0], dict(), "ATTN_E_INVALID_ARG"),
    ([-3], dict(), "ATTN_E_INVALID_ARG"),
    ([1025], dict(), "ATTN_E_PAST_PAGES"),
    ([1024], dict(num_pages=1 << 62), "ATTN_E_OVERFLOW"),
    ([1024], dict(num_chunks=-1), "ATTN_E_INVALID_ARG"),
    ([1024], dict(window=-1), "ATTN_E_INVALID_ARG"),
    ([1024], dict(kv_dtype=4), "ATTN_E_INVALID_ARG"),              # unknown element type
    ([1024], dict(kv_dtype=-1), "ATTN_E_INVALID_ARG"),
    ([1024], dict(k_scale=0.0), "ATTN_E_INVALID_ARG"),
    ([1024], dict(v_scale=-0.5), "ATTN_E_INVALID_ARG"),
    ([1024], dict(k_scale=float("inf")), "ATTN_E_INVALID_ARG"),
    ([1024], dict(v_scale=float("nan")), "ATTN_E_INVALID_ARG"),
    # FP8 rows: offsets and strides must be multiples of 16 elements (16 bytes)
    ([1024], dict(kv_dtype=2, v_offset=520), "ATTN_E_INVALID_ARG"),
    ([1024], dict(kv_dtype=2, row_stride=1032), "ATTN_E_INVALID_ARG"),
])
def test_plan_refusals(lens, fields, status):
    f = global_desc()
    f.update(fields)
    rc, _ = plan_status(lens, **f)
    assert rc == S[status], (rc, K.attn_decode_status_string(rc))


@pytest.mark.parametrize("kv_dtype", [0, 1, 2, 3])
def test_plan_accepts_served_element_types(kv_dtype):
    rc, p = plan_status([1024], **global_desc(1024, kv_dtype=kv_dtype, k_scale=0.5, v_scale=3.0))
    assert rc == 0
    assert p.desc.kv_dtype == kv_dtype and p.desc.k_scale == 0.5 and p.desc.v_scale == 3.0
    # 16-bit rows accept 8-element alignment; FP8 rows need 16
    rc, _ = plan_status([1024], **global_desc(1024, kv_dtype=kv_dtype, v_offset=520,
                                              row_stride=1032, head_stride=256 * 1032,
                                              page_stride=4 * 256 * 1032))
    assert rc == (0 if kv_dtype != 2 else S["ATTN_E_INVALID_ARG"])


def test_plan_accepts_exact_capacity_and_refuses_one_past():
    rc, _ = plan_status([1024], **global_desc(1024))
    assert rc == 0
    rc, _ = plan_status([1025], **global_desc(1024))
    assert rc == S["ATTN_E_PAST_PAGES"]


def test_positions_near_two_to_the_31_refused():
    """Key positions are 32-bit in the kernels: a plan whose chunks would end within 1024
    positions of 2^31 (lengths near it round up to whole tiles) is refused; one a little
    shorter is accepted and its chunks end below that bound."""
    big = dict(global_desc(), max_pages_per_seq=(1 << 23) + 4, num_pages=(1 << 23) + 8)
    for L in (2**31 - 1, 2**31 - 1024):
        rc, _ = plan_status([L], **big)
        assert rc == S["ATTN_E_OVERFLOW"], L
        rc, _ = prefill_status([L], [0, 1], **big)
        assert rc == S["ATTN_E_OVERFLOW"], L
    L = 2**31 - 70000
    rc, p = plan_status([L], **big)
    assert rc == 0
    pair = p.chunk_len + p.chunk_len_odd
    cover = (p.num_chunks // 2) * pair + (p.num_chunks % 2) * p.chunk_len
    assert L <= cover <= 2**31 - 1 - 1024
    rc, _ = prefill_status([L], [0, 1], **big)
    assert rc == 0


def test_plan_fuzz_under_sanitizers(tmp_path):
    """Host-side fuzz of the planning calls built with AddressSanitizer and
    UndefinedBehaviorSanitizer (g++, host code only): 200,000 seeded descriptors from
    valid shapes with up to two hostile fields, invariants of every accepted plan."""
    exe = tmp_path / "plan_fuzz"
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                    os.path.join(ROOT, "paged_split_kv_02_amd", "csrc", "plan.cpp"),
                    os.path.join(ROOT, "tests", "host", "plan_fuzz.cpp"), "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr
    m = re.search(r"(\d+) decode plans accepted, (\d+) refused, (\d+) prefill plans accepted", res.stdout)
    assert m and int(m.group(1)) > 10000 and int(m.group(2)) > 10000 and int(m.group(3)) > 10000, res.stdout


def test_null_pointers_refused():
    d = K.make_desc(**global_desc())
    p = K.AttnDecodePlan()
    lens = np.array([1024], dtype=np.int32)
    assert K._lib.attn_decode_plan(None, lens.ctypes.data, ctypes.byref(p)) == S["ATTN_E_INVALID_ARG"]
    assert K._lib.attn_decode_plan(ctypes.byref(d), None, ctypes.byref(p)) == S["ATTN_E_INVALID_ARG"]
    assert K._lib.attn_decode_plan(ctypes.byref(d), lens.ctypes.data, None) == S["ATTN_E_INVALID_ARG"]


def test_workspace_matches_gem_scratch_contract():
    """At P = 32, Hq = 32, D = 512 the workspace is the byte contract the gem design
    note prints: 4,096 + 4,096 + 2,097,152 = 2,105,344 bytes."""
    gold = load_golden("gem_scratch_contract.txt")
    rc, p = plan_status([8192], **global_desc(8192, num_chunks=gold["partitions"]))
    assert rc == 0
    assert p.num_chunks == gold["partitions"]
    assert p.off_part_m == 0
    assert p.off_part_l - p.off_part_m == gold["maxima_bytes"]
    assert p.off_part_o - p.off_part_l == gold["denominators_bytes"]
    assert p.workspace_bytes - p.off_part_o == gold["numerators_bytes"]
    assert p.workspace_bytes == gold["total_bytes"]


def test_size_limits_fail_closed():
    """A pool whose element count passes 2^60, or a merge grid past 65535 rows, is refused."""
    rc, _ = plan_status([1024], **global_desc(1024, num_pages=1 << 62))
    assert rc == S["ATTN_E_OVERFLOW"]
    # page_stride is 2^20 elements: 2^40 pages reach the limit exactly, one more passes it
    rc, _ = plan_status([1024], **global_desc(1024, num_pages=1 << 40))
    assert rc == 0
    rc, _ = plan_status([1024], **global_desc(1024, num_pages=(1 << 40) + 1))
    assert rc == S["ATTN_E_OVERFLOW"]
    hkv = 8191
    f = global_desc(1024, batch=9, num_q_heads=8 * hkv, num_kv_heads=hkv,
                    page_stride=hkv * 256 * 1024, num_pages=8)
    rc, _ = plan_status([1024] * 9, **f)
    assert rc == S["ATTN_E_OVERFLOW"], rc       # 9 x 65528 merge rows
    f["batch"] = 1
    rc, p = plan_status([1024], **f)
    assert rc == 0 and p.workspace_bytes > 0


def test_merge_group_bounds():
    rc, p = plan_status([8192], **global_desc(8192, num_chunks=64, merge_group=8))
    assert rc == 0 and p.num_groups == 8
    rc, _ = plan_status([8192], **global_desc(8192, num_chunks=64, merge_group=7))
    assert rc == S["ATTN_E_UNSUPPORTED"]
    rc, p = plan_status([8192], **global_desc(8192, num_chunks=64))
    assert rc == 0 and p.merge_group == 8 and p.num_groups == 8
    rc, p = plan_status([8192], **global_desc(8192, num_chunks=5))
    assert rc == 0 and p.merge_group == 1 and p.num_groups == 5


def chunk_ranges(p, L):
    """Chunks as the header lays them out: even-numbered ones chunk_len keys, odd-numbered
    ones chunk_len_odd, from the request's start, cut to the visible keys."""
    lo = max(0, L - p.desc.window) if p.desc.window > 0 else 0
    a = lo // p.tile * p.tile
    out = []
    for c in range(p.num_chunks):
        n = p.chunk_len if c % 2 == 0 else p.chunk_len_odd
        out.append((max(a, lo), min(a + n, L)))
        a += n
    return lo, out


@pytest.mark.parametrize("lens,fields,expect", [
    ([1024], dict(num_chunks=8), dict(num_chunks=8, chunk_len=128, chunk_len_odd=128)),
    # automatic chunking of a long context: even-numbered chunks (on the even XCDs) take
    # 42 tiles per quarter, odd ones 38, instead of 40 each
    ([163336], dict(), dict(num_chunks=64, chunk_len=2688, chunk_len_odd=2432)),
    ([81653], dict(), dict(num_chunks=64, chunk_len=1344, chunk_len_odd=1216)),
    ([10602], dict(), dict(num_chunks=56, chunk_len=192, chunk_len_odd=192)),
    ([100], dict(num_chunks=16), dict(num_chunks=16, chunk_len=64, chunk_len_odd=64)),
])
def test_chunking(lens, fields, expect):
    L = lens[0]
    f = global_desc(L, **fields)
    rc, p = plan_status(lens, **f)
    assert rc == 0
    for k, v in expect.items():
        assert getattr(p, k) == v, (k, getattr(p, k))
    assert p.chunk_len % (4 * p.tile) == 0 and p.chunk_len_odd % (4 * p.tile) == 0
    assert p.tile == 16
    assert p.chunk_len_odd == p.chunk_len or p.num_chunks % 2 == 0  # skew: even chunk count
    lo, ranges = chunk_ranges(p, L)
    covered = [x for a, b in ranges for x in range(a, b)]
    assert covered == list(range(lo, L)), "chunks must tile [lo, L) in order"
    assert p.num_groups == -(-p.num_chunks // p.merge_group)


def test_sliding_chunking_covers_every_window():
    rng = np.random.default_rng(0)
    lens = rng.integers(1, 4097, size=16)
    f = dict(batch=16, num_q_heads=32, num_kv_heads=16, head_dim=256, format=0, rot_cols=0,
             page_size=64, max_pages_per_seq=64, window=1024, num_chunks=0, merge_group=0,
             scale=1 / 16, num_pages=300, page_stride=16 * 64 * 512, head_stride=64 * 512,
             row_stride=512, k_offset=0, v_offset=256)
    rc, p = plan_status(lens, **f)
    assert rc == 0
    for L in lens:
        lo, ranges = chunk_ranges(p, int(L))
        covered = [x for a, b in ranges for x in range(a, b)]
        assert covered == list(range(lo, int(L)))
        assert int(L) - lo == min(int(L), 1024)


def test_stream_read_refuses_before_any_launch():
    fake = 1 << 20  # never dereferenced: every refusal below returns before a launch
    L = K._lib
    assert L.attn_stream_read(None, 1024, fake, None) == S["ATTN_E_INVALID_ARG"]
    assert L.attn_stream_read(fake, 1024, None, None) == S["ATTN_E_INVALID_ARG"]
    assert L.attn_stream_read(fake, 1000, fake, None) == S["ATTN_E_INVALID_ARG"]   # not whole words
    assert L.attn_stream_read(fake + 8, 1024, fake, None) == S["ATTN_E_INVALID_ARG"]  # misaligned
    assert L.attn_stream_read(fake, 1024, fake + 4, None) == S["ATTN_E_INVALID_ARG"]
    text = open(os.path.join(ROOT, "include", "attn_measure.h")).read()
    assert int(re.search(r"#define ATTN_STREAM_READ_GROUPS (\d+)", text).group(1)) == K.STREAM_READ_GROUPS


def test_split_and_merge_refuse_before_any_launch():
    rc, p = plan_status([1024], **global_desc())
    assert rc == 0
    fake = 1 << 20  # never dereferenced: every refusal below returns before a launch
    ws = p.workspace_bytes
    bad = K.AttnDecodePlan.from_buffer_copy(p)
    bad.magic = 0
    L = K._lib
    assert L.attn_decode_split(ctypes.byref(bad), fake, fake, fake, fake, fake, ws, None) == S["ATTN_E_PLAN"]
    assert L.attn_decode_merge(ctypes.byref(bad), fake, ws, fake, None) == S["ATTN_E_PLAN"]
    assert L.attn_decode_split(ctypes.byref(p), None, fake, fake, fake, fake, ws, None) == S["ATTN_E_INVALID_ARG"]
    assert L.attn_decode_split(ctypes.byref(p), fake, fake, fake, fake, fake, ws - 1, None) == S["ATTN_E_WORKSPACE"]
    assert L.attn_decode_split(ctypes.byref(p), fake, fake, fake, fake, fake + 4, ws, None) == S["ATTN_E_WORKSPACE"]
    assert L.attn_decode_merge(ctypes.byref(p), fake, ws - 1, fake, None) == S["ATTN_E_WORKSPACE"]
    assert L.attn_decode_merge(ctypes.byref(p), fake, ws, None, None) == S["ATTN_E_INVALID_ARG"]
    assert L.attn_decode_split(None, fake, fake, fake, fake, fake, ws, None) == S["ATTN_E_INVALID_ARG"]
    assert L.attn_kv_write(ctypes.byref(bad), fake, fake, 1, fake, fake, fake, None, None) == S["ATTN_E_PLAN"]
    assert L.attn_kv_write(ctypes.byref(p), fake, fake, 0, fake, fake, fake, None, None) == S["ATTN_E_INVALID_ARG"]
    assert L.attn_kv_write(ctypes.byref(p), None, fake, 1, fake, fake, fake, None, None) == S["ATTN_E_INVALID_ARG"]
    assert L.attn_query_fold(ctypes.byref(p), fake, fake, fake, None) == S["ATTN_E_UNSUPPORTED"]  # split plan
    assert L.attn_query_fold(ctypes.byref(bad), fake, fake, fake, None) == S["ATTN_E_PLAN"]
    # buffers the kernels move in 16-byte vectors must be 16-byte aligned
    mis = fake + 4
    assert L.attn_decode_split(ctypes.byref(p), mis, fake, fake, fake, fake, ws, None) == S["ATTN_E_INVALID_ARG"]
    assert L.attn_decode_split(ctypes.byref(p), fake, mis, fake, fake, fake, ws, None) == S["ATTN_E_INVALID_ARG"]
    assert L.attn_decode_merge(ctypes.byref(p), fake, ws, mis, None) == S["ATTN_E_INVALID_ARG"]
    assert L.attn_kv_write(ctypes.byref(p), mis, fake, 1, fake, fake, fake, None, None) == S["ATTN_E_INVALID_ARG"]
    assert L.attn_kv_write(ctypes.byref(p), fake, fake, 1, fake, mis, fake, None, None) == S["ATTN_E_INVALID_ARG"]
    odd = fake + 2  # int32 arrays at their element size
    assert L.attn_decode_split(ctypes.byref(p), fake, fake, odd, fake, fake, ws, None) == S["ATTN_E_INVALID_ARG"]
    assert L.attn_decode_split(ctypes.byref(p), fake, fake, fake, odd, fake, ws, None) == S["ATTN_E_INVALID_ARG"]
    assert L.attn_kv_write(ctypes.byref(p), fake, fake, 1, odd, fake, fake, None, None) == S["ATTN_E_INVALID_ARG"]


def test_tree_split_refuses_before_any_launch():
    """The tree entry point: a bad plan, a plan of one query row, null masks and the
    ordinary argument checks are all refused before a launch."""
    rc, p4 = plan_status([1024], **global_desc(num_rows=4))
    rc1, p1 = plan_status([1024], **global_desc())
    assert rc == 0 and rc1 == 0
    fake = 1 << 20  # never dereferenced
    ws = p4.workspace_bytes
    bad = K.AttnDecodePlan.from_buffer_copy(p4)
    bad.magic = 0
    T = K._lib.attn_decode_split_tree
    assert T(ctypes.byref(bad), fake, fake, fake, fake, fake, fake, ws, None) == S["ATTN_E_PLAN"]
    assert T(None, fake, fake, fake, fake, fake, fake, ws, None) == S["ATTN_E_INVALID_ARG"]
    assert T(ctypes.byref(p1), fake, fake, fake, fake, fake, fake, ws, None) == S["ATTN_E_INVALID_ARG"]
    assert T(ctypes.byref(p4), fake, fake, fake, fake, None, fake, ws, None) == S["ATTN_E_INVALID_ARG"]
    assert T(ctypes.byref(p4), None, fake, fake, fake, fake, fake, ws, None) == S["ATTN_E_INVALID_ARG"]
    assert T(ctypes.byref(p4), fake, fake, fake, fake, fake, fake, ws - 1, None) == S["ATTN_E_WORKSPACE"]


def test_status_strings():
    for name, code in S.items():
        s = K.attn_decode_status_string(code)
        assert s and s != "unknown status", name
    assert K.attn_decode_status_string(12345) == "unknown status"


def test_rows_plan():
    rc, p = plan_status([1000, 2000], **global_desc(2048, batch=2, num_rows=4))
    assert rc == 0 and p.num_rows == 4 and p.row_groups == 1 and p.grid_x == p.num_chunks
    assert p.chunk_len % 16 == 0 and p.chunk_len_odd == p.chunk_len  # rows: uniform chunks
    rc, p = plan_status([163336], **global_desc(163336, num_rows=4))
    assert rc == 0 and p.chunk_len_odd == p.chunk_len
    rc, p = plan_status([1000], **global_desc(1024, num_rows=8))
    assert rc == 0 and p.row_groups == 2 and p.grid_x == -(-p.num_chunks // 8) * 8 * 2
    # workspace counts request x row states
    rc, p1 = plan_status([1000], **global_desc(1024, num_rows=1, num_chunks=16))
    rc, p3 = plan_status([1000], **global_desc(1024, num_rows=3, num_chunks=16))
    assert p3.workspace_bytes >= 3 * (p1.workspace_bytes - 512)
    rc, _ = plan_status([3], **global_desc(1024, num_rows=4))
    assert rc == S["ATTN_E_INVALID_ARG"]          # fewer keys than rows
    rc, _ = plan_status([1000], **global_desc(1024, num_rows=65))
    assert rc == S["ATTN_E_INVALID_ARG"]
    rc, _ = plan_status([1000], **global_desc(1024, num_rows=-1))
    assert rc == S["ATTN_E_INVALID_ARG"]


def test_rows_plan_tile_choice():
    """Several rows at head dim 512 over bf16 pages of whole 32-key tiles: 32-key tiles
    (chunk starts and lengths in whole tiles); one row, other element types or pages of
    16 keep 16-key tiles."""
    for fmt, rot, v_off, cols in ((0, 0, 512, 1024), (1, 128, 128, 640)):
        f = global_desc(163336, num_rows=4, format=fmt, rot_cols=rot, v_offset=v_off,
                        row_stride=cols, head_stride=256 * cols, page_stride=4 * 256 * cols)
        rc, p = plan_status([163336], **f)
        assert rc == 0 and p.tile == 32 and p.chunk_len % 32 == 0
        assert p.num_chunks * p.chunk_len >= 163336 and p.grid_x == p.num_chunks
    # a window: chunks start at the first row's window start rounded down to 32
    rc, p = plan_status([5000], **global_desc(5000, num_rows=3, window=1024, num_chunks=3))
    assert rc == 0 and p.tile == 32 and p.max_span == 5000 - (5000 - 3 + 1 - 1024) // 32 * 32
    rc, p = plan_status([1000], **global_desc(1024, num_rows=1))
    assert rc == 0 and p.tile == 16
    rc, p = plan_status([1000], **global_desc(1024, num_rows=4, kv_dtype=1))
    assert rc == 0 and p.tile == 16                    # f16: the 16-key rows kernel
    rc, p = plan_status([1000], **global_desc(1024, num_rows=4, kv_dtype=2))
    assert rc == 0 and p.tile == 32                    # FP8: widened on the 32-key kernel
    rc, p = plan_status([1000], **global_desc(1024, num_rows=4, page_size=16,
                                              max_pages_per_seq=64, page_stride=4 * 16 * 1024,
                                              head_stride=16 * 1024, num_pages=70))
    assert rc == 0 and p.tile == 16



# ---------------------------------------------------------------------------- prefill plan

def prefill_status(lens, starts, **fields):
    d = K.make_desc(**fields)
    p = K.AttnPrefillPlan()
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    starts = np.ascontiguousarray(starts, dtype=np.int32)
    return K._lib.attn_prefill_plan(ctypes.byref(d), lens.ctypes.data, starts.ctypes.data,
                                    ctypes.byref(p)), p


def test_prefill_plan_layout_matches_header(tmp_path):
    pfields = [f for f, _ in K.AttnPrefillPlan._fields_]
    src = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', "int main(void){",
           'printf("%zu\\n", sizeof(attn_prefill_plan_t));']
    src += [f'printf("%zu\\n", offsetof(attn_prefill_plan_t, {f}));' for f in pfields]
    src += ["return 0;}"]
    c = tmp_path / "layout.c"
    c.write_text("\n".join(src))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-o", str(exe), str(c)], check=True)
    vals = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                           check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(K.AttnPrefillPlan)
    assert vals[1:] == [getattr(K.AttnPrefillPlan, f).offset for f in pfields]


def test_prefill_plan_accepts_f16():
    rc, p = prefill_status([1024], [0, 1000], **global_desc(kv_dtype=1))
    assert rc == 0 and p.row_tile == 8 and p.desc.kv_dtype == 1


def test_prefill_plan_accepts_fp8():
    rc, p = prefill_status([1024], [0, 1000], **global_desc(kv_dtype=2, k_scale=0.02, v_scale=0.03))
    assert rc == 0 and p.row_tile == 8 and p.desc.kv_dtype == 2


def test_prefill_plan_tiles():
    rc, p = prefill_status([1024], [0, 1000], **global_desc())
    assert rc == 0 and p.row_tile == 8 and p.key_tile == 32 and p.total_rows == 1000
    assert p.max_rows == 1000 and p.grid_x == 125 and p.group_size == 8
    f = dict(batch=3, num_q_heads=32, num_kv_heads=16, head_dim=256, format=0, rot_cols=0,
             page_size=64, max_pages_per_seq=64, window=1024, scale=1 / 16, num_pages=200,
             page_stride=16 * 64 * 512, head_stride=64 * 512, row_stride=512, k_offset=0,
             v_offset=256)
    rc, p = prefill_status([4096, 30, 700], [0, 4096, 4096, 4196], **f)
    assert rc == 0 and p.row_tile == 64 and p.max_rows == 4096 and p.grid_x == 64
    assert p.total_rows == 4196


@pytest.mark.parametrize("lens,starts,fields,status", [
    ([1024], [1, 1000], dict(), "ATTN_E_INVALID_ARG"),            # offsets must start at 0
    ([1024], [0, 1025], dict(), "ATTN_E_INVALID_ARG"),            # more rows than keys
    ([10, 10], [0, 5, 4], dict(batch=2), "ATTN_E_INVALID_ARG"),   # decreasing offsets
    ([1025], [0, 1], dict(), "ATTN_E_PAST_PAGES"),
    ([1024], [0, 8], dict(page_size=16, max_pages_per_seq=64), "ATTN_E_UNSUPPORTED"),
    ([1024], [0, 8], dict(head_dim=128), "ATTN_E_UNSUPPORTED"),
    ([1024], [0, 8], dict(row_stride=1020), "ATTN_E_INVALID_ARG"),
    ([1024], [0, 8], dict(batch=0), "ATTN_E_INVALID_ARG"),
    # rows of a tile must be reachable with 32-bit offsets
    ([1024], [0, 8], dict(row_stride=1 << 26, head_stride=1 << 34, page_stride=1 << 36),
     "ATTN_E_OVERFLOW"),
])
def test_prefill_plan_refusals(lens, starts, fields, status):
    f = global_desc()
    f.update(fields)
    rc, _ = prefill_status(lens, starts, **f)
    assert rc == S[status], (rc, status)


def test_prefill_plan_allows_empty_requests():
    rc, p = prefill_status([1024, 5], [0, 0, 0], **global_desc(batch=2))
    assert rc == 0 and p.total_rows == 0 and p.grid_x == 0


def test_prefill_refuses_before_any_launch():
    rc, p = prefill_status([1024], [0, 100], **global_desc())
    assert rc == 0
    fake = 1 << 20  # never dereferenced: every refusal below returns before a launch
    bad = K.AttnPrefillPlan.from_buffer_copy(p)
    bad.magic = 0
    L = K._lib
    assert L.attn_prefill(ctypes.byref(bad), fake, fake, fake, fake, fake, fake, None) == S["ATTN_E_PLAN"]
    assert L.attn_prefill(None, fake, fake, fake, fake, fake, fake, None) == S["ATTN_E_INVALID_ARG"]
    for k in range(6):
        args = [fake] * 6
        args[k] = None
        assert L.attn_prefill(ctypes.byref(p), *args, None) == S["ATTN_E_INVALID_ARG"], k
    for k in (0, 1, 5):  # q, pool and out move in 16-byte vectors
        args = [fake] * 6
        args[k] = fake + 4
        assert L.attn_prefill(ctypes.byref(p), *args, None) == S["ATTN_E_INVALID_ARG"], k
    # a decode plan is not a prefill plan
    rc, dp = plan_status([1024], **global_desc())
    assert L.attn_prefill(ctypes.cast(ctypes.byref(dp), ctypes.POINTER(K.AttnPrefillPlan)),
                          fake, fake, fake, fake, fake, fake, None) == S["ATTN_E_PLAN"]


def test_python_plan_refuses_wrong_length_count():
    """The binding checks that the host lengths hold exactly `batch` entries before the
    library reads them (a short array would be read past its end)."""
    d = K.make_desc(**global_desc(1024, batch=2, max_pages_per_seq=4))
    with pytest.raises(ValueError):
        K.attn_decode_plan(d, np.array([1024], dtype=np.int32))
    with pytest.raises(ValueError):
        K.attn_decode_plan(d, np.array([1024, 1024, 1024], dtype=np.int32))
    assert K.attn_decode_plan(d, np.array([1024, 1000], dtype=np.int32)).num_chunks >= 1


def test_loaded_library_matches_the_sources():
    """The library the binding loaded was built from the sources in the tree (the loader
    rebuilds a library whose recorded source digest differs)."""
    from paged_split_kv_02_amd import build as B
    assert B.is_current(), "libattn_decode.so is older than its sources"
    assert B.built_digest() == B.source_digest()


def test_noalloc_step_refuses_before_any_device_call():
    """The allocation-free step refuses a bad plan, null or misaligned buffers, masks with a
    one-row plan and a plan larger than its static array, all before touching a device."""
    rc, p = plan_status([1024], **global_desc())
    rc4, p4 = plan_status([1024], **global_desc(num_rows=4))
    assert rc == 0 and rc4 == 0
    # 16 requests of 163,336 tokens with 64-chunk states: more than the static array holds
    big_lens = [163336] * 16
    rcb, pb = plan_status(big_lens, **global_desc(163336, batch=16, num_chunks=64))
    assert rcb == 0 and pb.workspace_bytes > K.NOALLOC_SCRATCH_BYTES
    text = open(HEADER).read()
    assert re.search(r"#define ATTN_NOALLOC_SCRATCH_BYTES \(32u << 20\)", text)
    fake = 1 << 20  # never dereferenced
    bad = K.AttnDecodePlan.from_buffer_copy(p)
    bad.magic = 0
    N = K._lib.attn_decode_step_noalloc
    assert N(ctypes.byref(bad), fake, fake, fake, fake, None, fake, None) == S["ATTN_E_PLAN"]
    assert N(None, fake, fake, fake, fake, None, fake, None) == S["ATTN_E_INVALID_ARG"]
    assert N(ctypes.byref(p), fake, fake, fake, fake, None, None, None) == S["ATTN_E_INVALID_ARG"]
    assert N(ctypes.byref(p), None, fake, fake, fake, None, fake, None) == S["ATTN_E_INVALID_ARG"]
    assert N(ctypes.byref(p), fake, fake, fake, fake, None, fake + 4, None) == S["ATTN_E_INVALID_ARG"]
    assert N(ctypes.byref(p), fake, fake, fake, fake, fake, fake, None) == S["ATTN_E_INVALID_ARG"]
    assert N(ctypes.byref(p4), fake, fake, fake, fake, fake + 4, fake, None) == S["ATTN_E_INVALID_ARG"]
    assert N(ctypes.byref(pb), fake, fake, fake, fake, None, fake, None) == S["ATTN_E_SCRATCH"]


def test_sliding_plan_workgroups_per_cu():
    """One query row at head dim 256: one workgroup per CU in one round for the 16-bit and
    FP8 pools (the 16-request sliding batch, 16 x 16 KV heads, in one chunk per (request, KV
    head): 256 workgroups), two per CU for f32 pools (two chunks: 512 workgroups; a shorter
    request's second chunk is empty); a 4-request batch takes four chunks, and more over f32."""
    rng = np.random.default_rng(4)
    lens = rng.integers(1, 4097, size=16)
    f = dict(batch=16, num_q_heads=32, num_kv_heads=16, head_dim=256, format=0, rot_cols=0,
             page_size=64, max_pages_per_seq=64, window=1024, num_chunks=0, merge_group=0,
             scale=1 / 16, num_pages=300, page_stride=16 * 64 * 512, head_stride=64 * 512,
             row_stride=512, k_offset=0, v_offset=256)
    for kv_dtype in (0, 1, 2):  # bf16, f16, FP8 E4M3
        rc, p = plan_status(lens, **f, kv_dtype=kv_dtype)
        assert rc == 0 and p.num_chunks == 1 and p.grid_x == 1
    rc, p = plan_status(lens, **f, kv_dtype=3)  # f32: strides are in elements, as for bf16
    assert rc == 0 and p.num_chunks == 2 and p.grid_x == 2
    assert p.num_chunks * 16 * 16 == 512
    rc, p = plan_status(lens[:4], **dict(f, batch=4))
    assert rc == 0 and p.num_chunks == 4
    rc, p = plan_status(lens[:4], **dict(f, batch=4), kv_dtype=3)
    assert rc == 0 and p.num_chunks > 4  # eight asked for, fewer after rounding to whole quarters


def test_f32_rows_plan():
    """f32 windows of several rows: 16 / G rows per row group (2 at head dim 512), each wave
    a quarter of a chunk, 16-key tiles; the row groups of a chunk 8 workgroups apart."""
    rc, p = plan_status([5000], **global_desc(5000, kv_dtype=3, num_rows=5))
    assert rc == 0 and p.num_rows == 5 and p.row_groups == 3 and p.tile == 16
    assert p.chunk_len % (4 * 16) == 0
    assert p.grid_x == -(-p.num_chunks // 8) * 8 * 3


def test_f32_prefill_plan():
    rc, p = prefill_status([1024], [0, 1000], **global_desc(kv_dtype=3))
    assert rc == 0 and p.row_tile == 2 and p.key_tile == 16 and p.grid_x == 500


def test_f32_folded_plans_accepted():
    """f32 pools hold split or folded rows, for decode (one or several rows) and prefill."""
    f = global_desc(kv_dtype=3, format=1, rot_cols=128, v_offset=128, row_stride=640,
                    head_stride=256 * 640, page_stride=4 * 256 * 640)
    rc, p = plan_status([1024], **f)
    assert rc == 0 and p.tile == 16
    f["num_rows"] = 3
    rc, p = plan_status([1024], **f)
    assert rc == 0 and p.row_groups == 2
    f["num_rows"] = 0
    rc, p = prefill_status([1024], [0, 100], **f)
    assert rc == 0 and p.row_tile == 2
