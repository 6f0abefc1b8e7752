"""C-ABI tests that need no GPU: the library loads, exports every symbol the
header declares, rejects bad arguments before launching anything, and plans
decode splits (host-only logic) consistently with the pages' arithmetic."""

import ctypes
import json
import math
import os
import re
import subprocess

import numpy as np
import pytest

from tests.conftest import ROOT, load_golden

HEADER = os.path.join(ROOT, "include", "attn.h")


@pytest.fixture(scope="module")
def lib():
    from online_softmax_tiled_amd import api
    if not os.path.exists(api.LIB_PATH):
        from online_softmax_tiled_amd.build import build
        build()
    return api.load()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(attn_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    syms = declared_symbols()
    for name in ("attn_prefill_fwd", "attn_decode_plan", "attn_decode_split", "attn_merge_states",
                 "attn_paged_gather", "attn_last_error"):
        assert name in syms


def test_library_exports_every_declared_symbol(lib):
    from online_softmax_tiled_amd import api
    out = subprocess.run(["nm", "-D", "--defined-only", api.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s(attn_\w+)$", out, re.M))
    for name in declared_symbols():
        assert name in exported, name
        assert hasattr(lib, name)
    assert set(api.EXPORTS) == set(declared_symbols())


def test_one_hip_runtime_is_mapped(lib):
    maps = open("/proc/self/maps").read()
    paths = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    assert len(paths) == 1, paths


def test_version_and_empty_error(lib):
    from online_softmax_tiled_amd import api
    assert "gfx950" in api.version()


NULL = None


def prefill_call(lib, **kw):
    args = dict(q=1, k=1, v=1, km=NULL, rm=NULL, o=1, lse=NULL, B=1, h=4, h_kv=1, T_q=8, T_k=8,
                d=128, dtype=1, scale=0.088, causal=1)
    args.update(kw)
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.attn_prefill_fwd(p(args["q"]), p(args["k"]), p(args["v"]), p(args["km"]), p(args["rm"]),
                                p(args["o"]), p(args["lse"]), args["B"], args["h"], args["h_kv"],
                                args["T_q"], args["T_k"], args["d"], args["dtype"], args["scale"],
                                args["causal"], None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(d=64), 2, "head size"),
    (dict(dtype=5), 2, "dtype"),
    (dict(h=6, h_kv=4), 1, "multiple"),
    (dict(h_kv=0), 1, "positive"),
    (dict(scale=0.0), 1, "scale"),
    (dict(scale=float("nan")), 1, "scale"),
    (dict(T_q=9, T_k=8, causal=1), 2, "T_q <= T_k"),
    (dict(B=-1), 1, "negative"),
    (dict(q=None), 1, "NULL"),
    (dict(k=None), 1, "NULL"),
    (dict(B=1 << 20, h=1 << 12, h_kv=1 << 12, T_q=1, T_k=1, causal=0), 2, "B * h"),
])
def test_prefill_rejects_before_launch(lib, kw, code, msg):
    from online_softmax_tiled_amd import api
    assert prefill_call(lib, **kw) == code
    assert msg in api.last_error()


def test_prefill_empty_problem_is_ok_without_launch(lib):
    assert prefill_call(lib, B=0, q=None, k=None, v=None, o=None) == 0
    assert prefill_call(lib, T_q=0, T_k=0, causal=0, q=None, k=None, v=None, o=None) == 0


def split_call(lib, **kw):
    args = dict(q=1, k=1, v=1, bt=NULL, max_pages=0, page_size=16, num_pages=0, sl=1, s_max=64, B=1,
                h=8, h_kv=1, d=128, chunk=64, splits=1, dtype=1, scale=0.088, po=1, pm=1, pl=1)
    args.update(kw)
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.attn_decode_split(p(args["q"]), p(args["k"]), p(args["v"]), p(args["bt"]), args["max_pages"],
                                 args["page_size"], args["num_pages"], p(args["sl"]), args["s_max"], args["B"],
                                 args["h"], args["h_kv"], args["d"], args["chunk"], args["splits"],
                                 args["dtype"], args["scale"], p(args["po"]), p(args["pm"]), p(args["pl"]), None)


@pytest.mark.parametrize("kw,code", [
    (dict(h=514, h_kv=2), 2),              # 257 query heads per KV head
    (dict(chunk=40), 1),                   # not a multiple of 16
    (dict(chunk=0), 1),
    (dict(splits=0), 1),
    (dict(bt=1, page_size=8, max_pages=4, num_pages=4), 2),   # page not a multiple of 16
    (dict(bt=1, page_size=16, max_pages=0, num_pages=4), 1),
    (dict(pm=None), 1),
    (dict(d=96), 2),
    (dict(s_max=(1 << 23) + 1), 2),        # more keys per sequence than supported
    (dict(bt=1, page_size=1 << 16, max_pages=1 << 16, num_pages=4), 2),   # 2^32 addressable keys
    (dict(bt=1, page_size=16, max_pages=(1 << 19) + 1, num_pages=4), 2),
])
def test_decode_split_rejects_before_launch(lib, kw, code):
    assert split_call(lib, **kw) == code


def decode_call(lib, **kw):
    args = dict(q=1, k=1, v=1, bt=NULL, max_pages=0, page_size=16, num_pages=0, sl=1, s_max=64, B=1,
                h=8, h_kv=1, d=128, chunk=64, splits=1, dtype=1, scale=0.088, po=1, pm=1, pl=1, o=1,
                lse=NULL)
    args.update(kw)
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.attn_decode(p(args["q"]), p(args["k"]), p(args["v"]), p(args["bt"]), args["max_pages"],
                           args["page_size"], args["num_pages"], p(args["sl"]), args["s_max"], args["B"],
                           args["h"], args["h_kv"], args["d"], args["chunk"], args["splits"], args["dtype"],
                           args["scale"], p(args["po"]), p(args["pm"]), p(args["pl"]), p(args["o"]),
                           p(args["lse"]), None)


@pytest.mark.parametrize("kw,code", [
    (dict(h=514, h_kv=2), 2),
    (dict(chunk=40), 1),
    (dict(splits=0), 1),
    (dict(bt=1, page_size=8, max_pages=4, num_pages=4), 2),
    (dict(d=96), 2),
    (dict(dtype=2), 2),
    (dict(scale=0.0), 1),
    (dict(o=None), 1),
    (dict(po=None), 1),
    (dict(sl=None), 1),
    (dict(s_max=(1 << 23) + 1), 2),
])
def test_decode_rejects_before_launch(lib, kw, code):
    assert decode_call(lib, **kw) == code
    assert "attn_decode" in lib.attn_last_error().decode()


def fp8_call(lib, one_call, **kw):
    args = dict(q=1, k=1, v=1, bt=NULL, max_pages=0, page_size=16, num_pages=0, sl=1, s_max=64, B=1,
                h=8, h_kv=1, d=128, chunk=64, splits=1, dtype=1, scale=0.088, ks=0.5, vs=2.0, po=1, pm=1, pl=1,
                o=1, lse=NULL)
    args.update(kw)
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    head = (p(args["q"]), p(args["k"]), p(args["v"]), p(args["bt"]), args["max_pages"], args["page_size"],
            args["num_pages"], p(args["sl"]), args["s_max"], args["B"], args["h"], args["h_kv"], args["d"],
            args["chunk"], args["splits"], args["dtype"], args["scale"], args["ks"], args["vs"],
            p(args["po"]), p(args["pm"]), p(args["pl"]))
    if one_call:
        return lib.attn_decode_fp8kv(*head, p(args["o"]), p(args["lse"]), None)
    return lib.attn_decode_split_fp8kv(*head, None)


@pytest.mark.parametrize("one_call", [False, True])
@pytest.mark.parametrize("kw,code", [
    (dict(ks=0.0), 1),                     # scales finite and > 0
    (dict(vs=-1.0), 1),
    (dict(ks=float("inf")), 1),
    (dict(vs=float("nan")), 1),
    (dict(scale=0.0), 1),
    (dict(h=514, h_kv=2), 2),
    (dict(chunk=40), 1),
    (dict(splits=0), 1),
    (dict(bt=1, page_size=8, max_pages=4, num_pages=4), 2),
    (dict(d=96), 2),
    (dict(dtype=2), 2),
    (dict(pl=None), 1),
    (dict(k=None), 1),
    (dict(s_max=(1 << 23) + 1), 2),
])
def test_fp8kv_decode_rejects_before_launch(lib, one_call, kw, code):
    assert fp8_call(lib, one_call, **kw) == code
    assert "fp8kv" in lib.attn_last_error().decode()


def test_fp8kv_decode_needs_o_only_in_one_call(lib):
    assert fp8_call(lib, True, o=None) == 1
    assert fp8_call(lib, False, o=None, B=0) == 0
    assert fp8_call(lib, True, B=0, q=None, k=None, v=None, sl=None, po=None, pm=None, pl=None, o=None) == 0


def test_decode_empty_batch_is_ok_without_launch(lib):
    assert decode_call(lib, B=0, q=None, k=None, v=None, sl=None, po=None, pm=None, pl=None, o=None) == 0


def test_merge_and_gather_reject_before_launch(lib):
    p = ctypes.c_void_p
    assert lib.attn_merge_lse(p(1), p(1), p(1), p(1), -1, 128, p(1), None, 1, None) == 1
    assert lib.attn_merge_lse(p(1), None, p(1), p(1), 8, 128, p(1), None, 1, None) == 1
    assert lib.attn_merge_lse(p(1), p(1), p(1), p(1), 8, 64, p(1), None, 1, None) == 2
    assert lib.attn_merge_lse(p(1), p(1), p(1), p(1), 8, 128, p(1), None, 7, None) == 2
    assert lib.attn_merge_lse(None, None, None, None, 0, 128, None, None, 1, None) == 0
    assert lib.attn_merge_states(p(1), p(1), p(1), p(1), 0, 1, 8, 4, 128, p(1), None, 1, None) == 1
    assert lib.attn_merge_states(p(1), p(1), p(1), p(1), 64, 1, 8, 0, 128, p(1), None, 1, None) == 1
    assert lib.attn_merge_states(p(1), None, p(1), p(1), 64, 1, 8, 4, 128, p(1), None, 1, None) == 1
    assert lib.attn_merge_states(p(1), p(1), p(1), p(1), 64, 1, 8, 4, 64, p(1), None, 1, None) == 2
    assert lib.attn_paged_gather(p(1), p(1), p(1), 1, 8, 128, 0, 4, 4, 64, 1, p(1), None) == 1
    # more addressable keys than an int holds
    assert lib.attn_paged_gather(p(1), p(1), p(1), 1, 8, 128, 1 << 16, 1 << 15, 4, 64, 1, p(1), None) == 2
    assert lib.attn_paged_gather(p(1), None, p(1), 1, 8, 128, 16, 4, 4, 64, 1, p(1), None) == 1
    assert lib.attn_paged_gather(p(1), p(1), p(1), 1, 8, 128, 16, 4, 4, 64, 3, p(1), None) == 2


# ---------------------------------------------------------------- decode plan

def plan(lens, h, h_kv, cus):
    from online_softmax_tiled_amd import api
    return api.decode_plan(lens, h, h_kv, num_cus=cus)


def test_plan_reaches_first_wave_split_count_of_the_pages(lib):
    # "The grid": S* = ceil(N_SM / G_2D); at batch 1 the unsplit grid is one
    # workgroup per KV head here, and the plan must give at least S* splits.
    g = load_golden("decode_shape_arithmetic.json")
    for case, h, h_kv in zip(g["first_wave_splits"], (32, 8), (8, 1)):
        assert case["unsplit_grid"] == h_kv
        s_star = math.ceil(case["num_sm"] / case["unsplit_grid"])
        assert s_star == case["splits"]
        for s in (2560, 8192, 32768):
            chunk, splits = plan([s], h, h_kv, case["num_sm"])
            if s >= s_star * 64:
                assert math.ceil(s / chunk) >= s_star


def test_plan_properties(lib):
    rng = np.random.default_rng(0)
    for _ in range(200):
        B = int(rng.integers(1, 65))
        h_kv = int(rng.choice([1, 2, 4, 8]))
        lens = rng.integers(0, 40000, size=B)
        cus = int(rng.choice([132, 256, 304]))
        chunk, splits = plan(lens, h_kv * 4, h_kv, cus)
        assert chunk % 64 == 0 and chunk >= 64
        assert splits == max(1, math.ceil(int(lens.max()) / chunk))
        units = h_kv * sum(math.ceil(int(s) / chunk) for s in lens)
        if units < cus:       # only when the keys cannot fill the GPU
            assert chunk == 64
        assert plan(lens, h_kv * 4, h_kv, cus) == (chunk, splits)      # deterministic


def test_plan_on_the_measured_workloads(lib):
    # 70B TP8 shard, batch 1, 32768 keys on 256 CUs: one slice per CU.
    assert plan([32768], 8, 1, 256) == (128, 256)
    # 64 ragged sequences at Llama-3-8B shape: about 12 slices per CU, <=16 per sequence.
    rng = np.random.default_rng(1004)
    lens = rng.integers(512, 16384, size=64, endpoint=True)
    chunk, splits = plan(lens, 32, 8, 256)
    units = 8 * sum(math.ceil(int(s) / chunk) for s in lens)
    assert units >= 12 * 256 * 0.9 and splits <= 16


def test_plan_for_large_groups(lib):
    # more than 16 heads per KV head run on the row form, one workgroup per
    # CU: the plan aims at one workgroup of work per CU
    assert plan([32768] * 32, 128, 1, 256) == (4096, 8)
    assert plan([16384] * 64, 32, 1, 256) == (4096, 4)
    # the 16-head kernel's target (12 per CU) up to 16 heads
    chunk16, _ = plan([16384] * 64, 16, 1, 256)
    assert chunk16 < 4096
    rng = np.random.default_rng(2)
    for _ in range(100):
        B = int(rng.integers(1, 65))
        h_kv = int(rng.choice([1, 2, 4]))
        g = int(rng.choice([17, 24, 32, 64, 128]))
        lens = rng.integers(0, 40000, size=B)
        chunk, splits = plan(lens, h_kv * g, h_kv, 256)
        assert chunk % 64 == 0 and chunk >= 64
        units = h_kv * sum(math.ceil(int(s) / chunk) for s in lens)
        assert units >= 256 or chunk == 64
        assert units <= 2 * 256 or chunk == 128        # about one per CU, never far above


def test_plan_rejects_bad_input(lib):
    from online_softmax_tiled_amd import api
    with pytest.raises(api.AttnError):
        plan([-1], 8, 1, 256)
    with pytest.raises(api.AttnError):
        plan([10], 8, 1, 0)
    with pytest.raises(api.AttnError):
        plan([10], 8, 3, 256)


def test_partial_state_bytes_arithmetic():
    # "What the merge costs": S (d_h + 2) 4 bytes per token-head.
    g = load_golden("decode_shape_arithmetic.json")["partial_bytes_per_token_head"]
    assert g["splits"] * (g["head_dim"] + 2) * 4 == g["bytes"]


def test_prefill_rejects_sequences_beyond_32bit_offsets(lib):
    assert prefill_call(lib, T_q=1, T_k=(1 << 23) + 1, causal=0) == 2


def paged_prefill_call(lib, **kw):
    args = dict(q=1, cu=1, max_q=8, kp=1, vp=1, bt=1, sk=1, B=1, h=8, h_kv=2, d=128, page=16, max_pages=4,
                num_pages=4, dtype=1, scale=0.088, causal=1, o=1, lse=NULL)
    args.update(kw)
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.attn_prefill_paged(p(args["q"]), p(args["cu"]), args["max_q"], p(args["kp"]), p(args["vp"]),
                                  p(args["bt"]), p(args["sk"]), None, args["B"], args["h"], args["h_kv"], args["d"],
                                  args["page"], args["max_pages"], args["num_pages"], args["dtype"], args["scale"],
                                  args["causal"], p(args["o"]), p(args["lse"]), None)


@pytest.mark.parametrize("kw,code", [
    (dict(page=24), 2),          # not a power of two
    (dict(page=8), 2),           # below 16
    (dict(d=64), 2),
    (dict(dtype=3), 2),
    (dict(h=6, h_kv=4), 1),
    (dict(max_pages=0), 1),
    (dict(num_pages=0), 1),
    (dict(scale=-1.0), 1),
    (dict(B=-1), 1),
    (dict(bt=None), 1),
    (dict(cu=None), 1),
    (dict(max_pages=1 << 20, page=16), 2),   # more keys per sequence than supported
])
def test_paged_prefill_rejects_before_launch(lib, kw, code):
    assert paged_prefill_call(lib, **kw) == code


def test_paged_prefill_empty_is_ok_without_launch(lib):
    assert paged_prefill_call(lib, B=0, q=None, o=None) == 0
    assert paged_prefill_call(lib, max_q=0, q=None, o=None) == 0


def test_fixed_decode_plan_is_batch_independent(lib):
    # attn_decode_plan_fixed through the C ABI: the split length is the
    # caller's, a sequence's split count depends on its own length only, and
    # the grid covers the longest sequence
    import ctypes
    from online_softmax_tiled_amd import api

    def fixed(lens, split):
        arr = np.ascontiguousarray(np.asarray(lens, dtype=np.int32))
        chunk, splits = ctypes.c_int32(-5), ctypes.c_int32(-5)
        rc = lib.attn_decode_plan_fixed(int(arr.size), arr.ctypes.data_as(ctypes.c_void_p) if arr.size else None,
                                        split, ctypes.byref(chunk), ctypes.byref(splits))
        return rc, chunk.value, splits.value

    assert fixed([3000], 256) == (0, 256, 12)
    assert fixed([3000, 20000, 5], 256) == (0, 256, 79)
    assert fixed([], 2048) == (0, 2048, 1)
    assert fixed([0, 0], 2048) == (0, 2048, 1)
    assert fixed([2048], 2048) == (0, 2048, 1)
    assert fixed([2049], 2048) == (0, 2048, 2)
    rng = np.random.default_rng(5)
    for _ in range(100):
        lens = rng.integers(0, 1 << 20, size=int(rng.integers(1, 65)))
        split = 16 * int(rng.integers(1, 512))
        rc, chunk, splits = fixed(lens, split)
        assert rc == 0 and chunk == split
        assert splits == max(1, -(-int(lens.max()) // split))
        # one sequence alone gets the same slices as inside the batch: its
        # own split count does not depend on the companions
        b = int(rng.integers(0, lens.size))
        rc1, chunk1, splits1 = fixed(lens[b:b + 1], split)
        assert chunk1 == chunk and -(-int(lens[b]) // split) <= splits1 <= splits
    # invalid and unsupported inputs leave the outputs untouched
    assert fixed([10], 100)[0] == 1 and fixed([10], 100)[1:] == (-5, -5)
    assert fixed([10], 0)[0] == 1
    assert fixed([-1], 64)[0] == 1
    assert fixed([(1 << 23)], 16)[0] == 2                  # 524288 splits > 65535
    assert lib.attn_decode_plan_fixed(1, None, 64, ctypes.byref(ctypes.c_int32()), ctypes.byref(ctypes.c_int32())) == 1
    # the binding returns the library's plan and raises on its errors
    assert api.decode_plan_fixed([3000, 20000, 5], 256) == (256, 79)
    with pytest.raises(api.AttnError):
        api.decode_plan_fixed([10], 100)


def test_stream_read_rejects_before_launch(lib):
    p = ctypes.c_void_p
    assert lib.attn_stream_read(p(16), 64, 0, p(16), None) == 1          # no workgroup
    assert lib.attn_stream_read(p(16), 64, 65537, p(16), None) == 1
    assert lib.attn_stream_read(p(16), 60, 4, p(16), None) == 1          # not a multiple of 16 bytes
    assert lib.attn_stream_read(None, 64, 4, p(16), None) == 1
    assert lib.attn_stream_read(p(16), 64, 4, None, None) == 1
    assert lib.attn_stream_read(p(24), 64, 4, p(16), None) == 1          # misaligned source
    assert "attn_stream_read" in lib.attn_last_error().decode()


# ---------------------------------------------------------------- bounds-checking debug build

def test_no_bit_cast_of_a_subscripted_vector_element():
    # The device compiler lowers __builtin_bit_cast(T, v[i]) of an element of
    # an ext-vector as a load of the vector's first element, whatever i is
    # (the subscript is computed and dropped). Kernel sources copy such an
    # element to a scalar before a bit cast; this keeps the pattern out.
    csrc = os.path.join(ROOT, "online_softmax_tiled_amd", "csrc")
    pat = re.compile(r"__builtin_bit_cast\(\s*[\w:<>, ]+?,\s*[A-Za-z_][\w.]*\s*\[[^\]]*\]\s*(\[[^\]]*\]\s*)*\)")
    hits = []
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h", ".cpp")):
            for no, line in enumerate(open(os.path.join(csrc, name)), 1):
                if pat.search(line):
                    hits.append(f"{name}:{no}: {line.strip()}")
    assert not hits, "\n".join(hits)
    # the pattern matches the form it is meant to catch
    assert pat.search("m = max(m, __builtin_bit_cast(uint32_t, acc[i][e]) & 1u);")
    assert not pat.search("__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi))")


def test_checked_library_exports_every_declared_symbol(lib):
    from online_softmax_tiled_amd import api
    if not os.path.exists(api.CHECKED_LIB_PATH):
        from online_softmax_tiled_amd.build import build
        build()
    out = subprocess.run(["nm", "-D", "--defined-only", api.CHECKED_LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s(attn_\w+)$", out, re.M))
    assert set(declared_symbols()) <= exported
    with api.checked_library() as checked:
        assert "bounds checks" in api.version()
        # rejected before any device call
        hits = (ctypes.c_uint32 * 8)()
        assert checked.attn_check_report(ctypes.cast(hits, ctypes.c_void_p), 8) == 1
        assert checked.attn_check_report(None, 64) == 1
        assert checked.attn_check_selftest(None, None) == 1
    assert "bounds checks" not in api.version()   # the product library again


def test_product_library_has_no_bounds_checks(lib):
    hits = (ctypes.c_uint32 * 64)()
    assert lib.attn_check_report(ctypes.cast(hits, ctypes.c_void_p), 64) == 2
    assert "without device bounds checks" in lib.attn_last_error().decode()
    assert lib.attn_check_clear() == 2
    assert lib.attn_check_selftest(ctypes.c_void_p(16), None) == 2


@pytest.mark.parametrize("n", [2, 8])
def test_bench_refuses_more_than_one_gpu(n):
    # The bench measures one GPU; a request for more exits before any GPU
    # work (and before torch is imported) with a message naming the count.
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert r.stdout == ""
    assert f"--gpus {n}" in r.stderr and "one GPU" in r.stderr
