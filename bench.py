"""Benchmark of the tiled online-softmax attention kernels on one MI355X.

A step is one attn_prefill_fwd call over the Llama-3-8B layer prefill
workload (B=1, h=32, h_kv=8, d_h=128, T=8192, causal, bf16, synthetic N(0,1)
inputs already resident in HBM). ``value`` is its useful-FLOP throughput:
4 * d_h * h * T(T+1)/2 = 5.498e11 FLOP per step (causal: only key/query
pairs with j <= t count).

Also reported, on the same line:
* ``roofline``: the prefill kernel's achieved TFLOP/s (algorithmic FLOP per
  launch over the mean launch time measured with HIP events on the launch
  stream) against MI355X's dense bf16 MFMA peak, 2.5 PFLOP/s;
* ``decode``: split-KV decode (stage 1 + merge) on the batch-1 70B-TP8 shard
  shape (32768 contiguous keys; 40 distinct KV copies rotated so that every
  step reads from HBM, not from the 256 MB last-level cache) and on the
  64-sequence paged Llama-3-8B shape, as KV GB/s against 8 TB/s; the paged
  gather as GB/s moved;
* ``prefill_other``: the tiny and the numerics-stress prefill shapes, and
  the chunked prefill of 8 sequences against a paged cache;
* ``merge_lse``: the two-operand (O, LSE) merge on the Llama-3-8B prefill
  output shape, as GB/s against 8 TB/s;
* ``cpu_baseline``: the float64 oracle timed on the host CPU on a bounded
  sample of the same prefill workload (blocks of random query rows, about
  15 s of oracle time).

``python bench.py --gpus N --steps K --warmup W``. Only one GPU is used; N > 1
exits with a message.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill TFLOP/s (% MFMA peak); decode KV GB/s (% HBM peak) on 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E, published

# HBM bytes per prefill launch, from two rocprofv3 counter passes (FETCH_SIZE,
# WRITE_SIZE) scaled by what the same counters read for a plain device copy of
# known size. Valid only for the kernel source they were taken on.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_llama3_8b_t8192_traffic.json")
KERNEL_SOURCES = ("online_softmax_tiled_amd/csrc/prefill.hip", "online_softmax_tiled_amd/csrc/common.h")


def kernel_source_sha256():
    """SHA-256 of the prefill kernel's code: the sources with comments and
    blank space removed, so that only a code change invalidates the record."""
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per launch of the prefill kernel as recorded by the counter
    passes, or None when there is no record or the kernel source changed."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_sha256():
        return None
    return int(rec["hbm_bytes_per_launch"])
HEAD_DIM = 128


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def causal_pairs(t_q, t_k):
    off = t_k - t_q
    return sum(min(t_k, t + off + 1) for t in range(t_q)) if t_q <= 4096 else \
        t_q * (t_q + 1) // 2 + off * t_q


def visible_pairs(inp):
    """Number of visible (query, key) pairs per head, summed over the batch."""
    total = 0
    for b in range(inp["B"]):
        km = np.ones(inp["T_k"], dtype=bool) if inp["key_mask"] is None else inp["key_mask"][b] != 0
        rm = np.ones(inp["T_q"], dtype=bool) if inp["row_mask"] is None else inp["row_mask"][b] != 0
        cum = np.concatenate([[0], np.cumsum(km)])
        off = inp["T_k"] - inp["T_q"]
        t = np.arange(inp["T_q"])
        lim = np.minimum(inp["T_k"], t + off + 1) if inp["causal"] else np.full(inp["T_q"], inp["T_k"])
        total += int((cum[lim] * rm).sum())
    return total


def time_loop(fn, steps, warmup):
    """Mean ms per call of eager launches: HIP events on torch's current
    stream (the stream the library launches on), bracketed by device
    synchronisations."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall = time.perf_counter()
    t0.record()
    for i in range(steps):
        fn(i)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall
    return t0.elapsed_time(t1) / steps, wall


def time_graph(fn, steps, reps=5):
    """Mean ms per call when ``steps`` calls are captured in one HIP graph and
    the graph is replayed ``reps`` times: the device time of the kernels and
    the gaps between them, without the host's per-call launch cost."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(steps):
            fn(i)
    graph.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        graph.replay()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / (reps * steps)
    del graph
    return ms


def bench_prefill(name, steps, warmup, dev):
    import torch
    from online_softmax_tiled_amd import api
    from online_softmax_tiled_amd.workloads import make_config
    inp = make_config(name)
    q, k, v = (inp[n].to(dev) for n in "qkv")
    km = None if inp["key_mask"] is None else torch.from_numpy(inp["key_mask"]).to(dev)
    rm = None if inp["row_mask"] is None else torch.from_numpy(inp["row_mask"]).to(dev)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    flop = 4.0 * HEAD_DIM * inp["h"] * visible_pairs(inp)

    def step(i=0):
        api.prefill(q, k, v, causal=inp["causal"], scale=inp["scale"], key_mask=km, row_mask=rm,
                    out=out, lse=lse)

    ms, wall = time_loop(step, steps, warmup)
    return dict(inp=inp, flop=flop, ms=ms, wall=wall, tflops=flop / (ms * 1e-3) / 1e12)


def bench_chunked_prefill(steps, warmup, dev):
    """attn_prefill_paged on the chunked-prefill workload: 8 sequences with
    1024..8192 cached keys each, 256..1024 of them new (the query rows),
    16-token pages. Useful FLOP = 4 d h x visible (query, key) pairs."""
    import torch
    from online_softmax_tiled_amd import api
    from online_softmax_tiled_amd.workloads import make_config
    c = make_config("chunked_prefill_llama3_8b_b8")
    args = [t.to(dev) if isinstance(t, torch.Tensor) else torch.from_numpy(t).to(dev)
            for t in (c["q"], c["cu_seqlens_q"], c["k_pool"], c["v_pool"], c["block_table"], c["seq_lens_k"])]
    q, cu, kp, vp, bt, sk = args
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    tq = c["q_lens"].astype(np.int64)
    tk = c["seq_lens_k"].astype(np.int64)
    pairs = int((tq * (tk - tq) + tq * (tq + 1) // 2).sum())
    flop = 4.0 * c["d"] * c["h"] * pairs

    def step(i=0):
        api.prefill_paged(q, cu, c["max_q"], kp, vp, bt, sk, causal=True, scale=c["scale"], out=o, lse=lse,
                          seq_lens_k_host=c["seq_lens_k"])

    ms, _ = time_loop(step, steps, warmup)
    return dict(ms=ms, tflops=flop / (ms * 1e-3) / 1e12, flop=flop, new_tokens=int(tq.sum()),
                cached_keys=int(tk.sum()))


def bench_merge_lse(steps, warmup, dev, copies=3):
    """attn_merge_lse on the Llama-3-8B prefill output shape (two [1, 32, 8192,
    128] bf16 outputs with their LSEs, e.g. a cascade's prefix and suffix).
    ``copies`` input sets (3 x 268 MB) are rotated so each call reads HBM,
    not the 256 MB last-level cache. GB/s = bytes moved / call time."""
    import torch
    from online_softmax_tiled_amd import api
    g = torch.Generator(device="cpu").manual_seed(2024)
    shape, lead = (1, 32, 8192, 128), (1, 32, 8192)
    sets = []
    for _ in range(copies):
        sets.append(tuple(t.to(dev) for t in (
            torch.randn(shape, generator=g).to(torch.bfloat16), (torch.randn(lead, generator=g) * 4).float(),
            torch.randn(shape, generator=g).to(torch.bfloat16), (torch.randn(lead, generator=g) * 4).float())))
    o = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(lead, dtype=torch.float32, device=dev)
    rows = 32 * 8192
    nbytes = rows * (2 * 128 * 2 + 2 * 4 + 128 * 2 + 4)

    def step(i=0):
        oa, la, ob, lb = sets[i % copies]
        api.merge_lse(oa, la, ob, lb, out=o, lse=lse)

    ms, _ = time_loop(step, steps, warmup)
    return dict(workload="merge_lse_llama3_8b_t8192", rows=rows, bytes=nbytes, us=ms * 1e3,
                gbs=nbytes / (ms * 1e-3) / 1e9, frac_hbm=nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                rotated_input_sets=copies)


def bench_decode_large_group(steps, warmup, dev, paged=False, kv8=False, scales=(0.37, 0.29)):
    """Decode with a 128-head group on one KV head (g = 128, the heads as
    the rows of the prefill kernel): 32 sequences of 32768 keys, 537 MB of
    K+V (more than the 256 MB last-level cache), synthetic N(0,1) drawn on
    the device; contiguous, or (paged) in 16-token pages placed by a seeded
    permutation of the pool. kv8: K and V as E4M3 codes drawn on the device
    (sign, mantissa and an exponent field in 4..9 uniform; 268 MB), decoded
    with ``scales``. GB/s = K+V bytes / (split + merge time)."""
    import torch
    from online_softmax_tiled_amd import api
    B, h, h_kv, s, d = 32, 128, 1, 32768, 128
    g = torch.Generator(device=dev).manual_seed(1007)
    q = torch.randn((B, h, d), generator=g, device=dev).to(torch.bfloat16)
    if kv8:
        def codes():
            r = torch.randint(0, 96, (B, h_kv, s, d), generator=g, device=dev, dtype=torch.int32)
            return ((r // 48) * 128 + (4 + (r % 48) // 8) * 8 + r % 8).to(torch.uint8)
        k, v = codes(), codes()
    else:
        k = torch.randn((B, h_kv, s, d), generator=g, device=dev).to(torch.bfloat16)
        v = torch.randn((B, h_kv, s, d), generator=g, device=dev).to(torch.bfloat16)
    bt, page = None, 16
    if paged:
        n_pg = s // page
        perm = torch.randperm(B * n_pg, generator=torch.Generator().manual_seed(1008)).to(dev)
        k_pool = torch.empty((B * n_pg, page, h_kv, d), dtype=k.dtype, device=dev)
        v_pool = torch.empty_like(k_pool)
        k_pool[perm] = k.permute(0, 2, 1, 3).reshape(B * n_pg, page, h_kv, d)
        v_pool[perm] = v.permute(0, 2, 1, 3).reshape(B * n_pg, page, h_kv, d)
        bt = perm.view(B, n_pg).to(torch.int32).contiguous()
        k, v = k_pool, v_pool
    lens = np.full(B, s, dtype=np.int32)
    sl = torch.from_numpy(lens).to(dev)
    chunk, splits = api.decode_plan(lens, h, h_kv, device=dev)
    po = torch.empty((B, h, splits, d), dtype=torch.float32, device=dev)
    pm = torch.empty((B, h, splits), dtype=torch.float32, device=dev)
    pl = torch.empty_like(pm)
    o = torch.empty((B, h, d), dtype=q.dtype, device=dev)
    lse = torch.empty((B, h), dtype=torch.float32, device=dev)
    kv_bytes = 2 * B * h_kv * s * d * (1 if kv8 else 2)

    def full(i=0):
        if kv8:
            api.decode_split_fp8kv(q, k, v, sl, chunk, splits, scales[0], scales[1], block_table=bt, page_size=page,
                                   part_o=po, part_m=pm, part_l=pl)
        else:
            api.decode_split(q, k, v, sl, chunk, splits, block_table=bt, page_size=page, part_o=po, part_m=pm,
                             part_l=pl)
        api.merge_states(po, pm, pl, sl, chunk, q.dtype, out=o, lse=lse)

    ms, _ = time_loop(full, steps, warmup)
    return dict(kv_bytes=kv_bytes, us_per_step=ms * 1e3, gbs=kv_bytes / (ms * 1e-3) / 1e9,
                frac_hbm=kv_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, plan=[chunk, splits],
                shape="B=32 h=128 h_kv=1 s=32768 d=128 bf16" + (", E4M3 K/V" if kv8 else "")
                + (", 16-token pages" if paged else ""))


def bench_decode_contiguous(steps, warmup, dev, copies=40):
    """Batch-1 decode on the 70B-TP8 shard: attn_decode (split, then merge),
    HIP-graph timed over ``copies`` distinct K/V copies in turn (671 MB,
    beyond the 256 MB MALL, so every step reads cold data). Beside it, two
    floors on the same rotation: a plain read of the step's 16.8 MB of K/V
    (the copy's K and V, stored next to each other, with attn_stream_read) and
    one tiny kernel launch."""
    import torch
    from online_softmax_tiled_amd import api
    from online_softmax_tiled_amd.workloads import make_config
    dec = make_config("decode_70b_tp8_s32768")
    q = dec["q"].to(dev)
    sl = torch.from_numpy(dec["seq_lens"]).to(dev)
    k0, v0 = dec["k"].to(dev), dec["v"].to(dev)
    kvs = []
    for _ in range(copies):
        kv = torch.empty((2,) + tuple(k0.shape), dtype=k0.dtype, device=dev)
        kv[0].copy_(k0)
        kv[1].copy_(v0)
        kvs.append(kv)
    del k0, v0
    B, h, d = q.shape
    h_kv = kvs[0].shape[2]
    chunk, splits = api.decode_plan(dec["seq_lens"], h, h_kv, device=dev)
    po = torch.empty((B, h, splits, d), dtype=torch.float32, device=dev)
    pm = torch.empty((B, h, splits), dtype=torch.float32, device=dev)
    pl = torch.empty_like(pm)
    o = torch.empty((B, h, d), dtype=q.dtype, device=dev)
    lse = torch.empty((B, h), dtype=torch.float32, device=dev)
    kv_bytes = 2 * int(dec["seq_lens"].sum()) * h_kv * d * q.element_size()
    rd = torch.empty(1024, dtype=torch.int32, device=dev)
    tiny = torch.empty(16, dtype=torch.float32, device=dev)

    def split_only(i=0):
        kv = kvs[i % copies]
        api.decode_split(q, kv[0], kv[1], sl, chunk, splits, scale=dec["scale"], part_o=po, part_m=pm, part_l=pl)

    def full(i=0):
        kv = kvs[i % copies]
        api.decode_call(q, kv[0], kv[1], sl, chunk, splits, scale=dec["scale"], part_o=po, part_m=pm, part_l=pl,
                        out=o, lse=lse)

    def read_floor(i=0):
        api.stream_read(kvs[i % copies], chunks=1024, out=rd)

    def launch_floor(i=0):
        tiny.fill_(float(i))

    ms_eager, _ = time_loop(full, steps, warmup)
    ms_split = time_graph(split_only, copies * 5)
    ms = time_graph(full, copies * 5)
    ms_read = time_graph(read_floor, copies * 5)
    ms_launch = time_graph(launch_floor, copies * 5)
    return dict(workload="decode_70b_tp8_s32768", kv_bytes=kv_bytes, us_per_step=ms * 1e3,
                gbs=kv_bytes / (ms * 1e-3) / 1e9, frac_hbm=kv_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                split_us=ms_split * 1e3, eager_us_per_step=ms_eager * 1e3, plan=[chunk, splits],
                read_floor_us=ms_read * 1e3, read_floor_gbs=kv_bytes / (ms_read * 1e-3) / 1e9,
                read_floor_frac_hbm=kv_bytes / (ms_read * 1e-3) / 1e9 / PEAK_HBM_GBS,
                launch_floor_us=ms_launch * 1e3, rotated_kv_copies=copies,
                timing="HIP graph of attn_decode steps (split + merge), replayed; read_floor = attn_stream_read "
                       "over the same 16.8 MB of K/V (1024 contiguous chunks); launch_floor = one 64-byte fill kernel")


def bench_decode_fp8kv(steps, warmup, dev, name, copies=1, scales=(0.37, 0.29)):
    """Split-KV decode over 8-bit E4M3 K/V (attn_decode_fp8kv, split then
    merge) on a named decode workload with its K/V drawn as E4M3 codes. KV
    bytes = one byte per element. ``copies`` > 1 rotates that many K/V copies
    and times a HIP graph of the steps (batch-1 shape); else eager launches."""
    import torch
    from online_softmax_tiled_amd import api
    from online_softmax_tiled_amd.workloads import make_config
    dec = make_config(name, kv_codes=True)
    q = dec["q"].to(dev)
    sl = torch.from_numpy(dec["seq_lens"]).to(dev)
    B, h, d = q.shape
    paged = dec["paged"]
    if paged:
        kvs = [(dec["k_pool"].to(dev), dec["v_pool"].to(dev))]
        bt = torch.from_numpy(dec["block_table"]).to(dev)
        h_kv, ps = kvs[0][0].shape[2], dec["page_size"]
    else:
        k0, v0 = dec["k"].to(dev), dec["v"].to(dev)
        kvs = [(k0.clone(), v0.clone()) for _ in range(copies)]
        del k0, v0
        bt, h_kv, ps = None, dec["k"].shape[1], 16
    chunk, splits = api.decode_plan(dec["seq_lens"], h, h_kv, device=dev)
    po = torch.empty((B, h, splits, d), dtype=torch.float32, device=dev)
    pm = torch.empty((B, h, splits), dtype=torch.float32, device=dev)
    pl = torch.empty_like(pm)
    o = torch.empty((B, h, d), dtype=q.dtype, device=dev)
    lse = torch.empty((B, h), dtype=torch.float32, device=dev)
    kv_bytes = 2 * int(dec["seq_lens"].sum()) * h_kv * d

    def full(i=0):
        k, v = kvs[i % len(kvs)]
        api.decode_fp8kv_call(q, k, v, sl, chunk, splits, scales[0], scales[1], block_table=bt, page_size=ps,
                              scale=dec["scale"], part_o=po, part_m=pm, part_l=pl, out=o, lse=lse)

    if copies > 1:
        ms = time_graph(full, copies * 5)
        timing = f"HIP graph of attn_decode_fp8kv steps over {copies} rotated K/V copies"
    else:
        ms, _ = time_loop(full, steps, warmup)
        timing = "eager attn_decode_fp8kv steps"
    return dict(kv_bytes=kv_bytes, kv_format="E4M3 bytes, per-tensor fp32 scales", us_per_step=ms * 1e3,
                gbs=kv_bytes / (ms * 1e-3) / 1e9, frac_hbm=kv_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                plan=[chunk, splits], timing=timing)


def bench_decode_paged(steps, warmup, dev, dec, fixed_split=None, gather=True):
    """Paged split-KV decode on the 64-sequence workload, with the adaptive
    plan or (``fixed_split``) a batch-invariant fixed split length."""
    import torch
    from online_softmax_tiled_amd import api
    q = dec["q"].to(dev)
    sl = torch.from_numpy(dec["seq_lens"]).to(dev)
    kp, vp = dec["k_pool"].to(dev), dec["v_pool"].to(dev)
    bt = torch.from_numpy(dec["block_table"]).to(dev)
    B, h, d = q.shape
    h_kv = kp.shape[2]
    if fixed_split is None:
        chunk, splits = api.decode_plan(dec["seq_lens"], h, h_kv, device=dev)
    else:
        chunk, splits = api.decode_plan_fixed(dec["seq_lens"], fixed_split)
    po = torch.empty((B, h, splits, d), dtype=torch.float32, device=dev)
    pm = torch.empty((B, h, splits), dtype=torch.float32, device=dev)
    pl = torch.empty_like(pm)
    o = torch.empty((B, h, d), dtype=q.dtype, device=dev)
    lse = torch.empty((B, h), dtype=torch.float32, device=dev)
    kv_bytes = 2 * int(dec["seq_lens"].sum()) * h_kv * d * q.element_size()

    def split_only(i=0):
        api.decode_split(q, kp, vp, sl, chunk, splits, block_table=bt, page_size=dec["page_size"],
                         scale=dec["scale"], part_o=po, part_m=pm, part_l=pl)

    def full(i=0):
        api.decode_call(q, kp, vp, sl, chunk, splits, block_table=bt, page_size=dec["page_size"],
                        scale=dec["scale"], part_o=po, part_m=pm, part_l=pl, out=o, lse=lse)

    ms_split, _ = time_loop(split_only, steps, warmup)
    ms, _ = time_loop(full, steps, warmup)
    if not gather:
        return dict(kv_bytes=kv_bytes, us_per_step=ms * 1e3, split_us=ms_split * 1e3,
                    gbs=kv_bytes / (ms * 1e-3) / 1e9, frac_hbm=kv_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                    plan=[chunk, splits])
    ms_graph = time_graph(full, 10, reps=2)
    s_max = int(dec["seq_lens"].max())
    gout = torch.empty((B, h_kv, s_max, d), dtype=q.dtype, device=dev)

    def gather(i=0):
        api.paged_gather(kp, bt, sl, s_max, out=gout)

    ms_g, _ = time_loop(gather, max(3, steps // 4), 2)
    del gout
    gather_bytes = kv_bytes  # K pool rows read + the same bytes written (one pool)
    return dict(workload="paged_decode_llama3_8b_b64", kv_bytes=kv_bytes, us_per_step=ms * 1e3,
                split_us=ms_split * 1e3, graph_us_per_step=ms_graph * 1e3,
                gbs=kv_bytes / (ms * 1e-3) / 1e9,
                frac_hbm=kv_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, plan=[chunk, splits],
                gather_us=ms_g * 1e3, gather_gbs=gather_bytes / (ms_g * 1e-3) / 1e9)


def cpu_baseline(inp, budget_s=15.0):
    """The float64 oracle on the host CPU over a bounded sample of the prefill
    workload: blocks of 256 random query rows, one query head at a time, until
    about budget_s seconds of oracle time have been spent."""
    import threadpoolctl
    from oracle import attention_ref
    threads = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] or [1])
    t_q, g = inp["T_q"], inp["h"] // inp["h_kv"]
    rng = np.random.default_rng(0)
    heads = rows_total = 0
    flop = spent = 0.0
    while spent < budget_s and rows_total < 64 * t_q:
        i = heads % inp["h"]
        rows = np.sort(rng.choice(t_q, size=min(256, t_q), replace=False))
        t = time.perf_counter()
        attention_ref(inp["q"][:, i:i + 1], inp["k"][:, i // g:i // g + 1], inp["v"][:, i // g:i // g + 1],
                      inp["scale"], inp["causal"], rows=rows)
        spent += time.perf_counter() - t
        flop += 4.0 * HEAD_DIM * float(np.minimum(rows + 1, inp["T_k"]).sum())
        rows_total += rows.size
        heads += 1
    return dict(value=flop / spent / 1e12, unit="TFLOP/s", cores=int(threads), kind="oracle",
                sample=f"{rows_total} random query rows ({heads} blocks of 256, cycling over the heads) of the T=8192 causal "
                       f"prefill, float64 numpy materialised attention, {spent:.1f} s of oracle time",
                affinity_cores=len(os.sched_getaffinity(0)), cpu_model=cpu_model(), blas=blas_config(),
                threads_note="cores = BLAS threads of the matmuls; the exponentials (np.exp) run on one thread")


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None if unreadable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def blas_config():
    """numpy's BLAS as threadpoolctl reports it, and the thread variables."""
    import threadpoolctl
    libs = [{k: p.get(k) for k in ("internal_api", "version", "threading_layer", "num_threads", "architecture")}
            for p in threadpoolctl.threadpool_info() if p.get("user_api") == "blas"]
    env = {k: os.environ[k] for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")
           if k in os.environ}
    return {"libraries": libs, "env": env}


def run_only(args, dev):
    """One workload, for profiler counter runs: the prefill layer, a decode
    workload, or a plain device copy of a known size (the calibration point
    for the HBM byte counters)."""
    import torch
    if args.only == "prefill":
        r = bench_prefill("llama3_8b_prefill_t8192", args.steps, args.warmup, dev)
        print(json.dumps({"workload": "llama3_8b_prefill_t8192", "ms": r["ms"], "tflops": r["tflops"]}))
    elif args.only == "stress":
        r = bench_prefill("stress_prefill_t4096", args.steps, args.warmup, dev)
        print(json.dumps({"workload": "stress_prefill_t4096", "ms": r["ms"], "tflops": r["tflops"]}))
    elif args.only == "chunked":
        r = bench_chunked_prefill(args.steps, args.warmup, dev)
        print(json.dumps({"workload": "chunked_prefill_llama3_8b_b8", "ms": r["ms"], "tflops": r["tflops"]}))
    elif args.only == "decode_fp8":
        r = bench_decode_fp8kv(args.steps, args.warmup, dev, "paged_decode_llama3_8b_b64")
        print(json.dumps(r))
    elif args.only == "decode_fp8_70b":
        r = bench_decode_fp8kv(args.steps, args.warmup, dev, "decode_70b_tp8_s32768", copies=40)
        print(json.dumps(r))
    elif args.only == "decode_70b":
        r = bench_decode_contiguous(args.steps, args.warmup, dev)
        print(json.dumps(r))
    elif args.only == "merge_lse":
        print(json.dumps(bench_merge_lse(args.steps, args.warmup, dev)))
    elif args.only == "decode_g128":
        print(json.dumps(bench_decode_large_group(args.steps, args.warmup, dev)))
    elif args.only == "decode_g128_fp8":
        print(json.dumps(bench_decode_large_group(args.steps, args.warmup, dev, kv8=True)))
    elif args.only == "decode_paged":
        from online_softmax_tiled_amd.workloads import make_config
        r = bench_decode_paged(args.steps, args.warmup, dev, make_config("paged_decode_llama3_8b_b64"))
        print(json.dumps(r))
    else:
        n = args.copy_mb * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        ms, _ = time_loop(lambda i=0: dst.copy_(src), args.steps, args.warmup)
        print(json.dumps({"workload": "device copy", "bytes_read": n, "bytes_written": n, "ms": ms}))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="only the headline prefill")
    ap.add_argument("--only", choices=["prefill", "stress", "chunked", "decode_70b", "decode_paged", "decode_g128",
                                       "decode_fp8", "decode_fp8_70b", "decode_g128_fp8", "merge_lse", "copy"],
                    default=None,
                    help="run one workload only (for profiler counter runs) and print its timing")
    ap.add_argument("--copy-mb", type=int, default=1024,
                    help="bytes moved by the plain device copy of --only copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested); "
              "the attention kernels here run on a single MI355X.", file=sys.stderr)
        sys.exit(2)

    import torch
    from online_softmax_tiled_amd import api
    dev = torch.device("cuda:0")
    log(f"device: {torch.cuda.get_device_name(dev)}, {api.version()}")
    if args.only is not None:
        run_only(args, dev)
        return

    res = bench_prefill("llama3_8b_prefill_t8192", args.steps, args.warmup, dev)
    log(f"prefill T=8192: {res['ms']:.3f} ms/step, {res['tflops']:.1f} TFLOP/s")
    tflops = res["tflops"]
    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama3_8b_prefill_t8192", "B": 1, "h": 32, "h_kv": 8, "T": 8192,
                   "d_h": 128, "causal": True, "flop_per_step": res["flop"]},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic()},
    }
    inp = res.pop("inp")
    if not args.no_extras:
        other = {}
        for name in ("tiny_prefill", "stress_prefill_t4096"):
            r = bench_prefill(name, max(10, args.steps), 3, dev)
            other[name] = {"ms": round(r["ms"], 4), "tflops": round(r["tflops"], 2),
                           "frac_mfma": round(r["tflops"] / PEAK_BF16_TFLOPS, 4)}
            log(f"prefill {name}: {r['ms']:.4f} ms, {r['tflops']:.1f} TFLOP/s")
        rc = bench_chunked_prefill(max(10, args.steps), 3, dev)
        other["chunked_prefill_llama3_8b_b8"] = {"ms": round(rc["ms"], 4), "tflops": round(rc["tflops"], 2),
                                                  "frac_mfma": round(rc["tflops"] / PEAK_BF16_TFLOPS, 4),
                                                  "new_tokens": rc["new_tokens"], "cached_keys": rc["cached_keys"]}
        log(f"chunked prefill b8 (paged): {rc['ms']:.4f} ms, {rc['tflops']:.1f} TFLOP/s")
        line["prefill_other"] = other
        decode = {}
        r3 = bench_decode_contiguous(max(200, args.steps), 20, dev)
        log(f"decode 70b-tp8: {r3['us_per_step']:.2f} us/step ({r3['split_us']:.2f} split), {r3['gbs']:.0f} GB/s; "
            f"read floor {r3['read_floor_us']:.2f} us ({r3['read_floor_gbs']:.0f} GB/s), "
            f"launch floor {r3['launch_floor_us']:.2f} us")
        decode[r3.pop("workload")] = r3
        from online_softmax_tiled_amd.workloads import make_config
        log("generating the paged decode workload ...")
        dec = make_config("paged_decode_llama3_8b_b64")
        r4 = bench_decode_paged(max(20, args.steps), 3, dev, dec)
        log(f"decode paged b64: {r4['us_per_step']:.1f} us/step ({r4['split_us']:.1f} split), {r4['gbs']:.0f} GB/s; "
            f"gather {r4['gather_gbs']:.0f} GB/s")
        decode[r4.pop("workload")] = r4
        r5 = bench_decode_paged(max(20, args.steps), 3, dev, dec, fixed_split=2048, gather=False)
        log(f"decode paged b64, batch-invariant split 2048: {r5['us_per_step']:.1f} us/step, {r5['gbs']:.0f} GB/s")
        decode["paged_decode_llama3_8b_b64_fixed_split_2048"] = r5
        r6 = bench_decode_large_group(max(20, args.steps), 3, dev)
        log(f"decode g=128 b32 s32768: {r6['us_per_step']:.1f} us/step, {r6['gbs']:.0f} GB/s, plan {r6['plan']}")
        decode["decode_g128_b32_s32768"] = r6
        r7 = bench_decode_large_group(max(20, args.steps), 3, dev, paged=True)
        log(f"decode g=128 b32 s32768 paged: {r7['us_per_step']:.1f} us/step, {r7['gbs']:.0f} GB/s, plan {r7['plan']}")
        decode["decode_g128_b32_s32768_paged"] = r7
        r8 = bench_decode_fp8kv(max(200, args.steps), 20, dev, "decode_70b_tp8_s32768", copies=40)
        log(f"decode 70b tp8 fp8 KV: {r8['us_per_step']:.2f} us/step, {r8['gbs']:.0f} GB/s")
        decode["decode_70b_tp8_s32768_fp8kv"] = r8
        r9 = bench_decode_fp8kv(max(20, args.steps), 3, dev, "paged_decode_llama3_8b_b64")
        log(f"decode paged b64 fp8 KV: {r9['us_per_step']:.1f} us/step, {r9['gbs']:.0f} GB/s")
        decode["paged_decode_llama3_8b_b64_fp8kv"] = r9
        r10 = bench_decode_large_group(max(20, args.steps), 3, dev, kv8=True)
        log(f"decode g=128 b32 s32768 fp8 KV: {r10['us_per_step']:.1f} us/step, {r10['gbs']:.0f} GB/s")
        decode["decode_g128_b32_s32768_fp8kv"] = r10
        r11 = bench_decode_large_group(max(20, args.steps), 3, dev, paged=True, kv8=True)
        log(f"decode g=128 b32 s32768 paged fp8 KV: {r11['us_per_step']:.1f} us/step, {r11['gbs']:.0f} GB/s")
        decode["decode_g128_b32_s32768_paged_fp8kv"] = r11
        for v in decode.values():
            for key in list(v):
                if isinstance(v[key], float):
                    v[key] = round(v[key], 4)
        line["decode"] = decode
        rm = bench_merge_lse(max(30, args.steps), 5, dev)
        log(f"merge_lse llama3-8b t8192: {rm['us']:.1f} us, {rm['gbs']:.0f} GB/s")
        line["merge_lse"] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in rm.items()
                             if k != "workload"}
    if not args.no_cpu_baseline:
        log("timing the float64 oracle on the host CPU ...")
        line["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
