"""GPU parity: every kernel, called through the C ABI, against the float64
oracle on the same seeded inputs.

Tolerances (max abs error on outputs; LSE relative error |d| / max(1, |LSE|)):
fp16 outputs 2e-3, bf16 outputs 1e-2, LSE 1e-4; the paged gather and the
outputs of rows with no visible key (+0.0 bits, LSE -inf) are bit-exact.

The output gate is flat: every element must lie within the tolerance of the
exact result. The one exception is an element whose exact value the output
format cannot hold that closely: half the format's spacing at the exact
value exceeds the tolerance and the exact value is not itself a format
value (bf16 from |O| >= 4, fp16 from |O| >= 8). Such an element must be
within the tolerance plus half that spacing, i.e. a rounding of a value
within the tolerance. The excepted set depends on the exact values only, not
on the GPU's; each check asserts a bound on its size and records its counts
in the session summary.
"""

import math

import numpy as np
import pytest
import torch

from oracle import (attention_ref, decode_ref, finalize_ref, merge_partials_ref, paged_gather_ref,
                    split_states_ref)
from online_softmax_tiled_amd import api
from online_softmax_tiled_amd.workloads import make_config, make_decode, make_prefill

pytestmark = pytest.mark.gpu

TOL = {"f16": 2e-3, "bf16": 1e-2}
MANT_BITS = {"f16": 10, "bf16": 7}
LSE_TOL = 1e-4
DEV = torch.device("cuda:0")


def to_dev(x):
    if x is None:
        return None
    if isinstance(x, np.ndarray):
        x = torch.from_numpy(np.ascontiguousarray(x))
    return x.to(DEV).contiguous()


def lse_rel(a, b):
    return np.abs(a - b) / np.maximum(1.0, np.abs(b))


TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16}
GATE_RECORDS = []   # (what, elements, excepted, beyond the flat gate, max abs err)


def format_exception(exact, dtype):
    """Elements whose exact value the output format cannot hold within the
    tolerance: half its spacing there exceeds TOL and the exact value is not
    a format value. Returns (mask, half spacing at the exact value)."""
    mag = np.abs(exact)
    half = np.where(mag > 0, np.exp2(np.floor(np.log2(np.where(mag > 0, mag, 1.0))) - MANT_BITS[dtype] - 1), 0.0)
    rne = torch.from_numpy(np.ascontiguousarray(exact)).to(TORCH_DT[dtype]).double().numpy()
    return (half > TOL[dtype]) & (rne != exact), half


def assert_outputs(o_gpu_t, lse_gpu, o_ref, lse_ref, dtype, what, max_excepted_frac=2e-5):
    """o_gpu_t: torch output (any leading shape, last dim d); refs float64.
    Flat gate everywhere except the format's exception set (module
    docstring), whose size must stay within max(2, max_excepted_frac * n)."""
    o_gpu = o_gpu_t.float().cpu().numpy().astype(np.float64)
    empty = np.isneginf(lse_ref)
    diff = np.abs(o_gpu - o_ref)
    err = float(np.max(diff)) if o_ref.size else 0.0
    exc, half = format_exception(o_ref, dtype)
    bad = np.where(exc, diff > TOL[dtype] + half, diff > TOL[dtype])
    if bad.any():
        idx = np.argwhere(bad)[:6]
        detail = "; ".join(f"at {tuple(int(x) for x in i)}: exact {o_ref[tuple(i)]:.6f} "
                           f"got {o_gpu[tuple(i)]:.6f}" for i in idx)
        raise AssertionError(f"{what}: max abs err {err:.3e}; {int(bad.sum())} elements beyond the gate "
                             f"(flat {TOL[dtype]}, or {TOL[dtype]} + half the format spacing where the format "
                             f"cannot hold the exact value): {detail}")
    n_exc = int(exc.sum())
    n_beyond = int((diff > TOL[dtype]).sum())
    GATE_RECORDS.append((what, int(diff.size), n_exc, n_beyond, err))
    limit = max(2, int(max_excepted_frac * diff.size))
    assert n_exc <= limit, f"{what}: {n_exc} of {diff.size} elements in the format's exception set (limit {limit})"
    if lse_gpu is not None:
        assert np.array_equal(np.isneginf(lse_gpu), empty), f"{what}: empty-row LSE mismatch"
        fin = ~empty
        if fin.any():
            rel = float(lse_rel(lse_gpu[fin], lse_ref[fin]).max())
            assert rel <= LSE_TOL, f"{what}: LSE rel err {rel:.3e}"
    if empty.any():
        bits = o_gpu_t.view(torch.int16).cpu().numpy()
        assert np.all(bits[empty] == 0), f"{what}: empty rows are not +0.0 bits"
    return err


# ------------------------------------------------------------------ prefill

def run_prefill(inp, rows=None):
    o, lse = api.prefill(to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"]), causal=inp["causal"],
                         scale=inp["scale"], key_mask=to_dev(inp["key_mask"]),
                         row_mask=to_dev(inp["row_mask"]))
    torch.cuda.synchronize()
    o_ref, lse_ref = attention_ref(inp["q"], inp["k"], inp["v"], inp["scale"], inp["causal"],
                                   inp["key_mask"], inp["row_mask"], rows=rows)
    lse_g = lse.cpu().numpy().astype(np.float64)
    if rows is not None:
        o = o[:, :, torch.from_numpy(np.asarray(rows)).to(DEV)]
        lse_g = lse_g[:, :, rows]
    return o, lse_g, o_ref, lse_ref


def test_prefill_tiny_config():
    inp = make_config("tiny_prefill")
    o, lse, o_ref, lse_ref = run_prefill(inp)
    assert_outputs(o, lse, o_ref, lse_ref, "f16", "tiny prefill")


@pytest.mark.parametrize("B,h,h_kv,T_q,T_k,dtype,causal", [
    (1, 4, 1, 1, 1, "bf16", True),
    (1, 4, 1, 33, 33, "bf16", True),
    (2, 8, 2, 100, 100, "f16", True),
    (1, 8, 8, 70, 70, "bf16", True),       # g = 1
    (1, 8, 4, 64, 200, "bf16", True),      # g = 2, T_q < T_k (bottom-right)
    (1, 16, 2, 96, 96, "bf16", False),     # g = 8, no mask
    (2, 4, 1, 130, 257, "f16", False),
    (1, 32, 8, 300, 300, "bf16", True),
])
def test_prefill_shapes(B, h, h_kv, T_q, T_k, dtype, causal):
    inp = make_prefill(B, h, h_kv, T_q, T_k, 128, dtype, seed=T_q * 7 + T_k + h, causal=causal)
    o, lse, o_ref, lse_ref = run_prefill(inp)
    assert_outputs(o, lse, o_ref, lse_ref, dtype, f"prefill {B}x{h}/{h_kv} {T_q}x{T_k}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_prefill_masks_and_empty_rows(dtype):
    # per-key mask, tile masks, masked rows, and rows left empty by masked
    # early tiles under the causal mask
    inp = make_prefill(2, 8, 2, 200, 200, 128, dtype, seed=5, causal=True, key_tile=64,
                       key_tile_p=0.3, key_p=0.2, row_mask_count=7)
    inp["key_mask"][0, :70] = 0          # rows 0..69 of batch 0 see nothing
    inp["key_mask"][1, 128:192] = 0
    o, lse, o_ref, lse_ref = run_prefill(inp)
    assert np.isneginf(lse_ref[0, :, :70]).all()
    assert_outputs(o, lse, o_ref, lse_ref, dtype, "masked prefill")


@pytest.mark.parametrize("dtype,causal", [("f16", False), ("bf16", True)])
def test_prefill_skips_fully_masked_tiles(dtype, causal):
    # tiles with no visible key are skipped: only the last, partial tile
    # visible (batch 0); only one middle tile (batch 1); the first tiles
    # masked, so early causal rows see nothing (batch 2); a run of masked
    # tiles between visible ones (batch 3); T_k = 300 is not a tile multiple
    inp = make_prefill(4, 8, 2, 300, 300, 128, dtype, seed=17 + causal, causal=causal)
    km = np.ones((4, 300), dtype=np.uint8)
    km[0, :256] = 0
    km[1, :128] = 0
    km[1, 192:] = 0
    km[2, :130] = 0
    km[3, 64:256] = 0
    km[3, 10] = 0                      # and one partial tile
    inp["key_mask"] = km
    o, lse, o_ref, lse_ref = run_prefill(inp)
    if causal:
        assert np.isneginf(lse_ref[2, :, :130]).all()
    assert_outputs(o, lse, o_ref, lse_ref, dtype, f"prefill with masked tiles causal={causal}")


def test_prefill_key_mask_longer_than_tile_list():
    # 4097 tiles of keys: more than the list of visible tiles holds, so the
    # kernel walks every tile (masked ones included); checked on sampled rows
    T_k = 4097 * 64
    inp = make_prefill(1, 4, 1, 64, T_k, 128, "bf16", seed=19, causal=False, key_tile_p=0.25)
    rows = np.array([0, 1, 17, 31, 32, 63])
    o, lse, o_ref, lse_ref = run_prefill(inp, rows=rows)
    assert_outputs(o, lse, o_ref, lse_ref, "bf16", "prefill key mask over 4097 tiles (sampled rows)")


def test_prefill_all_keys_masked():
    inp = make_prefill(1, 4, 1, 40, 40, 128, "bf16", seed=6, causal=False)
    inp["key_mask"] = np.zeros((1, 40), dtype=np.uint8)
    o, lse, o_ref, lse_ref = run_prefill(inp)
    assert np.isneginf(lse).all()
    assert_outputs(o, lse, o_ref, lse_ref, "bf16", "all keys masked")


def test_prefill_stress_config_reduced():
    inp = make_config("stress_prefill_t4096", T_q=1024, T_k=1024)
    o, lse, o_ref, lse_ref = run_prefill(inp)
    assert_outputs(o, lse, o_ref, lse_ref, "bf16", "stress prefill T=1024", max_excepted_frac=1e-4)


def test_prefill_stress_config_full():
    inp = make_config("stress_prefill_t4096")
    o, lse, o_ref, lse_ref = run_prefill(inp)
    assert np.isneginf(lse_ref).any()
    assert_outputs(o, lse, o_ref, lse_ref, "bf16", "stress prefill T=4096", max_excepted_frac=1e-4)


def test_prefill_llama3_8b_t8192_every_row_block():
    # the full-size launch the bench times: two random rows from every
    # 32-row block (one in each half), the same for every head, so every
    # (head, row block) pair -- i.e. every wave of every workgroup -- is
    # compared with the oracle, plus the edge rows
    inp = make_config("llama3_8b_prefill_t8192")
    rng = np.random.default_rng(2)
    blocks = np.arange(0, 8192, 32)
    rows = np.unique(np.concatenate([blocks + rng.integers(0, 16, blocks.size),
                                     blocks + 16 + rng.integers(0, 16, blocks.size),
                                     [0, 1, 31, 32, 63, 64, 4095, 8190, 8191]]))
    o, lse, o_ref, lse_ref = run_prefill(inp, rows=rows)
    assert_outputs(o, lse, o_ref, lse_ref, "bf16", f"llama3-8b prefill T=8192 ({rows.size} rows per head)")


def test_prefill_causal_single_key_row_is_exact():
    # row 0 under a causal mask sees only key 0: its output is v_0 exactly
    inp = make_prefill(1, 8, 2, 64, 64, 128, "bf16", seed=8, causal=True)
    o, lse = api.prefill(to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"]), causal=True,
                         scale=inp["scale"])
    torch.cuda.synchronize()
    for i in range(8):
        assert torch.equal(o[0, i, 0].cpu(), inp["v"][0, i // 4, 0])


@pytest.mark.parametrize("upper", [False, True])
def test_prefill_row_max_on_either_half_wave(upper):
    # In the kernel's transposed score layout a row's scores are split
    # between two lanes of a wave: keys 0-3 of every aligned group of 8 on
    # one, keys 4-7 on the other. Here each row has two dominant keys (18
    # log2 units above the rest) at offsets of one kind only, so the row
    # maximum and the final sums must cross between the lanes: a half that
    # kept its own maximum would hold its sums at another reference.
    T, h, h_kv, d = 256, 4, 1, 128
    inp = make_prefill(1, h, h_kv, T, T, d, "bf16", seed=77 + upper, causal=False, qk_std=0.05)
    q, k = inp["q"].clone(), inp["k"].clone()
    for p in range(T):
        k[0, 0, p, p % d] = 12.0                 # key p points along e_(p mod 128)
    off = 4 if upper else 0
    for j in range(h):
        for i in range(T):
            p = 8 * ((i + 5 * j) % 16) + off + (i % 4)   # p % 8 in the chosen half; p + 128 shares e_p
            q[0, j, i, p] = 12.0
    inp = dict(inp, q=q, k=k)
    o, lse, o_ref, lse_ref = run_prefill(inp)
    assert_outputs(o, lse, o_ref, lse_ref, "bf16", f"dominant keys on the {'upper' if upper else 'lower'} lanes")


# ------------------------------------------------------------------ gather

@pytest.mark.parametrize("page_size,spare", [(16, 0), (16, 5), (32, 3), (48, 1)])
def test_paged_gather_bit_exact(page_size, spare):
    dec = make_decode(B=6, h=8, h_kv=2, d=128, dtype="bf16", seed=page_size + spare,
                      len_range=(1, 300), paged=True, page_size=page_size, spare_pages=spare)
    dec["seq_lens"][2] = 0
    s_max = int(dec["seq_lens"].max()) + 5
    sentinel = torch.full((6, 2, s_max, 128), -7.0, dtype=torch.bfloat16)
    out = api.paged_gather(to_dev(dec["k_pool"]), to_dev(dec["block_table"]), to_dev(dec["seq_lens"]),
                           s_max, out=to_dev(sentinel.clone()))
    torch.cuda.synchronize()
    ref = paged_gather_ref(dec["k_pool"], dec["block_table"], dec["seq_lens"], s_max, out=sentinel.clone())
    assert torch.equal(out.cpu().view(torch.int16), ref.view(torch.int16))
    for b in range(6):
        s = int(dec["seq_lens"][b])
        assert torch.equal(out[b, :, :s].cpu(), dec["k_seqs"][b][:, :s])


@pytest.fixture(scope="module")
def paged_llama():
    return make_config("paged_decode_llama3_8b_b64")


def test_paged_gather_llama3_8b_b64_full(paged_llama):
    dec = paged_llama
    s_max = int(dec["seq_lens"].max())
    bt, sl = to_dev(dec["block_table"]), to_dev(dec["seq_lens"])
    for pool, seqs in ((dec["k_pool"], dec["k_seqs"]), (dec["v_pool"], dec["v_seqs"])):
        out = api.paged_gather(to_dev(pool), bt, sl, s_max)
        torch.cuda.synchronize()
        out = out.cpu()
        for b in range(dec["B"]):
            s = int(dec["seq_lens"][b])
            assert torch.equal(out[b, :, :s].view(torch.int16), seqs[b].reshape(8, s, 128).view(torch.int16))
        del out


# ------------------------------------------------------------------ merge

def test_merge_on_oracle_partials():
    rng = np.random.default_rng(9)
    B, h, h_kv, S, chunk = 5, 8, 2, 6, 64
    lens = np.array([0, 1, 64, 200, 384], dtype=np.int32)
    q = rng.normal(size=(B, h, 128))
    po = np.full((B, h, S, 128), np.nan, dtype=np.float32)     # unused slots poisoned
    pm = np.full((B, h, S), np.nan, dtype=np.float32)
    pl = np.full((B, h, S), np.nan, dtype=np.float32)
    o_ref = np.zeros((B, h, 128))
    lse_ref = np.full((B, h), -np.inf)
    for b in range(B):
        s = int(lens[b])
        k = rng.normal(size=(h_kv, s, 128)) * 2
        v = rng.normal(size=(h_kv, s, 128))
        m, l, a = split_states_ref(q[b], k, v, s, 0.25, chunk)
        n = m.shape[1]
        if b == 3:                       # make one split empty
            m[:, 1], l[:, 1], a[:, 1] = -np.inf, 0.0, 0.0
        po[b, :, :n], pm[b, :, :n], pl[b, :, :n] = a, m, l
        for i in range(h):
            o_ref[b, i], lse_ref[b, i] = merge_partials_ref(pm[b, i, :n], pl[b, i, :n], po[b, i, :n])
    o, lse = api.merge_states(to_dev(po), to_dev(pm), to_dev(pl), to_dev(lens), chunk, torch.bfloat16)
    torch.cuda.synchronize()
    assert_outputs(o, lse.cpu().numpy().astype(np.float64), o_ref, lse_ref, "bf16", "merge")
    of, lf = api.merge_states(to_dev(po), to_dev(pm), to_dev(pl), to_dev(lens), chunk, torch.float16)
    torch.cuda.synchronize()
    assert_outputs(of, lf.cpu().numpy().astype(np.float64), o_ref, lse_ref, "f16", "merge f16")


@pytest.mark.parametrize("S", [256, 300, 700])
def test_merge_many_splits(S):
    # Many splits and few rows take the four-slice layout; up to 256 splits its
    # preloaded rows hold every split (the maximum is taken from them), beyond
    # that the maximum is read in a loop. Sequence 1 has fewer valid splits
    # than max_splits: its rows past the valid count hold NaN and must not count.
    rng = np.random.default_rng(10 + S)
    B, h, chunk = 2, 8, 128
    m = rng.normal(0, 20, size=(B, h, S)).astype(np.float32)
    l = (rng.random((B, h, S)) * 30 + 1).astype(np.float32)
    a = (rng.normal(size=(B, h, S, 128)) * l[..., None]).astype(np.float32)
    n_valid = [S, S - 37]
    lens = np.array([n * chunk - 5 for n in n_valid], dtype=np.int32)
    m[1, :, n_valid[1]:] = np.nan
    l[1, :, n_valid[1]:] = np.nan
    a[1, :, n_valid[1]:] = np.nan
    o, lse = api.merge_states(to_dev(a), to_dev(m), to_dev(l), to_dev(lens), chunk, torch.float16)
    torch.cuda.synchronize()
    o_ref = np.zeros((B, h, 128))
    lse_ref = np.zeros((B, h))
    for b in range(B):
        n = n_valid[b]
        for i in range(h):
            o_ref[b, i], lse_ref[b, i] = merge_partials_ref(m[b, i, :n], l[b, i, :n], a[b, i, :n])
    assert_outputs(o, lse.cpu().numpy().astype(np.float64), o_ref, lse_ref, "f16", f"merge {S} splits")


@pytest.mark.parametrize("n_max", [5, 8, 13, 16])
def test_merge_bits_do_not_depend_on_max_splits(n_max):
    # A row's merged bits depend only on its own split count: the same
    # partials merged with max_splits = n_max and with the buffers padded to
    # 40 splits (NaN rows beyond each row's valid count) agree bit for bit,
    # including a column whose every term is -0.0.
    rng = np.random.default_rng(40 + n_max)
    B, h, chunk = 3, 4, 64
    n_valid = [n_max, max(1, n_max - 2), 1]
    lens = np.array([n * chunk - 3 for n in n_valid], dtype=np.int32)
    m = rng.normal(0, 5, size=(B, h, n_max)).astype(np.float32)
    l = (rng.random((B, h, n_max)) * 30 + 1).astype(np.float32)
    a = (rng.normal(size=(B, h, n_max, 128)) * l[..., None]).astype(np.float32)
    a[0, 0, :, 7] = -0.0                       # a column whose every term is -0
    outs = []
    for S in (n_max, 40):
        pm = np.full((B, h, S), np.nan, dtype=np.float32)
        pl = np.full((B, h, S), np.nan, dtype=np.float32)
        po = np.full((B, h, S, 128), np.nan, dtype=np.float32)
        for b in range(B):
            k = n_valid[b]
            pm[b, :, :k], pl[b, :, :k], po[b, :, :k] = m[b, :, :k], l[b, :, :k], a[b, :, :k]
        o, lse = api.merge_states(to_dev(po), to_dev(pm), to_dev(pl), to_dev(lens), chunk, torch.bfloat16)
        torch.cuda.synchronize()
        outs.append((o.view(torch.int16).cpu().numpy(), lse.view(torch.int32).cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    o_ref = np.zeros((B, h, 128))
    lse_ref = np.zeros((B, h))
    for b in range(B):
        for i in range(h):
            k = n_valid[b]
            o_ref[b, i], lse_ref[b, i] = merge_partials_ref(m[b, i, :k], l[b, i, :k], a[b, i, :k])
    o_dev = torch.from_numpy(outs[0][0]).view(torch.bfloat16)
    assert_outputs(o_dev, outs[0][1].view(np.float32).astype(np.float64), o_ref, lse_ref, "bf16",
                   f"merge of at most {n_max} splits")


# ------------------------------------------------------------------ decode

def run_decode(dec, plan=None, one_call=True):
    paged = dec["paged"]
    q = to_dev(dec["q"])
    sl = to_dev(dec["seq_lens"])
    if paged:
        k, v, bt = to_dev(dec["k_pool"]), to_dev(dec["v_pool"]), to_dev(dec["block_table"])
        ps = dec["page_size"]
    else:
        k, v, bt, ps = to_dev(dec["k"]), to_dev(dec["v"]), None, 16
    o, lse, plan = api.decode(q, k, v, sl, seq_lens_host=dec["seq_lens"], block_table=bt, page_size=ps,
                              scale=dec["scale"], plan=plan, one_call=one_call)
    torch.cuda.synchronize()
    return o, lse.cpu().numpy().astype(np.float64), plan


@pytest.mark.parametrize("one_call", [True, False])
@pytest.mark.parametrize("paged,page_size", [(False, 16), (True, 16), (True, 32)])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_decode_small(paged, page_size, dtype, one_call):
    # one_call: attn_decode; else attn_decode_split + attn_merge_states
    lens = [1, 5, 16, 17, 63, 64, 65, 300, 1000, 0]
    dec = make_decode(B=len(lens), h=16, h_kv=4, d=128, dtype=dtype, seed=11 + page_size, seq_lens=lens,
                      paged=paged, page_size=page_size, spare_pages=3)
    o_ref, lse_ref = decode_ref(dec["q"], dec["k_seqs"], dec["v_seqs"], dec["seq_lens"], dec["scale"])
    # includes the last split taking the rest
    for plan in (None, (64, 16), (1024, 1), (64, 2), (16, 63)):
        o, lse, used = run_decode(dec, plan, one_call)
        assert_outputs(o, lse, o_ref, lse_ref, dtype, f"decode paged={paged} plan={used} one_call={one_call}")


@pytest.mark.parametrize("h", [8, 64])
def test_decode_no_keys_at_all(h):
    # every sequence empty and s_max = 0: K/V are empty (NULL) tensors, the
    # output is zeros and the LSE -inf (16-head blocks and the row form)
    B, h_kv = 3, 1
    q = torch.randn((B, h, 128), device=DEV).to(torch.bfloat16)
    kv = torch.empty((B, h_kv, 0, 128), dtype=torch.bfloat16, device=DEV)
    sl = torch.zeros(B, dtype=torch.int32, device=DEV)
    o, lse, plan = api.decode(q, kv, kv, sl, seq_lens_host=np.zeros(B, dtype=np.int32), scale=0.088)
    torch.cuda.synchronize()
    assert torch.count_nonzero(o.float()) == 0
    assert bool(torch.all(torch.isneginf(lse)))


def test_decode_split_partials_match_slices():
    dec = make_decode(B=2, h=8, h_kv=1, d=128, dtype="bf16", seed=12, seq_lens=[700, 129], paged=False)
    chunk, S = 128, 6
    po, pm, pl = api.decode_split(to_dev(dec["q"]), to_dev(dec["k"]), to_dev(dec["v"]), to_dev(dec["seq_lens"]),
                                  chunk, S, scale=dec["scale"])
    torch.cuda.synchronize()
    po, pm, pl = po.cpu().numpy(), pm.cpu().numpy(), pl.cpu().numpy()
    for b in range(2):
        s = int(dec["seq_lens"][b])
        qb = dec["q"][b].double().numpy()
        kb = dec["k_seqs"][b].double().numpy()
        vb = dec["v_seqs"][b].double().numpy()
        m, l, a = split_states_ref(qb, kb, vb, s, dec["scale"], chunk)
        n = min(S, math.ceil(s / chunk))
        for i in range(8):
            for sp in range(n):
                o_g, lse_g = finalize_ref((float(pm[b, i, sp]), float(pl[b, i, sp]), po[b, i, sp].astype(np.float64)))
                o_r, lse_r = finalize_ref((m[i, sp], l[i, sp], a[i, sp]))
                assert np.max(np.abs(o_g - o_r)) < 1e-2
                assert abs(lse_g - lse_r) / max(1.0, abs(lse_r)) < LSE_TOL
                # the stored reference lags the slice's largest logit by at most 8 ln 2
                slack = 1e-4 * max(1.0, abs(m[i, sp]))
                assert m[i, sp] - 8 * math.log(2) - slack <= float(pm[b, i, sp]) <= m[i, sp] + slack


@pytest.mark.parametrize("plan", [(1024, 3), (4096, 1)])
@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_decode_reference_moves_mid_split(paged, dtype, plan):
    # The decode kernels keep a reference maximum that moves only when a
    # head's logit passes it by more than 2^8; N(0,1) logits hardly ever do
    # after a split's first tile. Here q is scaled by 8 (logits of std about
    # 8 nats, whose running maximum keeps rising over the first tiles) and
    # each KV head gets one late key equal to 0.05 q of its group's first
    # head (a logit about 36 nats, some 9 above the others' maximum), so the
    # reference moves, and O~ is rescaled, in the middle of long splits.
    lens = [700, 1500, 2900]
    dec = make_decode(B=3, h=8, h_kv=2, d=128, dtype=dtype, seed=77, seq_lens=lens, paged=paged, page_size=16)
    dec["q"] = (dec["q"].float() * 8).to(dec["q"].dtype)
    g = dec["h"] // dec["h_kv"]
    for b, s_b in enumerate(lens):
        for kvh in range(dec["h_kv"]):
            j = s_b - 40 - 7 * kvh
            key = (dec["q"][b, kvh * g].float() * 0.05).to(dec["q"].dtype)
            dec["k_seqs"][b][kvh, j] = key
            if paged:
                dec["k_pool"][dec["block_table"][b, j // 16], j % 16, kvh] = key
            else:
                dec["k"][b, kvh, j] = key
    o_ref, lse_ref = decode_ref(dec["q"], dec["k_seqs"], dec["v_seqs"], dec["seq_lens"], dec["scale"])
    assert lse_ref[:, 0].min() > 30          # the planted key dominates head 0 of each sequence
    o, lse, used = run_decode(dec, plan=plan)
    assert_outputs(o, lse, o_ref, lse_ref, dtype, f"decode, moving reference, paged={paged} plan={used}")


def test_decode_70b_tp8_s32768():
    dec = make_config("decode_70b_tp8_s32768")
    o_ref, lse_ref = decode_ref(dec["q"], dec["k_seqs"], dec["v_seqs"], dec["seq_lens"], dec["scale"])
    for one_call in (True, False):
        for plan in (None, (32768, 1), (64, 512), (16, 2048)):
            o, lse, used = run_decode(dec, plan, one_call)
            assert_outputs(o, lse, o_ref, lse_ref, "bf16", f"70b-tp8 decode plan={used} one_call={one_call}")


def test_decode_llama3_8b_b64_paged(paged_llama):
    dec = paged_llama
    o_ref, lse_ref = decode_ref(dec["q"], dec["k_seqs"], dec["v_seqs"], dec["seq_lens"], dec["scale"])
    for one_call in (True, False):
        o, lse, used = run_decode(dec, None, one_call)
        assert_outputs(o, lse, o_ref, lse_ref, "bf16", f"paged decode B=64 plan={used} one_call={one_call}")


def test_decode_one_call_graph_replay():
    # attn_decode (split and merge on the caller's partial buffers) captured
    # in a HIP graph: every replay, with eager calls and synchronisations
    # between, reproduces the eager bits
    dec = make_decode(B=4, h=8, h_kv=2, d=128, dtype="bf16", seed=27, seq_lens=[7, 6000, 2000, 129],
                      paged=True, page_size=16)
    q, sl = to_dev(dec["q"]), to_dev(dec["seq_lens"])
    kp, vp, bt = to_dev(dec["k_pool"]), to_dev(dec["v_pool"]), to_dev(dec["block_table"])
    chunk, splits = 64, 94
    po = torch.empty((4, 8, splits, 128), dtype=torch.float32, device=DEV)
    pm = torch.empty((4, 8, splits), dtype=torch.float32, device=DEV)
    pl = torch.empty_like(pm)
    o = torch.empty((4, 8, 128), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((4, 8), dtype=torch.float32, device=DEV)

    def step():
        api.decode_call(q, kp, vp, sl, chunk, splits, block_table=bt, scale=dec["scale"], part_o=po, part_m=pm,
                        part_l=pl, out=o, lse=lse)

    step()
    torch.cuda.synchronize()
    o_eager, lse_eager = o.clone(), lse.clone()
    o_ref, lse_ref = decode_ref(dec["q"], dec["k_seqs"], dec["v_seqs"], dec["seq_lens"], dec["scale"])
    assert_outputs(o, lse.cpu().numpy().astype(np.float64), o_ref, lse_ref, "bf16", "attn_decode, eager")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        o.fill_(1.0)
        lse.fill_(0.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_eager.view(torch.int16)), rep
        assert torch.equal(lse, lse_eager), rep
        step()
        torch.cuda.synchronize()


# ------------------------------------------------------------------ (O, LSE) merge

@pytest.mark.parametrize("dtype,T_k,split", [("bf16", 300, 128), ("f16", 257, 1), ("bf16", 200, 199)])
def test_merge_lse_cascade_prefix_suffix(dtype, T_k, split):
    # A shared prefix and a suffix of the keys attended separately (key
    # masks), then combined in (O, LSE) form: the result is attention over
    # all keys, checked against the oracle at the prefill tolerances.
    inp = make_prefill(2, 8, 2, 96, T_k, 128, dtype, seed=T_k * 3 + split, causal=False)
    km_a = np.zeros((2, T_k), dtype=np.uint8)
    km_a[:, :split] = 1
    km_b = (1 - km_a).astype(np.uint8)
    q, k, v = to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"])
    oa, la = api.prefill(q, k, v, causal=False, scale=inp["scale"], key_mask=to_dev(km_a))
    ob, lb = api.prefill(q, k, v, causal=False, scale=inp["scale"], key_mask=to_dev(km_b))
    o, lse = api.merge_lse(oa, la, ob, lb)
    torch.cuda.synchronize()
    o_ref, lse_ref = attention_ref(inp["q"], inp["k"], inp["v"], inp["scale"], False)
    assert_outputs(o, lse.cpu().numpy().astype(np.float64), o_ref, lse_ref, dtype,
                   f"cascade merge {dtype} split {split}/{T_k}")


def _merge_lse_case(dtype, rows, seed):
    """Random (O, LSE) pairs with every kind of empty side. O of an empty side
    is NaN on the device (it must never be read) and zero for the oracle."""
    rng = np.random.default_rng(seed)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    oa = torch.from_numpy(rng.standard_normal((rows, 128)).astype(np.float32)).to(tdt)
    ob = torch.from_numpy(rng.standard_normal((rows, 128)).astype(np.float32)).to(tdt)
    la = rng.normal(0.0, 6.0, rows).astype(np.float32)
    lb = rng.normal(0.0, 6.0, rows).astype(np.float32)
    la[0:10] = -np.inf                       # a empty
    lb[10:20] = np.inf                       # b empty, +inf convention
    la[20:30], lb[20:30] = np.inf, -np.inf   # both empty
    la[30:40], lb[30:40] = -np.inf, -np.inf  # both empty
    la[40:50] = np.inf                       # a empty, +inf convention
    la[50:60], lb[50:60] = 80.0, -80.0       # one side dominates
    la[60:70] = lb[60:70]                    # equal masses
    empty_a = np.isinf(la)
    empty_b = np.isinf(lb)
    oa_ref = oa.float().numpy().astype(np.float64)
    ob_ref = ob.float().numpy().astype(np.float64)
    oa_ref[empty_a] = 0.0
    ob_ref[empty_b] = 0.0
    oa_dev, ob_dev = oa.clone(), ob.clone()
    oa_dev[torch.from_numpy(empty_a)] = float("nan")
    ob_dev[torch.from_numpy(empty_b)] = float("nan")
    return (to_dev(oa_dev), to_dev(la), to_dev(ob_dev), to_dev(lb)), (oa_ref, la.astype(np.float64),
                                                                       ob_ref, lb.astype(np.float64))


def _check_merge_lse(o, lse, o_ref, lse_ref, dtype, what):
    # fp32 arithmetic then one rounding: within half an output ulp plus 1e-5
    o_gpu = o.float().cpu().numpy().astype(np.float64)
    mag = np.abs(o_gpu)
    half_ulp = np.where(mag > 0, np.exp2(np.floor(np.log2(np.where(mag > 0, mag, 1.0))) - MANT_BITS[dtype] - 1), 0.0)
    diff = np.abs(o_gpu - o_ref)
    assert np.all(diff <= half_ulp + 1e-5 * np.maximum(1.0, np.abs(o_ref))), f"{what}: max err {diff.max():.3e}"
    lse_g = lse.cpu().numpy().astype(np.float64)
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_g), empty), f"{what}: empty rows differ"
    assert float(lse_rel(lse_g[~empty], lse_ref[~empty]).max()) <= 1e-5, f"{what}: LSE"
    assert np.all(o.view(torch.int16).cpu().numpy()[empty] == 0), f"{what}: empty rows are not +0.0 bits"


@pytest.mark.parametrize("dtype,rows", [("bf16", 1000), ("f16", 1000), ("bf16", 17), ("bf16", 1)])
def test_merge_lse_against_oracle_with_empty_sides(dtype, rows):
    from oracle import merge_lse_ref
    rows = max(rows, 70) if rows > 1 else rows
    (oa, la, ob, lb), (oa_r, la_r, ob_r, lb_r) = _merge_lse_case(dtype, rows, seed=rows)
    o, lse = api.merge_lse(oa, la, ob, lb)
    torch.cuda.synchronize()
    o_ref, lse_ref = merge_lse_ref(oa_r, la_r, ob_r, lb_r)
    _check_merge_lse(o, lse, o_ref, lse_ref, dtype, f"merge_lse {dtype} rows {rows}")
    # in place over the first operand gives the same bits
    o2, lse2 = api.merge_lse(oa, la, ob, lb, out=oa, lse=la)
    torch.cuda.synchronize()
    assert torch.equal(o2.view(torch.int16), o.view(torch.int16)) and torch.equal(lse2, lse)


def test_merge_lse_llama3_8b_shape_sampled():
    # Full prefill-output shape [1, 32, 8192, 128], in the launch configuration
    # the bench times; checked on 4096 sampled rows.
    from oracle import merge_lse_ref
    g = torch.Generator().manual_seed(7)
    oa = torch.randn((1, 32, 8192, 128), generator=g).to(torch.bfloat16)
    ob = torch.randn((1, 32, 8192, 128), generator=g).to(torch.bfloat16)
    la = (torch.randn((1, 32, 8192), generator=g) * 4).float()
    lb = (torch.randn((1, 32, 8192), generator=g) * 4).float()
    o, lse = api.merge_lse(to_dev(oa), to_dev(la), to_dev(ob), to_dev(lb))
    torch.cuda.synchronize()
    idx = np.random.default_rng(8).choice(32 * 8192, size=4096, replace=False)
    flat = lambda t: t.reshape(32 * 8192, *t.shape[3:])
    o_ref, lse_ref = merge_lse_ref(flat(oa).float().numpy()[idx].astype(np.float64),
                                   flat(la).numpy()[idx].astype(np.float64),
                                   flat(ob).float().numpy()[idx].astype(np.float64),
                                   flat(lb).numpy()[idx].astype(np.float64))
    sel = torch.from_numpy(idx).to(DEV)
    _check_merge_lse(flat(o)[sel], flat(lse)[sel], o_ref, lse_ref, "bf16", "merge_lse llama3-8b sampled")


# ------------------------------------------------------------------ paged (chunked) prefill

def _run_paged_prefill(c, causal, rows_per_block=False, host_order=False, max_excepted_frac=2e-5):
    """attn_prefill_paged on a chunked-prefill case; checks every sequence
    against the oracle over its ground-truth contiguous K/V (every query row,
    or with rows_per_block one random row from each 32-row block)."""
    from online_softmax_tiled_amd.workloads import DTYPES
    q = to_dev(c["q"])
    o, lse = api.prefill_paged(q, to_dev(c["cu_seqlens_q"]), c["max_q"], to_dev(c["k_pool"]), to_dev(c["v_pool"]),
                               to_dev(c["block_table"]), to_dev(c["seq_lens_k"]), causal=causal, scale=c["scale"],
                               seq_lens_k_host=c["seq_lens_k"] if host_order else None)
    torch.cuda.synchronize()
    cu = c["cu_seqlens_q"]
    excluded = c.get("excluded_keys", {})
    for b in range(c["B"]):
        tq, tk = int(cu[b + 1] - cu[b]), int(c["seq_lens_k"][b])
        if tq == 0:
            continue
        qb = c["q"][cu[b]:cu[b + 1]].permute(1, 0, 2).unsqueeze(0)
        kb = c["k_seqs"][b].unsqueeze(0)
        vb = c["v_seqs"][b].unsqueeze(0)
        km = None
        if b in excluded:
            km = np.ones((1, tk), dtype=np.uint8)
            km[0, excluded[b]] = 0
        rows = None
        if rows_per_block and tq > 32:
            # one random row from every 32-row block of the sequence
            starts = np.arange(0, tq, 32)
            rows = np.minimum(starts + np.random.default_rng(b).integers(0, 32, starts.size), tq - 1)
            rows = np.unique(np.concatenate([rows, [0, tq - 1]]))
        o_ref, lse_ref = attention_ref(qb, kb, vb, c["scale"], causal, key_mask=km, rows=rows)
        sel = np.arange(tq) if rows is None else rows
        ob = o[cu[b]:cu[b + 1]][torch.from_numpy(sel).to(DEV)].permute(1, 0, 2).unsqueeze(0)
        lb = lse[cu[b]:cu[b + 1]].cpu().numpy().astype(np.float64)[sel].T[None]
        assert_outputs(ob, lb, o_ref, lse_ref, c["dtype"], f"paged prefill seq {b} ({tq} new / {tk} keys)",
                       max_excepted_frac=max_excepted_frac)


# pools just under the largest addressed with 32-bit offsets (pool + one page
# <= 2^32 - 256 bytes) and just over 4 GB (64-bit addressing)
_UNDER_4GB = lambda page_bytes: 0xFFFFFF00 // page_bytes - 1
_OVER_4GB = lambda page_bytes: (1 << 32) // page_bytes + 64


@pytest.mark.parametrize("size", ["under_4gb", "over_4gb"])
def test_paged_prefill_large_pools(size):
    # the chunked-prefill kernel on pools of 16-key pages x 2 KV heads at the
    # edges of the 32-bit addressing (NaN-filled), half the used pages at the
    # top of the pool
    from online_softmax_tiled_amd.workloads import make_chunked_prefill
    c = make_chunked_prefill(3, 8, 2, 128, "bf16", seed=77, ctx_range=(100, 400), new_range=(10, 90), page_size=16)
    page_bytes = 16 * 2 * 128 * 2
    n_big = (_UNDER_4GB if size == "under_4gb" else _OVER_4GB)(page_bytes)
    assert (n_big * page_bytes + page_bytes <= 0xFFFFFF00) == (size == "under_4gb")
    n_used = c["k_pool"].shape[0]
    new_id = np.array([n_big - 1 - p if p % 2 == 0 else p for p in range(n_used)], dtype=np.int64)
    k_big = torch.full((n_big, 16, 2, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    v_big = torch.full_like(k_big, float("nan"))
    idx = torch.from_numpy(new_id).to(DEV)
    k_big[idx] = to_dev(c["k_pool"])
    v_big[idx] = to_dev(c["v_pool"])
    bt = c["block_table"].astype(np.int64)
    c = dict(c, k_pool=k_big, v_pool=v_big,
             block_table=np.where(bt >= 0, new_id[np.maximum(bt, 0)], -1).astype(np.int32))
    _run_paged_prefill(c, True)
    del c, k_big, v_big
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype,page_size,causal,host_order", [("bf16", 16, True, False), ("f16", 32, True, True),
                                                               ("bf16", 64, False, True), ("bf16", 16, False, False)])
def test_paged_prefill_small(dtype, page_size, causal, host_order):
    from online_softmax_tiled_amd.workloads import make_chunked_prefill
    c = make_chunked_prefill(5, 8, 2, 128, dtype, seed=page_size + 3 * causal, ctx_range=(1, 300),
                             new_range=(1, 120), page_size=page_size, spare_pages=3)
    _run_paged_prefill(c, causal, host_order=host_order)


def test_paged_prefill_edge_sequences():
    # an empty sequence (no new tokens), a fully new one (T_q = T_k), a
    # one-token one, and a block-table entry outside the pool (its keys are
    # excluded, as the oracle's key mask says)
    from online_softmax_tiled_amd.workloads import make_chunked_prefill
    c = make_chunked_prefill(4, 8, 2, 128, "bf16", seed=11, ctx_range=(40, 200), new_range=(1, 60),
                             page_size=16)
    tk = c["seq_lens_k"]
    q_lens = np.array([0, int(tk[1]), 1, min(37, int(tk[3]))], dtype=np.int32)
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    g = torch.Generator().manual_seed(12)
    c["q"] = torch.randn((int(cu[-1]), 8, 128), generator=g).to(torch.bfloat16)
    c.update(q_lens=q_lens, cu_seqlens_q=cu, max_q=int(q_lens.max()))
    bt = c["block_table"].copy()
    bt[3, 1] = -1                     # keys 16..31 of sequence 3 are not in the pool
    c["block_table"] = bt
    c["excluded_keys"] = {3: np.arange(16, 32)}
    _run_paged_prefill(c, True)


def test_paged_prefill_chunked_llama3_8b_b8():
    # the measured chunked-prefill workload, in the bench's launch
    # configuration, on one random query row from every 32-row block of
    # every sequence (every wave's rows are compared)
    c = make_config("chunked_prefill_llama3_8b_b8")
    _run_paged_prefill(c, True, rows_per_block=True, host_order=True)


def test_paged_prefill_matches_contiguous_prefill():
    # one sequence whose pages happen to be consecutive: bits equal to the
    # contiguous kernel on the same keys (same tiling, same arithmetic)
    inp = make_prefill(1, 8, 2, 70, 200, 128, "bf16", seed=5, causal=True)
    k, v = inp["k"][0], inp["v"][0]                       # [h_kv, T_k, d]
    pad = (-200) % 16                                     # 200 keys -> 13 pages, the last zero-padded
    kt = torch.cat([k.permute(1, 0, 2), torch.zeros(pad, 2, 128, dtype=k.dtype)]).reshape(-1, 16, 2, 128)
    vt = torch.cat([v.permute(1, 0, 2), torch.zeros(pad, 2, 128, dtype=v.dtype)]).reshape(-1, 16, 2, 128)
    bt = torch.arange(kt.shape[0], dtype=torch.int32)[None]
    q_tok = inp["q"][0].permute(1, 0, 2).contiguous()     # [T_q, h, d]
    o_p, l_p = api.prefill_paged(to_dev(q_tok), to_dev(torch.tensor([0, 70], dtype=torch.int32)), 70,
                                 to_dev(kt.contiguous()), to_dev(vt.contiguous()), to_dev(bt),
                                 to_dev(torch.tensor([200], dtype=torch.int32)), causal=True, scale=inp["scale"])
    o_c, l_c = api.prefill(to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"]), causal=True, scale=inp["scale"])
    torch.cuda.synchronize()
    assert torch.equal(o_p.permute(1, 0, 2).unsqueeze(0).contiguous().view(torch.int16), o_c.view(torch.int16))
    assert torch.equal(l_p.T.unsqueeze(0).contiguous(), l_c)


# ------------------------------------------------------------------ batch-invariant decode

@pytest.mark.parametrize("h,one_call", [(8, True), (8, False), (64, True)])
@pytest.mark.parametrize("paged", [False, True])
def test_decode_batch_invariant_with_fixed_split(paged, h, one_call):
    # One sequence decoded alone and inside a batch whose longest sequence
    # needs >= 64 splits (the merge then runs its 4-slice layout): with the
    # same fixed split length its output bits are identical, for 8 heads per
    # KV head (16-head blocks) and 64 (the heads as rows, staging waves).
    h_kv, d, split = 1, 128, 256
    lens = [3000, 100, 20000, 777, 5000]
    dec = make_decode(len(lens), h, h_kv, d, "bf16", seed=31, seq_lens=lens, paged=paged, page_size=16)
    alone = make_decode(1, h, h_kv, d, "bf16", seed=32, seq_lens=[3000], paged=paged, page_size=16)
    # sequence 0 of the batch gets the lone sequence's query, keys and values
    dec["q"][0] = alone["q"][0]
    if paged:
        kp, vp, bt = dec["k_pool"], dec["v_pool"], dec["block_table"]
        kp_a, vp_a, bt_a = alone["k_pool"], alone["v_pool"], alone["block_table"]
        for p_log in range((3000 + 15) // 16):
            kp[bt[0, p_log]] = kp_a[bt_a[0, p_log]]
            vp[bt[0, p_log]] = vp_a[bt_a[0, p_log]]
    else:
        dec["k"][0, :, :3000] = alone["k"][0]
        dec["v"][0, :, :3000] = alone["v"][0]

    def run(c):
        sl = to_dev(np.asarray(c["seq_lens"], dtype=np.int32))
        plan = api.decode_plan_fixed(c["seq_lens"], split)
        if paged:
            o, lse, _ = api.decode(to_dev(c["q"]), to_dev(c["k_pool"]), to_dev(c["v_pool"]), sl,
                                   block_table=to_dev(c["block_table"]), page_size=16, scale=c["scale"], plan=plan,
                                   one_call=one_call)
        else:
            o, lse, _ = api.decode(to_dev(c["q"]), to_dev(c["k"]), to_dev(c["v"]), sl, scale=c["scale"], plan=plan,
                                   one_call=one_call)
        torch.cuda.synchronize()
        return o, lse, plan

    o_b, lse_b, plan_b = run(dec)
    o_a, lse_a, plan_a = run(alone)
    assert plan_b[1] >= 64 and plan_a[1] < 64     # the two merges take different layouts
    assert torch.equal(o_b[0].view(torch.int16), o_a[0].view(torch.int16))
    assert torch.equal(lse_b[0], lse_a[0])
    o_ref, lse_ref = decode_ref(alone["q"], alone["k_seqs"], alone["v_seqs"], alone["seq_lens"], alone["scale"])
    assert_outputs(o_a, lse_a.cpu().numpy().astype(np.float64), o_ref, lse_ref, "bf16", "batch-invariant decode")
    # and run to run
    o_b2, _, _ = run(dec)
    assert torch.equal(o_b2.view(torch.int16), o_b.view(torch.int16))



# ------------------------------------------------------------------ large head groups (decode)

@pytest.mark.parametrize("dtype,paged,page_size,plans", [
    ("bf16", False, 16, [None, (80, 19), (1504, 1), (64, 2)]),   # split ends inside 64-key tiles; last takes the rest
    ("f16", False, 16, [None, (992, 2)]),
    ("bf16", True, 32, [None, (208, 8)]),
    ("f16", True, 16, [(64, 24), (400, 2)]),
    ("bf16", True, 48, [None, (96, 16)]),    # page size not a power of two: the 16-head block kernel
])
def test_decode_head_rows(dtype, paged, page_size, plans):
    # g = 40 on two KV heads: the heads of a group are the rows of two waves,
    # the second one part-filled; empty, one-key and tile-edge sequences
    lens = [0, 1, 63, 64, 65, 700, 1500]
    dec = make_decode(B=len(lens), h=80, h_kv=2, d=128, dtype=dtype, seed=31 + page_size, seq_lens=lens,
                      paged=paged, page_size=page_size, spare_pages=3)
    o_ref, lse_ref = decode_ref(dec["q"], dec["k_seqs"], dec["v_seqs"], dec["seq_lens"], dec["scale"])
    for plan in plans:
        o, lse, used = run_decode(dec, plan)
        assert_outputs(o, lse, o_ref, lse_ref, dtype, f"decode g=40 paged={paged} P={page_size} plan={used}")


def test_decode_head_rows_repeatable():
    # g = 128, contiguous: waves 4-7 only stage, and reach
    # iteration 0's store of K(2) into K(0)'s slot long before the other
    # waves; a barrier after the reads of K(0) keeps that store out of them.
    # Short splits put a first tile in every workgroup; every run must give
    # the same bits, within tolerance of the oracle.
    lens = [1500, 700, 64, 65, 1]
    dec = make_decode(B=len(lens), h=128, h_kv=1, d=128, dtype="bf16", seed=43, seq_lens=lens, paged=False)
    o_ref, lse_ref = decode_ref(dec["q"], dec["k_seqs"], dec["v_seqs"], dec["seq_lens"], dec["scale"])
    first = None
    for _ in range(20):
        o, lse, used = run_decode(dec, (80, 19))
        if first is None:
            assert_outputs(o, lse, o_ref, lse_ref, "bf16", "decode g=128 plan=(80, 19)")
            first = o.clone()
        else:
            assert torch.equal(o.view(torch.int16), first.view(torch.int16))


def test_decode_head_rows_page_outside_pool():
    # a block-table entry outside the pool: its 16 keys are excluded, so the
    # exact result is attention over the remaining keys
    lens = [300, 90]
    dec = make_decode(B=2, h=128, h_kv=1, d=128, dtype="bf16", seed=41, seq_lens=lens, paged=True, page_size=16)
    bt = dec["block_table"].copy()
    bt[0, 2] = dec["k_pool"].shape[0] + 5      # keys 32..47 of sequence 0
    bt[1, 5] = -7                              # keys 80..89 of sequence 1
    keep0 = np.r_[0:32, 48:300]
    keep1 = np.arange(80)
    k_seqs = [dec["k_seqs"][0][:, keep0], dec["k_seqs"][1][:, keep1]]
    v_seqs = [dec["v_seqs"][0][:, keep0], dec["v_seqs"][1][:, keep1]]
    o_ref, lse_ref = decode_ref(dec["q"], k_seqs, v_seqs, np.array([keep0.size, keep1.size]), dec["scale"])
    sl = to_dev(dec["seq_lens"])
    for plan in (None, (64, 5)):
        o, lse, used = api.decode(to_dev(dec["q"]), to_dev(dec["k_pool"]), to_dev(dec["v_pool"]), sl,
                                  seq_lens_host=dec["seq_lens"], block_table=to_dev(bt), page_size=16,
                                  scale=dec["scale"], plan=plan)
        torch.cuda.synchronize()
        assert_outputs(o, lse.cpu().numpy().astype(np.float64), o_ref, lse_ref, "bf16",
                       f"decode g=128 pages outside the pool plan={used}")


@pytest.mark.parametrize("size", ["under_4gb", "over_4gb"])
def test_decode_head_rows_large_pools(size):
    # pools of 16-key pages (NaN-filled) just under the largest addressed
    # with 32-bit offsets and just over 4 GB (64-bit addressing), for the row
    # form with staging waves (g = 64) and with every wave computing (g = 256);
    # half the pages sit at the top of the pool, one table entry is outside
    # the pool (its rows must read as zeros, not as the NaN of pool row 0),
    # the rest stay low
    page_bytes = 16 * 128 * 2
    n_big = (_UNDER_4GB if size == "under_4gb" else _OVER_4GB)(page_bytes)
    assert (n_big * page_bytes + page_bytes <= 0xFFFFFF00) == (size == "under_4gb")
    k_big = torch.empty((n_big, 16, 1, 128), dtype=torch.bfloat16, device=DEV)
    v_big = torch.empty_like(k_big)
    lens = [500, 77]
    for h in (64, 256):
        dec = make_decode(B=2, h=h, h_kv=1, d=128, dtype="bf16", seed=44 + h, seq_lens=lens, paged=True,
                          page_size=16)
        n_used = dec["k_pool"].shape[0]
        new_id = np.array([n_big - 1 - p if p % 2 == 0 else p for p in range(n_used)], dtype=np.int64)
        assert 0 not in new_id
        k_big.fill_(float("nan"))
        v_big.fill_(float("nan"))
        idx = torch.from_numpy(new_id).to(DEV)
        k_big[idx] = to_dev(dec["k_pool"])
        v_big[idx] = to_dev(dec["v_pool"])
        bt = dec["block_table"].astype(np.int64)
        bt = np.where(bt >= 0, new_id[np.maximum(bt, 0)], -1).astype(np.int32)
        bt[0, 3] = n_big + 9                       # keys 48..63 of sequence 0
        keep0 = np.r_[0:48, 64:500]
        k_seqs = [dec["k_seqs"][0][:, keep0], dec["k_seqs"][1]]
        v_seqs = [dec["v_seqs"][0][:, keep0], dec["v_seqs"][1]]
        o_ref, lse_ref = decode_ref(dec["q"], k_seqs, v_seqs, np.array([keep0.size, 77]), dec["scale"])
        sl = to_dev(dec["seq_lens"])
        for plan in (None, (64, 9)):
            o, lse, used = api.decode(to_dev(dec["q"]), k_big, v_big, sl, seq_lens_host=dec["seq_lens"],
                                      block_table=to_dev(bt), page_size=16, scale=dec["scale"], plan=plan)
            torch.cuda.synchronize()
            assert_outputs(o, lse.cpu().numpy().astype(np.float64), o_ref, lse_ref, "bf16",
                           f"decode g={h} on {size} pools of {n_big} pages plan={used}")
    del k_big, v_big
    torch.cuda.empty_cache()


def test_decode_head_rows_partials_match_slices():
    # the row kernel's stage-1 states, finalised one by one, against the
    # oracle on each key slice (m in natural-log units, l the sum of weights)
    dec = make_decode(B=2, h=40, h_kv=1, d=128, dtype="bf16", seed=13, seq_lens=[700, 129], paged=False)
    chunk, S = 144, 5
    po, pm, pl = api.decode_split(to_dev(dec["q"]), to_dev(dec["k"]), to_dev(dec["v"]), to_dev(dec["seq_lens"]),
                                  chunk, S, scale=dec["scale"])
    torch.cuda.synchronize()
    po, pm, pl = po.cpu().numpy(), pm.cpu().numpy(), pl.cpu().numpy()
    for b in range(2):
        s = int(dec["seq_lens"][b])
        qb = dec["q"][b].double().numpy()
        kb = dec["k_seqs"][b].double().numpy()
        vb = dec["v_seqs"][b].double().numpy()
        m, l, a = split_states_ref(qb, kb, vb, s, dec["scale"], chunk)
        n = min(S, math.ceil(s / chunk))
        for i in range(40):
            for sp in range(n):
                o_g, lse_g = finalize_ref((float(pm[b, i, sp]), float(pl[b, i, sp]), po[b, i, sp].astype(np.float64)))
                o_r, lse_r = finalize_ref((m[i, sp], l[i, sp], a[i, sp]))
                assert np.max(np.abs(o_g - o_r)) < 1e-2
                assert abs(lse_g - lse_r) / max(1.0, abs(lse_r)) < LSE_TOL


@pytest.mark.parametrize("h,h_kv,paged,page_size", [(32, 1, False, 16), (48, 2, True, 16), (128, 1, False, 16),
                                                    (128, 1, True, 16), (17, 1, False, 16),
                                                    (48, 2, True, 48), (17, 1, True, 80), (160, 2, True, 48),
                                                    (256, 1, True, 32), (256, 1, False, 16)])
def test_decode_large_groups(h, h_kv, paged, page_size):
    # g = 32, 24, 128 (MLA-style), 17: the heads as the rows of the prefill
    # kernel (with staging waves up to 128 heads, every wave computing at
    # 256); pages of 48 or 80 tokens (not a power of two): blocks of 16
    # heads, one per wave (head mode), with g = 80 spread over two workgroups
    dec = make_decode(3, h, h_kv, 128, "bf16", seed=h + h_kv, len_range=(1, 700), paged=paged, page_size=page_size)
    sl = to_dev(np.asarray(dec["seq_lens"], dtype=np.int32))
    if paged:
        o, lse, plan = api.decode(to_dev(dec["q"]), to_dev(dec["k_pool"]), to_dev(dec["v_pool"]), sl,
                                  block_table=to_dev(dec["block_table"]), page_size=page_size, scale=dec["scale"])
    else:
        o, lse, plan = api.decode(to_dev(dec["q"]), to_dev(dec["k"]), to_dev(dec["v"]), sl, scale=dec["scale"])
    torch.cuda.synchronize()
    o_ref, lse_ref = decode_ref(dec["q"], dec["k_seqs"], dec["v_seqs"], dec["seq_lens"], dec["scale"])
    assert_outputs(o, lse.cpu().numpy().astype(np.float64), o_ref, lse_ref, "bf16",
                   f"decode g={h // h_kv} paged={paged} plan={plan}")


# ------------------------------------------------------------------ PV product operand type

def _check_big_column(o, lse, o_ref, lse_ref, col, what):
    """Flat gate on every output column but ``col``; on ``col`` (which holds
    weighted sums of a value of 2^17) a relative bound of 2^-7: bf16 weights
    and the bf16 output each round to 2^-9 relative, while a value clamped to
    the fp16 maximum would be off by up to half."""
    keep = [c for c in range(o_ref.shape[-1]) if c != col]
    assert_outputs(o[..., keep], lse, o_ref[..., keep], lse_ref, "bf16", what)
    got = o[..., col].float().cpu().numpy().astype(np.float64)
    ref = o_ref[..., col]
    assert np.abs(ref).max() >= 100          # the big value carries real weight somewhere
    rel = np.abs(got - ref) / np.maximum(np.abs(ref), 1.0)
    assert float(rel.max()) <= 2.0 ** -7, f"{what}: column {col} rel err {rel.max():.3e}"


def test_bf16_values_beyond_fp16_range_take_the_bf16_pass():
    # The PV product runs on fp16 operands (bf16 V converted exactly when it
    # is staged). A bf16 value of magnitude 65536 or more does not fit fp16:
    # the workgroups that stage one must rerun with bf16 operands, so the
    # result is the exact one up to bf16 rounding, not one computed with a
    # value clamped to 65504. One V value of 2^17 in each form that stages V.
    from online_softmax_tiled_amd.workloads import make_chunked_prefill
    big = float(2 ** 17)
    # contiguous prefill, with and without a key mask
    for km in (0.0, 0.2):
        inp = make_prefill(1, 8, 2, 96, 96, 128, "bf16", seed=61, causal=True, key_p=km)
        inp["v"][0, 1, 5, 3] = big
        o, lse, o_ref, lse_ref = run_prefill(inp)
        _check_big_column(o, lse, o_ref, lse_ref, 3, f"prefill with V = 2^17 (key mask p={km})")
    # paged (chunked) prefill: sequence 1, key 7, column 9
    c = make_chunked_prefill(2, 8, 2, 128, "bf16", seed=62, ctx_range=(60, 200), new_range=(20, 60), page_size=16)
    b, key = 1, 7
    c["v_pool"][c["block_table"][b, key // 16], key % 16, 0, 9] = big
    c["v_seqs"][b][0, key, 9] = big
    q = to_dev(c["q"])
    o, lse = api.prefill_paged(q, to_dev(c["cu_seqlens_q"]), c["max_q"], to_dev(c["k_pool"]), to_dev(c["v_pool"]),
                               to_dev(c["block_table"]), to_dev(c["seq_lens_k"]), causal=True, scale=c["scale"])
    torch.cuda.synchronize()
    cu = c["cu_seqlens_q"]
    qb = c["q"][cu[b]:cu[b + 1]].permute(1, 0, 2).unsqueeze(0)
    o_ref, lse_ref = attention_ref(qb, c["k_seqs"][b].unsqueeze(0), c["v_seqs"][b].unsqueeze(0), c["scale"], True)
    ob = o[cu[b]:cu[b + 1]].permute(1, 0, 2).unsqueeze(0)
    lb = lse[cu[b]:cu[b + 1]].cpu().numpy().astype(np.float64).T[None]
    _check_big_column(ob, lb, o_ref, lse_ref, 9, "paged prefill with V = 2^17")
    # decode with the heads as rows (staging waves), contiguous: column 100
    dec = make_decode(B=2, h=64, h_kv=1, d=128, dtype="bf16", seed=63, seq_lens=[300, 90], paged=False)
    dec["v"][0, 0, 17, 100] = -big
    dec["v_seqs"][0][0, 17, 100] = -big
    o_ref, lse_ref = decode_ref(dec["q"], dec["k_seqs"], dec["v_seqs"], dec["seq_lens"], dec["scale"])
    o, lse, used = run_decode(dec)
    _check_big_column(o, lse, o_ref, lse_ref, 100, "row-form decode with V = -2^17")


@pytest.mark.parametrize("db,g4,half", [(db, g4, hf) for db in range(4) for g4 in range(4) for hf in range(2)])
def test_bf16_large_v_found_in_every_accumulator_register(db, g4, half):
    # A wave's output tile sits in 64 accumulator registers per lane: column
    # d = 32 db + 8 g4 + 4 half + k lives in register 4 g4 + k of block db on
    # the lanes of half-wave `half`. The fp16 pass sends a V value of 2^17 in
    # column d to that register only (as inf or NaN), so the test that starts
    # the bf16 pass must read every register; one run per (db, g4, half), k
    # varied with them.
    col = 32 * db + 8 * g4 + 4 * half + (db + g4 + half) % 4
    inp = make_prefill(1, 4, 1, 64, 64, 128, "bf16", seed=200 + col, causal=True)
    inp["v"][0, 0, 9, col] = -float(2 ** 17)
    o, lse, o_ref, lse_ref = run_prefill(inp)
    _check_big_column(o, lse, o_ref, lse_ref, col, f"prefill with V = -2^17 in column {col}")


def test_stream_read_reads_every_word_once():
    # the read-rate calibration kernel: chunk c's output is the xor of the
    # 32-bit words of its contiguous chunk (bit for bit), for sizes that do
    # and do not divide into the chunks
    for n_words, chunks in ((1 << 20, 1024), (4 * 1001, 7), (4 * 3, 5)):
        g = torch.Generator().manual_seed(n_words)
        src = torch.randint(-2 ** 31, 2 ** 31 - 1, (n_words,), generator=g, dtype=torch.int64).to(torch.int32)
        out = api.stream_read(to_dev(src), chunks=chunks)
        torch.cuda.synchronize()
        words = src.numpy().view(np.uint32)
        per16 = -(-(n_words // 4) // chunks)                  # 16-byte units per chunk
        want = np.zeros(chunks, dtype=np.uint32)
        for c in range(chunks):
            part = words[c * per16 * 4:(c + 1) * per16 * 4]
            want[c] = np.bitwise_xor.reduce(part) if part.size else 0
        assert np.array_equal(out.cpu().numpy().view(np.uint32), want)
