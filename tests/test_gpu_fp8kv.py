"""GPU parity of split-KV decode over 8-bit E4M3 K/V (attn_decode_split_fp8kv,
attn_decode_fp8kv) against the float64 oracle.

The oracle side decodes the stored codes with oracle.fp8 (OCP E4M3 times
the tensor's scale) and runs the plain float64 decode on those values; the
gate is the same as for 16-bit K/V (assert_outputs). Inputs come from
make_decode(kv_codes=True): codes with exponent field 4..9 and the NaN code
0x7F in every slot that must not be read (unused page slots, spare pages,
padding past a sequence's length).
"""

import numpy as np
import pytest
import torch

from oracle import decode_ref, e4m3_decode
from online_softmax_tiled_amd import api
from online_softmax_tiled_amd.workloads import make_decode

from tests.test_gpu_parity import DEV, assert_outputs, to_dev

pytestmark = pytest.mark.gpu

# Not powers of two, so both must enter the arithmetic; about 1/3, so that
# the decoded K and V (codes of rms about 3) have unit scale like the other
# decode checks' N(0,1) values, which the absolute output gate is set for.
K_SCALE, V_SCALE = 0.37, 0.29


def oracle_fp8(dec, k_scale, v_scale):
    k_f = [e4m3_decode(ks, k_scale) for ks in dec["k_seqs"]]
    v_f = [e4m3_decode(vs, v_scale) for vs in dec["v_seqs"]]
    return decode_ref(dec["q"], k_f, v_f, dec["seq_lens"], dec["scale"])


def run_fp8(dec, k_scale, v_scale, plan=None, one_call=True):
    q = to_dev(dec["q"])
    sl = to_dev(dec["seq_lens"])
    if dec["paged"]:
        k, v, bt, ps = to_dev(dec["k_pool"]), to_dev(dec["v_pool"]), to_dev(dec["block_table"]), dec["page_size"]
    else:
        k, v, bt, ps = to_dev(dec["k"]), to_dev(dec["v"]), None, 16
    if plan is None:
        plan = api.decode_plan(dec["seq_lens"], dec["h"], dec["h_kv"], device=DEV)
    chunk, splits = plan
    if one_call:
        o, lse = api.decode_fp8kv_call(q, k, v, sl, chunk, splits, k_scale, v_scale, block_table=bt, page_size=ps,
                                       scale=dec["scale"])
    else:
        parts = api.decode_split_fp8kv(q, k, v, sl, chunk, splits, k_scale, v_scale, block_table=bt, page_size=ps,
                                       scale=dec["scale"])
        o, lse = api.merge_states(*parts, sl, chunk, q.dtype)
    torch.cuda.synchronize()
    return o, lse.cpu().numpy().astype(np.float64), plan


@pytest.mark.parametrize("plan", [(1024, 3), (4096, 1)])
@pytest.mark.parametrize("paged", [False, True])
def test_fp8kv_decode_reference_moves_mid_split(paged, plan):
    # q scaled by 8 against E4M3 keys of magnitude up to 8 (k_scale 0.37):
    # logits of std about 10 nats, whose running maximum keeps rising over the
    # first tiles of each long split, so the kernel's lagging reference moves
    # (and O~ is rescaled) after the first tile.
    lens = [700, 1500, 2900]
    dec = make_decode(B=3, h=8, h_kv=2, d=128, dtype="bf16", seed=78, seq_lens=lens, paged=paged, page_size=16,
                      kv_codes=True)
    dec["q"] = (dec["q"].float() * 8).to(dec["q"].dtype)
    o_ref, lse_ref = oracle_fp8(dec, K_SCALE, V_SCALE)
    o, lse, used = run_fp8(dec, K_SCALE, V_SCALE, plan)
    assert_outputs(o, lse, o_ref, lse_ref, "bf16", f"fp8 KV decode, moving reference, paged={paged} plan={used}")


@pytest.mark.parametrize("one_call", [True, False])
@pytest.mark.parametrize("paged,page_size", [(False, 16), (True, 16), (True, 48)])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_fp8kv_decode_small(paged, page_size, dtype, one_call):
    lens = [1, 5, 16, 17, 63, 64, 65, 300, 1000, 0]
    dec = make_decode(B=len(lens), h=16, h_kv=4, d=128, dtype=dtype, seed=31 + page_size, seq_lens=lens,
                      paged=paged, page_size=page_size, spare_pages=3, kv_codes=True)
    o_ref, lse_ref = oracle_fp8(dec, K_SCALE, V_SCALE)
    for plan in (None, (64, 16), (1024, 1), (64, 2), (16, 63)):
        o, lse, used = run_fp8(dec, K_SCALE, V_SCALE, plan, one_call)
        assert_outputs(o, lse, o_ref, lse_ref, dtype, f"fp8 KV decode paged={paged} plan={used} one_call={one_call}")


@pytest.mark.parametrize("h,h_kv,paged,page_size", [(64, 2, False, 32), (128, 1, True, 32), (40, 2, True, 48),
                                                   (256, 1, False, 16), (160, 1, True, 48)])
def test_fp8kv_decode_large_groups(h, h_kv, paged, page_size):
    # more than 16 query heads per KV head: the heads as rows (up to 128,
    # power-of-two pages), else head blocks of 16 on the split kernel (pages
    # of 48 keys, 160 and 256 heads)
    dec = make_decode(B=3, h=h, h_kv=h_kv, d=128, dtype="bf16", seed=h + h_kv, seq_lens=[777, 64, 2049],
                      paged=paged, page_size=page_size, spare_pages=2, kv_codes=True)
    o_ref, lse_ref = oracle_fp8(dec, K_SCALE, V_SCALE)
    o, lse, _ = run_fp8(dec, K_SCALE, V_SCALE)
    assert_outputs(o, lse, o_ref, lse_ref, "bf16", f"fp8 KV decode g={h // h_kv}")


@pytest.mark.parametrize("layout", ["contiguous", "paged16", "paged64"])
@pytest.mark.parametrize("g", [17, 24, 32, 64, 128])
def test_fp8kv_decode_heads_as_rows(g, layout):
    # 17-128 query heads per KV head (power-of-two pages) take the prefill
    # kernel with the heads as its rows; its staging waves convert the codes
    # as they store the K/V tiles
    paged = layout != "contiguous"
    h_kv = 2 if g <= 32 else 1
    dtype = "f16" if g in (24, 128) else "bf16"
    dec = make_decode(B=3, h=g * h_kv, h_kv=h_kv, d=128, dtype=dtype, seed=900 + g, seq_lens=[1000, 33, 2500],
                      paged=paged, page_size=64 if layout == "paged64" else 16, spare_pages=2, kv_codes=True)
    o_ref, lse_ref = oracle_fp8(dec, K_SCALE, V_SCALE)
    for plan in (None, (64, 40), (512, 5), (16, 157)):
        o, lse, used = run_fp8(dec, K_SCALE, V_SCALE, plan, one_call=plan != (512, 5))
        assert_outputs(o, lse, o_ref, lse_ref, dtype, f"fp8 KV decode rows g={g} {layout} plan={used}")


_UNDER_4GB = lambda page_bytes: 0xFFFFFF00 // page_bytes - 1
_OVER_4GB = lambda page_bytes: (1 << 32) // page_bytes + 64


@pytest.mark.parametrize("size", ["under_4gb", "over_4gb"])
def test_fp8kv_decode_rows_large_pools(size):
    # 8-bit pools of 16-key pages (NaN code 0x7F everywhere else) just under
    # the largest the rows form addresses with 32-bit offsets, and just over
    # 4 GB (blocks of 16 heads then); half the used pages at the top of the
    # pool, one table entry outside the pool (its keys are excluded)
    page_bytes = 16 * 128
    n_big = (_UNDER_4GB if size == "under_4gb" else _OVER_4GB)(page_bytes)
    assert (n_big * page_bytes + page_bytes <= 0xFFFFFF00) == (size == "under_4gb")
    k_big = torch.empty((n_big, 16, 1, 128), dtype=torch.uint8, device=DEV)
    v_big = torch.empty_like(k_big)
    lens = [500, 77]
    dec = make_decode(B=2, h=64, h_kv=1, d=128, dtype="bf16", seed=47, seq_lens=lens, paged=True, page_size=16,
                      kv_codes=True)
    n_used = dec["k_pool"].shape[0]
    new_id = np.array([n_big - 1 - p if p % 2 == 0 else p for p in range(n_used)], dtype=np.int64)
    assert 0 not in new_id
    k_big.fill_(0x7F)
    v_big.fill_(0x7F)
    idx = torch.from_numpy(new_id).to(DEV)
    k_big[idx] = to_dev(dec["k_pool"])
    v_big[idx] = to_dev(dec["v_pool"])
    bt = dec["block_table"].astype(np.int64)
    bt = np.where(bt >= 0, new_id[np.maximum(bt, 0)], -1).astype(np.int32)
    bt[0, 3] = n_big + 9                       # keys 48..63 of sequence 0
    keep0 = np.r_[0:48, 64:500]
    kept = dict(dec, k_seqs=[dec["k_seqs"][0][:, keep0], dec["k_seqs"][1]],
                v_seqs=[dec["v_seqs"][0][:, keep0], dec["v_seqs"][1]], seq_lens=np.array([keep0.size, 77]))
    o_ref, lse_ref = oracle_fp8(kept, K_SCALE, V_SCALE)
    sl = to_dev(dec["seq_lens"])
    for plan in (None, (64, 9)):
        o, lse, used = api.decode_fp8kv(to_dev(dec["q"]), k_big, v_big, sl, K_SCALE, V_SCALE,
                                        seq_lens_host=dec["seq_lens"], block_table=to_dev(bt), page_size=16,
                                        scale=dec["scale"], plan=plan)
        torch.cuda.synchronize()
        assert_outputs(o, lse.cpu().numpy().astype(np.float64), o_ref, lse_ref, "bf16",
                       f"fp8 KV decode g=64 on {size} pools of {n_big} pages plan={used}")
    del k_big, v_big
    torch.cuda.empty_cache()


def test_fp8kv_every_finite_code():
    # keys and values run through every finite E4M3 code (subnormals, both
    # zeros, 448), so each one is converted on the device at least once (to
    # fp16 for both K and V here)
    dec = make_decode(B=2, h=8, h_kv=1, d=128, dtype="f16", seed=5, seq_lens=[254, 130], kv_codes=True)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    for b, s in enumerate(dec["seq_lens"]):
        n = int(s) * 128
        codes = torch.from_numpy(np.resize(np.roll(finite, 17 * b), n).reshape(1, int(s), 128))
        dec["k_seqs"][b][:] = codes
        dec["v_seqs"][b][:] = torch.from_numpy(np.resize(np.roll(finite, 101 + b), n).reshape(1, int(s), 128))
        dec["k"][b, :, :s] = dec["k_seqs"][b]
        dec["v"][b, :, :s] = dec["v_seqs"][b]
    # small k_scale: with codes up to 448 the logits stay moderate
    o_ref, lse_ref = oracle_fp8(dec, 0.002, 0.01)
    o, lse, _ = run_fp8(dec, 0.002, 0.01, plan=(64, 4))
    assert_outputs(o, lse, o_ref, lse_ref, "f16", "fp8 KV decode over every finite code")


def test_fp8kv_decode_70b_tp8_s32768():
    # the batch-1 decode shape (8 query heads, one KV head, 32768 keys) in full
    dec = make_decode(B=1, h=8, h_kv=1, d=128, dtype="bf16", seed=4242, seq_lens=[32768], kv_codes=True)
    o_ref, lse_ref = oracle_fp8(dec, K_SCALE, V_SCALE)
    o, lse, plan = run_fp8(dec, K_SCALE, V_SCALE)
    assert_outputs(o, lse, o_ref, lse_ref, "bf16", f"fp8 KV decode 70B TP8 shard, plan {plan}")


def test_fp8kv_matches_16bit_path_on_decoded_values():
    # the same keys and values given as fp16 (the decoded codes times
    # power-of-two scales are exact in fp16) give, through attn_decode, the
    # results of attn_decode_fp8kv up to the order of the fp32 sums (the two
    # kernels walk the head dimension's chunks in different orders): the
    # scales enter once per score and once per split's O~, not per element
    dec = make_decode(B=4, h=16, h_kv=2, d=128, dtype="f16", seed=77, seq_lens=[100, 513, 2, 4000],
                      paged=True, page_size=16, spare_pages=1, kv_codes=True)
    ks, vs = 0.5, 2.0
    kp = torch.from_numpy(e4m3_decode(dec["k_pool"], ks)).to(torch.float16)
    vp = torch.from_numpy(e4m3_decode(dec["v_pool"], vs)).to(torch.float16)
    q, sl, bt = to_dev(dec["q"]), to_dev(dec["seq_lens"]), to_dev(dec["block_table"])
    plan = api.decode_plan(dec["seq_lens"], 16, 2, device=DEV)
    o8, l8 = api.decode_fp8kv_call(q, to_dev(dec["k_pool"]), to_dev(dec["v_pool"]), sl, *plan, ks, vs,
                                   block_table=bt, page_size=16, scale=dec["scale"])
    o16, l16 = api.decode_call(q, to_dev(kp), to_dev(vp), sl, *plan, block_table=bt, page_size=16,
                               scale=dec["scale"])
    torch.cuda.synchronize()
    assert torch.allclose(o8.float(), o16.float(), rtol=0, atol=2e-3)
    assert torch.allclose(l8, l16, rtol=2e-6, atol=2e-6)
