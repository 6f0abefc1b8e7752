"""attn_decode_noalloc: attn_decode with the split-KV partial states in the
library's per-GPU device scratch (for callers that cannot allocate).

Checked through the C ABI against attn_decode on the same inputs: the two
run the same kernels on the same partial-state layout, so the outputs and
LSE must be bitwise equal; each call is also checked against the float64
oracle at the parity tolerances. Three calls in a row, each on a smaller
problem than the one before, so a later call runs on scratch the earlier
one left behind. Problems whose partial states do not fit the scratch are
rejected before anything is launched (CPU)."""

import ctypes

import numpy as np
import pytest
import torch

from oracle import decode_ref
from online_softmax_tiled_amd import api
from online_softmax_tiled_amd.workloads import make_decode
from tests.test_gpu_parity import DEV, assert_outputs, to_dev


def _both(dec, plan):
    q, sl = to_dev(dec["q"]), to_dev(dec["seq_lens"])
    if dec["paged"]:
        k, v, bt, ps = to_dev(dec["k_pool"]), to_dev(dec["v_pool"]), to_dev(dec["block_table"]), dec["page_size"]
    else:
        k, v, bt, ps = to_dev(dec["k"]), to_dev(dec["v"]), None, 16
    chunk, splits = plan
    o_n, l_n = api.decode_noalloc(q, k, v, sl, chunk, splits, block_table=bt, page_size=ps, scale=dec["scale"])
    torch.cuda.synchronize()
    o_a, l_a = api.decode_call(q, k, v, sl, chunk, splits, block_table=bt, page_size=ps, scale=dec["scale"])
    torch.cuda.synchronize()
    return o_n, l_n, o_a, l_a


@pytest.mark.gpu
def test_decode_noalloc_matches_attn_decode_on_successive_calls():
    cases = [
        # paged, 16 heads per KV head group of 4, ragged lengths: 12 sequences x 32 heads x 40 splits
        (make_decode(B=12, h=32, h_kv=8, d=128, dtype="bf16", seed=71, len_range=(1, 5000), paged=True,
                     page_size=16), (128, 40)),
        # contiguous, fewer sequences and splits, an empty sequence
        (make_decode(B=3, h=8, h_kv=1, d=128, dtype="f16", seed=72, seq_lens=[2000, 0, 333], paged=False), (64, 32)),
        # 64 heads per KV head (the row form), one sequence
        (make_decode(B=1, h=64, h_kv=1, d=128, dtype="bf16", seed=73, seq_lens=[700], paged=False), (64, 11)),
    ]
    for dec, plan in cases:
        o_n, l_n, o_a, l_a = _both(dec, plan)
        what = f"decode_noalloc B={dec['q'].shape[0]} h={dec['q'].shape[1]} plan={plan}"
        assert torch.equal(o_n.view(torch.int16), o_a.view(torch.int16)), what
        assert torch.equal(l_n, l_a), what
        o_ref, lse_ref = decode_ref(dec["q"], dec["k_seqs"], dec["v_seqs"], dec["seq_lens"], dec["scale"])
        dt = "bf16" if dec["q"].dtype == torch.bfloat16 else "f16"
        assert_outputs(o_n, l_n.cpu().numpy().astype(np.float64), o_ref, lse_ref, dt, what)


def test_decode_noalloc_rejects_what_the_scratch_cannot_hold():
    # 64 x 32 x 40 partial states need 42.6 MB (> 32 MiB): rejected as
    # unsupported before any launch; 64528 states (33.56 MB) would fit
    lib = api.load()
    p = lambda x: ctypes.c_void_p(x)
    rc = lib.attn_decode_noalloc(p(16), p(16), p(16), None, 0, 16, 0, p(16), 40 * 128, 64, 32, 8, 128, 128, 40, 1,
                                 0.088, p(16), None, None)
    assert rc == 2
    msg = lib.attn_last_error().decode()
    assert "attn_decode_noalloc" in msg and "scratch" in msg
    # the usual argument checks come first
    assert lib.attn_decode_noalloc(p(16), p(16), p(16), None, 0, 16, 0, p(16), 64, 1, 8, 1, 128, 40, 1, 1, 0.088,
                                   p(16), None, None) == 1        # chunk not a multiple of 16
    assert lib.attn_decode_noalloc(p(16), p(16), p(16), None, 0, 16, 0, p(16), 64, 1, 8, 1, 128, 64, 1, 1, 0.088,
                                   None, None, None) == 1         # no output
