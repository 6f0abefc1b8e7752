"""GPU parity on randomly drawn small configurations.

Each case draws its shape, dtype, masks, page size and split plan from a
seeded generator and checks the kernels, called through the C ABI, against
the float64 oracle with the tolerances of test_gpu_parity. The fixed cases
there pin the edges one by one; these mix them (GQA ratios, ragged lengths,
tile-edge split boundaries, partial pages, key and row masks, empty
sequences) in combinations nobody wrote down.
"""

import numpy as np
import pytest
import torch

from oracle import attention_ref, decode_ref
from online_softmax_tiled_amd import api
from online_softmax_tiled_amd.workloads import make_chunked_prefill, make_decode, make_prefill
from tests.test_gpu_parity import _run_paged_prefill, assert_outputs, run_decode, run_prefill

pytestmark = pytest.mark.gpu

N_CASES = 40


@pytest.mark.parametrize("case", range(N_CASES))
def test_prefill_random(case):
    rng = np.random.default_rng(5000 + case)
    h_kv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 3, 4, 5, 8]))
    causal = bool(rng.integers(2))
    t_q = int(rng.integers(1, 301))
    t_k = int(rng.integers(t_q if causal else 1, 401))
    dtype = str(rng.choice(["bf16", "f16"]))
    key_tile_p = float(rng.choice([0.0, 0.0, 0.25, 0.5]))
    key_p = float(rng.choice([0.0, 0.0, 0.1]))
    rows = int(rng.choice([0, 0, 3]))
    inp = make_prefill(int(rng.integers(1, 4)), h_kv * g, h_kv, t_q, t_k, 128, dtype, seed=6000 + case,
                       causal=causal, key_tile_p=key_tile_p, key_p=key_p, row_mask_count=min(rows, t_q) or None)
    o, lse, o_ref, lse_ref = run_prefill(inp)
    assert_outputs(o, lse, o_ref, lse_ref, dtype,
                   f"random prefill {case}: h={h_kv * g}/{h_kv} {t_q}x{t_k} causal={causal} "
                   f"tile_p={key_tile_p} key_p={key_p} rows={rows}")


@pytest.mark.parametrize("case", range(N_CASES))
def test_paged_prefill_random(case):
    rng = np.random.default_rng(7000 + case)
    h_kv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 4, 6]))
    page = int(rng.choice([16, 32, 64, 128]))
    causal = bool(rng.integers(2))
    c = make_chunked_prefill(int(rng.integers(1, 7)), h_kv * g, h_kv, 128, str(rng.choice(["bf16", "f16"])),
                             seed=8000 + case, ctx_range=(1, int(rng.integers(2, 700))),
                             new_range=(1, int(rng.integers(1, 200))), page_size=page,
                             spare_pages=int(rng.integers(0, 4)))
    _run_paged_prefill(c, causal, host_order=bool(rng.integers(2)))


@pytest.mark.parametrize("case", range(N_CASES))
def test_decode_random(case):
    rng = np.random.default_rng(9000 + case)
    h_kv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 4, 8, 16, 17, 24, 32, 40, 64, 128]))
    g = min(g, 256 // h_kv)
    paged = bool(rng.integers(2))
    page = int(rng.choice([16, 32, 48, 64]))
    dtype = str(rng.choice(["bf16", "f16"]))
    lens = rng.integers(0, 1500, size=int(rng.integers(1, 6)))
    lens[rng.random(lens.size) < 0.15] = 0
    dec = make_decode(B=lens.size, h=h_kv * g, h_kv=h_kv, d=128, dtype=dtype, seed=10000 + case,
                      seq_lens=lens.tolist(), paged=paged, page_size=page, spare_pages=2)
    plan = None
    if rng.integers(2):
        chunk = 16 * int(rng.integers(1, 80))
        need = max(1, -(-int(lens.max()) // chunk))
        plan = (chunk, int(rng.integers(max(1, need // 2), need + 1)))   # fewer splits: the last takes the rest
    o_ref, lse_ref = decode_ref(dec["q"], dec["k_seqs"], dec["v_seqs"], dec["seq_lens"], dec["scale"])
    one_call = bool(np.random.default_rng(9500 + case).integers(2))    # attn_decode, or split + merge
    o, lse, used = run_decode(dec, plan, one_call)
    assert_outputs(o, lse, o_ref, lse_ref, dtype,
                   f"random decode {case}: h={h_kv * g}/{h_kv} paged={paged} P={page} lens={lens.tolist()} plan={used} "
                   f"one_call={one_call}")
