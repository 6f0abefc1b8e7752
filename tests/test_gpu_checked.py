"""Parity cases run again through libattn_checked.so, the debug build of the
same sources whose kernels test every global access not made through a
range-checked buffer resource (and every buffer range they build) against
the extent of its tensor, computed from the call's sizes (include/attn.h,
attn_check_report). Each case keeps its own checks against the oracle; on
top, no access site may have failed its test.

The cases are called from their modules (test_gpu_parity, test_gpu_fp8kv,
test_zz_no_alloc) so that pytest does not collect them twice. They cover
every kernel and launch form: contiguous and paged prefill (masks, tile
lists, the bf16 pass, pools either side of 4 GB), the split-KV decode in
all its forms (16-head blocks, heads as rows, 8-bit K/V, pools either side
of 4 GB), the merges, the gather, the no-allocation entry point and the
stream read.
"""

import pytest
import torch

from online_softmax_tiled_amd import api
from tests import test_gpu_fp8kv as F8
from tests import test_gpu_parity as P
from tests import test_zz_no_alloc as NA

pytestmark = pytest.mark.gpu


def test_checker_flags_an_address_past_the_extent():
    # the checker's own test: an address inside a 64-byte extent (site 62)
    # and one past it (site 63), tested on the device and not accessed
    x = torch.zeros(64, dtype=torch.uint8, device=P.DEV)
    with api.checked_library():
        assert "bounds checks" in api.version()
        api.check_clear()
        assert api.check_report() == []
        api.check_selftest(x)
        assert api.check_report() == [63]
        api.check_clear()
        assert api.check_report() == []


CASES = [
    ("prefill_tiny", lambda: P.test_prefill_tiny_config()),
    ("prefill_gqa_bottom_right", lambda: P.test_prefill_shapes(1, 8, 4, 64, 200, "bf16", True)),
    ("prefill_ragged_f16", lambda: P.test_prefill_shapes(2, 4, 1, 130, 257, "f16", False)),
    ("prefill_masks_empty_rows", lambda: P.test_prefill_masks_and_empty_rows("bf16")),
    ("prefill_tile_list", lambda: P.test_prefill_skips_fully_masked_tiles("bf16", True)),
    ("prefill_walk_all_tiles", lambda: P.test_prefill_key_mask_longer_than_tile_list()),
    ("prefill_all_keys_masked", lambda: P.test_prefill_all_keys_masked()),
    ("prefill_stress_reduced", lambda: P.test_prefill_stress_config_reduced()),
    ("prefill_bf16_pass", lambda: P.test_bf16_values_beyond_fp16_range_take_the_bf16_pass()),
    ("paged_prefill_16", lambda: P.test_paged_prefill_small("bf16", 16, True, False)),
    ("paged_prefill_32_order", lambda: P.test_paged_prefill_small("f16", 32, True, True)),
    ("paged_prefill_edges", lambda: P.test_paged_prefill_edge_sequences()),
    ("paged_prefill_pool_under_4gb", lambda: P.test_paged_prefill_large_pools("under_4gb")),
    ("paged_prefill_pool_over_4gb", lambda: P.test_paged_prefill_large_pools("over_4gb")),
    ("gather_48", lambda: P.test_paged_gather_bit_exact(48, 1)),
    ("gather_16_spare", lambda: P.test_paged_gather_bit_exact(16, 5)),
    ("merge_oracle_partials", lambda: P.test_merge_on_oracle_partials()),
    ("merge_many_splits", lambda: P.test_merge_many_splits(256)),
    ("merge_many_splits_loop", lambda: P.test_merge_many_splits(700)),
    ("decode_contiguous", lambda: P.test_decode_small(False, 16, "bf16", True)),
    ("decode_paged_32", lambda: P.test_decode_small(True, 32, "f16", False)),
    ("decode_no_keys", lambda: P.test_decode_no_keys_at_all(64)),
    ("decode_70b_tp8", lambda: P.test_decode_70b_tp8_s32768()),
    ("decode_moving_reference", lambda: P.test_decode_reference_moves_mid_split(True, "bf16", (1024, 3))),
    ("decode_rows_paged_32", lambda: P.test_decode_head_rows("bf16", True, 32, [None, (208, 8)])),
    ("decode_head_mode_48", lambda: P.test_decode_head_rows("bf16", True, 48, [None, (96, 16)])),
    ("decode_rows_pool_under_4gb", lambda: P.test_decode_head_rows_large_pools("under_4gb")),
    ("decode_rows_pool_over_4gb", lambda: P.test_decode_head_rows_large_pools("over_4gb")),
    ("decode_g256_all_compute", lambda: P.test_decode_large_groups(256, 1, False, 16)),
    ("decode_g80_head_mode", lambda: P.test_decode_large_groups(160, 2, True, 48)),
    ("merge_lse_cascade", lambda: P.test_merge_lse_cascade_prefix_suffix("bf16", 300, 128)),
    ("merge_lse_empty_sides", lambda: P.test_merge_lse_against_oracle_with_empty_sides("bf16", 17)),
    ("stream_read", lambda: P.test_stream_read_reads_every_word_once()),
    ("fp8_decode_paged", lambda: F8.test_fp8kv_decode_small(True, 16, "bf16", True)),
    ("fp8_decode_moving_reference", lambda: F8.test_fp8kv_decode_reference_moves_mid_split(False, (1024, 3))),
    ("fp8_decode_rows_paged", lambda: F8.test_fp8kv_decode_heads_as_rows(32, "paged16")),
    ("fp8_decode_rows_contiguous", lambda: F8.test_fp8kv_decode_heads_as_rows(128, "contiguous")),
    ("fp8_decode_pool_under_4gb", lambda: F8.test_fp8kv_decode_rows_large_pools("under_4gb")),
    ("fp8_decode_pool_over_4gb", lambda: F8.test_fp8kv_decode_rows_large_pools("over_4gb")),
    ("fp8_decode_head_mode", lambda: F8.test_fp8kv_decode_large_groups(160, 1, True, 48)),
    ("decode_noalloc", lambda: NA.test_decode_noalloc_matches_attn_decode_on_successive_calls()),
]


@pytest.mark.parametrize("case", [c[1] for c in CASES], ids=[c[0] for c in CASES])
def test_no_access_outside_its_tensor(case):
    with api.checked_library():
        api.check_clear()
        case()
        hits = api.check_report()
    assert hits == [], f"accesses that failed their bounds test, at sites {hits} (include/attn.h, CheckSite)"
