"""Plant plausible mistakes in the oracle (on the CPU) and check that at least
one pin catches each of them: evidence that the pins constrain the oracle."""

import numpy as np
import pytest

import oracle.paged_attention as ora
from tests import test_oracle as pins


def _wrong_offset(table_row, t, bs):
    return int(table_row[t // bs]), (t + 1) % bs


def _bf16_bad_shift(bits, dtype, _orig=ora.to_f64):
    if dtype == "bf16":
        a = np.asarray(bits)
        return (a.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)
    return _orig(bits, dtype)


def _interleaved_heads(h, num_q_heads, num_kv_heads):
    return h % num_kv_heads


def _unnormalised(scores):
    return np.exp(scores - scores.max())


def _no_shift_wrong_sign(scores):
    w = np.exp(-(scores - scores.max()))
    return w / w.sum()


def _reads_whole_last_block(cache, table_row, kv_head, start, stop, bs, dtype,
                            _orig=ora.gather_rows):
    """Masks the last block's tail by multiplying it by zero instead of
    leaving it out (NaN * 0 is NaN)."""
    rows = _orig(cache, table_row, kv_head, start, stop, bs, dtype)
    if stop % bs == 0 or stop <= start:
        return rows
    tail = cache[int(table_row[(stop - 1) // bs]), kv_head, stop % bs:]
    return rows + 0.0 * ora.to_f64(tail, dtype).sum()


def _copy_k_only(k_cache, v_cache, block_pairs):
    kc = np.array(k_cache, copy=True)
    for src, dst in block_pairs:
        if src >= 0 and dst >= 0:
            kc[dst] = kc[src]
    return kc, np.array(v_cache, copy=True)


def _copy_swapped(k_cache, v_cache, block_pairs, _orig=ora.copy_blocks):
    return _orig(k_cache, v_cache, [(d, s) for s, d in block_pairs])


def _causal_off_by_one(L, T, j):
    return max(0, L - T + j)


def _not_causal(L, T, j):
    return max(0, L)


MUTANTS = {
    "multi_mask_off_by_one": ("query_context_len", _causal_off_by_one),
    "multi_not_causal": ("query_context_len", _not_causal),
    "cow_copies_k_only": ("copy_blocks", _copy_k_only),
    "cow_src_dst_swapped": ("copy_blocks", _copy_swapped),
    "offset_off_by_one": ("physical_slot", _wrong_offset),
    "bf16_decode_shift": ("to_f64", _bf16_bad_shift),
    "gqa_interleaved": ("kv_head_of", _interleaved_heads),
    "softmax_not_normalised": ("softmax_weights", _unnormalised),
    "softmax_sign_flip": ("softmax_weights", _no_shift_wrong_sign),
    "reads_tail_slots": ("gather_rows", _reads_whole_last_block),
}

PIN_CHECKS = [
    pins.test_decode_bf16_bit_patterns,
    pins.test_golden_block_table_examples,
    lambda: pins.test_paged_equals_dense_sdpa(8, 2, 16),
    lambda: pins.test_paged_equals_dense_sdpa(8, 1, 1),
    pins.test_brute_force_tiny,
    pins.test_probabilities_sum_to_one,
    pins.test_gqa_mapping_contiguous_groups,
    pins.test_poison_in_unread_slots_does_not_leak,
    pins.test_bf16_storage_path_equals_upcast_f32,
    pins.test_copy_blocks_bytes_and_untouched_blocks,
    pins.test_copy_on_write_flow_equals_private_copies,
    lambda: pins.test_multi_equals_dense_causal_sdpa(3, 8, 2),
    pins.test_multi_brute_force_tiny,
    pins.test_multi_is_causal_among_new_tokens,
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(ora, attr, fn)
    caught = []
    for check in PIN_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check()
        except AssertionError:
            caught.append(check)
    # a pin must fail on a wrong value, not merely crash
    assert caught, f"no pin caught the planted mistake {name!r}"


def test_unmutated_oracle_passes_every_check():
    for check in PIN_CHECKS:
        check()
