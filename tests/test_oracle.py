"""The oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle_pins as pins
from oracle import attention, brute


def test_hand_cases():
    pins.pin_hand_cases(attention.forward, attention.backward)


@pytest.mark.parametrize("pin", pins.FORWARD_PINS, ids=lambda p: p.__name__)
def test_forward_pin(pin):
    pin(attention.forward)


def test_torch_backward():
    pins.pin_torch_backward(attention.backward)


def test_finite_differences():
    pins.pin_finite_differences(attention.forward, attention.backward)


def test_backward_identities():
    pins.pin_backward_identities(attention.backward)


def test_torch_gqa():
    pins.pin_torch_gqa(attention.forward, attention.backward)


def test_gqa_matches_copied_heads():
    pins.pin_gqa_matches_copied_heads(attention.forward, attention.backward)


def test_gqa_rejects_bad_groups():
    q = np.zeros((1, 4, 3, 2))
    with pytest.raises(ValueError):
        attention.forward(q, np.zeros((1, 3, 3, 2)), np.zeros((1, 3, 3, 2)), False, 1.0)


def test_torch_lower_right():
    pins.pin_torch_lower_right(attention.forward, attention.backward)


def test_window_closed_forms():
    pins.pin_window_closed_forms(attention.forward)


def test_window_equals_key_slice():
    pins.pin_window_equals_key_slice(attention.forward)


def test_brute_force_masks():
    pins.pin_brute_force_masks(attention.forward, attention.backward, brute)


def test_finite_differences_masks():
    pins.pin_finite_differences_masks(attention.forward, attention.backward)


def test_empty_rows():
    pins.pin_empty_rows(attention.forward, attention.backward)


def test_varlen_padded():
    pins.pin_varlen_padded(attention.forward_varlen, attention.backward_varlen)


def test_varlen_rejects_bad_offsets():
    q = np.zeros((5, 1, 2))
    for cu_k in ([0, 5], [0, 6, 5], [1, 3, 5], [0, 2, 4], [0, 3, 2, 5]):
        with pytest.raises(ValueError):
            attention.forward_varlen(q, q, q, [0, 2, 5], cu_k, False, 1.0)


def test_brute_force():
    pins.pin_brute_force(attention.forward, attention.backward, brute)


def test_softmax_rows_sum_to_one():
    s = np.random.default_rng(0).standard_normal((64, 300)) * 10
    s[:, 7] = -np.inf
    p, lse = attention.softmax_rows(s)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=1e-14)
    assert (p[:, 7] == 0).all()
    np.testing.assert_allclose(lse, np.log(np.exp(np.where(np.isinf(s), -np.inf, s)).sum(axis=1)), rtol=1e-13)


def test_row_subset_matches_full():
    rng = np.random.default_rng(1)
    q, k, v = (rng.standard_normal((2, 2, 300, 8)) for _ in range(3))
    rows = np.array([0, 1, 5, 100, 299])
    for causal in (False, True):
        o, lse = attention.forward(q, k, v, causal, 0.35)
        o_s, lse_s = attention.forward(q, k, v, causal, 0.35, rows=rows)
        np.testing.assert_allclose(o_s, o[:, :, rows], atol=1e-14)
        np.testing.assert_allclose(lse_s, lse[:, :, rows], atol=1e-14)


def test_block_mask_all_true():
    pins.pin_block_mask_all_true(attention.forward, attention.backward)


def test_block_mask_torch():
    pins.pin_block_mask_torch(attention.forward, attention.backward)


def test_block_mask_drops_keys():
    pins.pin_block_mask_drops_keys(attention.forward)


def test_block_mask_brute():
    pins.pin_block_mask_brute(attention.forward, attention.backward, brute)


def test_dq_rows_brute():
    pins.pin_dq_rows_brute(attention.backward_dq_rows, brute)


def test_dq_rows_torch():
    pins.pin_dq_rows_torch(attention.backward_dq_rows)


def test_kv_rows_brute():
    pins.pin_kv_rows_brute(attention.backward_kv_rows, brute)


def test_kv_rows_torch():
    pins.pin_kv_rows_torch(attention.backward_kv_rows)
