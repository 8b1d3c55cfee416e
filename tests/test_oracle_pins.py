"""The float64 oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle
from tests import oracle_pins as pins


def fwd(q, k, v, scale, causal, cu):
    return oracle.attention_forward(q, k, v, scale, causal, cu)


def bwd(q, k, v, do, scale, causal, cu):
    return oracle.attention_backward(q, k, v, do, scale, causal, cu)


@pytest.mark.parametrize("pin", pins.ALL_FWD_PINS, ids=lambda f: f.__name__)
def test_forward_pins(pin):
    pin(fwd, bwd)


@pytest.mark.parametrize("pin", [pins.pin_finite_differences, pins.pin_gradient_invariants],
                         ids=lambda f: f.__name__)
def test_backward_pins(pin):
    pin(fwd, bwd)


def test_row_subset_is_exact():
    """Rows computed alone equal the same rows of the full computation."""
    rng = np.random.default_rng(3)
    q, k, v = rng.standard_normal((1, 40, 2, 8)), rng.standard_normal((1, 40, 1, 8)), rng.standard_normal((1, 40, 1, 8))
    o, lse = oracle.attention_forward(q, k, v, 0.3, True, None)
    rows = np.array([0, 5, 39])
    o2, lse2 = oracle.attention_forward(q, k, v, 0.3, True, None, rows=lambda s, L: rows)
    assert np.array_equal(o2[:, rows], o[:, rows])
    assert np.array_equal(lse2[:, :, rows], lse[:, :, rows])
    others = np.setdiff1d(np.arange(40), rows)
    assert np.all(np.isnan(o2[:, others])) and np.all(np.isnan(lse2[:, :, others]))


def test_backward_rowdot_against_softmax_identity():
    pins.pin_rowdot(oracle.backward_rowdot)


def test_empty_sequence_is_skipped():
    rng = np.random.default_rng(5)
    cu = np.array([0, 3, 3, 5], dtype=np.int32)
    q, k, v = rng.standard_normal((5, 2, 4)), rng.standard_normal((5, 1, 4)), rng.standard_normal((5, 1, 4))
    o, lse = oracle.attention_forward(q, k, v, 0.5, True, cu)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    dq, dk, dv = oracle.attention_backward(q, k, v, rng.standard_normal((5, 2, 4)), 0.5, True, cu)
    assert np.all(np.isfinite(dq)) and np.all(np.isfinite(dk)) and np.all(np.isfinite(dv))



def test_dq_rows_match_torch_autograd():
    """The row-sampled dQ equals PyTorch fp64 autograd's dQ on those rows."""
    pins.pin_dq_rows(oracle.head_backward_dq_rows)


def test_split_and_merge_pins():
    pins.pin_split(oracle.attention_forward_split, oracle.merge_partials)


def test_fp8_pins():
    pins.pin_fp8(oracle.attention_forward_fp8, oracle.e4m3_to_float)


def test_pin_fp8_blocks():
    pins.pin_fp8_blocks(oracle.attention_forward_fp8)
