"""The CPU oracle against what the pages and the mathematics fix (no GPU)."""
import pytest

import pins


@pytest.mark.parametrize("check", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(oracle_impl, check):
    check(oracle_impl)


def test_oracle_rejects_bad_arguments(oracle_impl):
    import numpy as np

    with pytest.raises(ValueError):
        oracle_impl.topk_mask_shape(-1, 1, 1)
    idx = np.zeros((1, 2, 3), dtype=np.int32)
    with pytest.raises(ValueError):  # words too small for key_len
        oracle_impl.topk_mask_build(idx, 200, words=4)
    with pytest.raises(ValueError):  # reserved word would overlap a bit word
        oracle_impl.topk_mask_build(idx, 128, key_starts=np.zeros(1, dtype=np.int32), words=4)
