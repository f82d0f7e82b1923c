"""The oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle.attention as A
from oracle_pins import PINS, f64_case, run, close


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


def test_row_blocking_changes_nothing():
    """Materialising the score block in row slices changes nothing beyond the
    last bit (rows are independent; BLAS may round a slice's products in a
    different order)."""
    c = f64_case(201, 2, 2, 37, 29, 8, causal=True, mask="random")
    O, lse = run(c, row_block=4096)
    for rb in (1, 5, 16):
        O2, lse2 = run(c, row_block=rb)
        close(O2, O, 1e-14, f"O row_block={rb}")
        close(lse2, lse, 1e-14, f"lse row_block={rb}")


def test_sampled_rows_match_full():
    """attention_rows_fp64 (used for sampled checks at full size) equals the
    full evaluation on the rows it is asked for."""
    c = f64_case(202, 2, 3, 41, 33, 8, causal=True, mask="lengths")
    O, lse = run(c)
    picks = [(0, 1, np.array([0, 5, 40])), (1, 2, np.arange(0, 41, 7))]
    got = A.attention_rows_fp64(c["q"], c["k"], c["v"], c["scale"], c["causal"], c["kpm"], picks)
    for (b, h, rows), (o, l) in zip(picks, got):
        close(o, O[b, h, rows], 1e-15, "rows O")
        close(l, lse[b, h, rows], 1e-15, "rows lse")


def test_shape_errors():
    c = f64_case(203, 1, 1, 4, 4, 4)
    with pytest.raises(ValueError):
        A.attention_fp64(c["q"], c["k"][..., :2], c["v"], c["scale"])
    with pytest.raises(ValueError):
        A.attention_fp64(c["q"], c["k"], c["v"], c["scale"], key_padding_mask=np.zeros((2, 4), np.uint8))
