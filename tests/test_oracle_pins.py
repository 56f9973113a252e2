"""The oracle against what the pages and mathematics fix (CPU only)."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(oracle_lib, pin):
    pin()


def test_dilution_rows_in_batches_match_row_by_row(oracle_lib):
    """When one head is spread over the host threads, the oracle takes the
    dilution rows in batches (bids row by row, shares key by key, sums in key
    order); with enough heads each thread walks its head one row at a time.
    Both forms evaluate the same expression per (row, key) pair and sum in the
    same order, so the results are the same bits (T = 300: several batches and
    a ragged last one)."""
    import numpy as np

    from transformer_attention_causal_amd.workloads import draw_qkv

    H = max(2, oracle_lib.num_threads())
    inp = draw_qkv(1, H, 300, 64, "bf16", seed=11, heavy_frac=0.05)
    q, k, v = (oracle_lib.Bf16(x) for x in (inp.q, inp.k, inp.v))
    for eps in (1e-6, 0.0):
        out, lse, dem = oracle_lib.dilution_fwd(q, k, v, 1.0, eps)
        for h in (0, H - 1):
            o1, l1, d1 = oracle_lib.dilution_fwd(q, k, v, 1.0, eps, heads=[h])
            assert np.array_equal(o1[:, h], out[:, h])
            assert np.array_equal(l1[:, h], lse[:, h])
            assert np.array_equal(d1[:, h], dem[:, h])
