"""The fp64 oracle against its pins (CPU only)."""
import pytest

import oracle
import pins


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle.LIB_PATH)


def test_rows_entry_matches_full():
    import numpy as np
    import torch
    g = torch.Generator().manual_seed(21)
    q = torch.randn(3, 4, 8, 64, generator=g).to(torch.bfloat16)
    k = torch.randn(3, 50, 2, 64, generator=g).to(torch.bfloat16)
    v = torch.randn(3, 50, 2, 64, generator=g).to(torch.bfloat16)
    sl = np.array([50, 3, 17], np.int32)
    o, l = oracle.attention(q, k, v, sl, True)
    rows = [(b, h, i) for b in range(3) for h in range(8) for i in range(4)]
    orow, lrow = oracle.attention_rows(q, k, v, rows, sl, True)
    for r, (b, h, i) in enumerate(rows):
        assert np.array_equal(orow[r], o[b, i, h])
        assert lrow[r] == l[b, h, i] or (np.isneginf(lrow[r]) and np.isneginf(l[b, h, i]))


def test_rejects_bad_arguments():
    import torch
    q = torch.zeros(1, 1, 3, 8, dtype=torch.float16)
    k = torch.zeros(1, 4, 2, 8, dtype=torch.float16)
    with pytest.raises(ValueError):
        oracle.attention(q, k, k)          # Hq % Hkv != 0
    with pytest.raises(ValueError):
        oracle.attention_rows(q[:, :, :2].contiguous(), k, k, [(0, 5, 0)])
