"""CPU checks of the parity rules' f16 query-rounding term (oracle/compare.py)."""
import numpy as np
import torch

from oracle.compare import f16_query_rounding


def test_no_rounding_for_ordinary_queries():
    g = torch.Generator().manual_seed(0)
    iq = torch.randn(4, 128, generator=g, dtype=torch.float64).to(torch.bfloat16).to(torch.float64)
    assert (f16_query_rounding(iq) == 0).all()


def test_scaled_vectors_keep_every_element_within_range():
    # largest 3 -> scale 2^13; 2^-20 -> 2^-7 exact; 2^-40 -> 2^-27 is an f16
    # subnormal (counted whole); a 1.5 x 2^20 vector scales down instead of
    # overflowing (bf16 inputs: 8 significant bits, exact in f16 once in range)
    x = torch.zeros(3, 128, dtype=torch.float64)
    x[0, :3] = torch.tensor([3.0, 2.0 ** -20, -(2.0 ** -40)])
    x[1, :2] = torch.tensor([1.5 * 2.0 ** 20, 3.0])
    x[2] = 0.0
    r = f16_query_rounding(x).numpy()
    assert r[0, 0] == 0 and r[0, 1] == 0 and r[0, 2] == 2.0 ** -40
    assert r[1, 0] == 0 and r[1, 1] == 0 and np.isfinite(r).all()
    assert (r[2] == 0).all()
