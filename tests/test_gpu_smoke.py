"""The entry point's smoke run (quantize, dequant, GEMV with k slices, GEMM
on a 256 x 512 dyadic weight against the oracle) as a GPU test."""

import pytest

pytestmark = pytest.mark.gpu


def test_graft_entry_smoke():
    import __graft_entry__
    __graft_entry__.smoke()
