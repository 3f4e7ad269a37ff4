"""CPU checks of the element band the GPU parity tests apply: bf16-sized
rounding passes, including in rows far above the average magnitude, while a
wrong tile or a wrong row fails."""
import numpy as np
import pytest
import torch

from parity_util import band_scale, compare


def _bf16(x):
    return torch.from_numpy(x).to(torch.bfloat16).double().numpy()


def _ref():
    rng = np.random.default_rng(0)
    r = rng.standard_normal((2048, 1024))
    r[0] *= 13.0  # one row far above the average, like the first token's gradient
    return r


def test_rounding_passes_in_every_row():
    r = _ref()
    compare("rounded", _bf16(r), r, "bf16", verbose=False)


def test_wrong_tile_fails():
    r = _ref()
    g = _bf16(r)
    rng = np.random.default_rng(1)
    # one 32 x 32 tile off by 0.3 of the rms (say a missing k-part): the
    # Frobenius norm over the matrix stays under the bar, the band does not
    g[256:288, 160:192] += 0.3 * rng.standard_normal((32, 32))
    with pytest.raises(AssertionError, match="out of bound"):
        compare("wrong_tile", g, r, "bf16", verbose=False)


def test_wrong_big_row_fails():
    r = _ref()
    g = _bf16(r)
    g[0] = -g[0]  # the large row with a sign error
    with pytest.raises(AssertionError):
        compare("wrong_row", g, r, "bf16", verbose=False)


def test_small_rows_keep_the_global_floor():
    r = _ref()
    sc = band_scale(r)
    assert sc.shape == (2048, 1)
    assert np.all(sc >= np.sqrt(np.mean(r * r)) - 1e-15)
    assert sc[0, 0] > 5 * np.sqrt(np.mean(r * r))
