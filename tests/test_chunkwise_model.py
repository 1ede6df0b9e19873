"""The chunk / superchunk algebra of the HIP kernels, modelled in fp64 numpy
(tests/chunkwise_model.py), equals the sequential oracle for any chunk size,
superchunk size, ragged tail, block count and initial state."""
import numpy as np
import pytest

import oracle
from chunkwise_model import chunkwise
from test_oracle_pins import RNG, _inputs, _relerr, _state


@pytest.mark.parametrize("T,L,G", [(1, 64, 4), (60, 64, 4), (64, 16, 1), (200, 16, 3),
                                   (333, 32, 2), (257, 64, 1), (130, 7, 5)])
@pytest.mark.parametrize("nb", [1, 2])
@pytest.mark.parametrize("with_state", [False, True])
def test_chunkwise_equals_oracle(T, L, G, nb, with_state):
    rng = RNG(T * 7 + L + G + nb)
    B, H, dqk, dv = 1, 2, 8, 12
    q, k, v, ip, fp, op, bs = _inputs(rng, B, H, T, dqk, dv)
    st = _state(rng, B, H, dqk, dv, nb) if with_state else (None, None, None)
    ref = oracle.mlstm_fwd(q, k, v, ip, fp, op, bs, *st, num_blocks=nb)
    got = chunkwise(q, k, v, ip, fp, op, bs, *st, nb=nb, L=L, G=G)
    assert _relerr(got[0], ref[0]) < 1e-12
    assert _relerr(got[1], ref[1]) < 1e-12
    assert _relerr(got[2], ref[2]) < 1e-12
    assert np.max(np.abs(got[3] - ref[3])) < 1e-12


def test_chunkwise_retention_no_normaliser():
    rng = RNG(99)
    B, H, T, d = 2, 4, 150, 6
    q, k, v = (rng.standard_normal((B, H, T, d)) for _ in range(3))
    g = 1.0 - 2.0 ** (-5.0 - np.arange(H))
    fp = np.broadcast_to(np.log(g / (1 - g))[None, :, None], (B, H, T)).copy()
    got = chunkwise(q, k, v, np.zeros((B, H, T)), fp, nb=1, L=16, G=3, normalise=False)
    out, S = oracle.retention_fwd(q, k, v)
    assert _relerr(got[0], out) < 1e-12
    assert _relerr(got[1][:, :, 0], S) < 1e-12
