"""dbf_linear_forward_i8: exact int32 sign sums against the oracle."""
import numpy as np
import pytest
import torch

import bit_adapters_amd as D
import oracle as O
from bit_adapters_amd import synth as S
from dbfutil import DEV, assert_close, device_terms, to_np

pytestmark = pytest.mark.gpu


def _run(layer, xq, with_beta, with_alpha=True, want_s2=False):
    N, M, R, L = layer["N"], layer["M"], layer["R"], len(layer["terms"])
    T = xq.shape[0]
    terms = device_terms(layer, gamma=False, alpha=with_alpha, beta=with_beta)
    xd = torch.from_numpy(xq).to(DEV)
    s1 = torch.empty((L, T, R), dtype=torch.int32, device=DEV)
    s2 = torch.empty((L, T, N), dtype=torch.int32, device=DEV) if want_s2 else None
    y = torch.empty((T, N), dtype=torch.float32, device=DEV)
    D.dbf_linear_forward_i8(terms, N, M, R, xd, s1=s1, s2=s2, y=y)
    torch.cuda.synchronize()
    return s1.cpu().numpy(), (s2.cpu().numpy() if want_s2 else None), to_np(y)


def test_config1_int8_with_scales():
    layer = S.make_layer(1)
    xq = S.make_x(1, 1, "i8")
    s1, _, y = _run(layer, xq, with_beta=True)
    r1, _ = O.default().forward_int(layer["terms"], xq)
    assert np.array_equal(s1, r1)
    terms = O.terms64(layer)
    for t in terms:
        t["gamma"] = np.ones_like(t["gamma"])
    ref = O.default().forward(terms, xq.astype(np.float64))
    assert_close(y, ref)


def test_config1_int8_unit_scales_bit_exact():
    layer = S.make_layer(1)
    xq = S.make_x(1, 1, "i8")
    s1, s2, y = _run(layer, xq, with_beta=False, with_alpha=False, want_s2=True)
    r1, r2 = O.default().forward_int(layer["terms"], xq)
    assert np.array_equal(s1, r1)
    assert np.array_equal(s2, r2)
    # |S2| < 2^24 here, so y = float(S2) is exact as well
    assert np.abs(r2).max() < 2 ** 24
    assert np.array_equal(y, r2.sum(axis=0).astype(np.float64))


@pytest.mark.parametrize("N,M,R,L,T", [(65, 33, 17, 2, 3), (130, 300, 70, 3, 5),
                                       (1, 1, 1, 1, 1), (300, 2000, 100, 1, 6)])
def test_odd_shapes_exact(N, M, R, L, T):
    layer, xq = S.make_custom(N, M, R, L, T, seed=5, x_kind="i8")
    s1, s2, _ = _run(layer, xq, with_beta=False, want_s2=True)
    r1, r2 = O.default().forward_int(layer["terms"], xq)
    assert np.array_equal(s1, r1)
    assert np.array_equal(s2, r2)
