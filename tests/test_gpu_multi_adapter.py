"""lordba_multi_adapter_forward (several LoRDBA adapters beside one bf16
base, one adapter per token) against the oracle.  As in the single-adapter
tests, the adapter part is also checked with W0 = 0, since it is ~1e-4 of y
in the LoRDBA-sized layer."""
import numpy as np
import pytest
import torch

import bit_adapters_amd as D
import oracle as O
from bit_adapters_amd import synth as S
from dbfutil import DEV, assert_close, bf16_dev, device_terms, to_np, x64, x_dev

pytestmark = pytest.mark.gpu


def _setup(N, M, R, K, T, seed, lo=0.01, hi=0.05):
    ads = [S.make_custom(N, M, R, 1, 1, seed=seed * 100 + a, scale_lo=lo, scale_hi=hi)[0]
           for a in range(K)]
    layer, x = S.make_custom(N, M, R, 1, T, seed=seed, base=True)
    return ads, layer["w0"], x


def _run(ads, w0, x, idx, N, M, R, zero_w0=False, ws=None):
    adapters = [device_terms(a)[0] for a in ads]
    w = bf16_dev(w0)
    if zero_w0:
        w = torch.zeros_like(w)
    it = torch.tensor(idx, dtype=torch.int32, device=DEV)
    y = D.lordba_multi_adapter_forward(w, adapters, N, M, R, it, x_dev(x), ws=ws)
    torch.cuda.synchronize()
    return to_np(y)


def _ref(ads, w0, x, idx, zero_w0=False):
    o = O.default()
    w = O.widen_bf16(w0)
    if zero_w0:
        w = np.zeros_like(w)
    return o.multi_adapter(w, [O.terms64(a)[0] for a in ads], idx, x64(x))


@pytest.mark.parametrize("N,M,R,K,T", [(4096, 4096, 16, 4, 5), (4096, 4096, 64, 8, 16),
                                       (300, 777, 32, 3, 33), (65, 130, 17, 2, 3),
                                       (1000, 2048, 96, 32, 40), (128, 512, 8, 1, 1)])
def test_multi_adapter(N, M, R, K, T):
    print("multi adapter", N, M, R, K, T, flush=True)
    ads, w0, x = _setup(N, M, R, K, T, seed=N + K)
    g = np.random.default_rng([0xDBF, 107, N, K, T])
    idx = g.integers(-1, K, T).tolist()
    assert_close(_run(ads, w0, x, idx, N, M, R, zero_w0=True), _ref(ads, w0, x, idx, True),
                 what="adapters only")
    assert_close(_run(ads, w0, x, idx, N, M, R), _ref(ads, w0, x, idx), what="with base")


def test_all_base_only_and_deterministic():
    ads, w0, x = _setup(256, 1024, 16, 3, 9, seed=5)
    idx = [-1] * 9
    y = _run(ads, w0, x, idx, 256, 1024, 16)
    assert_close(y, O.default().dense(O.widen_bf16(w0), x64(x)))
    idx = [2, 0, 1, 1, 2, 0, -1, 2, 1]
    a = _run(ads, w0, x, idx, 256, 1024, 16)
    b = _run(ads, w0, x, idx, 256, 1024, 16)
    assert np.array_equal(a, b)


def test_index_out_of_range_is_flagged():
    ads, w0, x = _setup(128, 512, 16, 2, 4, seed=6)
    ws = torch.zeros(D.dbf_workspace_bytes(128, 512, 16, 1, 4, D.DBF_PATH_DECODE),
                     dtype=torch.uint8, device=DEV)
    idx = [0, 5, 1, -3]
    y = _run(ads, w0, x, idx, 128, 512, 16, zero_w0=True, ws=ws)
    with pytest.raises(D.DbfError) as e:
        D.dbf_workspace_check(ws)
    assert e.value.code == D.DBF_EINVAL
    # the flagged tokens got no adapter term; the others are right
    ref = _ref(ads, w0, x, [0, -1, 1, -1], zero_w0=True)
    assert_close(y, ref)
    assert not ws[:D.DBF_WS_HEAD_BYTES].any()
    # the buffer serves the next call again
    y = _run(ads, w0, x, [1, 1, 0, 0], 128, 512, 16, zero_w0=True, ws=ws)
    D.dbf_workspace_check(ws)
    assert_close(y, _ref(ads, w0, x, [1, 1, 0, 0], zero_w0=True))
