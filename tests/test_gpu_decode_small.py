"""The decode path at one and two tokens on layers whose products both have
whole 128-feature K-blocks (M and R above 96, four packed words per row per
tile), against the fp64 oracle.

These shapes cover what the decode kernel's indexing depends on at small
token counts: N not a multiple of 16 or 64 (a partial row tile), R and M not
multiples of 16, 64 or 128 (ragged last K-block, zero pad bits), M not a
multiple of 4 (element-wise activation loads), several passes per product
(more than 2048 features or ranks), K-splits of the first product, several
terms, both token counts, and the configurations at one and two tokens."""
import numpy as np
import pytest
import torch

import bit_adapters_amd as D
import oracle as O
from bit_adapters_amd import synth as S
from dbfutil import (DEV, assert_close, assert_close_bf16, device_terms, to_np, x64,
                     x_dev)

pytestmark = pytest.mark.gpu

DEC = D.DBF_PATH_DECODE

SHAPES = [(17, 97, 97, 1, 1), (100, 300, 130, 2, 2), (4100, 2100, 2050, 1, 1),
          (333, 5001, 700, 3, 2), (8191, 4099, 2047, 1, 2), (257, 4096, 2048, 8, 1),
          (1000, 129, 4500, 2, 1), (48, 20000, 160, 1, 2)]


@pytest.mark.parametrize("N,M,R,L,T", SHAPES)
@pytest.mark.parametrize("xk", ["bf16", "f16"])
def test_shapes(N, M, R, L, T, xk):
    print("decode", N, M, R, L, T, xk, flush=True)
    layer, x = S.make_custom(N, M, R, L, T, seed=N + 2 * M + 3 * R + L, x_kind=xk)
    terms = device_terms(layer)
    y = D.dbf_linear_forward(terms, N, M, R, x_dev(x), path=DEC)
    torch.cuda.synchronize()
    ref = O.default().forward(O.terms64(layer), x64(x))
    assert_close(to_np(y), ref)


@pytest.mark.parametrize("config,T", [(1, 2), (2, 2), (4, 2), (5, 1), (5, 2)])
def test_configs(config, T):
    print("decode config", config, "T", T, flush=True)
    layer = S.make_layer(config)
    x = S.make_x(config, T)
    y = D.dbf_linear_forward(device_terms(layer), layer["N"], layer["M"], layer["R"], x_dev(x),
                             path=D.DBF_PATH_AUTO)
    torch.cuda.synchronize()
    ref = O.default().forward(O.terms64(layer), x64(x))
    assert_close(to_np(y), ref, what="config %d T %d" % (config, T))


@pytest.mark.parametrize("T", [1, 2])
def test_dtypes_accumulate_strides_determinism(T):
    N, M, R, L = 301, 1000, 200, 2
    layer, x = S.make_custom(N, M, R, L, T, seed=44 + T)
    ref = O.default().forward(O.terms64(layer), x64(x))
    terms = device_terms(layer)
    xd = torch.zeros((T, 1008), dtype=torch.bfloat16, device=DEV)
    xd[:, :M] = x_dev(x)
    xs = xd[:, :M]  # ldx = 1008
    nb = D.dbf_workspace_bytes(N, M, R, L, T, DEC)
    ws = torch.zeros(nb, dtype=torch.uint8, device=DEV)
    big = torch.full((T, 320), 7.0, dtype=torch.float32, device=DEV)
    D.dbf_linear_forward(terms, N, M, R, xs, y=big[:, :N], ws=ws, path=DEC)
    torch.cuda.synchronize()
    assert_close(to_np(big[:, :N]), ref)
    assert torch.all(big[:, N:] == 7.0)
    first = big[:, :N].clone()
    base = torch.randn((T, N), dtype=torch.float32, device=DEV)
    y2 = base.clone()
    D.dbf_linear_forward(terms, N, M, R, xs, y=y2, accumulate=True, ws=ws, path=DEC)
    torch.cuda.synchronize()
    assert_close(to_np(y2), ref + to_np(base))
    for dt in (torch.bfloat16, torch.float16):
        yb = D.dbf_linear_forward(terms, N, M, R, xs, y_dtype=dt, ws=ws, path=DEC)
        torch.cuda.synchronize()
        if dt == torch.bfloat16:
            assert_close_bf16(to_np(yb), ref)
        else:
            assert_close(to_np(yb), ref)
    # bitwise reproducible, and the workspace head is left zero
    for _ in range(3):
        D.dbf_linear_forward(terms, N, M, R, xs, y=big[:, :N], ws=ws, path=DEC)
        D.dbf_workspace_check(ws)
        assert torch.equal(big[:, :N], first)
        assert not ws[:D.DBF_WS_HEAD_BYTES].any()


def test_row_flip():
    # flipping every sign of row 77 of B1 negates output 77 exactly and
    # leaves the other outputs bit for bit
    layer, x = S.make_custom(200, 600, 300, 1, 1, seed=9)
    y = to_np(D.dbf_linear_forward(device_terms(layer), 200, 600, 300, x_dev(x), path=DEC))
    layer["terms"][0]["b1"][77, :] *= -1
    y2 = to_np(D.dbf_linear_forward(device_terms(layer), 200, 600, 300, x_dev(x), path=DEC))
    torch.cuda.synchronize()
    rest = [n for n in range(200) if n != 77]
    assert np.array_equal(y2[:, rest], y[:, rest])
    assert np.array_equal(y2[:, 77], -y[:, 77])
