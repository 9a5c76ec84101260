"""dbf_linear_forward on the decode path against the fp64 oracle."""
import numpy as np
import pytest
import torch

import bit_adapters_amd as D
import oracle as O
from bit_adapters_amd import synth as S
from dbfutil import (DEV, assert_close, assert_close_bf16, bf16_dev, device_terms, to_np, x64,
                     x_dev)

pytestmark = pytest.mark.gpu

PATH = D.DBF_PATH_DECODE


def run(layer, x, path=PATH, **kw):
    terms = device_terms(layer)
    y = D.dbf_linear_forward(terms, layer["N"], layer["M"], layer["R"], x_dev(x),
                             path=path, **kw)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("config,T", [(1, 1), (2, 1), (2, 4), (2, 16), (4, 1),
                                      (4, 8)])
def test_configs(config, T):
    print("decode config", config, "T", T, flush=True)
    layer = S.make_layer(config)
    x = S.make_x(config, T)
    y = to_np(run(layer, x))
    ref = O.default().forward(O.terms64(layer), x64(x))
    assert_close(y, ref, what="config %d T %d" % (config, T))


ODD = [(1, 1, 1, 1, 1), (65, 33, 17, 2, 3), (130, 300, 70, 3, 5),
       (64, 128, 64, 1, 2), (200, 1000, 96, 1, 16), (77, 129, 33, 2, 7),
       (4096, 64, 16, 1, 2), (33, 4100, 130, 1, 17)]


@pytest.mark.parametrize("N,M,R,L,T", ODD)
@pytest.mark.parametrize("xk", ["bf16", "f16"])
def test_odd_shapes(N, M, R, L, T, xk):
    print("decode odd", N, M, R, L, T, xk, flush=True)
    layer, x = S.make_custom(N, M, R, L, T, seed=N + M + R, x_kind=xk)
    y = to_np(run(layer, x))
    ref = O.default().forward(O.terms64(layer), x64(x))
    assert_close(y, ref)


def test_output_dtypes_accumulate_and_strides():
    layer, x = S.make_custom(96, 200, 40, 2, 5, seed=3)
    ref = O.default().forward(O.terms64(layer), x64(x))
    terms = device_terms(layer)
    xd = torch.zeros((5, 208), dtype=torch.bfloat16, device=DEV)
    xd[:, :200] = x_dev(x)
    xs = xd[:, :200]                                   # ldx = 208
    # fp32 output into a strided view with a guard band
    big = torch.full((5, 100), 7.0, dtype=torch.float32, device=DEV)
    y = big[:, :96]
    D.dbf_linear_forward(terms, 96, 200, 40, xs, y=y, path=PATH)
    torch.cuda.synchronize()
    assert_close(to_np(y), ref)
    assert torch.all(big[:, 96:] == 7.0)
    # accumulate onto a known base
    base = torch.randn((5, 96), dtype=torch.float32, device=DEV)
    y2 = base.clone()
    D.dbf_linear_forward(terms, 96, 200, 40, xs, y=y2, accumulate=True, path=PATH)
    torch.cuda.synchronize()
    assert_close(to_np(y2), ref + to_np(base))
    # bf16 and fp16 outputs, compared with the oracle rounded the same way
    yb = D.dbf_linear_forward(terms, 96, 200, 40, xs, y_dtype=torch.bfloat16, path=PATH)
    torch.cuda.synchronize()
    assert_close_bf16(to_np(yb), ref)
    yh = D.dbf_linear_forward(terms, 96, 200, 40, xs, y_dtype=torch.float16, path=PATH)
    torch.cuda.synchronize()
    assert_close(to_np(yh), ref.astype(np.float16).astype(np.float64))


def test_deterministic():
    layer = S.make_layer(2)
    x = S.make_x(2, 4)
    a = run(layer, x).cpu()
    b = run(layer, x).cpu()
    assert torch.equal(a, b)


def test_zero_tokens():
    layer, _ = S.make_custom(8, 8, 8, 1, 1, seed=1)
    terms = device_terms(layer)
    x = torch.empty((0, 8), dtype=torch.bfloat16, device=DEV)
    y = D.dbf_linear_forward(terms, 8, 8, 8, x, path=PATH)
    assert y.shape == (0, 8)


def test_row_flip_on_gpu():
    # the pages' structure: flipping row n0 of B1 negates output n0 only
    layer, x = S.make_custom(128, 256, 64, 1, 2, seed=11)
    y = to_np(run(layer, x))
    layer["terms"][0]["b1"][5, :] *= -1
    y2 = to_np(run(layer, x))
    np.testing.assert_allclose(y2[:, 5], -y[:, 5], rtol=1e-5, atol=1e-5)
    rest = [n for n in range(128) if n != 5]
    assert np.array_equal(y2[:, rest], y[:, rest])


@pytest.mark.parametrize("N,M,R,L,T", [(256, 4096, 2048, 1, 1), (64, 4096, 64, 1, 1),
                                       (128, 1536, 256, 2, 1), (128, 8192, 512, 1, 2)])
def test_partial_passes(N, M, R, L, T):
    # K-splits shorter than a pass (the last waves of a pass have no block)
    layer, x = S.make_custom(N, M, R, L, T, seed=21)
    y = to_np(run(layer, x))
    ref = O.default().forward(O.terms64(layer), x64(x))
    assert_close(y, ref)


def test_shared_workspace_head_stays_clear():
    # one workspace serves decode, MFMA and adapter (published-intermediate
    # rank path) calls in turn: after each the handoff head is zero again and
    # no wait gave up
    N, M, R, L, T = 200, 1000, 64, 2, 5
    layer, x = S.make_custom(N, M, R, L, T, seed=3, base=True, scale_lo=0.01,
                             scale_hi=0.05)
    terms = device_terms(layer)
    nb = max(D.dbf_workspace_bytes(N, M, R, L, T, p)
             for p in (D.DBF_PATH_DECODE, D.DBF_PATH_MFMA))
    ws = torch.zeros(nb, dtype=torch.uint8, device=DEV)
    o = O.default()
    ref = o.forward(O.terms64(layer), x64(x))
    for path in (D.DBF_PATH_DECODE, D.DBF_PATH_MFMA, D.DBF_PATH_DECODE):
        y = D.dbf_linear_forward(terms, N, M, R, x_dev(x), ws=ws, path=path)
        D.dbf_workspace_check(ws)
        assert not ws[:D.DBF_WS_HEAD_BYTES].any()
        assert_close(to_np(y), ref)
    w0 = bf16_dev(layer["w0"])
    y = D.lordba_adapter_forward(w0, terms, N, M, R, x_dev(x), ws=ws)
    D.dbf_workspace_check(ws)
    assert not ws[:D.DBF_WS_HEAD_BYTES].any()
    assert_close(to_np(y), ref + o.dense(O.widen_bf16(layer["w0"]), x64(x)))


def _shared_layer(N, M, R, L, T, seed, share_b2=True):
    # LoRDBA's envelope form: every term on the same B1 (and B2), own scales
    layer, x = S.make_custom(N, M, R, L, T, seed=seed)
    for t in layer["terms"][1:]:
        t["b1"] = layer["terms"][0]["b1"]
        if share_b2:
            t["b2"] = layer["terms"][0]["b2"]
    return layer, x


def _shared_terms(layer, share_b2=True):
    terms = device_terms(layer)
    out = [terms[0]]
    for t in terms[1:]:
        out.append(D.DbfTerm(terms[0].b1, terms[0].b2 if share_b2 else t.b2, t.alpha,
                             t.beta, t.gamma))
    return out


@pytest.mark.parametrize("N,M,R,L,T", [(256, 512, 128, 2, 1), (300, 1000, 96, 3, 5),
                                       (65, 33, 17, 4, 3), (4096, 4096, 2048, 3, 1),
                                       (1000, 4096, 512, 4, 3), (1000, 4096, 512, 4, 16), (130, 300, 70, 5, 2),
                                       (512, 2048, 256, 2, 20)])
def test_shared_carriers(N, M, R, L, T):
    # terms that alias one B1 and one B2 run as separate terms; the sums
    # are exact to the tolerance and bitwise reproducible
    print("shared carriers", N, M, R, L, T, flush=True)
    layer, x = _shared_layer(N, M, R, L, T, seed=L + N)
    terms = _shared_terms(layer)
    y = D.dbf_linear_forward(terms, N, M, R, x_dev(x), path=PATH)
    torch.cuda.synchronize()
    ref = O.default().forward(O.terms64(layer), x64(x))
    assert_close(to_np(y), ref)
    y2 = D.dbf_linear_forward(terms, N, M, R, x_dev(x), path=PATH)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)


def test_partly_shared_carriers():
    # B1 shared, B2 not
    layer, x = _shared_layer(200, 700, 64, 3, 4, seed=77, share_b2=False)
    terms = _shared_terms(layer, share_b2=False)
    y = D.dbf_linear_forward(terms, 200, 700, 64, x_dev(x), path=PATH)
    torch.cuda.synchronize()
    assert_close(to_np(y), O.default().forward(O.terms64(layer), x64(x)))


@pytest.mark.parametrize("slot,code", [(2, D.DBF_ESTALLED), (3, D.DBF_EINVAL)])
def test_workspace_check_reports_and_clears(slot, code):
    # A handoff wait that gave up (slot 2) or an adapter index out of range
    # (slot 3) is a flag in the workspace head.  The flag is set here from
    # the host, so no kernel has to stall: dbf_workspace_check must report
    # it, clear the whole head, and leave the buffer usable.
    layer, x = S.make_custom(130, 300, 70, 1, 2, seed=21)
    nb = D.dbf_workspace_bytes(130, 300, 70, 1, 2, D.DBF_PATH_DECODE)
    ws = torch.zeros(nb, dtype=torch.uint8, device=DEV)
    head = ws[:D.DBF_WS_HEAD_BYTES].view(torch.int32)
    head[slot] = 1
    head[0] = 5   # a consumer ticket
    head[64] = 7  # a producer counter
    torch.cuda.synchronize()
    with pytest.raises(D.DbfError) as e:
        D.dbf_workspace_check(ws)
    assert e.value.code == code
    assert not ws[:D.DBF_WS_HEAD_BYTES].any()
    D.dbf_workspace_check(ws)  # clean now
    y = D.dbf_linear_forward(device_terms(layer), 130, 300, 70, x_dev(x), ws=ws,
                             path=D.DBF_PATH_DECODE)
    D.dbf_workspace_check(ws)
    assert not ws[:D.DBF_WS_HEAD_BYTES].any()
    assert_close(to_np(y), O.default().forward(O.terms64(layer), x64(x)))
