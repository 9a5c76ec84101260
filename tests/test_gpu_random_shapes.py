"""Seeded random shapes for every float entry point against the fp64 oracle.

The hand-picked odd shapes of the other files pin the edges that were
thought of; these draw sizes, term counts, token counts, activation dtypes
and paths at random (fixed seed, so every run checks the same cases), so
that a tiling, split or padding rule that fails only for some combination of
sizes shows up.  Every case compares the whole output at the float tolerance.
"""
import numpy as np
import pytest
import torch

import bit_adapters_amd as D
import oracle as O
from bit_adapters_amd import synth as S
from dbfutil import (assert_close, bf16_dev, device_terms, f16_dev, pack_signs, to_np, x64,
                     x_dev)

pytestmark = pytest.mark.gpu

DEC, MF, AUTO = D.DBF_PATH_DECODE, D.DBF_PATH_MFMA, D.DBF_PATH_AUTO
_g = np.random.default_rng(0xDBF5EED)


def _size(hi, lo=1):
    # half the draws log-uniform (small sizes and single tiles), half uniform
    # (several tiles and ragged tails)
    if _g.integers(0, 2):
        return int(_g.integers(lo, hi + 1))
    return min(hi, int(np.exp(_g.uniform(np.log(lo), np.log(hi + 1)))))


FORWARD = [(_size(700), _size(1500), _size(300), int(_g.integers(1, 5)), _size(300),
            ["bf16", "f16"][int(_g.integers(0, 2))], [AUTO, DEC, MF][int(_g.integers(0, 3))])
           for _ in range(64)]
ADAPTER = [(_size(400), int(_g.integers(1, 12)) * 128 if i % 2 == 0 else _size(1500),
            _size(130), int(_g.integers(0, 3)), 1 if i % 3 else _size(20))
           for i in range(32)]
BOOL = [(_size(500), _size(1200), int(_g.integers(1, 4)), _size(120),
         [AUTO, DEC, MF][int(_g.integers(0, 3))]) for _ in range(32)]
BACKWARD = [(_size(300), _size(600), _size(150), int(_g.integers(1, 3)), _size(80),
             [DEC, MF][i % 2]) for i in range(16)]


@pytest.mark.parametrize("N,M,R,L,T,xk,path", FORWARD)
def test_forward(N, M, R, L, T, xk, path):
    print("random forward", N, M, R, L, T, xk, path, flush=True)
    layer, x = S.make_custom(N, M, R, L, T, seed=N * 7 + M * 3 + R + T, x_kind=xk)
    y = D.dbf_linear_forward(device_terms(layer), N, M, R, x_dev(x), path=path)
    torch.cuda.synchronize()
    assert_close(to_np(y), O.default().forward(O.terms64(layer), x64(x)))


@pytest.mark.parametrize("N,M,R,L,T", ADAPTER)
def test_adapter(N, M, R, L, T):
    print("random adapter", N, M, R, L, T, flush=True)
    layer, x = S.make_custom(N, M, R, max(L, 1), T, seed=N + M * 5 + R * 11 + T, base=True,
                             scale_lo=-0.05, scale_hi=0.05)
    terms = device_terms(layer)[:L]
    w0 = bf16_dev(layer["w0"])
    y = D.lordba_adapter_forward(w0, terms, N, M, R, x_dev(x))
    torch.cuda.synchronize()
    o = O.default()
    base = o.dense(O.widen_bf16(layer["w0"]), x64(x))
    ad = o.forward(O.terms64(layer)[:L], x64(x)) if L else 0.0
    assert_close(to_np(y), base + ad, what="full")
    if L:
        # the adapter is a small part of y: also at its own scale (W0 = 0)
        y0 = D.lordba_adapter_forward(torch.zeros_like(w0), terms, N, M, R, x_dev(x))
        torch.cuda.synchronize()
        assert_close(to_np(y0), ad, what="adapter only")


@pytest.mark.parametrize("N,M,K,T,path", BOOL)
def test_bool(N, M, K, T, path):
    print("random bool", N, M, K, T, path, flush=True)
    layer, x = S.make_custom_bool(N, M, K, T, seed=N + 2 * M + 3 * K + T)
    kernels = [D.DbfBoolKernel(pack_signs(k["w"]), f16_dev(k["s_in"]), f16_dev(k["s_out"]))
               for k in layer["kernels"]]
    y = D.dbf_bool_forward(kernels, N, M, x_dev(x), path=path)
    torch.cuda.synchronize()
    ok = [dict(w=k["w"], s_in=np.asarray(k["s_in"], np.float64),
               s_out=np.asarray(k["s_out"], np.float64)) for k in layer["kernels"]]
    assert_close(to_np(y), O.default().bool_forward(ok, x64(x)))


@pytest.mark.parametrize("N,M,R,L,T,path", BACKWARD)
def test_backward(N, M, R, L, T, path):
    print("random backward", N, M, R, L, T, path, flush=True)
    layer, x = S.make_custom(N, M, R, L, T, seed=3 * N + M + 5 * R + T)
    dy_np = np.random.default_rng([0xDBF, 108, N, T]).standard_normal((T, N)).astype(np.float32)
    terms = device_terms(layer)
    tts = [D.dbf_term_t(t, N, M, R) for t in terms]
    dx, scales = D.dbf_linear_backward(terms, tts, N, M, R, x_dev(x),
                                       torch.from_numpy(dy_np).to("cuda:0"), path=path)
    torch.cuda.synchronize()
    rdx, rda, rdb, rdg = O.default().backward(O.terms64(layer), x64(x), dy_np.astype(np.float64))
    assert_close(to_np(dx), rdx, what="dx")
    for i, (da, db, dg) in enumerate(scales):
        assert_close(to_np(da), rda[i], what="dalpha %d" % i)
        assert_close(to_np(db), rdb[i], what="dbeta %d" % i)
        assert_close(to_np(dg), rdg[i], what="dgamma %d" % i)


INT8 = [(_size(600), _size(1500), _size(300), int(_g.integers(1, 4)), _size(40))
        for _ in range(16)]
MULTI = [(_size(300), _size(1200), _size(64), int(_g.integers(1, 9)), _size(24))
         for _ in range(12)]


@pytest.mark.parametrize("N,M,R,L,T", INT8)
def test_int8_exact(N, M, R, L, T):
    # int8 activations, beta = 1: S1 and S2 must match the oracle bit for bit
    print("random int8", N, M, R, L, T, flush=True)
    layer, xq = S.make_custom(N, M, R, L, T, seed=N + M + 7 * R + T, x_kind="i8")
    terms = device_terms(layer, gamma=False, beta=False)
    xd = torch.from_numpy(xq).to("cuda:0")
    s1 = torch.empty((L, T, R), dtype=torch.int32, device="cuda:0")
    s2 = torch.empty((L, T, N), dtype=torch.int32, device="cuda:0")
    D.dbf_linear_forward_i8(terms, N, M, R, xd, s1=s1, s2=s2)
    torch.cuda.synchronize()
    r1, r2 = O.default().forward_int(layer["terms"], xq)
    assert np.array_equal(s1.cpu().numpy(), r1)
    assert np.array_equal(s2.cpu().numpy(), r2)


@pytest.mark.parametrize("N,M,R,K,T", MULTI)
def test_multi_adapter(N, M, R, K, T):
    # token t on adapter idx[t] in [-1, K): -1 is the base alone
    print("random multi-adapter", N, M, R, K, T, flush=True)
    ads = [S.make_custom(N, M, R, 1, 1, seed=N * 3 + a, scale_lo=-0.05, scale_hi=0.05)[0]
           for a in range(K)]
    layer, x = S.make_custom(N, M, R, 1, T, seed=M + T, base=True)
    idx = np.random.default_rng([0xDBF, 109, N, T]).integers(-1, K, T).astype(np.int32)
    adapters = [device_terms(a)[0] for a in ads]
    it = torch.from_numpy(idx).to("cuda:0")
    o = O.default()
    for zero in (False, True):
        w0 = bf16_dev(layer["w0"])
        if zero:
            w0 = torch.zeros_like(w0)
        y = D.lordba_multi_adapter_forward(w0, adapters, N, M, R, it, x_dev(x))
        torch.cuda.synchronize()
        w = np.zeros((N, M)) if zero else O.widen_bf16(layer["w0"])
        ref = o.multi_adapter(w, [O.terms64(a)[0] for a in ads], idx, x64(x))
        assert_close(to_np(y), ref, what="W0 = 0" if zero else "with base")
