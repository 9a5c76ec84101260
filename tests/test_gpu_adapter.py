"""lordba_adapter_forward (bf16 base + unmerged double-binary adapter) against
the oracle, with the adapter isolated (W0 = 0) and the base isolated
(n_terms = 0), since in the LoRDBA-sized layer the adapter is ~1e-4 of y and
a tolerance on y alone could not see it."""
import numpy as np
import pytest
import torch

import bit_adapters_amd as D
import oracle as O
from bit_adapters_amd import synth as S
from dbfutil import (DEV, assert_close, assert_close_bf16, bf16_dev, device_terms, to_np, x64,
                     x_dev)

pytestmark = pytest.mark.gpu


def _run(layer, x, n_terms=None, zero_w0=False, **kw):
    N, M, R = layer["N"], layer["M"], layer["R"]
    terms = device_terms(layer)
    if n_terms is not None:
        terms = terms[:n_terms]
    w0 = bf16_dev(layer["w0"])
    if zero_w0:
        w0 = torch.zeros_like(w0)
    y = D.lordba_adapter_forward(w0, terms, N, M, R, x_dev(x), **kw)
    torch.cuda.synchronize()
    return to_np(y)


@pytest.mark.parametrize("R", [16, 64])
@pytest.mark.parametrize("T", [1, 4, 16])
def test_lordba_config(R, T):
    print("adapter R", R, "T", T, flush=True)
    layer = S.make_layer(3, R=R)
    x = S.make_x(3, T)
    o = O.default()
    w0 = O.widen_bf16(layer["w0"])
    xx = x64(x)
    adapter_ref = o.forward(O.terms64(layer), xx)
    base_ref = o.dense(w0, xx)
    assert_close(_run(layer, x), adapter_ref + base_ref, what="full")
    assert_close(_run(layer, x, zero_w0=True), adapter_ref, what="adapter only")
    assert_close(_run(layer, x, n_terms=0), base_ref, what="base only")


# Ranks with L * ceil(R / 16) <= 4 take the in-workgroup rank path (every
# term count and rank-tile count it is built for appears here); larger ones
# take the published-intermediate path.
@pytest.mark.parametrize("N,M,R,L,T", [(65, 33, 17, 2, 3), (130, 300, 70, 3, 5),
                                       (1, 1, 1, 1, 1), (200, 1000, 64, 1, 20),
                                       (50, 520, 16, 1, 16), (96, 1280, 48, 1, 2),
                                       (300, 777, 32, 1, 5), (64, 2304, 10, 3, 1),
                                       (128, 4096, 16, 4, 4), (80, 1536, 16, 2, 33),
                                       (70, 600, 31, 2, 7), (256, 2048, 128, 1, 2),
                                       (40, 4096, 96, 1, 1)])
def test_odd_shapes(N, M, R, L, T):
    print("adapter odd", N, M, R, L, T, flush=True)
    layer, x = S.make_custom(N, M, R, L, T, seed=9, base=True, scale_lo=0.01,
                             scale_hi=0.05)
    o = O.default()
    xx = x64(x)
    ad = o.forward(O.terms64(layer), xx)
    base = o.dense(O.widen_bf16(layer["w0"]), xx)
    assert_close(_run(layer, x), ad + base)
    assert_close(_run(layer, x, zero_w0=True), ad)


def test_strided_x_and_bf16_output():
    layer, x = S.make_custom(96, 200, 32, 1, 4, seed=2, base=True)
    o = O.default()
    ref = o.adapter(O.widen_bf16(layer["w0"]), O.terms64(layer), x64(x))
    xd = torch.zeros((4, 216), dtype=torch.bfloat16, device=DEV)
    xd[:, :200] = x_dev(x)
    terms = device_terms(layer)
    y = D.lordba_adapter_forward(bf16_dev(layer["w0"]), terms, 96, 200, 32,
                                 xd[:, :200], y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert_close_bf16(to_np(y), ref)


def test_unaligned_activation_rows():
    # ldx = 605: no 16-byte loads, every feature takes the bounded step
    layer, x = S.make_custom(48, 600, 40, 1, 3, seed=4, base=True, scale_lo=0.01,
                             scale_hi=0.05)
    o = O.default()
    ref = o.adapter(O.widen_bf16(layer["w0"]), O.terms64(layer), x64(x))
    xd = torch.zeros((3, 605), dtype=torch.bfloat16, device=DEV)
    xd[:, :600] = x_dev(x)
    y = D.lordba_adapter_forward(bf16_dev(layer["w0"]), device_terms(layer), 48, 600, 40,
                                 xd[:, :600])
    torch.cuda.synchronize()
    assert_close(to_np(y), ref)


def test_adapter_deterministic():
    layer = S.make_layer(3, R=64)
    x = S.make_x(3, 4)
    a = _run(layer, x)
    b = _run(layer, x)
    assert np.array_equal(a, b)


# One token with M a multiple of 128 stages every operand through LDS: ragged
# rows, waves with no group (small M), one and two terms, every rank-tile
# count, and waves with many more groups than the ring holds (M = 12288 gives
# 12 per wave).
@pytest.mark.parametrize("N,M,R,L,lo", [(65, 256, 17, 2, 0.01), (50, 1280, 48, 1, 0.01),
                                        (33, 128, 16, 1, 0.01), (300, 5120, 33, 1, 0.01),
                                        (48, 12288, 64, 1, 0.01), (96, 2048, 32, 2, -0.05),
                                        (17, 4096, 1, 2, -0.05)])
def test_one_token_staged(N, M, R, L, lo):
    # lo < 0: scales of both signs
    print("adapter one token", N, M, R, L, lo, flush=True)
    layer, x = S.make_custom(N, M, R, L, 1, seed=13, base=True, scale_lo=lo,
                             scale_hi=0.05)
    o = O.default()
    xx = x64(x)
    ad = o.forward(O.terms64(layer), xx)
    base = o.dense(O.widen_bf16(layer["w0"]), xx)
    assert_close(_run(layer, x), ad + base, what="full")
    assert_close(_run(layer, x, zero_w0=True), ad, what="adapter only")
    assert_close(_run(layer, x, n_terms=0), base, what="base only")


# With four rank tiles and M <= 4096 the one-token kernel's stream waves read
# W0 rows into registers, 512 features a load: M not a multiple of 512 (a last
# load with idle lanes), M = 128 (one partial load), ragged rows (N not a
# multiple of 16), one or two terms.
@pytest.mark.parametrize("N,M,R,L", [(37, 640, 64, 1), (130, 3968, 64, 1), (20, 128, 50, 1),
                                     (64, 4096, 32, 2), (16, 4096, 64, 1)])
def test_one_token_register_stream(N, M, R, L):
    print("adapter one token, register stream", N, M, R, L, flush=True)
    layer, x = S.make_custom(N, M, R, L, 1, seed=31, base=True, scale_lo=-0.05, scale_hi=0.05)
    o = O.default()
    xx = x64(x)
    ad = o.forward(O.terms64(layer), xx)
    base = o.dense(O.widen_bf16(layer["w0"]), xx)
    assert_close(_run(layer, x), ad + base, what="full")
    assert_close(_run(layer, x, zero_w0=True), ad, what="adapter only")
    assert_close(_run(layer, x, n_terms=0), base, what="base only")


# The one-token kernel's LDS limit: rank 64 fits with M = 7168 (ring of two
# groups per stream wave) and not with M = 7296 (the older kernel runs);
# rank 16 at M = 8192 fits with a ring of three.
@pytest.mark.parametrize("M,R", [(7168, 64), (7296, 64), (8192, 16)])
def test_one_token_lds_limits(M, R):
    print("adapter one token, LDS limit", M, R, flush=True)
    layer, x = S.make_custom(40, M, R, 1, 1, seed=21, base=True, scale_lo=0.01, scale_hi=0.05)
    o = O.default()
    xx = x64(x)
    ref = o.forward(O.terms64(layer), xx) + o.dense(O.widen_bf16(layer["w0"]), xx)
    assert_close(_run(layer, x), ref)


def test_one_token_gamma_not_16_byte_aligned():
    # gamma is copied 16 bytes at a time; an offset gamma takes the older kernel
    layer, x = S.make_custom(64, 1024, 32, 1, 1, seed=22, base=True, scale_lo=0.01,
                             scale_hi=0.05)
    o = O.default()
    ref = o.adapter(O.widen_bf16(layer["w0"]), O.terms64(layer), x64(x))
    t = device_terms(layer)[0]
    g = torch.zeros(1024 + 8, dtype=torch.float16, device=DEV)
    g[4:4 + 1024] = t.gamma
    shifted = D.DbfTerm(t.b1, t.b2, t.alpha, t.beta, g[4:4 + 1024])
    y = D.lordba_adapter_forward(bf16_dev(layer["w0"]), [shifted], 64, 1024, 32, x_dev(x))
    torch.cuda.synchronize()
    assert_close(to_np(y), ref)


def test_one_token_strided_x():
    # x one row inside a wider buffer (ldx = 1152, still 16-byte rows)
    layer, x = S.make_custom(70, 1024, 40, 1, 1, seed=5, base=True, scale_lo=0.01,
                             scale_hi=0.05)
    o = O.default()
    ref = o.adapter(O.widen_bf16(layer["w0"]), O.terms64(layer), x64(x))
    xd = torch.zeros((1, 1152), dtype=torch.bfloat16, device=DEV)
    xd[:, :1024] = x_dev(x)
    y = D.lordba_adapter_forward(bf16_dev(layer["w0"]), device_terms(layer), 70, 1024, 40,
                                 xd[:, :1024])
    torch.cuda.synchronize()
    assert_close(to_np(y), ref)
