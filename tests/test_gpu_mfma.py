"""dbf_linear_forward on the MFMA path against the fp64 oracle.

The MFMA path rounds gamma . x and the per-token-scaled rank-R intermediate
to fp16 (relative ~2^-11 each), so it meets the same float tolerance as the
decode path.  The 4096-token configuration is compared in full in
test_gpu_c5_full.py."""
import numpy as np
import pytest
import torch

import bit_adapters_amd as D
import oracle as O
from bit_adapters_amd import synth as S
from dbfutil import (DEV, assert_close, assert_close_bf16, device_terms, to_np, x64,
                     x_dev)

pytestmark = pytest.mark.gpu

MF = D.DBF_PATH_MFMA


def run(layer, x, path=MF, **kw):
    terms = device_terms(layer)
    y = D.dbf_linear_forward(terms, layer["N"], layer["M"], layer["R"], x_dev(x),
                             path=path, **kw)
    torch.cuda.synchronize()
    return y


ODD = [(1, 1, 1, 1, 1), (65, 33, 17, 2, 3), (130, 300, 70, 3, 5),
       (300, 129, 257, 1, 130), (256, 256, 256, 1, 128), (77, 1000, 96, 2, 200),
       (513, 64, 600, 1, 17), (40, 4100, 130, 1, 33),
       # a row of one full 8192-feature prep segment and a ragged one
       (40, 9000, 130, 1, 33)]


@pytest.mark.parametrize("N,M,R,L,T", ODD)
@pytest.mark.parametrize("xk", ["bf16", "f16"])
def test_odd_shapes(N, M, R, L, T, xk):
    print("mfma odd", N, M, R, L, T, xk, flush=True)
    layer, x = S.make_custom(N, M, R, L, T, seed=N * 3 + M + R, x_kind=xk)
    y = to_np(run(layer, x))
    ref = O.default().forward(O.terms64(layer), x64(x))
    assert_close(y, ref)


@pytest.mark.parametrize("T", [64, 256])
def test_config4(T):
    print("mfma config 4 T", T, flush=True)
    layer = S.make_layer(4)
    x = S.make_x(4, T)
    y = to_np(run(layer, x, path=D.DBF_PATH_AUTO))
    ref = O.default().forward(O.terms64(layer), x64(x))
    assert_close(y, ref)


def test_config2_forced_mfma():
    layer = S.make_layer(2)
    x = S.make_x(2, 16)
    y = to_np(run(layer, x))
    ref = O.default().forward(O.terms64(layer), x64(x))
    assert_close(y, ref)


def test_config2_short_product_tiles():
    # 250 tokens of the 4096 x 4096, R 2048 layer: stage 2 (16 K steps)
    # runs on 32-row tiles, the last one ragged
    print("mfma config 2 T 250", flush=True)
    layer = S.make_layer(2)
    x = S.make_x(2, 250)
    y = to_np(run(layer, x))
    toks = np.array([0, 31, 32, 128, 223, 224, 249])
    ref = O.default().forward(O.terms64(layer), x64(x[toks]))
    assert_close(y[toks], ref)


def test_config4_eight_tokens_auto():
    # 8 tokens of the three-term layer: the automatic choice is the MFMA path
    # (the decode's sign work, 2 x 3 x 2048 x 15104, is above its threshold),
    # split along K
    print("config 4 T 8 auto", flush=True)
    layer = S.make_layer(4)
    x = S.make_x(4, 8)
    y = to_np(run(layer, x, path=D.DBF_PATH_AUTO))
    ref = O.default().forward(O.terms64(layer), x64(x))
    assert_close(y, ref)


@pytest.mark.parametrize("scale", [2.0 ** 20, 2.0 ** -20])
@pytest.mark.parametrize("L", [1, 3])
def test_extreme_activation_scale(scale, L):
    # |gamma . x| far above the fp16 range (inf without a scale), or far below
    # its normal range (subnormal): the per-token power of two keeps both fp16
    # intermediates in range, so the MFMA path meets the same tolerance
    layer, x = S.make_custom(200, 700, 130, L, 40, seed=77 + L)
    xs = S.f32_to_bf16_bits((x64(x) * scale).astype(np.float32))
    assert np.array_equal(x64(xs), x64(x) * scale)  # a power of two: exact
    y = to_np(run(layer, xs))
    assert np.all(np.isfinite(y))
    ref = O.default().forward(O.terms64(layer), x64(xs))
    assert_close(y, ref)
    # and scaling x scales y by the same power of two, bit for bit
    y1 = to_np(run(layer, x))
    assert np.array_equal(y, y1 * scale)


def test_mixed_token_scales():
    # tokens whose magnitudes differ by 2^40 in one batch: each token has its
    # own scale, so the small ones are not flushed by the large ones
    layer, x = S.make_custom(150, 600, 96, 2, 64, seed=12)
    f = 2.0 ** np.round(np.linspace(-20, 20, 64))
    xs = S.f32_to_bf16_bits((x64(x) * f[:, None]).astype(np.float32))
    y = to_np(run(layer, xs))
    ref = O.default().forward(O.terms64(layer), x64(xs))
    num = np.linalg.norm(y - ref, axis=1)
    assert np.all(num <= 2e-3 * np.linalg.norm(ref, axis=1))


def test_output_dtypes_accumulate_strides():
    layer, x = S.make_custom(96, 200, 40, 2, 150, seed=3)
    ref = O.default().forward(O.terms64(layer), x64(x))
    terms = device_terms(layer)
    xd = torch.zeros((150, 208), dtype=torch.bfloat16, device=DEV)
    xd[:, :200] = x_dev(x)
    xs = xd[:, :200]
    big = torch.full((150, 100), 7.0, dtype=torch.float32, device=DEV)
    y = big[:, :96]
    D.dbf_linear_forward(terms, 96, 200, 40, xs, y=y, path=MF)
    torch.cuda.synchronize()
    assert_close(to_np(y), ref)
    assert torch.all(big[:, 96:] == 7.0)
    base = torch.randn((150, 96), dtype=torch.float32, device=DEV)
    y2 = base.clone()
    D.dbf_linear_forward(terms, 96, 200, 40, xs, y=y2, accumulate=True, path=MF)
    torch.cuda.synchronize()
    assert_close(to_np(y2), ref + to_np(base))
    yb = D.dbf_linear_forward(terms, 96, 200, 40, xs, y_dtype=torch.bfloat16, path=MF)
    torch.cuda.synchronize()
    assert_close_bf16(to_np(yb), ref)


def test_deterministic_and_scale_invariant():
    layer, x = S.make_custom(300, 500, 200, 2, 140, seed=8)
    a = run(layer, x).cpu()
    b = run(layer, x).cpu()
    assert torch.equal(a, b)
    # a power-of-two scale of x scales y exactly (the per-token scale absorbs it)
    xs = x_dev(x) * 64.0
    terms = device_terms(layer)
    c = D.dbf_linear_forward(terms, 300, 500, 200, xs, path=MF)
    torch.cuda.synchronize()
    assert torch.equal(c.cpu(), a * 64.0)


@pytest.mark.parametrize("R", [80, 88, 95, 96])
@pytest.mark.parametrize("seed", [1, 2])
def test_first_row_block_small_rank(R, seed):
    # sign rows of 3 words (rank <= 96) with a single K step: every row block
    # of the tile must come out right (regression for an operand hazard that
    # corrupted the first 32 rows)
    layer, x = S.make_custom(40, 300, R, 1, 40, seed=seed)
    y = to_np(run(layer, x))
    ref = O.default().forward(O.terms64(layer), x64(x))
    assert_close(y, ref)


# Few output tiles: K is split across workgroups and the fp32 partials are
# summed in split order by a reduction kernel.  (300, 2000, 601, 3, 40):
# stage 2 has 3 x 5 steps over 7 splits, so splits straddle term boundaries;
# R and N not multiples of 4; (4096, 4096, 2048, 1, 33): 16 splits in stage 1.
SPLIT = [(300, 2000, 601, 3, 40), (1000, 4096, 2048, 1, 64), (4096, 4096, 2048, 1, 33),
         (701, 3000, 301, 2, 9), (130, 8192, 1030, 1, 2)]


@pytest.mark.parametrize("N,M,R,L,T", SPLIT)
def test_split_k(N, M, R, L, T):
    print("mfma split", N, M, R, L, T, flush=True)
    layer, x = S.make_custom(N, M, R, L, T, seed=N + 7 * R + L)
    ref = O.default().forward(O.terms64(layer), x64(x))
    a = to_np(run(layer, x))
    assert_close(a, ref)
    assert np.array_equal(a, to_np(run(layer, x)))


# The split sums are instantiated per split count (2 .. 16).  Shapes that
# give every count in the first product (M = 256 s at one token: s splits of
# two K steps) and in the second (the rest; found with the tile rule at the
# time of writing), each checked against the oracle with a bf16 output.
EVERY_SPLIT = ([(128, 256 * s, 128, 1, 1) for s in range(2, 17)] +
               [(128, 256, 256, 2, 1), (128, 256, 256, 3, 1), (128, 256, 512, 2, 1),
                (128, 256, 640, 2, 1), (128, 256, 512, 3, 1), (128, 256, 640, 3, 1),
                (128, 256, 1024, 2, 1), (128, 256, 768, 3, 1), (128, 256, 1280, 2, 1),
                (2816, 256, 1024, 3, 33), (128, 256, 1024, 3, 1), (2432, 256, 1280, 3, 33),
                (2304, 256, 1280, 3, 33), (128, 256, 1280, 3, 1), (128, 256, 2048, 2, 1)])


@pytest.mark.parametrize("N,M,R,L,T", EVERY_SPLIT)
def test_every_split_count(N, M, R, L, T):
    print("mfma every split", N, M, R, L, T, flush=True)
    layer, x = S.make_custom(N, M, R, L, T, seed=3 * N + M + R + L)
    ref = O.default().forward(O.terms64(layer), x64(x))
    assert_close_bf16(to_np(run(layer, x, y_dtype=torch.bfloat16)), ref)


def test_split_k_output_dtypes_accumulate_strides():
    N, M, R, L, T = 301, 3000, 300, 2, 20
    layer, x = S.make_custom(N, M, R, L, T, seed=5)
    ref = O.default().forward(O.terms64(layer), x64(x))
    terms = device_terms(layer)
    big = torch.full((T, 320), 7.0, dtype=torch.float32, device=DEV)
    base = torch.randn((T, N), dtype=torch.float32, device=DEV)
    big[:, :N] = base
    D.dbf_linear_forward(terms, N, M, R, x_dev(x), y=big[:, :N], accumulate=True, path=MF)
    torch.cuda.synchronize()
    assert_close(to_np(big[:, :N]), ref + to_np(base))
    assert torch.all(big[:, N:] == 7.0)
    yb = torch.full((T, 310), 3.0, dtype=torch.bfloat16, device=DEV)
    D.dbf_linear_forward(terms, N, M, R, x_dev(x), y=yb[:, :N], path=MF)
    torch.cuda.synchronize()
    assert_close_bf16(to_np(yb[:, :N]), ref)
    assert torch.all(yb[:, N:] == 3.0)


@pytest.mark.parametrize("path", [D.DBF_PATH_DECODE, MF])
def test_maximum_terms(path):
    # DBF_MAX_TERMS terms, separate carriers
    L = D.DBF_MAX_TERMS
    layer, x = S.make_custom(200, 640, 96, L, 6, seed=88)
    y = to_np(run(layer, x, path=path))
    assert_close(y, O.default().forward(O.terms64(layer), x64(x)))
