"""dbf_pack / dbf_unpack on the GPU against the oracle's packer: bit-exact."""
import numpy as np
import pytest
import torch

import bit_adapters_amd as D
import oracle as O
from bit_adapters_amd import synth as S
from dbfutil import DEV

pytestmark = pytest.mark.gpu

SHAPES = [(1, 1), (3, 31), (64, 32), (65, 33), (70, 97), (130, 300),
          (16, 4096), (4096, 16), (64, 2048), (2048, 4096)]


def _dev(v, kind):
    if kind == "bf16":
        return torch.from_numpy(v.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(v).to(DEV)


def _as64(v, kind):
    return O.widen_bf16(v) if kind == "bf16" else v.astype(np.float64)


@pytest.mark.parametrize("kind", ["f32", "f16", "bf16", "i8"])
@pytest.mark.parametrize("rows,k", SHAPES)
def test_pack_bit_exact(rows, k, kind):
    v = S.random_values(rows, k, seed=rows * 7 + k, kind=kind)
    print("pack", rows, k, kind, flush=True)
    got = D.dbf_pack(_dev(v, kind)).cpu().numpy().view(np.uint32)
    exp = O.default().pack(_as64(v, kind))
    assert np.array_equal(got, exp)
    back = D.dbf_unpack(torch.from_numpy(exp.view(np.int32)).to(DEV), rows, k)
    assert np.array_equal(back.cpu().numpy(), O.default().unpack(exp, rows, k))


def test_pack_strided_source_and_special_values():
    v = np.array([[0.0, -0.0, np.nan, -1e-30, 1e-30, -np.inf, np.inf, 2.0]],
                 dtype=np.float32)
    big = np.full((3, 40), -5.0, dtype=np.float32)
    big[1, :8] = v[0]
    t = torch.from_numpy(big).to(DEV)[:, :8]          # ld = 40 > k = 8
    got = D.dbf_pack(t).cpu().numpy().view(np.uint32)
    exp = O.default().pack(big[:, :8].astype(np.float64))
    assert np.array_equal(got, exp)
    assert np.array_equal(O.default().unpack(exp, 3, 8)[1], [1, 1, -1, -1, 1, -1, 1, 1])


def test_pack_overwrites_padding():
    rows, k = 65, 33
    out = torch.full((D.dbf_packed_bytes(rows, k) // 4,), -1, dtype=torch.int32,
                     device=DEV)
    s = np.ones((rows, k), dtype=np.int8)
    D.dbf_pack(torch.from_numpy(s).to(DEV), out=out)
    got = out.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, O.default().pack(s.astype(np.float64)))
    assert int(np.unpackbits(got.view(np.uint8)).sum()) == rows * k
