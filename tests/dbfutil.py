"""Helpers for the GPU parity tests: move a synthetic layer to the device
(signs packed by the library's own dbf_pack), and compare results with the
oracle to the stated tolerances."""
from __future__ import annotations

import numpy as np
import torch

import bit_adapters_amd as D
import oracle as O

DEV = "cuda:0"

# float tolerance for bf16 / fp16 activations with fp32 accumulation:
# relative L2 over the whole output and max-abs relative to max |y_ref|.
REL_L2 = 2e-3
MAX_ABS = 1e-2


def f16_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float16)).to(DEV)


def bf16_dev(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.to(DEV).view(torch.bfloat16)


def x_dev(x):
    if x.dtype == np.uint16:
        return bf16_dev(x)
    if x.dtype == np.float16:
        return f16_dev(x)
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def x64(x):
    """Activations as the oracle sees them (fp64, exact widening)."""
    return O.widen_bf16(x) if x.dtype == np.uint16 else x.astype(np.float64)


def pack_signs(s: np.ndarray) -> torch.Tensor:
    return D.dbf_pack(torch.from_numpy(np.ascontiguousarray(s)).to(DEV))


def device_terms(layer, gamma=True, alpha=True, beta=True):
    out = []
    for t in layer["terms"]:
        out.append(D.DbfTerm(pack_signs(t["b1"]), pack_signs(t["b2"]),
                             f16_dev(t["alpha"]) if alpha else None,
                             f16_dev(t["beta"]) if beta else None,
                             f16_dev(t["gamma"]) if gamma else None))
    torch.cuda.synchronize()
    return out


def errors(y, ref):
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = y - ref
    rel = np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300)
    mx = np.abs(d).max() / max(np.abs(ref).max(), 1e-300)
    return rel, mx


def assert_close(y, ref, rel_l2=REL_L2, max_abs=MAX_ABS, what=""):
    rel, mx = errors(y, ref)
    assert rel <= rel_l2 and mx <= max_abs, (
        "%s rel_l2 %.3e (<= %.1e) max_abs %.3e (<= %.1e)" % (what, rel, rel_l2, mx, max_abs))
    return rel, mx


def round_bf16(a):
    """fp64 -> bf16 (RNE, through fp32) -> fp64, for bf16-output checks."""
    from bit_adapters_amd.synth import f32_to_bf16_bits
    return O.widen_bf16(f32_to_bf16_bits(np.asarray(a, dtype=np.float32)))


def assert_close_bf16(y, ref, what=""):
    """A bf16 output against the oracle rounded the same way (RNE to bf16),
    at the float tolerance: the rounding of the output itself is then not
    charged to the kernel.  Where the kernel's fp32 result and the oracle lie
    on either side of a rounding boundary the two differ by one bf16 step, so
    additionally every element must be within one step (2^-7 relative, the
    spacing at the bottom of a binade) of the exact oracle value, or within
    1e-3 max|ref| for values near zero."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert_close(y, round_bf16(ref), what=what + " (bf16 output)")
    lim = np.abs(ref) * 2.0 ** -7 + 1e-3 * np.abs(ref).max()
    bad = np.abs(y - ref) > lim
    assert not bad.any(), "%s: %d elements more than one bf16 step from the oracle" % (
        what, int(bad.sum()))


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return O.widen_bf16(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.float().cpu().numpy().astype(np.float64) if t.dtype != torch.int32 \
        else t.cpu().numpy()
