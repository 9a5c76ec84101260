"""The prefill-sized layer (8192 x 8192, rank 6144, 4096 tokens of bf16 x)
on the path the library picks for it (the MFMA path), every output against
the fp64 oracle.

Every token is independent, so any wrong workgroup-to-tile mapping (two token
tiles or column tiles swapped, a tile written twice, a ragged edge left
unwritten) shows up as a large error somewhere in the output, and the whole
[4096 x 8192] output is compared: relative L2 and max-abs over the full
tensor, plus a per-token relative error so that a single wrong tile cannot
hide in the global norm.  The oracle takes about two minutes on 16 host
cores.
"""
import time

import numpy as np
import pytest
import torch

import bit_adapters_amd as D
import oracle as O
from bit_adapters_amd import synth as S
from dbfutil import assert_close, device_terms, errors, to_np, x64, x_dev

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(900)
def test_config5_every_token():
    print("config 5: 4096 tokens, every output against the oracle", flush=True)
    layer = S.make_layer(5)
    x = S.make_x(5, 4096)
    terms = device_terms(layer)
    y = D.dbf_linear_forward(terms, layer["N"], layer["M"], layer["R"], x_dev(x),
                             path=D.DBF_PATH_AUTO)
    torch.cuda.synchronize()
    got = to_np(y)
    del y
    t0 = time.perf_counter()
    ref = np.empty_like(got)
    xs = x64(x)
    step = 256
    for t in range(0, 4096, step):
        ref[t:t + step] = O.default().forward(O.terms64(layer), xs[t:t + step])
        print("  oracle tokens %d..%d (%.0f s)" % (t, t + step - 1, time.perf_counter() - t0),
              flush=True)
    assert_close(got, ref, what="config 5, 4096 tokens")
    # per token: every 128-token tile and every column tile is covered by
    # these rows, so a misplaced tile fails here even if the global norm
    # would absorb it
    num = np.linalg.norm(got - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    worst = int(np.argmax(num / den))
    assert np.all(num <= 2e-3 * den), "token %d rel_l2 %.3e" % (worst, num[worst] / den[worst])
    rel, mx = errors(got, ref)
    print("config 5 full: rel_l2 %.3e max_abs %.3e, worst token %d %.3e"
          % (rel, mx, worst, num[worst] / den[worst]), flush=True)
