"""HIP-graph replays: the entry points captured once and replayed several
times, with eager calls of the same and other paths on the same workspace
in between, every replay checked bit for bit against the eager result.  The
decode kernels' handoff counters are reset by the kernels themselves (no
memset node), so every replay must leave the workspace head clear."""
import numpy as np
import pytest
import torch

import bit_adapters_amd as D
from bit_adapters_amd import synth as S
from dbfutil import DEV, bf16_dev, device_terms, f16_dev, pack_signs, x_dev

pytestmark = pytest.mark.gpu


def _replays(call, eager_between, ws, n=4):
    """Capture call() once; replay n times, eager_between() after each."""
    ref = call().clone()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        out = call()
    for i in range(n):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "replay %d differs" % i
        if ws is not None:
            assert not ws[:D.DBF_WS_HEAD_BYTES].any(), "replay %d left the head set" % i
        eager_between()
        torch.cuda.synchronize()
    if ws is not None:
        D.dbf_workspace_check(ws)


def test_forward_paths_in_a_graph():
    layer, x = S.make_custom(300, 1000, 96, 2, 5, seed=41)
    terms = device_terms(layer)
    xd = x_dev(x)
    nb = max(D.dbf_workspace_bytes(300, 1000, 96, 2, 5, p)
             for p in (D.DBF_PATH_DECODE, D.DBF_PATH_MFMA))
    ws = torch.zeros(nb, dtype=torch.uint8, device=DEV)
    y = torch.empty((5, 300), dtype=torch.float32, device=DEV)
    y2 = torch.empty_like(y)
    for path in (D.DBF_PATH_DECODE, D.DBF_PATH_MFMA):
        other = D.DBF_PATH_MFMA if path == D.DBF_PATH_DECODE else D.DBF_PATH_DECODE
        _replays(lambda: D.dbf_linear_forward(terms, 300, 1000, 96, xd, y=y, ws=ws, path=path),
                 lambda: D.dbf_linear_forward(terms, 300, 1000, 96, xd, y=y2, ws=ws, path=other),
                 ws)


def test_adapter_bool_and_multi_adapter_in_graphs():
    N, M, R, T = 256, 1024, 64, 6
    layer, x = S.make_custom(N, M, R, 1, T, seed=42, base=True, scale_lo=0.01,
                             scale_hi=0.05)
    terms = device_terms(layer)
    w0 = bf16_dev(layer["w0"])
    xd = x_dev(x)
    ws = torch.zeros(D.dbf_workspace_bytes(N, M, R, 2, T, D.DBF_PATH_DECODE) + (1 << 20),
                     dtype=torch.uint8, device=DEV)
    y = torch.empty((T, N), dtype=torch.float32, device=DEV)
    y2 = torch.empty_like(y)
    # the adapter with two terms takes the published-intermediate path
    terms2 = terms + device_terms(S.make_custom(N, M, R, 1, T, seed=43)[0])
    _replays(lambda: D.lordba_adapter_forward(w0, terms2, N, M, R, xd, y=y, ws=ws),
             lambda: D.dbf_linear_forward(terms2, N, M, R, xd, y=y2, ws=ws,
                                          path=D.DBF_PATH_DECODE), ws)
    # boolean kernels on the decode path
    bl, bx = S.make_custom_bool(N, M, 2, T, seed=44)
    kernels = [D.DbfBoolKernel(pack_signs(k["w"]), f16_dev(k["s_in"]), f16_dev(k["s_out"]))
               for k in bl["kernels"]]
    bxd = x_dev(bx)
    _replays(lambda: D.dbf_bool_forward(kernels, N, M, bxd, y=y, ws=ws,
                                        path=D.DBF_PATH_DECODE),
             lambda: D.lordba_adapter_forward(w0, terms2, N, M, R, xd, y=y2, ws=ws), ws)
    # several adapters, one per token
    adapters = [terms2[0], terms2[1]]
    idx = torch.tensor([0, 1, -1, 1, 0, 0], dtype=torch.int32, device=DEV)
    _replays(lambda: D.lordba_multi_adapter_forward(w0, adapters, N, M, R, idx, xd, y=y, ws=ws),
             lambda: D.dbf_bool_forward(kernels, N, M, bxd, y=y2, ws=ws,
                                        path=D.DBF_PATH_DECODE), ws)


def test_backward_in_a_graph():
    N, M, R, T = 200, 700, 96, 24
    layer, x = S.make_custom(N, M, R, 2, T, seed=45)
    terms = device_terms(layer)
    tts = [D.dbf_term_t(t, N, M, R) for t in terms]
    xd = x_dev(x)
    dy = torch.from_numpy(np.random.default_rng(3).standard_normal((T, N)).astype(np.float32)).to(DEV)
    for path in (D.DBF_PATH_DECODE, D.DBF_PATH_MFMA):
        ws = torch.zeros(D.dbf_backward_workspace_bytes(N, M, R, 2, T, path),
                         dtype=torch.uint8, device=DEV)

        def call():
            dx, sc = D.dbf_linear_backward(terms, tts, N, M, R, xd, dy, ws=ws, path=path)
            return torch.cat([dx.reshape(-1)] + [v.reshape(-1) for trip in sc for v in trip])

        _replays(call, lambda: None, ws if path == D.DBF_PATH_DECODE else None)
