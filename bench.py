"""Throughput of the double-binary factorized linear layer on one MI355X.

Default workload: the Llama-7B-shaped projection as a one-term DBF layer
(N = M = 4096, R = 2048, ~1 bit/weight), decode batch of 1 token, bf16 x and
bf16 y.  A step is one forward, dbf_linear_forward, over one batch: both
sign-accumulate stages, the three scale vectors and the output.

Timing: the layer is replicated into distinct copies (>= 1 GiB in total);
W warm-up steps run eagerly, then K steps (one copy each, round robin) are
captured in one HIP graph.  The graph is replayed once untimed, then a 1 GiB
buffer is read and written (evicting the 256 MiB last-level cache and every
L2, whatever K is), then the graph is replayed between two HIP events on the
capturing stream; ms_per_step = elapsed / K.  So every step reads its signs
from HBM.  The graph's last output is checked against an eager call and
against the fp64 oracle.

The default run (the 4096 x 4096 layer at one token) also times the metric's
second operating point in the same process: the prefill-sized layer (8192 x
8192, R 6144) on 4096 tokens, reported as MFMA utilisation under the key
"mfma_4096" (--no-prefill skips it).

Other workloads: --config 3 --rank {16,64} (LoRDBA adapter on a bf16 base),
--config 4 (three-term layer), --config 5 (8192 x 8192, R = 6144, 4096
tokens), --config 6 / 7 (the Multi-Boolean form, dbf_bool_forward: two
4096 x 4096 or three 11008 x 4096 sign kernels with rank-one scales), with
--tokens T.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import bit_adapters_amd as D  # noqa: E402
from bit_adapters_amd import synth as S  # noqa: E402

METRIC = "DBF linear tokens/s; HBM GB/s frac @1 tok, MFMA util @4096 tok"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 / bf16 matrix peak
DEV = "cuda:0"


def kernel_sources_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_adapters_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def dev_f16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float16)).to(DEV)


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def dev_x(x_np):
    """Activations on the device: bf16 (stored as uint16 bits) or fp16."""
    if x_np.dtype == np.float16:
        return dev_f16(x_np)
    return dev_bf16(x_np)


def widen_x(x_np):
    """Activations as the oracle sees them (fp64, exact widening)."""
    import oracle as O
    return x_np.astype(np.float64) if x_np.dtype == np.float16 else O.widen_bf16(x_np)


def algorithmic(cfg, N, M, R, L, T, base):
    """Bytes the method must move per forward (packed signs at one bit each,
    fp16 scales, bf16 x and y, bf16 W0 if any) and its flops."""
    signs = L * R * (N + M) / 8.0
    scales = 2.0 * L * (N + R + M)
    xy = 2.0 * T * (M + N)
    w0 = 2.0 * N * M if base else 0.0
    flops = 2.0 * T * R * (N + M) * L + (2.0 * T * N * M if base else 0.0)
    return signs + scales + xy + w0, flops


def algorithmic_bool(N, M, K, T):
    """The same for K boolean kernels: N x M signs at one bit, s_in and s_out
    in fp16, bf16 x and y; one sign-accumulate product per kernel."""
    return K * N * M / 8.0 + 2.0 * K * (N + M) + 2.0 * T * (M + N), 2.0 * T * N * M * K


def algorithmic_backward(N, M, R, L, T):
    """The backward: the packed signs twice (the factors and their
    transposes), fp16 scales, bf16 x, dy and dx, fp32 scale gradients; four
    sign-accumulate products per term."""
    signs = 2 * L * R * (N + M) / 8.0
    scales = 2.0 * L * (N + R + M) + 4.0 * L * (N + R + M)
    io = 2.0 * T * (M + N) + 2.0 * T * M
    return signs + scales + io, 4.0 * T * R * (N + M) * L


def auto_path(T, L, blocks):
    # the library's automatic choice for the boolean kernels and the
    # backward products (dbf_abi.hip, resolve_path)
    return "decode" if T <= 4 or L * ((T + 3) // 4) <= blocks else "mfma"


def auto_bool_path(T, K):
    # the library's automatic choice for the boolean kernels (dbf_abi.hip,
    # resolve_bool_path): decode while its launch has one token block or
    # K times its token blocks is at most 4
    tb = 1 if T <= 1 else (2 if T <= 4 else 4)
    blocks = (T + tb - 1) // tb
    return "decode" if blocks == 1 or K * blocks <= 4 else "mfma"


def auto_dbf_path(N, M, R, L, T):
    # the library's automatic choice for the double-binary forward
    # (dbf_abi.hip, resolve_dbf_path): decode while T <= 4 or the sign work
    # of the 4-token blocks is at most 8.0e7 lookups
    return "decode" if T <= 4 or L * ((T + 3) // 4) * R * (N + M) <= 8.0e7 else "mfma"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--tokens", type=int, default=None)
    ap.add_argument("--rank", type=int, default=16)
    ap.add_argument("--path", type=int, default=D.DBF_PATH_AUTO)
    ap.add_argument("--rotate-gib", type=float, default=1.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--shared", action="store_true",
                    help="LoRDBA's envelope form: every term on term 0's B1 and B2 "
                         "(own scales); multi-term configurations")
    ap.add_argument("--multi", type=int, default=0,
                    help="config 3: K adapters beside one base, token t on adapter t %% K "
                         "(lordba_multi_adapter_forward)")
    ap.add_argument("--backward", action="store_true",
                    help="time dbf_linear_backward (dx and every scale gradient) instead")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 256 MiB device copy (counter calibration)")
    ap.add_argument("--no-prefill", action="store_true",
                    help="default run: skip the 4096-token prefill measurement")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only (--gpus 1): the layer is not sharded "
              "across GPUs in this library", file=sys.stderr)
        sys.exit(2)

    boolk = args.config in S.BOOL_CONFIGS
    cfgd = S.BOOL_CONFIGS[args.config] if boolk else S.CONFIGS[args.config]
    T = args.tokens if args.tokens is not None else min(cfgd["T"])
    base = bool(cfgd.get("base"))
    x_np = S.make_x(args.config, T)
    x = dev_x(x_np)

    # one packed copy, then clones for rotation
    terms0 = []
    if boolk:
        layer = S.make_bool_layer(args.config)
        N, M, L = layer["N"], layer["M"], len(layer["kernels"])
        R = None
        for k in layer["kernels"]:
            terms0.append(D.DbfBoolKernel(D.dbf_pack(torch.from_numpy(k["w"]).to(DEV)),
                                          dev_f16(k["s_in"]), dev_f16(k["s_out"])))
    else:
        layer = S.make_layer(args.config, R=args.rank if base else None)
        N, M, R, L = layer["N"], layer["M"], layer["R"], len(layer["terms"])
        if args.shared:
            if L < 2:
                print("--shared needs a multi-term configuration (4)", file=sys.stderr)
                sys.exit(2)
            for t in layer["terms"][1:]:
                t["b1"], t["b2"] = layer["terms"][0]["b1"], layer["terms"][0]["b2"]
        for t in layer["terms"]:
            terms0.append(D.DbfTerm(
                D.dbf_pack(torch.from_numpy(t["b1"]).to(DEV)),
                D.dbf_pack(torch.from_numpy(t["b2"]).to(DEV)),
                dev_f16(t["alpha"]), dev_f16(t["beta"]), dev_f16(t["gamma"])))
    if args.backward and (boolk or base):
        print("--backward is for the double-binary layers (configs 1, 2, 4, 5)", file=sys.stderr)
        sys.exit(2)
    if args.backward:
        # each copy carries its packed transposes as well
        terms0 = [(t, D.dbf_term_t(t, N, M, R)) for t in terms0]
        dy = dev_bf16(S.f32_to_bf16_bits(np.random.default_rng([0xDBF, 106, T, N]).standard_normal(
            (T, N), dtype=np.float32)))
    multi = args.multi
    if multi:
        if not base or multi > D.DBF_MAX_ADAPTERS:
            print("--multi K needs config 3 and 1 <= K <= %d" % D.DBF_MAX_ADAPTERS, file=sys.stderr)
            sys.exit(2)
        # K adapters of the configuration's rank: adapter 0 is the layer's own,
        # the others are its clones (same values, separate memory)
        terms0 = [terms0[0]] + [type(terms0[0])(*[v.clone() for v in terms0[0]])
                                for _ in range(multi - 1)]
        midx = torch.arange(T, dtype=torch.int32, device=DEV) % multi
    tcls = type(terms0[0])
    w0 = dev_bf16(layer["w0"]) if base else None
    def nbytes(t):
        if isinstance(t, tuple) and not hasattr(t, "_fields"):
            return sum(nbytes(u) for u in t)
        return sum(v.numel() * v.element_size() for v in t)

    if args.shared:
        terms0 = [terms0[0]] + [tcls(terms0[0].b1, terms0[0].b2, *t[2:]) for t in terms0[1:]]
    copy_bytes = sum(nbytes(t) for t in terms0)
    if base:
        copy_bytes += w0.numel() * 2
    ncopies = max(1, min(int(math.ceil(args.rotate_gib * 2 ** 30 / copy_bytes)), 4096))
    copies = [(terms0, w0)]
    for _ in range(ncopies - 1):
        if args.backward:
            copies.append(([(type(a)(*[v.clone() for v in a]), type(b)(*[v.clone() for v in b]))
                            for a, b in terms0], None))
        elif args.shared:
            b1, b2 = terms0[0].b1.clone(), terms0[0].b2.clone()
            copies.append(([tcls(b1, b2, *[v.clone() for v in t[2:]]) for t in terms0], None))
        else:
            copies.append(([tcls(*[v.clone() for v in t]) for t in terms0],
                           w0.clone() if base else None))

    y = torch.empty((T, N), dtype=torch.bfloat16, device=DEV)
    if args.backward:
        nws = D.dbf_backward_workspace_bytes(N, M, R, L, T, args.path)
        gdx = torch.empty((T, M), dtype=torch.bfloat16, device=DEV)
    elif boolk:
        nws = D.dbf_bool_workspace_bytes(N, M, L, T, args.path)
    elif base:
        nws = D.dbf_workspace_bytes(N, M, R, L, T, D.DBF_PATH_DECODE)
    else:
        nws = D.dbf_workspace_bytes(N, M, R, L, T, args.path)
    ws = torch.zeros(max(nws, 16), dtype=torch.uint8, device=DEV)

    def step(i):
        terms, w = copies[i % ncopies]
        if multi:
            D.lordba_multi_adapter_forward(w, terms, N, M, R, midx, x, y=y, ws=ws)
        elif args.backward:
            D.dbf_linear_backward([a for a, _ in terms], [b for _, b in terms], N, M, R, x, dy,
                                  dx_dtype=torch.bfloat16, ws=ws, path=args.path)
        elif boolk:
            D.dbf_bool_forward(terms, N, M, x, y=y, ws=ws, path=args.path)
        elif base:
            D.lordba_adapter_forward(w, terms, N, M, R, x, y=y, ws=ws)
        else:
            D.dbf_linear_forward(terms, N, M, R, x, y=y, ws=ws, path=args.path)

    ms = time_steps(step, args.steps, args.warmup)

    if args.backward:
        bytes_alg, flops = algorithmic_backward(N, M, R, L, T)
    elif multi:
        # W0 once, each adapter the batch uses once, x and y
        bytes_alg, flops = algorithmic(args.config, N, M, R, 1, T, True)
        used = min(multi, T)
        bytes_alg += (used - 1) * (R * (N + M) / 8.0 + 2.0 * (N + R + M))
    elif args.shared:
        # the signs once, every term's scales
        bytes_alg, flops = algorithmic(args.config, N, M, R, 1, T, False)
        bytes_alg += 2.0 * (L - 1) * (N + R + M)
        flops *= L
    elif boolk:
        bytes_alg, flops = algorithmic_bool(N, M, L, T)
    else:
        bytes_alg, flops = algorithmic(args.config, N, M, R, L, T, base)
    tok_s = T / (ms * 1e-3)
    gbs = bytes_alg / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    if args.backward:
        path = {1: "decode", 2: "mfma"}.get(args.path) or auto_path(T, 1, 4)
    else:
        path = "adapter" if base else ({1: "decode", 2: "mfma"}.get(args.path)
                                       or (auto_bool_path(T, L) if boolk
                                           else auto_dbf_path(N, M, R, L, T)))
    # achieved = algorithmic bytes (flops) per step / HIP-event time per step;
    # decode and adapter steps are one kernel launch each, the MFMA step is
    # three (prep, stage-1 GEMM, stage-2 GEMM) and is rated as a whole
    if path == "mfma":
        roof = {"bound": "mfma", "achieved": round(tflops, 2),
                "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)}
    roof["traffic"] = traffic_for(args, T)

    check = None
    if args.backward:
        args.no_check = True  # parity of the backward: tests/test_gpu_backward.py
    if not args.no_check:
        check = verify(layer, x_np, x, y, copies[(args.steps - 1) % ncopies], base,
                       N, M, R, T, args, step_index=args.steps - 1, ws=ws)

    cpu = None if args.no_cpu else cpu_baseline(layer, args.config, T, base, boolk,
                                                backward=args.backward)

    # the metric's second operating point, in the same run as the first
    prefill = None
    default_run = (args.config == 2 and args.tokens is None and args.path == D.DBF_PATH_AUTO
                   and not (args.backward or args.shared or multi))
    if default_run and not args.no_prefill:
        del copies
        torch.cuda.empty_cache()
        prefill = prefill_point(args)

    copy_probe = None
    if args.copy_probe:
        a = torch.empty(64 * 2 ** 20, dtype=torch.int32, device=DEV)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        copy_probe = {"bytes_read": a.numel() * 4, "bytes_written": b.numel() * 4}

    name = cfgd["name"] + ("-r%d" % R if base else "") + ("-backward" if args.backward else "")
    if args.shared:
        name = "lordba-envelope-%dx%d-r%d-l%d-shared" % (N, M, R, L)
    if multi:
        name += "-multi%d" % multi
    shape = ({"N": N, "M": M, "kernels": L} if boolk else
             {"N": N, "M": M, "R": R, "terms": L})
    out = {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # arithmetic the path computes in: fp32 table sums (decode), fp16
        # MFMA products with fp32 sums (MFMA), bf16 MFMA products (adapter)
        "dtype": {"decode": "f32", "mfma": "f16", "adapter": "bf16"}[path],
        "data": "synthetic (seeded i.i.d. signs and scales of the configuration)",
        "config": {"workload": name, **shape,
                   "tokens": T, "path": path,
                   "x_dtype": "f16" if x_np.dtype == np.float16 else "bf16",
                   "rotated_copies": ncopies,
                   "copies_touched": min(args.steps, ncopies),
                   "cache_scrub_bytes": SCRUB_BYTES,
                   "algorithmic_bytes": int(bytes_alg), "algorithmic_flops": int(flops),
                   "effective_GBps": round(gbs, 1), "effective_TFLOPs": round(tflops, 3)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "check": check,
    }
    if prefill is not None:
        out["mfma_4096"] = prefill
    if copy_probe:
        out["copy_probe"] = copy_probe
    print(json.dumps(out), flush=True)


SCRUB_BYTES = 1 << 30
_scrub = None


def time_steps(step, steps, warmup):
    """W eager steps, then K steps captured in one HIP graph; one untimed
    replay, a 1 GiB read-and-write of another buffer (so no step finds its
    inputs in the last-level cache or an L2), then the timed replay between
    two HIP events on the capturing stream.  Returns ms per step."""
    global _scrub
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(steps):
            step(i)
    g.replay()
    torch.cuda.synchronize()
    if _scrub is None:
        _scrub = torch.zeros(SCRUB_BYTES // 4, dtype=torch.int32, device=DEV)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        _scrub.add_(1)
        start.record(stream)
        g.replay()
        end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def prefill_point(args, T=4096, steps=10, warmup=2):
    """The 8192 x 8192, R 6144 layer on 4096 tokens (the path picks MFMA),
    timed as above, rated against the dense fp16 matrix peak; its output is
    checked against the oracle on one token of each 128-token tile."""
    import oracle as O

    layer = S.make_layer(5)
    N, M, R = layer["N"], layer["M"], layer["R"]
    x_np = S.make_x(5, T)
    x = dev_x(x_np)
    terms = [D.DbfTerm(D.dbf_pack(torch.from_numpy(t["b1"]).to(DEV)),
                       D.dbf_pack(torch.from_numpy(t["b2"]).to(DEV)),
                       dev_f16(t["alpha"]), dev_f16(t["beta"]), dev_f16(t["gamma"]))
             for t in layer["terms"]]
    y = torch.empty((T, N), dtype=torch.bfloat16, device=DEV)
    ws = torch.zeros(D.dbf_workspace_bytes(N, M, R, 1, T, D.DBF_PATH_AUTO), dtype=torch.uint8,
                     device=DEV)

    def step(i):
        D.dbf_linear_forward(terms, N, M, R, x, y=y, ws=ws)

    ms = time_steps(step, steps, warmup)
    bytes_alg, flops = algorithmic(5, N, M, R, 1, T, False)
    tflops = flops / (ms * 1e-3) / 1e12
    check = None
    if not args.no_check:
        toks = np.arange(0, T, 128) + (np.arange(T // 128) * 37) % 128
        ref = O.default().forward(O.terms64(layer), widen_x(x_np[toks]))
        got = O.widen_bf16(y[torch.from_numpy(toks).to(DEV)].view(torch.int16).cpu().numpy()
                           .view(np.uint16))
        from bit_adapters_amd.synth import f32_to_bf16_bits
        ref_b = O.widen_bf16(f32_to_bf16_bits(ref.astype(np.float32)))
        rel = float(np.linalg.norm(got - ref_b) / np.linalg.norm(ref_b))
        mx = float(np.abs(got - ref_b).max() / np.abs(ref_b).max())
        check = {"tokens_checked": len(toks), "rel_l2_vs_oracle_bf16": round(rel, 7),
                 "max_abs": round(mx, 7), "ok": rel <= 2e-3 and mx <= 1e-2}
    return {"workload": S.CONFIGS[5]["name"], "N": N, "M": M, "R": R, "terms": 1,
            "tokens": T, "path": "mfma", "dtype": "f16", "steps": steps, "warmup": warmup,
            "ms_per_step": round(ms, 6), "tokens_per_s": round(T / (ms * 1e-3), 1),
            "algorithmic_flops": int(flops), "algorithmic_bytes": int(bytes_alg),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                         "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4)},
            "check": check}


def traffic_for(args, T):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel sources; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        db = json.load(f)
    key = "c%d-t%d%s-p%d" % (args.config, T, "-r%d" % args.rank if args.config == 3 else "",
                             args.path)
    ent = db.get(key)
    if not ent or ent.get("sources") != kernel_sources_digest():
        return None
    return ent.get("bytes_per_launch")


def verify(layer, x_np, x, y, copy, base, N, M, R, T, args, step_index, ws):
    """The graph's last output vs an eager call on the same copy (bitwise) and
    vs the oracle on sampled rows."""
    import oracle as O

    yg = y.clone()
    terms, w = copy
    ye = torch.empty_like(y)
    boolk = args.config in S.BOOL_CONFIGS
    if args.multi:
        midx = torch.arange(T, dtype=torch.int32, device=DEV) % args.multi
        D.lordba_multi_adapter_forward(w, terms, N, M, R, midx, x, y=ye, ws=ws)
    elif boolk:
        D.dbf_bool_forward(terms, N, M, x, y=ye, ws=ws, path=args.path)
    elif base:
        D.lordba_adapter_forward(w, terms, N, M, R, x, y=ye, ws=ws)
    else:
        D.dbf_linear_forward(terms, N, M, R, x, y=ye, ws=ws, path=args.path)
    torch.cuda.synchronize()
    same = bool(torch.equal(yg, ye))
    toks = list(range(min(T, 4)))
    xs = widen_x(x_np[toks])
    if boolk:
        ref = O.default().bool_forward(bool64(layer), xs)
    else:
        ref = O.default().forward(O.terms64(layer), xs)
    if base:
        ref = ref + O.default().dense(O.widen_bf16(layer["w0"]), xs)
    from bit_adapters_amd.synth import f32_to_bf16_bits
    ref_b = O.widen_bf16(f32_to_bf16_bits(ref.astype(np.float32)))
    got = O.widen_bf16(yg[toks].view(torch.int16).cpu().numpy().view(np.uint16))
    rel = float(np.linalg.norm(got - ref_b) / np.linalg.norm(ref_b))
    mx = float(np.abs(got - ref_b).max() / np.abs(ref_b).max())
    ok = same and rel <= 2e-3 and mx <= 1e-2
    if not ok:
        print("bench check failed: graph==eager %s rel_l2 %.3e max_abs %.3e"
              % (same, rel, mx), file=sys.stderr)
    return {"graph_equals_eager": same, "tokens_checked": len(toks),
            "rel_l2_vs_oracle_bf16": round(rel, 7), "max_abs": round(mx, 7), "ok": ok}


def bool64(layer):
    return [dict(w=k["w"], s_in=np.asarray(k["s_in"], np.float64),
                 s_out=np.asarray(k["s_out"], np.float64)) for k in layer["kernels"]]


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(layer, config, T, base, boolk=False, budget_s=12.0, budget1_s=5.0,
                 backward=False):
    """The fp64 oracle on the host over a bounded sample of the same
    workload: whole tokens of the same layer, until about budget_s seconds on
    every thread the oracle uses, then about budget1_s seconds on one."""
    import oracle as O

    o = O.default()
    cfgd = S.BOOL_CONFIGS[config] if boolk else S.CONFIGS[config]
    terms = bool64(layer) if boolk else O.terms64(layer)
    xs = widen_x(S.make_x(config, max(cfgd["T"])))
    w0 = O.widen_bf16(layer["w0"]) if base else None

    def run(budget):
        done, t0 = 0, time.perf_counter()
        while True:
            tok = xs[done % xs.shape[0]][None, :]
            if boolk:
                o.bool_forward(terms, tok)
            elif backward:
                o.backward(terms, tok, np.ones((1, layer["N"])))
            else:
                o.forward(terms, tok)
            if base:
                o.dense(w0, tok)
            done += 1
            el = time.perf_counter() - t0
            if el >= budget or done >= 1 << 20:
                return done, el

    cores = o.threads()
    done, el = run(budget_s)
    o.set_threads(1)
    done1, el1 = run(budget1_s)
    o.set_threads(cores)
    what = "backwards" if backward else "forwards"
    return {"value": round(done / el, 3), "unit": "tokens/s", "cores": cores,
            "kind": "oracle", "cpu_model": cpu_model(),
            "value_1_thread": round(done1 / el1, 3),
            "sample": "%d single-token %s of the same layer on %d threads (%.1f s), then %d on "
                      "one thread (%.1f s), fp64" % (done, what, cores, el, done1, el1)}


if __name__ == "__main__":
    main()
