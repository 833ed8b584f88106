"""Throughput of the fused exact-attention path on one MI355X.

One step = the whole hot path over the long-context workload (B=1, H=16,
S=32768, d=128, bf16): forward + backward without mask, then forward +
backward with the causal mask.  FLOPs are counted the usual way for
attention: forward 4*B*H*S^2*d, backward 2.5x that, both halved under the
causal mask.  Inputs are seeded synthetic N(0,1) draws already resident in
HBM before the timed region.

Prints ONE JSON line (rank 0) with the step throughput, the per-part
figures, the roofline of the dominant kernel (its time measured with HIP
events on the launch stream inside the timed region) and the CPU oracle
timed on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --configs | --varlen | --ablation   (other measurements, see --help)
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention TFLOPS fwd/bwd, bf16 d=128 S=32k causal+noncausal; % MFMA peak"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA peak (published)
WORKLOAD = "long_b1_h16_s32768"
TRAFFIC_DIR = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["fa_common.h", "fa_fwd.hip", "fa_bwd.hip"]


def flops(B, H, S, d, causal, bwd):
    f = 4.0 * B * H * S * S * d
    if bwd:
        f *= 2.5
    return f / 2 if causal else f


def kernel_source_hash():
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "exact_attention_39_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_bytes(kname, causal):
    """HBM bytes per launch of a kernel from the committed counter summary
    (profiles/traffic_long_s32768.txt: FETCH_SIZE and WRITE_SIZE of each
    launch, scaled by what they read for a 1 GiB copy), or None if absent or
    taken on other kernel sources."""
    vals = {}
    try:
        with open(os.path.join(TRAFFIC_DIR, "traffic_long_s32768.txt")) as f:
            for line in f:
                parts = line.split()
                if len(parts) == 2 and not line.startswith("#"):
                    vals[parts[0]] = parts[1]
    except OSError:
        return None
    if vals.get("source_sha256") != kernel_source_hash():
        return None
    v = vals.get(f"{kname}{'_causal' if causal else ''}")
    return None if v is None else float(v)


def cpu_baseline(bits, S, d, scale, rows_n=2048):
    """The oracle as it stands on `rows_n` query rows of one head (non-causal):
    forward rows plus the dQ rows of the backward."""
    import numpy as np

    import attn_inputs as gen
    import oracle

    threads = min(os.cpu_count() or 1, 16)
    Q, K, V, dO = (gen.bf16_bits_to_f64(bits[t][0, 0]) for t in ("q", "k", "v", "do"))
    rows = np.linspace(0, S - 1, rows_n).astype(np.int64)
    t0 = time.perf_counter()
    oracle.forward_rows(Q, K, V, rows, scale, False, nthreads=threads)
    oracle.backward_dq_rows(Q, K, V, dO, rows, scale, False, nthreads=threads)
    dt = time.perf_counter() - t0
    counted = rows_n * (4.0 + 10.0) * S * d
    cpu = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), cpu)
    except OSError:
        pass
    return {"value": counted / dt / 1e12, "unit": "TFLOPS", "cores": threads, "kind": "oracle",
            "sample": f"{rows_n} query rows of head 0, non-causal S={S} d={d} on {threads} threads of "
                      f"{os.cpu_count()} ({cpu}): oracle forward_rows + "
                      f"backward_dq_rows, {dt:.1f} s; credited (4+10)*S*d FLOP per row like the GPU step "
                      f"(the dQ-rows routine does 8*S*d of the 10*S*d, so the CPU figure is flattered)"}


def _time(fn, reps=5, warm_calls=10):
    """Mean milliseconds of fn() over reps launches (events on the current
    stream) after 1 + warm_calls untimed ones: a fixed number of launches per
    call, so that counter runs can attribute dispatches to configurations."""
    import torch
    for _ in range(1 + warm_calls):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def _sweep(configs, rounds=3):
    """Median launch time of each (key, launch) in configs, the
    configurations interleaved over `rounds` rounds so that clock and
    warm-up drift do not favour any of them (after 300 ms of warm-up on the
    first configuration)."""
    times = {}
    print(f"[ablation] sweep of {len(configs)} configurations: {_warm(configs[0][1])} warm-up launches of the "
          "first, then per round and configuration 16 launches", file=sys.stderr, flush=True)
    for _ in range(rounds):
        for key, fn in configs:
            times.setdefault(key, []).append(_time(fn))
    return {k: sorted(v)[len(v) // 2] for k, v in times.items()}


def ablation(fa, gen, dev, q, k, v, do, B, H, S, d, scale):
    """One JSON line: kernel times under each softmax option and causal order
    (medians of three interleaved rounds)."""
    import torch
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    dq = torch.empty((B, H, S, d), dtype=torch.float32, device="cuda")
    dk, dv = torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, S, d) // 4, dtype=torch.float32, device="cuda")
    rows = []
    opts = [(8.0, 0, 3), (0.0, 0, 3), (8.0, 1, 3), (8.0, 2, 3), (8.0, 1, 5), (8.0, 2, 5)]

    def option_rows(wname, qq, kk, vv, oo, ll, sc, shape, options, causals):
        cfgs = [((opt, causal),
                 (lambda causal=causal, opt=opt: fa.fa_fwd(qq, kk, vv, oo, ll, sc, causal, opts=fa.Options(*opt))))
                for opt in options for causal in causals]
        med = _sweep(cfgs)
        for (opt, causal), ms in med.items():
            fl = flops(*shape, causal, False)
            rows.append({"kernel": "fwd", "workload": wname, "causal": causal, "tau": opt[0],
                         "poly_eighths": opt[1], "poly_degree": opt[2], "ms": round(ms, 4),
                         "tflops": round(fl / ms / 1e9, 1)})

    option_rows(WORKLOAD, q, k, v, o, lse, scale, (B, H, S, d), opts, (False, True))
    # the same options at a shorter sequence (B = 4, H = 16, S = 4096), and
    # the rescale threshold on the workload built to move the running max
    for wname, options, causals in (("fwd_b4_h16_s4096", opts[:4], (False, True)),
                                    ("causal_boost_b2_h16_s8192", [(0.0, 0, 3), (2.0, 0, 3), (8.0, 0, 3)],
                                     (True,))):
        w = gen.WORKLOADS[wname]
        bb = gen.workload_inputs(wname, ("q", "k", "v"))
        qs, ks, vs = (dev(bb[t]) for t in "qkv")
        os_ = torch.empty_like(qs)
        ls = torch.empty(qs.shape[:3], dtype=torch.float32, device="cuda")
        option_rows(wname, qs, ks, vs, os_, ls, gen.default_scale(w["d"]), (w["B"], w["H"], w["S"], w["d"]),
                    options, causals)
        del qs, ks, vs, os_, ls
    # causal block order: longest first (LPT) vs shortest first
    fa.fa_fwd(q, k, v, o, lse, scale, True)
    fa.fa_bwd_preprocess(o, do, lse, ws)
    kernels = (("fwd", lambda op: fa.fa_fwd(q, k, v, o, lse, scale, True, opts=op), flops(B, H, S, d, True, False)),
               ("bwd_dkdv", lambda op: fa.fa_bwd_dkdv(q, k, v, do, dk, dv, scale, True, ws, opts=op),
                0.8 * flops(B, H, S, d, True, True)),
               ("bwd_dq", lambda op: fa.fa_bwd_dq(q, k, v, do, dq, scale, True, ws, opts=op),
                0.2 * flops(B, H, S, d, True, True)))
    cfgs = [((name, lpt), (lambda fn=fn, lpt=lpt: fn(fa.Options(longest_first=lpt))))
            for lpt in (True, False) for name, fn, _ in kernels]
    med = _sweep(cfgs)
    fl_of = {name: fl for name, _, fl in kernels}
    for (name, lpt), ms in med.items():
        rows.append({"kernel": name, "workload": WORKLOAD, "causal": True, "longest_first": lpt,
                     "ms": round(ms, 4), "tflops": round(fl_of[name] / ms / 1e9, 1)})
    print(json.dumps({"ablation": rows}), flush=True)


def varlen_bench(fa, gen, args, name="prefill_varlen_h16_d128"):
    """Forward-only prefill over a packed batch of causal sequences of mixed
    lengths: TFLOPS = sum over sequences of 2 * H * L^2 * d (the causal half
    of 4 * H * L^2 * d) / mean time of one fa_fwd_varlen call."""
    import numpy as np
    import torch

    w = gen.VARLEN_WORKLOADS[name]
    print(f"[bench] generating inputs {name}", file=sys.stderr, flush=True)
    lens, bits = gen.varlen_inputs(name)
    H, d = w["H"], w["d"]
    total = int(lens.sum())
    scale = gen.default_scale(d)

    def dev(b):
        return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).cuda()

    q, k, v = (dev(bits[t]) for t in ("q", "k", "v"))
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).cuda()
    o = torch.empty_like(q)
    lse = torch.empty((H, total), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    maxlen = int(lens.max())
    call = lambda: fa.fa_fwd_varlen(q, k, v, o, lse, cu, maxlen, scale, w["causal"], stream)
    for _ in range(args.warmup):
        call()
    _warm(call)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    fl = float(sum(4.0 * H * float(L) ** 2 * d * (0.5 if w["causal"] else 1.0) for L in lens))
    tf = fl / (ms / 1e3) / 1e12
    print(json.dumps({
        "metric": "prefill forward TFLOPS, packed variable-length causal batch, bf16 d=128",
        "value": round(tf, 1), "unit": "TFLOPS", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 3), "higher_is_better": True, "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic", "pct_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
        "config": {"workload": name, "nseq": int(len(lens)), "total_tokens": total, "H": H, "d": d,
                   "min_len": int(lens.min()), "max_len": maxlen, "causal": w["causal"]},
    }))


GEMM_N = 16384


def gemm_ceiling(args):
    """The practical MFMA ceiling on this GPU: the library bf16 GEMM
    (torch.matmul -> hipBLASLt), n = 16384, on N(0,1) operands (the data the
    attention workloads feed their MFMAs) and on constant operands (all ones,
    which toggle no datapath bits and so draw less power).  3 warm-up calls,
    then 10 calls timed one by one with HIP events; TFLOPS = 2 n^3 / median.
    One JSON line per operand kind."""
    import torch
    n = GEMM_N
    g = torch.Generator(device="cuda")
    g.manual_seed(0xFA)
    for kind in ("normal", "ones"):
        if kind == "normal":
            a = torch.randn((n, n), device="cuda", generator=g).to(torch.bfloat16)
            b = torch.randn((n, n), device="cuda", generator=g).to(torch.bfloat16)
        else:
            a = torch.ones((n, n), device="cuda", dtype=torch.bfloat16)
            b = torch.ones((n, n), device="cuda", dtype=torch.bfloat16)
        c = torch.empty((n, n), device="cuda", dtype=torch.bfloat16)
        med, mn = _events_ms(lambda: torch.matmul(a, b, out=c), warmup=3, reps=10)
        tf = 2.0 * n ** 3 / (med / 1e3) / 1e12
        print(json.dumps({"metric": "library bf16 GEMM TFLOPS (median of 10 calls)", "operands": kind, "n": n,
                          "value": round(tf, 1), "unit": "TFLOPS", "ms_median": round(med, 4),
                          "ms_min": round(mn, 4), "pct_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2)}), flush=True)
        del a, b, c
        torch.cuda.empty_cache()


def gemm_ceiling_tflops():
    """The N(0,1) GEMM rate recorded in profiles/gemm_ceiling.txt (line
    `ceiling_tflops_normal V`), or None."""
    try:
        with open(os.path.join(TRAFFIC_DIR, "gemm_ceiling.txt")) as f:
            for line in f:
                parts = line.split()
                if len(parts) == 2 and parts[0] == "ceiling_tflops_normal":
                    return float(parts[1])
    except (OSError, ValueError):
        pass
    return None


def _warm(fn, min_ms=300.0, max_calls=2000):
    """Call fn() until at least min_ms of GPU time has passed (the clock of an
    idle GPU takes a while to come up; a few calls of a sub-millisecond
    kernel are not enough).  Returns the number of calls."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n, calls = 1, 0
    while True:
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        calls += n
        if e0.elapsed_time(e1) >= min_ms or n >= max_calls:
            return calls
        n = min(max_calls, n * 4)


def _events_ms(fn, warmup=3, reps=20):
    """Per-call milliseconds of fn() (HIP events on the current stream around
    each call) after `warmup` untimed calls and at least 300 ms of warm-up:
    (median, min)."""
    import torch
    for _ in range(warmup):
        fn()
    _warm(fn)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in evs:
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    t = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    return t[len(t) // 2], t[0]


def configs_bench(fa, gen, args):
    """Every workload of the suite, each direction it runs: 3 warm-up calls,
    then 20 calls timed one by one; TFLOPS = counted FLOPs / median time.
    One JSON line per (workload, mask, direction)."""
    import numpy as np
    import torch

    def dev(b):
        return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).cuda()

    for name, w in gen.WORKLOADS.items():
        B, H, S, d = w["B"], w["H"], w["S"], w["d"]
        scale = gen.default_scale(d)
        print(f"[bench] configs: {name}", file=sys.stderr, flush=True)
        tensors = ("q", "k", "v", "do") if w["bwd"] else ("q", "k", "v")
        bits = gen.workload_inputs(name, tensors)
        t = {k: dev(b) for k, b in bits.items()}
        del bits
        o = torch.empty_like(t["q"])
        lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
        for causal in w["causal"]:
            runs = [("fwd", lambda: fa.fa_fwd(t["q"], t["k"], t["v"], o, lse, scale, causal))]
            if w["bwd"]:
                fa.fa_fwd(t["q"], t["k"], t["v"], o, lse, scale, causal)
                dq = torch.empty((B, H, S, d), dtype=torch.float32, device="cuda")
                dk, dv = torch.empty_like(t["q"]), torch.empty_like(t["q"])
                ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, S, d) // 4, dtype=torch.float32, device="cuda")
                runs.append(("bwd", lambda: fa.fa_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], dq, dk, dv,
                                                      scale, causal, ws)))
                # the same backward with the stored-dS option (its own, larger workspace)
                on = fa.Options(stored_ds=True)
                ws2 = torch.empty((fa.fa_bwd_workspace_bytes(B, H, S, d, causal, on) + 3) // 4,
                                  dtype=torch.float32, device="cuda")
                runs.append(("bwd_stored_ds", lambda: fa.fa_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], dq, dk,
                                                                dv, scale, causal, ws2, opts=on)))
            for direction, fn in runs:
                med, mn = _events_ms(fn)
                fl = flops(B, H, S, d, causal, direction != "fwd")
                tf = fl / (med / 1e3) / 1e12
                print(json.dumps({
                    "metric": f"attention {direction} TFLOPS (median of 20 calls)", "value": round(tf, 1),
                    "unit": "TFLOPS", "n_gpus": 1, "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
                    "ms_median": round(med, 4), "ms_min": round(mn, 4), "pct_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
                    "config": {"workload": name, "B": B, "H": H, "S": S, "d": d, "causal": causal,
                               "boost": w["boost"]},
                }), flush=True)
            runs.clear()
            torch.cuda.empty_cache()
        del t, o, lse
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stored-ds", action="store_true",
                    help="skip the second timing of the step with the stored-dS backward")
    ap.add_argument("--cpu-rows", type=int, default=24576)
    ap.add_argument("--varlen", action="store_true",
                    help="time the packed variable-length prefill forward (fa_fwd_varlen) on the "
                         "prefill_varlen_h16_d128 batch instead of the step; prints its own JSON line")
    ap.add_argument("--configs", action="store_true",
                    help="time every workload of the suite and direction it runs (3 warm-up calls, "
                         "20 timed calls, median and minimum); one JSON line each, instead of the step")
    ap.add_argument("--ablation", action="store_true",
                    help="time the softmax options (hybrid exp share, polynomial degree, rescale "
                         "threshold) and the causal block order instead of the step")
    ap.add_argument("--gemm-ceiling", action="store_true",
                    help="time the library bf16 GEMM (n = 16384) on N(0,1) and on constant operands: "
                         "the practical MFMA ceiling the attention kernels are compared with")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: this build measures one MI355X "
              "(each head is independent; the multi-GPU sharding is described, not built)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import attn_inputs as gen
    import exact_attention_39_amd as fa

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    fa.load_library()
    if args.gemm_ceiling:
        gemm_ceiling(args)
        return
    if args.varlen:
        varlen_bench(fa, gen, args)
        return
    if args.configs:
        configs_bench(fa, gen, args)
        return
    w = gen.WORKLOADS[WORKLOAD]
    B, H, S, d = w["B"], w["H"], w["S"], w["d"]
    scale = gen.default_scale(d)
    print(f"[bench] generating inputs {WORKLOAD} B={B} H={H} S={S} d={d}", file=sys.stderr, flush=True)
    bits = gen.workload_inputs(WORKLOAD, ("q", "k", "v", "do"))

    def dev(b):
        return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).cuda()

    q, k, v, do = (dev(bits[t]) for t in ("q", "k", "v", "do"))
    if args.ablation:
        ablation(fa, gen, dev, q, k, v, do, B, H, S, d, scale)
        return
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    dq = torch.empty((B, H, S, d), dtype=torch.float32, device="cuda")
    dk, dv = torch.empty_like(q), torch.empty_like(q)
    stream = torch.cuda.current_stream()

    parts = [("fwd", False), ("bwd_pre", False), ("bwd_dkdv", False), ("bwd_dq", False),
             ("fwd", True), ("bwd_pre", True), ("bwd_dkdv", True), ("bwd_dq", True)]
    NP = len(parts) // 2
    step_flop = sum(flops(B, H, S, d, c, bwd) for c in (False, True) for bwd in (False, True))

    def timed_steps(opts, tag):
        """Warm-up, then args.steps timed steps of the whole path with these
        backward options; (ms per step by the host clock, mean ms per part by
        HIP events on the launch stream)."""
        nbytes = max(fa.fa_bwd_workspace_bytes(B, H, S, d, c, opts) for c in (False, True))
        ws = torch.empty((nbytes + 3) // 4, dtype=torch.float32, device="cuda")

        def launch(kind, causal):
            if kind == "fwd":
                fa.fa_fwd(q, k, v, o, lse, scale, causal, stream)
            elif kind == "bwd_pre":
                fa.fa_bwd_preprocess(o, do, lse, ws, stream)
            elif kind == "bwd_dkdv":
                fa.fa_bwd_dkdv(q, k, v, do, dk, dv, scale, causal, ws, stream, opts)
            else:
                fa.fa_bwd_dq(q, k, v, do, dq, scale, causal, ws, stream, opts)

        def step(events=None):
            for i, (kind, causal) in enumerate(parts):
                if events is not None:
                    events[i].record(stream)
                launch(kind, causal)
            if events is not None:
                events[len(parts)].record(stream)

        print(f"[bench] {tag}: warmup {args.warmup}", file=sys.stderr, flush=True)
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(parts) + 1)] for _ in range(args.steps)]
        print(f"[bench] {tag}: timing {args.steps} steps", file=sys.stderr, flush=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(args.steps):
            step(evs[s])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        part_ms = [float(np.mean([evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(args.steps)]))
                   for i in range(len(parts))]
        del ws
        torch.cuda.empty_cache()
        return wall * 1e3 / args.steps, part_ms, nbytes

    ms_step, part_ms, _ = timed_steps(None, "default backward")
    value = step_flop / (ms_step / 1e3) / 1e12

    detail = {}
    for causal in (False, True):
        tag = "causal" if causal else "noncausal"
        i0 = 0 if not causal else NP
        f_ms = part_ms[i0]
        b_ms = part_ms[i0 + 1] + part_ms[i0 + 2] + part_ms[i0 + 3]
        for name, ms, fl in (("fwd", f_ms, flops(B, H, S, d, causal, False)),
                             ("bwd", b_ms, flops(B, H, S, d, causal, True))):
            tf = fl / (ms / 1e3) / 1e12
            detail[f"{name}_{tag}"] = {"ms": round(ms, 4), "tflops": round(tf, 1),
                                       "pct_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2)}
        detail[f"bwd_{tag}"]["preprocess_ms"] = round(part_ms[i0 + 1], 4)
        detail[f"bwd_{tag}"]["dkdv_ms"] = round(part_ms[i0 + 2], 4)
        detail[f"bwd_{tag}"]["dq_ms"] = round(part_ms[i0 + 3], 4)

    # dominant kernel: the longest launch of the step.  Algorithmic FLOPs per
    # launch: fwd 4*B*H*S^2*d; dK/dV kernel: S, dP, dV and dK contractions
    # (8*B*H*S^2*d); dQ kernel: the dQ contraction only (2*B*H*S^2*d) -- its
    # recomputed S and dP are extra work, not credited.  Halved when causal.
    dom = int(np.argmax(part_ms))
    kind, causal = parts[dom]
    kname = {"fwd": "fwd_kernel", "bwd_pre": "bwd_pre_kernel", "bwd_dkdv": "bwd_dkdv_kernel",
             "bwd_dq": "bwd_dq_kernel"}[kind]
    cfac = 0.5 if causal else 1.0
    if kind == "bwd_pre":
        alg = 2.0 * B * H * S * d * 2 + 4.0 * B * H * S * 3  # bytes: O, dO, LSE read; D, LSE2 written
        roof = {"bound": "hbm", "achieved": alg / (part_ms[dom] / 1e3) / 1e9, "peak": 8000.0, "unit": "GB/s"}
    else:
        alg = {"fwd": 4.0, "bwd_dkdv": 8.0, "bwd_dq": 2.0}[kind] * B * H * S * S * d * cfac
        roof = {"bound": "mfma", "achieved": alg / (part_ms[dom] / 1e3) / 1e12, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    if roof["unit"] == "TFLOP/s":
        # the library GEMM's rate on N(0,1) operands (profiles/gemm_ceiling.txt): what the same MFMAs
        # reach on this GPU under its power limit; frac stays against the published peak
        roof["ceiling"] = gemm_ceiling_tflops()
    roof["achieved"] = round(roof["achieved"], 1)
    roof["frac"] = round(roof["frac"], 4)
    roof["kernel"] = f"{kname}<d=128,causal={int(causal)}>"
    roof["launch_ms"] = round(part_ms[dom], 4)
    roof["traffic"] = traffic_bytes(kname, causal)
    roof["launch_ms_all"] = {f"{k}{'_causal' if c else ''}": round(m, 4) for (k, c), m in zip(parts, part_ms)}

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "TFLOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{WORKLOAD}: fwd+bwd non-causal then fwd+bwd causal",
                   "B": B, "H": H, "S": S, "d": d, "scale": scale, "global_batch": B, "seq_len": S,
                   "parallelism": "single GPU"},
        "pct_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "parts": detail,
        "roofline": roof,
    }
    if not args.no_stored_ds:
        # the same step with the stored-dS backward (fa_options.stored_ds): dQ
        # from the dS the dK/dV kernel wrote to the workspace, no recompute
        ms2, part2, nbytes2 = timed_steps(fa.Options(stored_ds=True), "stored-dS backward")
        alt = {"ms_per_step": round(ms2, 3), "value": round(step_flop / (ms2 / 1e3) / 1e12, 1),
               "workspace_gib": round(nbytes2 / 2 ** 30, 2)}
        for causal in (False, True):
            i0 = NP if causal else 0
            b_ms = part2[i0 + 1] + part2[i0 + 2] + part2[i0 + 3]
            tf = flops(B, H, S, d, causal, True) / (b_ms / 1e3) / 1e12
            alt[f"bwd_{'causal' if causal else 'noncausal'}"] = {
                "ms": round(b_ms, 4), "tflops": round(tf, 1), "pct_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
                "dkdv_ms": round(part2[i0 + 2], 4), "dq_ms": round(part2[i0 + 3], 4)}
        out["stored_ds_step"] = alt
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle on a row sample)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(bits, S, d, scale, args.cpu_rows)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
