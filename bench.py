"""Decode-step benchmark: split-KV decode attention at a 1M-token context on
one MI355X.

One step = the append of the newest token of every (request, KV head) and
the attention over all slices with their LSE combine, on one stream, with
the cache already resident in HBM: by default one hx_decode_step call (the
append inside the partial kernel, then one fold of the slice partials into
the final O and LSE); --append codes runs hx_kv_append, hx_decode_attn_partial
and hx_lse_combine as separate calls.  Inputs are synthetic (seeded), shaped
like the named workload.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload NAME]
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

from long_context_decode_split_amd import api, configs, roofline, synth

DEFAULT_WORKLOAD = configs.LLAMA405B_SHARE.name
METRIC = "µs/layer/decode step and KV-read HBM GB/s (% of peak) at 1M-token context"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def make_pool(desc, inp, seed):
    """A block pool holding every request's n tokens: lists grown by the host
    allocator, then each request's blocks shuffled among themselves (seeded)
    so that consecutive 16-row groups of a slice sit at scattered places of
    the pool, as after a long run of interleaved growth and recycling."""
    need = 0
    for n in inp.ctx:
        for r in range(desc.P):
            need += -(-api.slice_len(n, desc.P, r) // 16)
    pool = api.KVPool(desc, need, device="cuda")
    rng = np.random.default_rng(seed + 7)
    for b, n in enumerate(inp.ctx):
        pool.reserve(b, n)
        ids = pool.table_host[b][pool.table_host[b] >= 0]
        pool.table_host[b][pool.table_host[b] >= 0] = rng.permutation(ids)
    pool.sync()
    return pool


def setup(w, seed, append_bf16=False, layout="dense", flags=0):
    t0 = time.time()
    inp = synth.make_inputs(w, seed, device="cuda")
    desc = api.KVDesc(P=w.P, B=w.B, Hkv=w.Hkv, Dk=w.Dk, Dv=w.Dv, v_alias_k=w.v_alias_k, dtype=w.dtype, cap=inp.cap,
                      flags=flags)
    if layout == "paged":
        cache = make_pool(desc, inp, seed)
        append = api.kv_append_paged
    else:
        cache = api.KVCache(desc, device="cuda")
        append = api.kv_append
    # the cache holds n-1 tokens of every request before the step
    append(cache, inp.k, inp.v, inp.k_scale, inp.v_scale, pos=[0] * w.B, count=[n - 1 for n in inp.ctx])
    last = [n - 1 for n in inp.ctx]

    def newest(t):
        if t is None:
            return None
        return torch.stack([t[b, :, last[b]:last[b] + 1] for b in range(w.B)]).contiguous()

    step_in = dict(k=newest(inp.k), v=newest(inp.v), ks=newest(inp.k_scale), vs=newest(inp.v_scale), pos=last)
    if append_bf16:
        # the newest token as the bf16 values a QKV projection would produce, quantised by the append
        g = torch.Generator(device="cuda").manual_seed(seed + 1)
        step_in["kb"] = (torch.randn(w.B, w.Hkv, 1, w.Dk, generator=g, device="cuda") * w.std).to(torch.bfloat16)
        step_in["vb"] = None if w.v_alias_k else \
            (torch.randn(w.B, w.Hkv, 1, w.Dv, generator=g, device="cuda") * w.std).to(torch.bfloat16)
    ws = torch.zeros(api.workspace_size(desc, w.Hq), dtype=torch.uint8, device="cuda")
    o_part = torch.empty(w.P, w.B, w.Hq, w.Dv, dtype=torch.float32, device="cuda")
    lse_part = torch.empty(w.P, w.B, w.Hq, dtype=torch.float32, device="cuda")
    o = torch.empty(w.B, w.Hq, w.Dv, dtype=torch.float32, device="cuda")
    lse = torch.empty(w.B, w.Hq, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    log(f"[bench] setup {w.name}: ctx={inp.ctx[:4]}{'...' if w.B > 4 else ''} cap={inp.cap} "
        f"cache={cache.nbytes() / 1e9:.3f} GB in {time.time() - t0:.1f}s")
    return inp, cache, step_in, ws, o_part, lse_part, o, lse


def traffic_key(w, layout):
    return w.name if layout == "dense" else f"{w.name}+{layout}"


def kernel_src_hash(w):
    """Hash of the partial kernel's sources for workload w, to tell whether
    recorded counters still describe the kernel that runs."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for p in ("decode_mla.hip" if w.v_alias_k else "decode_gqa.hip", "hx_common.h"):
        with open(os.path.join(here, "long_context_decode_split_amd", "csrc", p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(w, layout="dense"):
    """HBM bytes per launch of the partial kernel from the rocprofv3
    FETCH_SIZE / WRITE_SIZE passes recorded in profiles/traffic.json (scaled by
    a copy of known size), or None when none was recorded for this workload
    and cache layout, or the kernel sources changed since."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(traffic_key(w, layout))
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_src_sha16") != kernel_src_hash(w):
        return None
    return int(rec["fetch_bytes"]) + int(rec["write_bytes"])


def cpu_baseline(inp, budget_s=20.0, o=None, lse=None):
    """The oracle (fp64, numpy) on a bounded sample of the same step: whole
    (request, KV head) groups over their full context, as many as fit the
    time budget (at least one); scaled to KV-read GB/s like the GPU value.
    With the step's final outputs `o`, `lse` (device tensors) it also
    returns their largest deviations from the oracle over those groups."""
    from oracle import attention as oatt
    from oracle import codecs as ocod

    w = inp.w
    G = w.G
    per_tok = roofline.kv_bytes_per_token(w.Dk, w.Dv, w.v_alias_k, w.dtype)
    done_bytes, t_total, groups = 0.0, 0.0, 0
    err_o = err_l = 0.0
    oc = None if o is None else o.float().cpu().numpy()
    lc = None if lse is None else lse.float().cpu().numpy()
    order = [(b, g) for b in range(w.B) for g in range(w.Hkv)]
    for b, g in order:
        n = inp.ctx[b]
        # host copies of the generator's storage-format tensors (not timed)
        kc = inp.k[b, g, :n].cpu()
        vc = None if inp.v is None else inp.v[b, g, :n].cpu()
        ks = None if inp.k_scale is None else inp.k_scale[b, g, :n].cpu().numpy()
        vs = None if inp.v_scale is None else inp.v_scale[b, g, :n].cpu().numpy()
        q = ocod.bf16_bits_to_f64(inp.q[b, g * G:(g + 1) * G].cpu().view(torch.int16).numpy().view(np.uint16))
        t0 = time.perf_counter()
        if w.dtype == "bf16":
            K = ocod.bf16_bits_to_f64(kc.view(torch.int16).numpy().view(np.uint16))
            V = K[:, :w.Dv] if w.v_alias_k else ocod.bf16_bits_to_f64(vc.view(torch.int16).numpy().view(np.uint16))
        elif w.dtype == "fp8_e4m3":
            K = ocod.dequant_fp8(kc.numpy(), ks[::16])
            V = K[:, :w.Dv] if w.v_alias_k else ocod.dequant_fp8(vc.numpy(), vs[::16])
        else:
            K = ocod.dequant_mxfp4(kc.numpy(), ks)
            V = K[:, :w.Dv] if w.v_alias_k else ocod.dequant_mxfp4(vc.numpy(), vs)
        O, L = oatt.attend(q, K, V, w.softmax_scale)
        t_total += time.perf_counter() - t0
        if oc is not None:
            err_o = max(err_o, float(np.max(np.abs(oc[b, g * G:(g + 1) * G] - O))))
            err_l = max(err_l, float(np.max(np.abs(lc[b, g * G:(g + 1) * G] - L) / np.maximum(1.0, np.abs(L)))))
        done_bytes += n * per_tok
        groups += 1
        del K, V
        if t_total >= budget_s:
            break
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    parity = None if oc is None else {
        "groups": groups, "max_abs_dO": err_o, "max_rel_dLSE": err_l,
        "bound_abs_dO": 2e-3 if w.dtype == "bf16" else 2e-2, "bound_rel_dLSE": 1e-4,
        "reference": "the oracle on the same stored K/V (dequantised values for fp8 / MXFP4)"}
    return parity, {
        "value": done_bytes / t_total / 1e9,
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{groups} of {len(order)} (request, KV head) groups of the same step, full context each; "
                  f"fp64 numpy unsplit attention incl. decoding the stored K/V; {t_total:.1f}s",
        "us_per_layer_step_extrapolated": t_total / done_bytes * roofline.kv_bytes(w, inp.ctx) * 1e6,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(configs.ALL))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--append", choices=("fused", "codes", "bf16"), default="fused",
                    help="fused (default): the whole step is one hx_decode_step call (the newest token appended in "
                         "storage format inside the partial kernel, then the final O and LSE); codes: "
                         "hx_kv_append, then the attention calls of --attn; bf16: as codes, with bf16 values "
                         "quantised on the device (hx_kv_append_bf16)")
    ap.add_argument("--attn", choices=("partial+combine", "one-call"), default="partial+combine",
                    help="partial+combine: hx_decode_attn_partial then hx_lse_combine (the slice partials are "
                         "outputs); one-call: hx_decode_attn (final O and LSE only; one launch for small problems)")
    ap.add_argument("--layout", choices=("dense", "paged"), default="dense",
                    help="dense: [P][B][Hkv][cap/16] cache planes; paged: a block pool with per-(request, slice) "
                         "16-row block lists, each request's blocks shuffled among themselves (the *_paged calls)")
    ap.add_argument("--p-bf16", action="store_true",
                    help="HX_FLAG_P_BF16: the MLA value product takes P rounded once to bf16 (faster, less precise)")
    ap.add_argument("--graph", action="store_true",
                    help="time the step as one captured HIP graph per step (the partial call is still timed on "
                         "eager launches)")
    ap.add_argument("--flush-cache", action="store_true",
                    help="write a 1 GiB buffer before every step (outside the timed events) so that no KV bytes "
                         "survive in L2 or the 256 MB MALL; steps are then timed one by one")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes (5 times); used to scale the "
                         "HBM traffic counters of a profiler run")
    args = ap.parse_args()
    if args.calibrate_copy:
        src = torch.empty(args.calibrate_copy, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": args.calibrate_copy, "copies": 5}), flush=True)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: every KV-parallel slice lives in that GPU's HBM and the library has "
              "no collectives between GPUs; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    w = configs.ALL[args.workload]
    inp, cache, st, ws, o_part, lse_part, o, lse = setup(w, args.seed, append_bf16=args.append == "bf16",
                                                         layout=args.layout,
                                                         flags=api.HX_FLAG_P_BF16 if args.p_bf16 else 0)
    stream = torch.cuda.current_stream()
    paged = args.layout == "paged"
    append_bf16 = api.kv_append_bf16_paged if paged else api.kv_append_bf16
    append_codes = api.kv_append_paged if paged else api.kv_append
    attn_one = api.decode_attn_paged if paged else api.decode_attn
    attn_partial = api.decode_attn_partial_paged if paged else api.decode_attn_partial
    fused_step = api.decode_step_paged if paged else api.decode_step

    def step(ev=None, stream=stream):
        if args.append == "fused":
            if ev is not None:
                ev[0].record(stream)
            fused_step(cache, st["k"], st["v"], st["ks"], st["vs"], inp.q, inp.ctx, w.softmax_scale, o, lse, ws,
                       stream=stream)
            if ev is not None:
                ev[1].record(stream)
            return
        if args.append == "bf16":
            append_bf16(cache, st["kb"], st["vb"], pos=st["pos"], stream=stream)
        else:
            append_codes(cache, st["k"], st["v"], st["ks"], st["vs"], pos=st["pos"], stream=stream)
        if ev is not None:
            ev[0].record(stream)
        if args.attn == "one-call":
            attn_one(cache, inp.q, inp.ctx, w.softmax_scale, o, lse, ws, stream=stream)
            if ev is not None:
                ev[1].record(stream)
            return
        attn_partial(cache, inp.q, inp.ctx, w.softmax_scale, o_part, lse_part, ws, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        api.lse_combine(o_part, lse_part, o, lse, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    new_ev = lambda: torch.cuda.Event(enable_timing=True)
    kev = [(new_ev(), new_ev()) for _ in range(args.steps)]
    sev = [(new_ev(), new_ev()) for _ in range(args.steps)]
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda") if args.flush_cache else None
    start, end = new_ev(), new_ev()
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        if flush is not None:
            flush.fill_(i & 0xFF)
        sev[i][0].record(stream)
        step(kev[i])
        sev[i][1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    kern_ms = [a.elapsed_time(b) for a, b in kev]
    step_each_ms = [a.elapsed_time(b) for a, b in sev]
    kern_avg_ms = float(np.mean(kern_ms))
    # back-to-back steps: total over the timed region; flushed steps: each step on its own
    step_ms = float(np.mean(step_each_ms)) if flush is not None else start.elapsed_time(end) / args.steps
    if args.graph:
        # the same step captured once and replayed: no host launch work between its kernels
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step(stream=side)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step(stream=torch.cuda.current_stream())
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        gev = [(new_ev(), new_ev()) for _ in range(args.steps)]
        start.record(stream)
        for i in range(args.steps):
            if flush is not None:
                flush.fill_(i & 0xFF)
            gev[i][0].record(stream)
            graph.replay()
            gev[i][1].record(stream)
        end.record(stream)
        torch.cuda.synchronize()
        step_each_ms = [a.elapsed_time(b) for a, b in gev]
        step_ms = float(np.mean(step_each_ms)) if flush is not None else start.elapsed_time(end) / args.steps
    pct = lambda x: {f"p{q}": round(float(np.percentile(x, q)) * 1e3, 2) for q in (10, 50, 90)}

    nbytes = roofline.kv_bytes(w, inp.ctx)
    flops = roofline.attn_flops(w, inp.ctx)
    step_gbs = nbytes / (step_ms * 1e-3) / 1e9
    kern_gbs = nbytes / (kern_avg_ms * 1e-3) / 1e9
    peak_gbs = roofline.HBM_PEAK_BYTES_PER_S / 1e9
    log(f"[bench] step {step_ms * 1e3:.1f} us, partial kernel {kern_avg_ms * 1e3:.1f} us "
        f"(min {min(kern_ms) * 1e3:.1f}, max {max(kern_ms) * 1e3:.1f}), {kern_gbs:.0f} GB/s")

    cpu = parity = None
    if not args.no_cpu_baseline:
        parity, cpu = cpu_baseline(inp, args.cpu_budget, o, lse)
        log(f"[bench] cpu oracle: {cpu['value']:.3f} GB/s ({cpu['sample']}); "
            f"max |dO| {parity['max_abs_dO']:.2e}, LSE rel {parity['max_rel_dLSE']:.2e}")

    out = {
        "metric": METRIC,
        "value": round(step_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 6),
        "us_per_layer_step": round(step_ms * 1e3, 2),
        "frac_of_hbm_peak": round(step_gbs / peak_gbs, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8_e4m3": "fp8_e4m3 KV, bf16 MFMA, fp32 acc",
                  "mxfp4": "mxfp4 KV, bf16 MFMA, fp32 acc"}[w.dtype] if w.dtype != "bf16" else "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "Dk": w.Dk, "Dv": w.Dv,
            "v_alias_k": w.v_alias_k, "kv_dtype": w.dtype, "slices": w.P,
            "context": inp.ctx if w.ctx is None else w.ctx, "kv_bytes_per_step": nbytes, "seed": args.seed,
            "append": {"bf16": "bf16 values quantised on the device", "codes": "storage format",
                       "fused": "storage format, inside the attention call (hx_decode_step)"}[args.append],
            "attention": "one-call" if args.append == "fused" else args.attn,
            "layout": "block pool, 16-row blocks shuffled within each request" if paged else "dense planes",
            "launch": "one HIP graph replay per step" if args.graph else "eager launches",
            "p_in_value_product": ("bf16, rounded once" if args.p_bf16 or w.dtype != "bf16"
                                   else "bf16 high part + bf16 residual"),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": ("decode_step" if args.append == "fused" else "decode_attn" if args.attn == "one-call"
                       else "decode_attn_partial") + ("_paged" if paged else ""),
            "achieved": round(kern_gbs, 2),
            "peak": peak_gbs,
            "unit": "GB/s",
            "frac": round(kern_gbs / peak_gbs, 4),
            "traffic": recorded_traffic(w, args.layout),
            "kernel_avg_us": round(kern_avg_ms * 1e3, 2),
            "mfma_tflops": round(flops / (kern_avg_ms * 1e-3) / 1e12, 2),
        },
        "cpu_baseline": cpu,
        "parity": parity,
        "timing_us": {"step": pct(step_each_ms), "partial": pct(kern_ms),
                      "cache": "flushed before every step" if flush is not None else "hot (back-to-back steps)"},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
