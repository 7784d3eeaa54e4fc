"""Decode-step benchmark: split-KV decode attention at a 1M-token context on
one MI355X.

One step = the append of the newest token of every (request, KV head) and
the attention over all slices with their LSE combine, on one stream, with
the cache already resident in HBM: by default one hx_decode_step call (the
append inside the partial kernel, then one fold of the slice partials into
the final O and LSE); --append codes runs hx_kv_append, hx_decode_attn_partial
and hx_lse_combine as separate calls; --append bf16 gives the newest token as
bf16 values that hx_decode_step_bf16 quantises into the cache's format inside
the step.  Inputs are synthetic (seeded), shaped like the named workload.

The headline is the llama405b_tpa8_share step; by default the same run also
measures every other workload (tiny_gqa, deepseek_r1_mla, fp8_gqa,
mxfp4_ragged, wide_gqa_g64) under "workloads".  Every launch of the timed
steps is bracketed by the library's launch trace (HIP events recorded on the
launch's stream right after it), which gives each kernel's duration.  Prints
one JSON line.

    python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--workload NAME] [--no-extra]
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

from long_context_decode_split_amd import api, configs, roofline, synth

DEFAULT_WORKLOAD = configs.LLAMA405B_SHARE.name
EXTRA_WORKLOADS = [configs.TINY_GQA.name, configs.DEEPSEEK_MLA.name, configs.FP8_GQA.name,
                   configs.MXFP4_RAGGED.name, configs.WIDE_GQA_G64.name, configs.DEEPSEEK_MLA_FP8.name,
                   configs.DEEPSEEK_MLA_MXFP4.name]
METRIC = "µs/layer/decode step and KV-read HBM GB/s (% of peak) at 1M-token context"
PARTIAL_KERNELS = ("gqa_partial", "gqa_wide_partial", "mla_partial")


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


class Setup:
    """The cache (holding n - 1 tokens of every request), the step's inputs
    and outputs of workload w."""

    def __init__(self, w, seed, append, layout="dense", flags=0):
        t0 = time.time()
        self.w = w
        inp = self.inp = synth.make_inputs(w, seed, device="cuda")
        desc = api.KVDesc(P=w.P, B=w.B, Hkv=w.Hkv, Dk=w.Dk, Dv=w.Dv, v_alias_k=w.v_alias_k, dtype=w.dtype,
                          cap=inp.cap, flags=flags)
        self.paged = layout == "paged"
        if self.paged:
            self.cache = make_pool(desc, inp, seed)
            app = api.kv_append_paged
        else:
            self.cache = api.KVCache(desc, device="cuda")
            app = api.kv_append
        app(self.cache, inp.k, inp.v, inp.k_scale, inp.v_scale, pos=[0] * w.B, count=[n - 1 for n in inp.ctx])
        last = [n - 1 for n in inp.ctx]
        self.last = last

        def newest(t):
            if t is None:
                return None
            return torch.stack([t[b, :, last[b]:last[b] + 1] for b in range(w.B)]).contiguous()

        self.k, self.v, self.ks, self.vs = (newest(t) for t in (inp.k, inp.v, inp.k_scale, inp.v_scale))
        if append == "bf16":
            # the newest token as the bf16 values a QKV projection would produce
            g = torch.Generator(device="cuda").manual_seed(seed + 1)
            self.kb = (torch.randn(w.B, w.Hkv, 1, w.Dk, generator=g, device="cuda") * w.std).to(torch.bfloat16)
            self.vb = None if w.v_alias_k else \
                (torch.randn(w.B, w.Hkv, 1, w.Dv, generator=g, device="cuda") * w.std).to(torch.bfloat16)
        self.ws = torch.zeros(api.workspace_size(desc, w.Hq), dtype=torch.uint8, device="cuda")
        self.o_part = torch.empty(w.P, w.B, w.Hq, w.Dv, dtype=torch.float32, device="cuda")
        self.lse_part = torch.empty(w.P, w.B, w.Hq, dtype=torch.float32, device="cuda")
        self.o = torch.empty(w.B, w.Hq, w.Dv, dtype=torch.float32, device="cuda")
        self.lse = torch.empty(w.B, w.Hq, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        log(f"[bench] setup {w.name}: ctx={inp.ctx[:4]}{'...' if w.B > 4 else ''} cap={inp.cap} "
            f"cache={self.cache.nbytes() / 1e9:.3f} GB in {time.time() - t0:.1f}s")


def step_fn(s, append, attn):
    """One decode step of Setup s on a stream."""
    w, c = s.w, s.cache
    p = s.paged
    if append == "fused":
        fn = api.decode_step_paged if p else api.decode_step
        return lambda st: fn(c, s.k, s.v, s.ks, s.vs, s.inp.q, s.inp.ctx, w.softmax_scale, s.o, s.lse, s.ws, stream=st)
    if append == "bf16":
        fn = api.decode_step_bf16_paged if p else api.decode_step_bf16
        return lambda st: fn(c, s.kb, s.vb, s.inp.q, s.inp.ctx, w.softmax_scale, s.o, s.lse, s.ws, stream=st)
    app = api.kv_append_paged if p else api.kv_append
    one = api.decode_attn_paged if p else api.decode_attn
    part = api.decode_attn_partial_paged if p else api.decode_attn_partial

    def run(st):
        app(c, s.k, s.v, s.ks, s.vs, pos=s.last, stream=st)
        if attn == "one-call":
            one(c, s.inp.q, s.inp.ctx, w.softmax_scale, s.o, s.lse, s.ws, stream=st)
        else:
            part(c, s.inp.q, s.inp.ctx, w.softmax_scale, s.o_part, s.lse_part, s.ws, stream=st)
            api.lse_combine(s.o_part, s.lse_part, s.o, s.lse, stream=st)
    return run


def kernel_src_hash(w):
    """Hash of the partial kernel's sources for workload w, to tell whether
    recorded counters still describe the kernel that runs."""
    here = os.path.dirname(os.path.abspath(__file__))
    shared = ("hx_common.h", "hx_append.h", "hx_quant.h")   # the fused append / quantisation are part of it
    if w.v_alias_k:
        files = ("decode_mla.hip", "hx_gqa_frag.h") + shared
    elif w.G > 16:
        files = ("decode_gqa_wide.hip", "hx_gqa_frag.h") + shared
    else:
        files = ("decode_gqa.hip", "hx_gqa_frag.h") + shared
    h = hashlib.sha256()
    for p in files:
        with open(os.path.join(here, "long_context_decode_split_amd", "csrc", p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_key(w, layout, append="fused"):
    """Which recorded counters describe this run's partial kernel: one per
    workload, cache layout and append mode (the fused append and the fused
    quantisation are other instantiations of the kernel)."""
    key = w.name if layout == "dense" else f"{w.name}+{layout}"
    if append == "codes":
        return key + "+codes"
    return key + "+bf16append" if append == "bf16" and w.dtype != "bf16" else key


def recorded_traffic(w, layout="dense", append="fused"):
    """HBM bytes per launch of the partial kernel from the rocprofv3
    FETCH_SIZE / WRITE_SIZE passes recorded in profiles/traffic.json (scaled by
    a copy of known size), or None when none was recorded for this workload
    and cache layout, or the kernel sources changed since."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(traffic_key(w, layout, append))
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_src_sha16") != kernel_src_hash(w):
        return None
    return int(rec["fetch_bytes"]) + int(rec["write_bytes"])


def blas_threads():
    try:
        import threadpoolctl
        np.ones((2, 2)) @ np.ones((2, 2))
        info = [d for d in threadpoolctl.threadpool_info() if d.get("user_api") == "blas"]
        return int(info[0]["num_threads"]) if info else None
    except Exception:
        return None


def cpu_baseline(inp, budget_s, o, lse):
    """The oracle (fp64, numpy) on a bounded sample of the same step: whole
    (request, KV head) groups over their full context, as many as fit the
    time budget (at least one); scaled to KV-read GB/s like the GPU value.
    Also the largest deviations of the step's final O and LSE (device
    tensors) from the oracle over those groups."""
    from oracle import attention as oatt
    from oracle import codecs as ocod

    w = inp.w
    G = w.G
    per_tok = roofline.kv_bytes_per_token(w.Dk, w.Dv, w.v_alias_k, w.dtype)
    done_bytes, t_total, groups = 0.0, 0.0, 0
    err_o = err_l = 0.0
    max_o = 0.0
    oc = o.float().cpu().numpy()
    lc = lse.float().cpu().numpy()
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
        err_o = max(err_o, float(np.max(np.abs(oc[b, g * G:(g + 1) * G] - O))))
        err_l = max(err_l, float(np.max(np.abs(lc[b, g * G:(g + 1) * G] - L) / np.maximum(1.0, np.abs(L)))))
        max_o = max(max_o, float(np.max(np.abs(O))))
        done_bytes += n * per_tok
        groups += 1
        del K, V
        if t_total >= budget_s:
            break
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    parity = {"groups": groups, "heads_per_group": G, "max_abs_dO": err_o, "max_abs_O": max_o, "max_rel_dLSE": err_l,
              "bound_abs_dO": 2e-3 if w.dtype == "bf16" else 2e-2, "bound_rel_dLSE": 1e-4,
              "reference": "the oracle on the same stored K/V (dequantised values for fp8 / MXFP4)"}
    return parity, {
        "value": done_bytes / t_total / 1e9,
        "unit": "GB/s",
        "cores": threads,
        "blas_threads": blas_threads(),
        "kind": "oracle",
        "sample": f"{groups} of {len(order)} (request, KV head) groups of the same step, full context each; "
                  f"fp64 numpy unsplit attention incl. decoding the stored K/V; {t_total:.1f}s",
        "us_per_layer_step_extrapolated": t_total / done_bytes * roofline.kv_bytes(w, inp.ctx) * 1e6,
    }


def time_steps(step, steps, warmup, stream, flush=None):
    """Warm-up, then three passes of `steps` steps each.  Returns (ms per
    step, per-step ms list, {kernel: [ms per launch]}):
      * the timed region: `steps` back-to-back steps between two events and
        nothing else on the stream (with `flush`: each step between its own
        events, a cache flush before it, and the mean of those);
      * per-step events around each step (the distribution);
      * the library's launch trace, with the queue first filled by a plain
        read of 2 GiB so the host runs ahead of the GPU: each launch's entry
        is then its kernel's duration plus the dispatch gap before it, not
        time the GPU spent waiting for the host."""
    for _ in range(warmup):
        step(stream)
    torch.cuda.synchronize()
    new_ev = lambda: torch.cuda.Event(enable_timing=True)
    start, end = new_ev(), new_ev()
    sev = [(new_ev(), new_ev()) for _ in range(steps)]

    def per_step(flush_marks=None):
        for i in range(steps):
            if flush is not None:
                flush.fill_(i & 0xFF)
                if flush_marks is not None:
                    flush_marks.mark("flush", stream)   # the step's first launch is timed from here
            sev[i][0].record(stream)
            step(stream)
            sev[i][1].record(stream)

    torch.cuda.synchronize()
    if flush is None:
        start.record(stream)
        for _ in range(steps):
            step(stream)
        end.record(stream)
        torch.cuda.synchronize()
        total = start.elapsed_time(end) / steps
        per_step()
        torch.cuda.synchronize()
        each = [a.elapsed_time(b) for a, b in sev]
    else:
        per_step()
        torch.cuda.synchronize()
        each = [a.elapsed_time(b) for a, b in sev]
        total = float(np.mean(each))
    primer = torch.empty(2 << 30, dtype=torch.uint8, device="cuda") if flush is None else None
    torch.cuda.synchronize()
    with api.Trace(capacity=8 * steps + 8, stream=stream) as tr:
        if primer is not None:
            api.read_probe(primer, stream=stream)
            for _ in range(steps):
                step(stream)
        else:
            per_step(tr)
        torch.cuda.synchronize()
    del primer
    kern = tr.by_kernel()
    kern.pop("flush", None)
    kern.pop("read_probe", None)
    return total, each, kern


def graph_steps(step, steps, warmup, stream):
    """The same step captured once in a HIP graph and replayed."""
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step(side)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(torch.cuda.current_stream())
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        graph.replay()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def pct(x):
    return {f"p{q}": round(float(np.percentile(x, q)) * 1e3, 2) for q in (10, 50, 90)}


def measure(w, args, steps, warmup, append, attn, layout, cpu_budget, flags=0, flush=False, graph=False):
    """Time the step of workload w; returns a result dict."""
    s = Setup(w, args.seed, append, layout=layout, flags=flags)
    stream = torch.cuda.current_stream()
    step = step_fn(s, append, attn)
    flush_buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda") if flush else None
    step_ms, each, kern = time_steps(step, steps, warmup, stream, flush_buf)
    graph_ms = graph_steps(step, steps, warmup, stream) if graph else None
    pname = next((k for k in PARTIAL_KERNELS if k in kern), None)
    part = kern.get(pname, [float("nan")])
    part_ms = float(np.mean(part))
    nbytes = roofline.kv_bytes(w, s.inp.ctx)
    flops = roofline.attn_flops(w, s.inp.ctx)
    peak_gbs = roofline.HBM_PEAK_BYTES_PER_S / 1e9
    step_gbs = nbytes / (step_ms * 1e-3) / 1e9
    kern_gbs = nbytes / (part_ms * 1e-3) / 1e9
    res = {
        "config": {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "Dk": w.Dk, "Dv": w.Dv,
                   "v_alias_k": w.v_alias_k, "kv_dtype": w.dtype, "slices": w.P,
                   "context": s.inp.ctx if w.ctx is None else w.ctx, "kv_bytes_per_step": nbytes, "seed": args.seed,
                   "append": {"bf16": "bf16 values quantised on the device inside the step (hx_decode_step_bf16)",
                              "codes": "storage format, separate call",
                              "fused": "storage format, inside the attention call (hx_decode_step)"}[append],
                   "attention": "one-call" if append != "codes" else attn,
                   "layout": "block pool, 16-row blocks shuffled within each request" if layout == "paged"
                   else "dense planes",
                   "p_in_value_product": ("bf16, rounded once" if (flags or w.dtype != "bf16")
                                          else "bf16 high part + bf16 residual")},
        "step_us": round(step_ms * 1e3, 2),
        "step_gbs": round(step_gbs, 2),
        "step_frac_of_hbm_peak": round(step_gbs / peak_gbs, 4),
        "kernels_us": {k: round(float(np.mean(v)) * 1e3, 2) for k, v in kern.items()},
        "launches_per_step": round(sum(len(v) for v in kern.values()) / steps, 2),
        "roofline": {
            # the bound is whichever floor is higher: the KV bytes at the HBM
            # peak, or the algorithmic matrix flops at the bf16 matrix peak
            # (the MLA step with quantised rows: fewer bytes, the same flops)
            **({"bound": "mfma", "achieved": round(flops / (part_ms * 1e-3) / 1e12, 2),
                "peak": roofline.MFMA_BF16_DENSE_FLOPS / 1e12, "unit": "TFLOP/s",
                "frac": round(flops / (part_ms * 1e-3) / roofline.MFMA_BF16_DENSE_FLOPS, 4)}
               if flops / roofline.MFMA_BF16_DENSE_FLOPS > nbytes / roofline.HBM_PEAK_BYTES_PER_S else
               {"bound": "hbm", "achieved": round(kern_gbs, 2), "peak": peak_gbs, "unit": "GB/s",
                "frac": round(kern_gbs / peak_gbs, 4)}),
            "kernel": pname,
            "hbm_gbs": round(kern_gbs, 2),
            "hbm_frac": round(kern_gbs / peak_gbs, 4),
            "traffic": recorded_traffic(w, layout, append),
            "kernel_avg_us": round(part_ms * 1e3, 2),
            "mfma_tflops": round(flops / (part_ms * 1e-3) / 1e12, 2),
            "mfma_frac": round(flops / (part_ms * 1e-3) / roofline.MFMA_BF16_DENSE_FLOPS, 4),
            "algorithmic_flops": flops,
        },
        "timing_us": {"step": pct(each), "partial": pct(part),
                      "cache": "flushed before every step" if flush else "hot (back-to-back steps)",
                      "how": "step_us: the timed region (back-to-back steps between two events); step: each step "
                             "between its own events; partial and kernels_us: the launch trace with the queue "
                             "filled ahead (kernel duration plus the dispatch gap before it)"},
    }
    if graph_ms is not None:
        res["graph_step_us"] = round(graph_ms * 1e3, 2)
    log(f"[bench] {w.name}: step {step_ms * 1e3:.1f} us ({step_gbs:.0f} GB/s), kernels "
        + ", ".join(f"{k} {v:.1f} us" for k, v in res["kernels_us"].items())
        + f"; partial {kern_gbs:.0f} GB/s = {kern_gbs / peak_gbs:.1%} of HBM, {res['roofline']['mfma_frac']:.1%} of MFMA"
        + f" (bound: {res['roofline']['bound']})")
    if cpu_budget > 0:
        parity, cpu = cpu_baseline(s.inp, cpu_budget, s.o, s.lse)
        res["cpu_baseline"], res["parity"] = cpu, parity
        log(f"[bench] {w.name}: cpu oracle {cpu['value']:.3f} GB/s ({cpu['sample']}); "
            f"max |dO| {parity['max_abs_dO']:.2e} (max |O| {parity['max_abs_O']:.2e}), LSE rel {parity['max_rel_dLSE']:.2e}")
    del s
    torch.cuda.empty_cache()
    return res


def copy_rates(nbytes=4 << 30, reps=5):
    """Same-run device-to-device copy (bytes read + written per second) and a
    plain streaming read (hx_read_probe), as context for the HBM ceiling."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    dst.copy_(src)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    out = api.read_probe(src)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        api.read_probe(src, out)
    b.record()
    torch.cuda.synchronize()
    read_gbs = nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst, out
    torch.cuda.empty_cache()
    return {"copy_gbs": round(copy_gbs, 1), "read_gbs": round(read_gbs, 1), "bytes": nbytes,
            "how": "torch copy_ of 4 GiB (read + write bytes) and hx_read_probe, a plain streaming read of the "
                   "same 4 GiB with the kernels' 16-byte non-temporal loads (read bytes), HIP events"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(configs.ALL))
    ap.add_argument("--q-heads", type=int, default=0,
                    help="override the workload's query heads (GQA: a multiple of its KV heads, up to 128 per KV head)")
    ap.add_argument("--kv-dtype", choices=("bf16", "fp8_e4m3", "mxfp4"), default=None,
                    help="override the workload's cache format (GQA workloads)")
    ap.add_argument("--no-extra", action="store_true",
                    help="measure only --workload (default: also every other workload, under \"workloads\")")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work for the headline")
    ap.add_argument("--extra-cpu-budget", type=float, default=5.0, help="seconds of oracle work per extra workload")
    ap.add_argument("--append", choices=("fused", "codes", "bf16"), default="fused",
                    help="fused (default): the whole step is one hx_decode_step call (the newest token appended in "
                         "storage format inside the partial kernel, then the final O and LSE); codes: "
                         "hx_kv_append, then the attention calls of --attn; bf16: one hx_decode_step_bf16 call (the "
                         "newest token as bf16 values, quantised into the cache's format inside the step)")
    ap.add_argument("--attn", choices=("partial+combine", "one-call"), default="partial+combine",
                    help="with --append codes: partial+combine: hx_decode_attn_partial then hx_lse_combine (the "
                         "slice partials are outputs); one-call: hx_decode_attn")
    ap.add_argument("--layout", choices=("dense", "paged"), default="dense",
                    help="dense: [P][B][Hkv][cap/16] cache planes; paged: a block pool with per-(request, slice) "
                         "16-row block lists, each request's blocks shuffled among themselves (the *_paged calls)")
    ap.add_argument("--p-bf16", action="store_true",
                    help="HX_FLAG_P_BF16: the MLA value product takes P rounded once to bf16 (faster, less precise)")
    ap.add_argument("--graph", action="store_true", help="also time the step as one captured HIP graph per step")
    ap.add_argument("--flush-cache", action="store_true",
                    help="write a 1 GiB buffer before every step (outside the step's events) so that no KV bytes "
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

    t_start = time.time()
    flags = api.HX_FLAG_P_BF16 if args.p_bf16 else 0
    w = configs.ALL[args.workload]
    if args.q_heads or args.kv_dtype:
        if w.v_alias_k:
            print("--q-heads / --kv-dtype apply to GQA workloads", file=sys.stderr)
            sys.exit(2)
        w = w.scaled(name=f"{w.name}+Hq{args.q_heads or w.Hq}+{args.kv_dtype or w.dtype}",
                     Hq=args.q_heads or w.Hq, dtype=args.kv_dtype or w.dtype)
    head = measure(w, args, args.steps, args.warmup, args.append, args.attn, args.layout,
                   0 if args.no_cpu_baseline else args.cpu_budget, flags=flags, flush=args.flush_cache,
                   graph=args.graph)
    extras = {}
    if not args.no_extra:
        for name in EXTRA_WORKLOADS:
            if name == w.name:
                continue
            extras[name] = measure(configs.ALL[name], args, args.steps, args.warmup, args.append, args.attn,
                                   args.layout, 0 if args.no_cpu_baseline else args.extra_cpu_budget, flags=flags)
            if name == configs.TINY_GQA.name and not args.flush_cache:
                # the cache-resident step again with the caches flushed before every step
                fl = measure(configs.ALL[name], args, args.steps, args.warmup, args.append, args.attn, args.layout, 0,
                             flags=flags, flush=True)
                extras[name]["flushed"] = {"step_us": fl["step_us"], "timing_us": fl["timing_us"],
                                           "kernels_us": fl["kernels_us"]}
    rates = copy_rates()
    log(f"[bench] device copy {rates['copy_gbs']:.0f} GB/s (read + write), plain streaming read "
        f"{rates['read_gbs']:.0f} GB/s; run took {time.time() - t_start:.0f}s")

    step_us = head["step_us"]
    peak_gbs = roofline.HBM_PEAK_BYTES_PER_S / 1e9
    roof = dict(head["roofline"])
    roof.update(rates)
    out = {
        "metric": METRIC,
        "value": head["step_gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_us * 1e-3, 6),
        "us_per_layer_step": step_us,
        "frac_of_hbm_peak": round(head["step_gbs"] / peak_gbs, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8_e4m3": "fp8_e4m3 KV, bf16 MFMA, fp32 acc",
                  "mxfp4": "mxfp4 KV, bf16 MFMA, fp32 acc"}[w.dtype],
        "data": "synthetic",
        "config": dict(head["config"], launch="one HIP graph replay per step" if args.graph else "eager launches"),
        "roofline": roof,
        "cpu_baseline": head.get("cpu_baseline"),
        "parity": head.get("parity"),
        "kernels_us": head["kernels_us"],
        "timing_us": head["timing_us"],
    }
    if "graph_step_us" in head:
        out["graph_step_us"] = head["graph_step_us"]
    if extras:
        out["workloads"] = extras
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
