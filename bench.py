#!/usr/bin/env python3
"""Benchmark of the expert-cached MoE layer forward on one MI355X.

Headline (the JSON `value`): decode MoE layer in bf16 -- 16 tokens, d 4096,
256 routed experts all resident in HBM, SwiGLU intermediate 1024, top-6 --
whole-layer tokens/s with inputs resident in HBM.  A step is one full pass of
the layer (router GEMV, top-k, permutation, gate/up + SwiGLU, down, combine)
over one batch; 64 distinct seeded batches rotate so consecutive steps route to
different experts and the 256 MB Infinity Cache cannot serve the weights.
Decode steps replay one captured HIP graph per batch.

Alongside (`also`): decode at 1 and 4 tokens, bf16 prefill (4096 tokens), MXFP4
prefill (8192 tokens, I 2048, top-8), the 43-layer cached decode with 37% slots
and the q* split, the machine's B_P / B_H from ecf_bandwidth_profile, the
cached-decode policy ablation at equal capacity (q* at the configured and at the
measured ratio, every miss over PCIe, a static hot subset with every miss on the
host), the prefill layer prefetch overlap, and torch.bmm on the prefill
GEMM shapes (a vendor-library calibration).  `roofline` is for the
dominant kernel of the headline workload (decode gate/up GEMV); `cpu_baseline`
is the oracle on a bounded sample of the headline workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads ...]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HOST_EXPERTS = 8  # distinct host-generated experts behind --host-inputs
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
METRIC = "MoE-layer tokens/s (decode, prefill) + % HBM BW / % MFMA peak, 1 MI355X"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "expert_cache_ffn_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ---- achievable HBM bandwidth on this GPU (context for the roofline's 8 TB/s peak) ----------

def bench_hbm(torch, ecf, reps=10):
    """A plain streaming read of 4 GiB (libecf's ecf_stream_read: one contiguous
    chunk per block, two blocks per CU, 16 B per lane, eight loads in flight)
    and a 2 GiB device copy (torch), timed with HIP events: what simple kernels
    reach on this GPU."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.float32, device="cuda")  # contents do not matter for timing
    b = torch.empty(n // 2, dtype=torch.float32, device="cuda")
    c = torch.empty_like(b)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    out = {}
    read = lambda: ecf.ecf_stream_read(a.data_ptr(), 4 * n, sink.data_ptr(), torch.cuda.current_stream().cuda_stream)
    for name, fn, nbytes in (("read", read, 4 * n), ("copy", lambda: c.copy_(b), 2 * 4 * (n // 2))):
        fn()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(reps):
            fn()
        ev1.record()
        torch.cuda.synchronize()
        out[f"{name}_GBps"] = nbytes * reps / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
    # the MFMA rate under a GEMM-like load: bf16 MFMAs only, from registers, with
    # operands that change from one MFMA to the next (libecf's ecf_mfma_rate)
    mf = {}
    for bpc in (1, 2):
        st = torch.cuda.current_stream().cuda_stream
        ecf.ecf_mfma_rate(2000, bpc, sink.data_ptr(), st)  # warm-up
        ts = []
        for _ in range(5):
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record()
            flop = ecf.ecf_mfma_rate(20000, bpc, sink.data_ptr(), st)
            ev1.record()
            torch.cuda.synchronize()
            ts.append(ev0.elapsed_time(ev1) * 1e-3)
        mf[bpc] = flop / sorted(ts)[len(ts) // 2] / 1e12
    out["mfma_bf16_TFLOPs"] = max(mf.values())
    out["mfma_bf16_TFLOPs_by_waves_per_simd"] = {str(k): v for k, v in mf.items()}
    out["mfma_bf16_peak_TFLOPs"] = BF16_PEAK_TFLOPS
    del a, b, c, sink
    torch.cuda.empty_cache()
    out["peak_GBps"] = HBM_PEAK_GBS
    log(f"hbm: plain read {out['read_GBps']:.0f} GB/s, device copy {out['copy_GBps']:.0f} GB/s "
        f"(read+write), datasheet peak {HBM_PEAK_GBS:.0f}; bf16 MFMA-only loop {out['mfma_bf16_TFLOPs']:.0f} "
        f"TFLOP/s (datasheet {BF16_PEAK_TFLOPS:.0f})")
    return out


def one_launch_read_us(torch, ecf, nbytes, reps=5, launches=10):
    """Time per launch of ecf_stream_read over nbytes (rounded down to 16 B):
    the floor for any single kernel that streams that many bytes from HBM,
    launch and ramp included.  The launches are captured in one HIP graph, as
    the decode steps are, and replayed back to back; each reads a different
    region of a 4 GiB buffer whose pages have all been written, so none is
    served from the 256 MB last-level cache.  Median over repeats."""
    span = 1 << 32
    nbytes = max(16, nbytes // 16 * 16)
    buf = torch.empty(span, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    slots = max(1, span // nbytes)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(launches):
            ecf.ecf_stream_read(buf.data_ptr() + (i % slots) * nbytes, nbytes, sink.data_ptr(), stream.cuda_stream)
    ts = []
    with torch.cuda.stream(stream):
        for r in range(reps + 1):
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            g.replay()
            ev1.record(stream)
            stream.synchronize()
            if r >= 1:
                ts.append(1e3 * ev0.elapsed_time(ev1) / launches)
    del g, buf, sink
    torch.cuda.empty_cache()
    return sorted(ts)[len(ts) // 2]


def bench_vendor_gemm(torch, reps=5):
    """Calibration, not part of the layer: torch.bmm (the ROCm BLAS libraries)
    on the prefill layers' per-expert GEMM shapes with every expert holding
    exactly R/E rows and dense bf16 weights (no ragged tiles, no MXFP4
    expansion), plus one large square GEMM and one large dense torch.mm with
    the MXFP4 GEMM1's flop -- what the vendor's GEMMs reach on this GPU for
    the same work.  Right operands of bmm are contiguous [E, K, N]."""
    shapes = {  # name: (batch, M, K, N)
        "square_8192": (1, 8192, 8192, 8192),
        "prefill_bf16_gemm1": (256, 96, 4096, 2048),    # 4096 tokens x top-6 / 256 experts; [gate|up]
        "prefill_bf16_gemm2": (256, 96, 1024, 4096),
        "prefill_mxfp4_gemm1": (256, 256, 4096, 4096),  # 8192 tokens x top-8 / 256 experts
        "prefill_mxfp4_gemm2": (256, 256, 2048, 4096),
    }
    out = {}
    for name, (bt, m, kk, n) in shapes.items():
        a = torch.randn(bt, m, kk, device="cuda", dtype=torch.bfloat16)
        b = torch.randn(bt, kk, n, device="cuda", dtype=torch.bfloat16)
        c = torch.bmm(a, b)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(reps):
            torch.bmm(a, b, out=c)
        ev1.record()
        torch.cuda.synchronize()
        us = 1e3 * ev0.elapsed_time(ev1) / reps
        tf = 2.0 * bt * m * kk * n / (us * 1e-6) / 1e12
        out[name] = {"batch": bt, "M": m, "K": kk, "N": n, "us": us, "tflops": tf,
                     "mfma_frac": tf / BF16_PEAK_TFLOPS}
        del a, b, c
    torch.cuda.empty_cache()
    # one large dense GEMM with the MXFP4 prefill GEMM1's flop (torch.mm)
    m, kk, n = 65536, 4096, 4096
    a = torch.randn(m, kk, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, kk, device="cuda", dtype=torch.bfloat16)
    c = torch.mm(a, b.t())
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(reps):
        torch.mm(a, b.t(), out=c)
    ev1.record()
    torch.cuda.synchronize()
    us = 1e3 * ev0.elapsed_time(ev1) / reps
    tf = 2.0 * m * kk * n / (us * 1e-6) / 1e12
    out["dense_mm_65536x4096x4096"] = {"batch": 1, "M": m, "K": kk, "N": n, "us": us, "tflops": tf,
                                       "mfma_frac": tf / BF16_PEAK_TFLOPS}
    del a, b, c
    torch.cuda.empty_cache()
    log("vendor bmm/mm: " + ", ".join(f"{k} {v['us']:.0f} us ({v['tflops']:.0f} TF)" for k, v in out.items()))
    return out


# ---- decode (headline) ---------------------------------------------------------------

def bench_decode(torch, ecf, syn, Ts, steps, warmup, n_batches=64, use_graph=True, host_inputs=False,
                 w_dtype="bf16"):
    import dataclasses
    from expert_cache_ffn_amd.layer import ExpertPool, Layer, pack_expert
    cfg = dataclasses.replace(syn.CONFIGS["decode"], w_dtype=w_dtype)
    d, E, I, k = cfg.hidden, cfg.experts, cfg.inter, cfg.top_k
    shape = ecf.make_shape(d, I, E, k, w_dtype, "bf16")
    S = ecf.ecf_expert_bytes(shape)
    # gate + up bytes of one expert: the two weight sections (+ their scales for MXFP4)
    gu_expert = 2 * (I * d * 2 if w_dtype == "bf16" else I * d // 2 + I * d // 32)
    dn_expert = d * I * 2 if w_dtype == "bf16" else d * I // 2 + d * I // 32  # down weights (+ scales)
    pool = ExpertPool(shape, "cuda")
    # host_inputs: every input is generated on the host and copied, so the only
    # GPU kernels of the run are libecf's and the runtime's copies (a hardware
    # counter pass then sees nothing else).  Generating 6.4 GB on the host is slow,
    # so the expert blobs repeat HOST_EXPERTS distinct experts; routing (router
    # weights and activations) is the full recipe's, and kernel timing and traffic
    # do not depend on weight values.
    gen_dev = "cpu" if host_inputs else "cuda"
    if host_inputs:
        log(f"decode: {E} expert blobs ({E * S / 1e9:.2f} GB) from {HOST_EXPERTS} host-generated experts")
        blobs = []
        for h in range(HOST_EXPERTS):
            b = torch.empty(S, dtype=torch.uint8)
            pack_expert(shape, syn.expert_weights(cfg, 0, h, device="cpu"), b)
            blobs.append(b)
        for e in range(E):
            pool.buf[e].copy_(blobs[e % HOST_EXPERTS])
        del blobs
    else:
        log(f"decode: generating {E} experts ({E * S / 1e9:.2f} GB) on the GPU")
        for e in range(E):
            pool.load(e, syn.expert_weights(cfg, 0, e, device="cuda"))
    wr = syn.router_weights(cfg, device=gen_dev).to("cuda")
    lay = Layer(shape, max(Ts))
    stream = torch.cuda.Stream()
    results = {}
    for T in Ts:
        xs = [syn.activations(cfg, T, batch=b, device=gen_dev).to("cuda") for b in range(n_batches)]
        outs = [torch.empty((T, d), dtype=torch.float32, device="cuda") for _ in range(n_batches)]
        counts = torch.empty((n_batches, E), dtype=torch.int32, device="cuda")  # written by the layer
        # Everything above was queued on the default stream; the layer runs on `stream`.
        # Drain the device first: the caching allocator may have handed the workspace,
        # x and out blocks that generation temporaries (still pending on the default
        # stream) were writing, and nothing orders the two streams.
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            plain = [lay.args(router_w=wr, expert_ptrs=pool.ptrs, stream=stream) for _ in range(n_batches)]
            call = lambda b: ecf.lib().moe_layer_forward(plain[b], xs[b].data_ptr(), T, outs[b].data_ptr(), None)
            # routing of every batch (for the algorithmic byte counts)
            for b in range(n_batches):
                a = lay.args(router_w=wr, expert_ptrs=pool.ptrs, stream=stream, counts=counts[b])
                lay.forward(a, xs[b], outs[b], want_stats=False)
            stream.synchronize()
            U = (counts.cpu() > 0).sum(1).double()
            graphs = []
            if use_graph:
                for b in range(n_batches):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=stream):
                        rc = call(b)
                    assert rc == 0, ecf.lib().ecf_last_error()
                    graphs.append(g)
                step = lambda i: graphs[i % n_batches].replay()
            else:
                def step(i):
                    rc = call(i % n_batches)
                    assert rc == 0
            for i in range(warmup):
                step(i)
            stream.synchronize()
            torch.cuda.synchronize()
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record(stream)
            for i in range(steps):
                step(i)
            ev1.record(stream)
            stream.synchronize()
            torch.cuda.synchronize()
            ms = ev0.elapsed_time(ev1)
            # per-step spread: the same steps again with an event between steps
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
            evs[0].record(stream)
            for i in range(steps):
                step(i)
                evs[i + 1].record(stream)
            stream.synchronize()
            per_step = sorted(evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(steps))
            # per-kernel durations: same steps again, eager, each launch bracketed by HIP events
            ecf.ecf_profile_reset()
            ecf.ecf_profile_enable(True)
            for i in range(steps):
                assert call(i % n_batches) == 0
            stream.synchronize()
            prof = ecf.ecf_profile_get_all()
            ecf.ecf_profile_enable(False)
        used = [i % n_batches for i in range(steps)]
        U_avg = float(U[used].mean())
        R = T * k
        gu_bytes = U_avg * gu_expert + R * d * 2 + R * I * 4           # gate+up weights, x rows, h
        dn_bytes = U_avg * dn_expert + R * I * 4 + R * d * 4           # down weights, h, Y
        layer_bytes = U_avg * S + E * d * 2 + T * d * 2 + T * d * 4    # weights, router, x, out
        kern = {n: {"launches": c, "avg_us": 1e3 * t / max(c, 1)} for n, (c, t) in prof.items()}
        gu_us = kern["decode_gateup"]["avg_us"]
        results[T] = dict(
            tokens=T, ms_per_step=ms / steps, tokens_per_s=T * steps / (ms / 1e3), unique_experts_avg=U_avg,
            us_step_median=per_step[steps // 2], us_step_p10=per_step[steps // 10],
            us_step_p90=per_step[min(steps - 1, (9 * steps) // 10)],
            layer_bytes=layer_bytes, layer_GBps=layer_bytes / (ms / steps * 1e-3) / 1e9,
            layer_hbm_frac=layer_bytes / (ms / steps * 1e-3) / 1e9 / HBM_PEAK_GBS,
            gateup_bytes=gu_bytes, gateup_avg_us=gu_us, gateup_GBps=gu_bytes / (gu_us * 1e-6) / 1e9,
            down_bytes=dn_bytes, kernels=kern, graph=use_graph)
        if "decode_down" in kern:  # one token of MXFP4 runs down and combine as one kernel
            dn_us = kern["decode_down"]["avg_us"]
            results[T].update(down_avg_us=dn_us, down_GBps=dn_bytes / (dn_us * 1e-6) / 1e9)
        # the same bytes read by one plain streaming kernel: the floor for the
        # whole layer, which is a chain of dependent kernels
        # (not in the host-input mode used for hardware-counter passes: the floor
        # runs torch kernels, which that mode keeps out of the profiled process)
        if layer_bytes < (1 << 31) and not host_inputs:
            floor = one_launch_read_us(torch, ecf, int(layer_bytes))
            results[T]["one_launch_read_us"] = floor
            results[T]["layer_time_over_one_launch_read"] = ms / steps * 1e3 / floor
        floor_s = (f", one plain read of the layer's bytes {results[T]['one_launch_read_us']:.1f} us"
                   if "one_launch_read_us" in results[T] else "")
        log(f"decode {w_dtype} T={T}: {ms / steps * 1e3:.1f} us/step (median {per_step[steps // 2]:.1f}), "
            f"{results[T]['tokens_per_s']:.0f} tok/s, "
            f"U={U_avg:.1f}, layer {results[T]['layer_GBps']:.0f} GB/s, gate/up {results[T]['gateup_GBps']:.0f} GB/s"
            f"{floor_s}")
        del graphs
    def gpu_run(x_cpu):
        """One eager forward of the layer on x (host tensor); routing and output on the host."""
        T = x_cpu.shape[0]
        x = x_cpu.to("cuda")
        out = torch.empty((T, d), dtype=torch.float32, device="cuda")
        idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
        gate = torch.empty((T, k), dtype=torch.float32, device="cuda")
        cnt = torch.empty(E, dtype=torch.int32, device="cuda")
        perm = torch.empty(T * k, dtype=torch.int32, device="cuda")
        lgo = torch.empty((T, E), dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            a = lay.args(router_w=wr, expert_ptrs=pool.ptrs, stream=stream, topk_idx=idx, topk_gate=gate,
                         counts=cnt, perm=perm, logits_out=lgo)
            lay.forward(a, x, out, want_stats=False)
        stream.synchronize()
        return dict(idx=idx.cpu().numpy(), gate=gate.cpu().numpy(), counts=cnt.cpu().numpy(),
                    perm=perm.cpu().numpy(), out=out.cpu().numpy(), logits=lgo.cpu().numpy())

    sample = dict(pool=pool, wr=wr, cfg=cfg, gpu_run=gpu_run if w_dtype == "bf16" else None)
    return results, sample


def cpu_baseline_decode(torch, syn, sample, budget_s=15.0, T=16, max_batches=256):
    """The oracle (C, OpenMP over tokens) on whole T=16 batches until ~budget_s."""
    import numpy as np
    import oracle
    cfg, pool = sample["cfg"], sample["pool"]
    wr = sample["wr"].cpu()
    shape_sections = None
    from expert_cache_ffn_amd.layer import blob_sections
    import expert_cache_ffn_amd as ecf
    shape = ecf.make_shape(cfg.hidden, cfg.inter, cfg.experts, cfg.top_k, "bf16", "bf16")
    shape_sections = dict(blob_sections(shape))
    cache = {}

    def expert(e):
        if e not in cache:
            blob = pool.buf[e].cpu()
            d, I = cfg.hidden, cfg.inter
            n = d * I * 2
            cache[e] = {nm: blob[off:off + n].view(torch.bfloat16).view(I if nm != "w_down" else d,
                                                                         d if nm != "w_down" else I)
                        for nm, off in shape_sections.items()}
        return cache[e]

    # every timed batch is also run on the GPU and compared with the oracle: routing
    # exactly (rows whose fp32 logits agree; the others may differ by one ulp),
    # counts and permutation exactly where every row agrees, outputs within
    # 2e-2 x the oracle output's RMS
    gpu_run = sample.get("gpu_run")
    chk = dict(batches=0, tokens=0, rows_logit_1ulp=0, rows_routing_exact=0, batches_perm_counts_exact=0,
               max_err_over_rms=0.0, tolerance=2e-2, ok=True)
    done, elapsed, batches = 0, 0.0, 0
    while elapsed < budget_s and batches < max_batches:
        x = syn.activations(cfg, T, batch=batches)
        lg = oracle.logits(x, wr)
        idx, g = oracle.route(lg, cfg.top_k)
        experts = [None] * cfg.experts
        for e in set(int(v) for v in idx.ravel()):
            experts[e] = expert(e)
        t0 = time.perf_counter()
        res = oracle.moe_layer(x, experts, cfg.top_k, wr=wr)   # the whole layer, routing included
        elapsed += time.perf_counter() - t0
        done += T
        batches += 1
        assert np.all(np.isfinite(res["out"]))
        if gpu_run is not None:
            gr = gpu_run(x)
            same = np.all(gr["logits"] == res["logits"], axis=1)
            ulp = np.spacing(np.abs(res["logits"]).astype(np.float32))
            exact = same & np.all(gr["idx"] == res["idx"], axis=1)
            perm_ok = bool(same.all() and np.array_equal(gr["counts"], res["counts"])
                           and np.array_equal(gr["perm"], res["perm"]))
            rms = float(np.sqrt(np.mean(res["out"] ** 2)))
            err = float(np.max(np.abs(gr["out"] - res["out"]))) / rms
            chk["batches"] += 1
            chk["tokens"] += T
            chk["rows_logit_1ulp"] += int((~same).sum())
            chk["rows_routing_exact"] += int(exact.sum())
            chk["batches_perm_counts_exact"] += int(perm_ok)
            chk["max_err_over_rms"] = max(chk["max_err_over_rms"], err)
            chk["ok"] = chk["ok"] and bool(np.all(np.abs(gr["logits"] - res["logits"]) <= ulp)) \
                and int(exact.sum()) == int(same.sum()) and (perm_ok or not same.all()) and err <= 2e-2
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    out = {"value": done / elapsed, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"{batches} batches of {T} tokens of the headline decode workload (router, top-k, "
                     f"permutation, experts, combine in fp64), {elapsed:.1f} s of CPU time",
           "cpu_model": model, "nproc": os.cpu_count(), "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}
    if gpu_run is not None:
        out["checked_against_gpu"] = chk
        log(f"cpu baseline: GPU layer checked on the same {chk['batches']} batches: routing exact on "
            f"{chk['rows_routing_exact']}/{chk['tokens']} tokens ({chk['rows_logit_1ulp']} with 1-ulp logits), "
            f"max|err|/RMS {chk['max_err_over_rms']:.2e}, {'ok' if chk['ok'] else 'FAILED'}")
    return out


# ---- prefill (bf16 and MXFP4) ----------------------------------------------------------------

def cpu_oracle_prefill(torch, syn, cfg, x, lg, counts_gpu, out_gpu, sample=128):
    """The oracle on a bounded sample of a prefill layer: routing, counts and
    permutation of all T tokens, the expert FFNs and combine of the first
    `sample` tokens (every expert they reach), timed; those tokens' GPU outputs
    and the layer's expert counts are checked against it."""
    import numpy as np
    import oracle
    T, E, k = cfg.tokens[0], cfg.experts, cfg.top_k
    toks = np.arange(min(sample, T))
    lg_c, x_c = lg.float().cpu(), x.cpu()
    idx, _ = oracle.route(lg_c, k)
    need = sorted(set(int(v) for v in idx[toks].ravel()))
    experts = [None] * E
    for e in need:  # the same seeded tensors the GPU blobs were packed from
        experts[e] = {n: t.detach().cpu() for n, t in syn.expert_weights(cfg, 0, e, device="cuda").items()}
    t0 = time.perf_counter()
    res = oracle.moe_layer(x_c, experts, k, lg=lg_c, w_dtype=cfg.w_dtype, tokens=toks)
    el = time.perf_counter() - t0
    tol = 5e-2 if cfg.w_dtype == "mxfp4" else 2e-2
    got = out_gpu[: len(toks)].cpu().numpy()
    rms = float(np.sqrt(np.mean(res["out"] ** 2)))
    err = float(np.max(np.abs(got - res["out"]))) / rms
    counts_ok = bool(np.array_equal(counts_gpu.cpu().numpy(), res["counts"]))
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    r = {"value": len(toks) / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
         "sample": f"routing of all {T} tokens and the experts of the first {len(toks)} ({len(need)} experts), "
                   f"{el:.1f} s of CPU time",
         "checked_against_gpu": {"tokens": int(len(toks)), "counts_exact": counts_ok, "max_err_over_rms": err,
                                 "tolerance": tol, "ok": bool(counts_ok and err <= tol)}}
    log(f"{cfg.name}: oracle {r['value']:.1f} tok/s on {threads} threads ({r['sample']}); GPU counts "
        f"{'exact' if counts_ok else 'DIFFER'}, max|err|/RMS {err:.2e} on {len(toks)} tokens")
    return r


def bench_prefill(torch, ecf, syn, name, steps, warmup, cpu=False, host_inputs=False):
    from expert_cache_ffn_amd.layer import ExpertPool, Layer, pack_expert
    cfg = syn.CONFIGS[name]
    T, d, E, I, k = cfg.tokens[0], cfg.hidden, cfg.experts, cfg.inter, cfg.top_k
    shape = ecf.make_shape(d, I, E, k, cfg.w_dtype, "bf16")
    S = ecf.ecf_expert_bytes(shape)
    pool = ExpertPool(shape, "cuda")
    # host_inputs: every input is generated on the host and copied in, so the only
    # GPU kernels of the run are libecf's (a hardware counter pass then sees
    # nothing else); the expert blobs repeat HOST_EXPERTS host-generated experts,
    # routing inputs are the full recipe's (timing and traffic do not depend on
    # weight values)
    gen_dev = "cpu" if host_inputs else "cuda"
    if host_inputs:
        log(f"{name}: {E} expert blobs ({E * S / 1e9:.2f} GB, {cfg.w_dtype}) from {HOST_EXPERTS} host-generated experts")
        blobs = []
        for h in range(HOST_EXPERTS):
            b = torch.empty(S, dtype=torch.uint8)
            pack_expert(shape, syn.expert_weights(cfg, 0, h, device="cpu"), b)
            blobs.append(b)
        for e in range(E):
            pool.buf[e].copy_(blobs[e % HOST_EXPERTS])
        del blobs
    else:
        log(f"{name}: generating {E} experts ({E * S / 1e9:.2f} GB, {cfg.w_dtype}) on the GPU")
        for e in range(E):
            pool.load(e, syn.expert_weights(cfg, 0, e, device="cuda"))
    lay = Layer(shape, T)
    xs = [syn.activations(cfg, T, batch=b, device=gen_dev).to("cuda") for b in range(2)]
    lgs = [syn.router_logits(cfg, T, step=b, device=gen_dev).to("cuda") for b in range(2)]
    out = torch.empty((T, d), dtype=torch.float32, device="cuda")
    counts = torch.zeros(E, dtype=torch.int32).to("cuda")
    argsv = [lay.args(router_logits=lgs[b], expert_ptrs=pool.ptrs) for b in range(2)]
    call = lambda i: ecf.lib().moe_layer_forward(argsv[i % 2], xs[i % 2].data_ptr(), T, out.data_ptr(), None)
    lay.forward(lay.args(router_logits=lgs[0], expert_ptrs=pool.ptrs, counts=counts), xs[0], out, False)
    for i in range(warmup):
        assert call(i) == 0
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(steps):
        assert call(i) == 0
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record()
    for i in range(steps):
        assert call(i) == 0
        evs[i + 1].record()
    torch.cuda.synchronize()
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))
    ecf.ecf_profile_reset()
    ecf.ecf_profile_enable(True)
    for i in range(steps):
        assert call(i) == 0
    torch.cuda.synchronize()
    prof = ecf.ecf_profile_get_all()
    ecf.ecf_profile_enable(False)
    kern = {n: {"launches": c, "avg_us": 1e3 * t / max(c, 1)} for n, (c, t) in prof.items()}
    R = T * k
    flops = 2.0 * R * d * 3 * I
    n_active = int((counts.cpu() > 0).sum())
    wbytes = n_active * S
    res = dict(tokens=T, ms_per_layer=ms, tokens_per_s=T / (ms * 1e-3), active_experts=n_active,
               ms_median=per_step[steps // 2], ms_p10=per_step[steps // 10],
               ms_p90=per_step[min(steps - 1, (9 * steps) // 10)],
               tflops=flops / (ms * 1e-3) / 1e12, mfma_frac=flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
               weight_GBps=wbytes / (ms * 1e-3) / 1e9, hbm_frac_weights=wbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
               kernels=kern)
    g1 = kern.get("prefill_gemm1", {}).get("avg_us")
    g2 = kern.get("prefill_gemm2", {}).get("avg_us")
    if g1 and g2:
        res["gemm1_tflops"] = 2.0 * R * d * 2 * I / (g1 * 1e-6) / 1e12
        res["gemm2_tflops"] = 2.0 * R * I * d / (g2 * 1e-6) / 1e12
    # hardware-counter figures of these GEMMs (FETCH_SIZE / WRITE_SIZE copy-calibrated,
    # MFMA busy cycles), valid while the kernel sources match the recorded hash
    cpath = os.path.join(ROOT, "profiles", "prefill_grouped_gemm_bf16_T4096_mxfp4_T8192_counters.md")
    if os.path.exists(cpath):
        cj = json.loads(open(cpath).read().split("```json", 1)[1].split("```", 1)[0])
        if cj.get("source_hash") == src_hash("k_prefill.hip", "device_common.h"):
            fmt = "mxfp4" if cfg.w_dtype == "mxfp4" else "bf16"
            res["counters"] = {g: {kk: cj["gemms"][f"{fmt}_{g}"][kk] for kk in
                                   ("traffic_ratio", "mfma_util", "clock_ghz", "flop_counted_over_algorithmic")}
                               for g in ("gemm1", "gemm2")}
    if cpu and not host_inputs:  # the oracle beside it, on batch 0 (what `counts` holds)
        lay.forward(lay.args(router_logits=lgs[0], expert_ptrs=pool.ptrs), xs[0], out, False)
        torch.cuda.synchronize()
        # MXFP4 expert FFNs take the oracle ~0.15 s per token: a smaller sample
        res["cpu_oracle"] = cpu_oracle_prefill(torch, syn, cfg, xs[0], lgs[0], counts, out,
                                               sample=32 if cfg.w_dtype == "mxfp4" else 128)
    log(f"{name}: {ms:.3f} ms/layer (median {per_step[steps // 2]:.3f}), {res['tokens_per_s']:.0f} tok/s, "
        f"{res['tflops']:.0f} TFLOP/s "
        f"({100 * res['mfma_frac']:.1f}% MFMA), weights {res['weight_GBps']:.0f} GB/s")
    del pool
    torch.cuda.empty_cache()
    return res


def bench_prefetch(torch, ecf, syn, name="prefill", layers=8, reps=3):
    """Prefill stack through the shared slot pool: before layer l's forward call,
    prefetch_layer queues layer l+1's whole expert set (one contiguous host layer
    blob) into the cache's slots on a copy stream; the forward call of l+1 waits
    on device for it.  Slots: two layers.  Host pool: two distinct pinned layer
    blobs, aliased over the stack.  Timed with HIP events: the copy of a layer
    alone (median of `reps` warm copies), the layer's forward alone on resident
    slots (median of `reps`), and the stack.  From the start of layer 1's copy
    to the end of the last layer's copy the copy stream moves L-1 layers
    (t_copy per layer); from the same start to the end of the last layer's
    kernels the stack finishes L-1 layers (t_layer per layer); the last layer
    waits for its copy, so t_copy <= t_layer by construction.  overlap =
    max(t_copy, compute alone) / t_layer (1 = the shorter of the two is wholly
    hidden)."""
    from expert_cache_ffn_amd.layer import Layer, pack_expert
    cfg = syn.CONFIGS[name]
    T, d, E, I, k = cfg.tokens[0], cfg.hidden, cfg.experts, cfg.inter, cfg.top_k
    shape = ecf.make_shape(d, I, E, k, cfg.w_dtype, "bf16")
    S = ecf.ecf_expert_bytes(shape)
    LB = E * S
    log(f"{name} stream: pinning 2 host layer blobs ({2 * LB / 1e9:.1f} GB), {2 * E} slots ({2 * LB / 1e9:.1f} GB)")
    host = torch.empty((2, E, S), dtype=torch.uint8).pin_memory()
    slots = torch.empty((2 * E, S), dtype=torch.uint8, device="cuda")
    for h in range(2):
        for e in range(E):
            pack_expert(shape, syn.expert_weights(cfg, h, e, device="cuda"), slots[e])
        host[h].copy_(slots[:E].cpu())
    hb = host.data_ptr()
    pool = [hb + ((l % 2) * E + e) * S for l in range(layers) for e in range(E)]
    cache = ecf.ecf_cache_create(layers, E, 2 * E, 2 * E, S, slots.data_ptr(), pool, host_threads=1)
    lay = Layer(shape, T)
    xs = [syn.activations(cfg, T, layer=l % 2, device="cuda") for l in range(2)]
    lgs = [syn.router_logits(cfg, T, layer=l % 2, device="cuda") for l in range(2)]
    outs = [torch.empty((T, d), dtype=torch.float32, device="cuda") for _ in range(layers)]
    comp, copy = torch.cuda.current_stream(), torch.cuda.Stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    args = lambda l: lay.args(layer=l, router_logits=lgs[l % 2], cache=cache, path=ecf.ECF_PATH_PREFILL,
                              copy_stream=copy)
    torch.cuda.synchronize()
    med = lambda v: sorted(v)[len(v) // 2]
    # copy alone: drop every entry (resize to 0 and back), then one whole layer
    t_copy_solo = []
    for _ in range(reps):
        ecf.ecf_cache_resize(cache, 0)
        ecf.ecf_cache_resize(cache, 2 * E)
        a, b = ev(), ev()
        a.record(copy)
        ecf.prefetch_layer(cache, 0, S, copy.cuda_stream)
        b.record(copy)
        b.synchronize()
        t_copy_solo.append(a.elapsed_time(b))
    # compute alone: layer 0 resident in its slots (all hits)
    lay.forward(args(0), xs[0], outs[0], want_stats=False)
    t_gemm = []
    for _ in range(reps):
        a, b = ev(), ev()
        a.record(comp)
        lay.forward(args(0), xs[0], outs[0], want_stats=False)
        b.record(comp)
        b.synchronize()
        t_gemm.append(a.elapsed_time(b))
    # the stack, from an empty cache
    ecf.ecf_cache_resize(cache, 0)
    ecf.ecf_cache_resize(cache, 2 * E)
    torch.cuda.synchronize()
    c0 = [ev() for _ in range(layers)]
    c1 = [ev() for _ in range(layers)]
    done = [ev() for _ in range(layers)]
    t0 = ev()
    t0.record(comp)
    c0[0].record(copy)
    ecf.prefetch_layer(cache, 0, S, copy.cuda_stream)
    c1[0].record(copy)
    n_missing = 0
    for l in range(layers):
        if l + 1 < layers:
            c0[l + 1].record(copy)
            _, m = ecf.prefetch_layer(cache, l + 1, S, copy.cuda_stream)
            n_missing += m
            c1[l + 1].record(copy)
        lay.forward(args(l), xs[l % 2], outs[l], want_stats=False)
        done[l].record(comp)
    torch.cuda.synchronize()
    copies = [c0[l].elapsed_time(c1[l]) for l in range(1, layers)]
    gaps = [done[l - 1].elapsed_time(done[l]) for l in range(1, layers)]
    t_copy = c0[1].elapsed_time(c1[-1]) / (layers - 1)
    t_layer = c0[1].elapsed_time(done[-1]) / (layers - 1)
    t_comp = med(t_gemm)
    total = t0.elapsed_time(done[-1])
    # the last layer against the all-resident prefill on the same slots
    ptrs = torch.tensor([slots.data_ptr() + ecf.ecf_cache_slot_of(cache, layers - 1, e) * S for e in range(E)],
                        dtype=torch.int64, device="cuda")
    ref = torch.empty_like(outs[-1])
    lay.forward(lay.args(router_logits=lgs[(layers - 1) % 2], expert_ptrs=ptrs, path=ecf.ECF_PATH_PREFILL),
                xs[(layers - 1) % 2], ref, want_stats=False)
    torch.cuda.synchronize()
    same = bool(torch.equal(ref, outs[-1]))
    st = ecf.ecf_cache_get_stats(cache)
    ecf.ecf_cache_destroy(cache)
    res = dict(config=name, layers=layers, tokens=T, layer_bytes=LB, slots=2 * E,
               ms_copy_solo_median=med(t_copy_solo), ms_copy_solo_all=t_copy_solo,
               ms_copy_per_layer=t_copy, h2d_GBps=LB / (t_copy * 1e-3) / 1e9,
               ms_copy_in_stack_median=med(copies), ms_layer_interval_median=med(gaps),
               ms_compute_median=t_comp, ms_per_layer_streamed=t_layer, ms_stack_total=total,
               overlap_efficiency=max(t_copy, t_comp) / t_layer,
               tokens_per_s_streamed=T / (t_layer * 1e-3), experts_not_prefetched=n_missing,
               last_layer_equals_resident=same, cache_stats=st)
    log(f"{name} stream: copy {t_copy:.2f} ms/layer in the stack ({res['h2d_GBps']:.1f} GB/s; alone "
        f"{res['ms_copy_solo_median']:.1f}), compute alone {t_comp:.2f} ms, {t_layer:.2f} ms/layer streamed, "
        f"overlap {res['overlap_efficiency']:.4f}, last layer {'equals' if same else 'DIFFERS from'} the "
        f"resident layer")
    del slots, host
    torch.cuda.empty_cache()
    return res


# ---- cached decode (43 layers, 37% slots, q*) -------------------------------------------

def cached_setup(torch, ecf, syn, T=16, steps=16, warmup=16, n_blobs=256, w_dtype="bf16"):
    """Host pool, device slots, activations and per-step router logits of the
    43-layer cached-decode workload, shared by every policy run."""
    import dataclasses
    from expert_cache_ffn_amd.layer import Layer, pack_expert
    cfg = dataclasses.replace(syn.CONFIGS["cached"], w_dtype=w_dtype)
    L, d, E, I, k = cfg.layers, cfg.hidden, cfg.experts, cfg.inter, cfg.top_k
    shape = ecf.make_shape(d, I, E, k, w_dtype, "bf16")
    S = ecf.ecf_expert_bytes(shape)
    n_slots = int(0.37 * L * E)
    log(f"cached {w_dtype}: {L} layers x {E} experts, {n_slots} slots ({n_slots * S / 1e9:.1f} GB HBM), "
        f"host pool of {n_blobs} distinct blobs ({n_blobs * S / 1e9:.1f} GB pinned) aliased over layers")
    host = torch.empty((n_blobs, S), dtype=torch.uint8).pin_memory()
    stage = torch.empty((16, S), dtype=torch.uint8, device="cuda")
    for b0 in range(0, n_blobs, 16):
        for j in range(min(16, n_blobs - b0)):
            b = b0 + j
            pack_expert(shape, syn.expert_weights(cfg, b // E, b % E, device="cuda"), stage[j])
        host[b0:b0 + 16].copy_(stage[:min(16, n_blobs - b0)].cpu())
    del stage
    slots = torch.empty((n_slots, S), dtype=torch.uint8, device="cuda")
    hb = host.data_ptr()
    blob_of = lambda l, e: (l * 97 + e) % n_blobs
    pool = [hb + blob_of(l, e) * S for l in range(L) for e in range(E)]
    ctx = dict(cfg=cfg, shape=shape, S=S, L=L, E=E, d=d, n_slots=n_slots, host=host, slots=slots, w_dtype=w_dtype,
               pool=pool, blob_of=blob_of, n_blobs=n_blobs, steps=steps, warmup=warmup,
               cstream=torch.cuda.Stream())
    cached_tokens(torch, syn, ctx, T)
    return ctx


def cached_tokens(torch, syn, ctx, T):
    """Set the batch size of the cached-decode workload: per-step router logits
    (fresh every step, so no replayed trace inflates the hit rate), the layer's
    workspace, activations, the fp32 residual and the bf16 next-layer input."""
    from expert_cache_ffn_amd.layer import Layer
    cfg, L, d = ctx["cfg"], ctx["L"], ctx["d"]
    ctx.pop("lgs", None)
    n_logits = ctx["warmup"] + ctx["steps"]
    ctx.update(T=T, lgs=[[syn.router_logits(cfg, T, layer=l, step=s, device="cuda") for l in range(L)]
                         for s in range(n_logits)],
               layer=Layer(ctx["shape"], T), xa=syn.activations(cfg, T, device="cuda"),
               res_f=torch.empty((T, d), dtype=torch.float32, device="cuda"),
               act=torch.empty((T, d), dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()  # setup queued on the default stream lands before the copy stream fills slots


def static_hot_set(syn, cfg, n_slots):
    """The n_slots most popular (layer, expert) pairs of the Zipf recipe: the same
    top ranks in every layer (all layers share one popularity law), the
    remainder spread one more rank over the first layers."""
    L = cfg.layers
    per, extra = divmod(n_slots, L)
    hot = []
    for l in range(L):
        rank = syn.popularity_rank(cfg, l)
        n_l = per + (1 if l < extra else 0)
        hot.append(sorted(int(e) for e in (rank <= n_l).nonzero().flatten()))
    return hot


# cached-decode policies at equal capacity: (q mode, fixed or measured ratio, static hot set)
POLICIES = {
    "lru_qstar": "shared LRU, misses split by q* at the configured B_P/B_H = 0.4",
    "lru_qstar_measured": "shared LRU, misses split by q* at the B_P/B_H measured by ecf_bandwidth_profile",
    "lru_all_pcie": "shared LRU, every miss copied over PCIe (q = m)",
    "static_hot": "the most popular pairs pinned once (static hot subset), every miss on the host (q = 0)",
}


def cached_oracle_check(torch, syn, ctx, rec, lgs_step):
    """The oracle layer by layer on one recorded cached-decode step: each layer's
    GPU input (the previous layer's bf16 output) and residual in, through the
    oracle's MoE layer on that layer's (aliased) host blobs; the GPU's layer
    output must equal residual + MoE within 2e-2 of the MoE part's RMS.  Timed:
    the oracle's tokens/s over the 43 layers (a bounded sample of the cached
    workload: one step)."""
    import numpy as np
    import oracle
    from expert_cache_ffn_amd.layer import blob_sections
    cfg, L, E, d, I, k = ctx["cfg"], ctx["L"], ctx["E"], ctx["d"], ctx["cfg"].inter, ctx["cfg"].top_k
    secs = dict(blob_sections(ctx["shape"]))
    host = ctx["host"]
    cache = {}

    def expert(b):
        if b not in cache:
            blob = host[b]
            n = d * I * 2
            cache[b] = {nm: blob[off:off + n].view(torch.bfloat16).view(I if nm != "w_down" else d,
                                                                        d if nm != "w_down" else I)
                        for nm, off in secs.items()}
        return cache[b]

    worst, el, T = 0.0, 0.0, rec[0][0].shape[0]
    for l, (x_in, r_in, out) in enumerate(rec):
        experts = [expert(ctx["blob_of"](l, e)) for e in range(E)]
        t0 = time.perf_counter()
        moe = oracle.moe_layer(x_in, experts, k, lg=lgs_step[l].cpu())["out"]
        el += time.perf_counter() - t0
        err = float(np.max(np.abs(out - (r_in + moe)))) / float(np.sqrt(np.mean(moe ** 2)))
        worst = max(worst, err)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    r = {"value": T / el, "unit": "tokens/s (43-layer step)", "cores": threads, "kind": "oracle",
         "sample": f"one step of {T} tokens through all {L} layers ({el:.1f} s of CPU time)",
         "checked_against_gpu": {"layers": L, "max_err_over_moe_rms": worst, "tolerance": 2e-2,
                                 "ok": bool(worst <= 2e-2)}}
    log(f"cached oracle: {r['value']:.2f} tok/s over {L} layers on {threads} threads; GPU layers within "
        f"{worst:.2e} of the oracle's (x RMS of each layer's MoE output)")
    return r


def bench_cached(torch, ecf, syn, ctx, policy="lru_qstar", bw=None, oracle_check=False, track_misses=False):
    """One policy on the shared cached-decode setup; returns throughput and traffic.
    oracle_check: afterwards one more step is recorded layer by layer and checked
    against (and timed beside) the oracle.  track_misses: also return each timed
    step's (trace step, (misses, lookups)) over its layers."""
    L, E, T, S = ctx["L"], ctx["E"], ctx["T"], ctx["S"]
    steps, warmup, lgs, lay = ctx["steps"], ctx["warmup"], ctx["lgs"], ctx["layer"]
    n_logits = len(lgs)
    cache = ecf.ecf_cache_create(L, E, ctx["n_slots"], ctx["n_slots"], S, ctx["slots"].data_ptr(), ctx["pool"],
                                 host_threads=0)
    q_mode, b_p, b_h = ecf.ECF_Q_AUTO, 0.4, 1.0
    if policy == "lru_qstar_measured":
        b_p, b_h = bw["b_p_conc"], bw["b_h"]
    elif policy == "lru_all_pcie":
        q_mode = ecf.ECF_Q_ALL_GPU
    elif policy == "static_hot":
        q_mode = ecf.ECF_Q_ALL_HOST
        for l, hot in enumerate(static_hot_set(syn, ctx["cfg"], ctx["n_slots"])):
            ecf.expert_cache_lookup(cache, l, hot)
            slots, _ = ecf.expert_cache_evict(cache, l, hot)
            for e, sl in zip(hot, slots):
                ctx["slots"][sl].copy_(ctx["host"][ctx["blob_of"](l, e)], non_blocking=True)
        torch.cuda.synchronize()
    elif policy != "lru_qstar":
        raise ValueError(policy)
    totals = dict(unique=0, hits=0, gpu_experts=0, misses=0, q=0, host=0, h2d=0, hostb=0, wait=0.0, hostms=0.0)
    qhist = {}
    per_step = []
    res_f, act, xa = ctx["res_f"], ctx["act"], ctx["xa"]

    def one_step(s, record, layers_out=None):
        x = xa
        res_f.zero_()
        sm = [0, 0]
        for l in range(L):
            a = lay.args(layer=l, router_logits=lgs[s % n_logits][l], cache=cache, b_p=b_p, b_h=b_h,
                         q_mode=q_mode, copy_stream=ctx["cstream"], residual=res_f, out_act=act)
            if layers_out is not None:
                torch.cuda.synchronize()
                x_in, r_in = x.cpu().clone(), res_f.cpu().numpy().copy()
            st = lay.forward(a, x, res_f)
            if layers_out is not None:
                torch.cuda.synchronize()
                layers_out.append((x_in, r_in, res_f.cpu().numpy().copy()))
            x = act
            if record:
                totals["unique"] += st["n_unique"]
                totals["hits"] += st["hits"]
                totals["gpu_experts"] += st["n_unique"] - st["host"]
                totals["misses"] += st["misses"]
                totals["q"] += st["q"]
                totals["host"] += st["host"]
                totals["h2d"] += st["bytes_h2d"]
                totals["hostb"] += st["bytes_host"]
                totals["wait"] += st["ms_wait_route"]
                totals["hostms"] += st["ms_host_ffn"]
                qhist[st["q"]] = qhist.get(st["q"], 0) + 1
                sm[0] += st["misses"]
                sm[1] += st["n_unique"]
        if record and track_misses:
            per_step.append((s, tuple(sm)))

    torch.cuda.synchronize()
    st0 = ecf.ecf_cache_get_stats(cache)
    for s in range(warmup):
        one_step(s, False)
    torch.cuda.synchronize()
    st1 = ecf.ecf_cache_get_stats(cache)
    t0 = time.perf_counter()
    for s in range(steps):
        one_step(warmup + s, True)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    st2 = ecf.ecf_cache_get_stats(cache)
    oracle_res = None
    if oracle_check:
        rec = []
        one_step(warmup + steps, False, rec)
        oracle_res = cached_oracle_check(torch, syn, ctx, rec, lgs[(warmup + steps) % n_logits])
    ecf.ecf_cache_destroy(cache)
    miss_cold = (st1["misses"] - st0["misses"]) / max(1, st1["lookups"] - st0["lookups"])
    miss_steady = (st2["misses"] - st1["misses"]) / max(1, st2["lookups"] - st1["lookups"])
    res = dict(policy=policy, policy_desc=POLICIES[policy], w_dtype=ctx["w_dtype"], slot_bytes=S, b_p=b_p, b_h=b_h,
               tokens=T, layers=L, slots=ctx["n_slots"], steps=steps, warmup=warmup,
               ms_per_step=1e3 * el / steps, tokens_per_s=T * steps / el, miss_rate_steady=miss_steady,
               miss_rate_warmup=miss_cold, unique_per_layer=totals["unique"] / (steps * L),
               q_total=totals["q"], host_total=totals["host"],
               pcie_GBps=totals["h2d"] / el / 1e9, host_read_GBps=totals["hostb"] / el / 1e9,
               # expert weights the GPU kernels read from slots (hits and copied misses)
               hbm_expert_GBps=totals["gpu_experts"] * S / el / 1e9,
               ms_wait_route_per_step=totals["wait"] / steps, ms_host_ffn_per_step=totals["hostms"] / steps,
               q_hist={str(q): n for q, n in sorted(qhist.items())}, host_blobs=ctx["n_blobs"],
               host_threads="default (min(16, hardware threads))")
    if oracle_res is not None:
        res["cpu_oracle"] = oracle_res
    if track_misses:
        res["per_step_misses"] = per_step
    log(f"cached {ctx['w_dtype']} [{policy}]: {res['ms_per_step']:.1f} ms/step ({L} layers), {res['tokens_per_s']:.1f} tok/s, "
        f"steady miss rate {100 * miss_steady:.1f}%, PCIe {res['pcie_GBps']:.1f} GB/s, "
        f"host {res['host_read_GBps']:.1f} GB/s, HBM (expert weights) {res['hbm_expert_GBps']:.1f} GB/s")
    return res


DRIFT_POLICIES = ("lru_qstar", "lru_qstar_measured", "static_hot")


def bench_drift(torch, ecf, syn, ctx, bw, args):
    """The policy ablation at 16 tokens on a trace whose hot set moves: each
    layer's Zipf(1.1) ranking is redrawn every args.drift_steps steps (a new
    seeded permutation per phase).  The static subset is bound once from the
    first phase's law, as a placement fixed at load or prefill time is; the
    shared LRU follows the routing.  Besides the whole timed window, each
    policy's miss rate is split into the first 8 steps after each phase change
    and the rest."""
    import dataclasses
    saved = {n: ctx[n] for n in ("cfg", "steps", "warmup")}
    ctx.update(cfg=dataclasses.replace(saved["cfg"], drift_steps=args.drift_steps), steps=args.drift_timed,
               warmup=args.cached_warmup)
    cached_tokens(torch, syn, ctx, 16)
    out = {"drift_steps": args.drift_steps, "warmup": ctx["warmup"], "steps": ctx["steps"],
           "phases_timed": sorted({syn.phase_of(ctx["cfg"], s)
                                   for s in range(ctx["warmup"], ctx["warmup"] + ctx["steps"])})}
    for p in DRIFT_POLICIES:
        r = bench_cached(torch, ecf, syn, ctx, p, bw, track_misses=True)
        r.pop("q_hist")
        per = r.pop("per_step_misses")
        fresh = [m for s, m in per if s % args.drift_steps < 8]
        rest = [m for s, m in per if s % args.drift_steps >= 8]
        frac = lambda v: sum(m for m, _ in v) / max(1, sum(n for _, n in v))
        r["miss_rate_first8_after_change"] = frac(fresh)
        r["miss_rate_rest_of_phase"] = frac(rest)
        out[p] = r
        log(f"drift [{p}]: miss rate {100 * r['miss_rate_steady']:.1f}% (first 8 steps of a phase "
            f"{100 * r['miss_rate_first8_after_change']:.1f}%, rest {100 * r['miss_rate_rest_of_phase']:.1f}%), "
            f"{r['tokens_per_s']:.1f} tok/s")
    ctx.update(saved)
    ctx.pop("lgs", None)
    return out


def bench_bandwidth(torch, ecf, ctx, seconds=2.0):
    """ecf_bandwidth_profile on 16 blobs of the cached pool (the q* inputs)."""
    S = ctx["S"]
    n = min(16, ctx["n_blobs"])
    dbuf = torch.empty((4, S), dtype=torch.uint8, device="cuda")
    cs = torch.cuda.Stream()
    torch.cuda.synchronize()
    r = ecf.ecf_bandwidth_profile(ctx["shape"], [ctx["host"].data_ptr() + i * S for i in range(n)],
                                  dbuf.data_ptr(), dbuf.numel(), copy_stream=cs.cuda_stream, seconds=seconds)
    del dbuf
    r["ratio_b_p_over_b_h"] = r["b_p_conc"] / r["b_h"]
    log(f"bandwidth: B_P {r['b_p']:.1f} GB/s alone, {r['b_p_conc']:.1f} with host experts; host experts "
        f"{r['b_cpu']:.1f} alone, {r['b_cpu_conc']:.1f} with copies ({r['host_threads']} threads); plain read "
        f"{r['b_read']:.1f}; B_H = {r['b_h']:.1f} GB/s, B_P/B_H = {r['ratio_b_p_over_b_h']:.3f}")
    return r


# ---- main ----------------------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workloads",
                    default="hbm,decode,decode_fp4,prefill,prefill_fp4,vendor,prefetch,cached,bandwidth,policies,"
                            "drift,cached_fp4",
                    help="any of hbm, decode, decode_fp4, prefill, prefill_fp4, vendor, prefetch, cached, bandwidth, "
                         "policies, drift, cached_fp4 (policies: the cached-decode policy ablation at equal capacity; "
                         "drift: the same ablation on a trace whose popularity ranking moves; *_fp4: the same layers "
                         "with MXFP4 experts; vendor: torch.bmm on the prefill GEMM shapes)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--cached-steps", type=int, default=32, help="cached decode timed steps per policy and batch size")
    ap.add_argument("--cached-warmup", type=int, default=16, help="cached decode warm-up steps (the LRU fills)")
    ap.add_argument("--policies", default=",".join(POLICIES), help="policies the 'policies' workload compares")
    ap.add_argument("--cached-tokens", default="1,4,16", help="cached-decode batch sizes (cached, policies)")
    ap.add_argument("--drift-steps", type=int, default=32,
                    help="drift workload: steps per popularity phase (each layer's Zipf ranking redrawn)")
    ap.add_argument("--drift-timed", type=int, default=80, help="drift workload: timed steps per policy")
    ap.add_argument("--calib-copy", action="store_true",
                    help="first run one plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--host-inputs", action="store_true",
                    help="decode and prefill: generate inputs on the host (no GPU kernels but libecf's and copies; "
                         "expert blobs repeat a few distinct experts) - for hardware counter passes")
    ap.add_argument("--prefill-steps", type=int, default=None,
                    help="prefill layers per timed loop (default max(20, steps / 10))")
    ap.add_argument("--decode-tokens", default="1,4,16",
                    help="decode batch sizes (the headline is 16; others are reported alongside)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(expert parallelism across GPUs is a design note, not code); run with --gpus 1.", flush=True)
        sys.exit(2)

    import torch
    import ecf_synth as syn
    import expert_cache_ffn_amd as ecf

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    ecf.lib()
    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")  # contents do not matter
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: 1 GiB device to device")
        del src, dst
    wl = set(args.workloads.split(","))
    hbm = bench_hbm(torch, ecf) if "hbm" in wl else None
    Ts = tuple(int(t) for t in args.decode_tokens.split(","))
    head, also, cpu, sample = None, {}, None, None
    if "decode" in wl:
        dec, sample = bench_decode(torch, ecf, syn, Ts, args.steps, args.warmup, use_graph=not args.no_graph,
                                   host_inputs=args.host_inputs)
        head = dec.get(16)
        also.update({f"decode_T{T}": dec[T] for T in Ts if T != 16})
    if "decode_fp4" in wl:
        dec4, _ = bench_decode(torch, ecf, syn, (1, 16), args.steps, args.warmup, use_graph=not args.no_graph,
                               host_inputs=args.host_inputs, w_dtype="mxfp4")
        also.update({f"decode_mxfp4_T{T}": dec4[T] for T in dec4})
        torch.cuda.empty_cache()
    psteps = args.prefill_steps or max(20, args.steps // 10)
    if "prefill" in wl:
        also["prefill_bf16_T4096"] = bench_prefill(torch, ecf, syn, "prefill", psteps,
                                                   max(2, args.warmup // 5), cpu=not args.no_cpu_baseline,
                                                   host_inputs=args.host_inputs)
    if "prefill_fp4" in wl:
        also["prefill_mxfp4_T8192"] = bench_prefill(torch, ecf, syn, "prefill_fp4", psteps,
                                                    max(2, args.warmup // 5), cpu=not args.no_cpu_baseline,
                                                    host_inputs=args.host_inputs)
    if "vendor" in wl:
        also["vendor_bmm_calibration"] = bench_vendor_gemm(torch)
    # each prefill layer's MFMA rate against what the MFMA pipes sustain on this
    # GPU with nothing else to do (ecf_mfma_rate), beside the datasheet fraction
    if hbm:
        for key in ("prefill_bf16_T4096", "prefill_mxfp4_T8192"):
            if key in also:
                also[key]["mfma_frac_of_mfma_only_loop"] = also[key]["tflops"] / hbm["mfma_bf16_TFLOPs"]
    if sample is not None and not args.no_cpu_baseline:
        log("cpu baseline: oracle on sampled decode batches")
        cpu = cpu_baseline_decode(torch, syn, sample)
        log(f"cpu baseline: {cpu['value']:.2f} tok/s on {cpu['cores']} threads")
    del sample
    torch.cuda.empty_cache()
    if "prefetch" in wl:
        also["prefill_bf16_streamed_stack"] = bench_prefetch(torch, ecf, syn, "prefill")
        also["prefill_mxfp4_streamed_stack"] = bench_prefetch(torch, ecf, syn, "prefill_fp4")
    if wl & {"cached", "bandwidth", "policies", "drift"}:
        cw = args.cached_steps if args.cached_warmup is None else args.cached_warmup
        ctx = cached_setup(torch, ecf, syn, steps=args.cached_steps, warmup=cw)
        bw = None
        if wl & {"bandwidth", "policies", "drift"}:
            bw = also["bandwidth_profile"] = bench_bandwidth(torch, ecf, ctx)
        for T in (int(t) for t in args.cached_tokens.split(",") if wl & {"cached", "policies"}):
            cached_tokens(torch, syn, ctx, T)
            if "cached" in wl:
                also[f"cached_decode_43L_T{T}"] = bench_cached(
                    torch, ecf, syn, ctx, "lru_qstar", oracle_check=T == 16 and not args.no_cpu_baseline)
            if "policies" in wl:
                pol = {p: (dict(also[f"cached_decode_43L_T{T}"]) if p == "lru_qstar" and "cached" in wl
                           else bench_cached(torch, ecf, syn, ctx, p, bw))
                       for p in POLICIES if p in args.policies.split(",")}
                for r in pol.values():
                    r.pop("q_hist")
                also[f"cached_policies_43L_T{T}"] = pol
        if "drift" in wl:
            also["cached_policies_43L_T16_drift"] = bench_drift(torch, ecf, syn, ctx, bw, args)
        del ctx
        torch.cuda.empty_cache()
    if "cached_fp4" in wl:
        cw = args.cached_steps if args.cached_warmup is None else args.cached_warmup
        ctx = cached_setup(torch, ecf, syn, steps=args.cached_steps, warmup=cw, w_dtype="mxfp4")
        bw4 = also["bandwidth_profile_mxfp4"] = bench_bandwidth(torch, ecf, ctx)
        for p in ("lru_qstar", "lru_qstar_measured"):
            r = bench_cached(torch, ecf, syn, ctx, p, bw4)
            r.pop("q_hist")
            also[f"cached_decode_mxfp4_43L_T16_{p}"] = r
        del ctx
        torch.cuda.empty_cache()
    if head is None:  # a partial run (profiling): no headline line
        print(json.dumps({"partial": True, "also": also}), flush=True)
        return

    traffic = None
    tpath = os.path.join(ROOT, "profiles", "decode_gateup_T16_traffic.md")
    if head is not None and os.path.exists(tpath):
        # measured HBM bytes / algorithmic bytes of the same launches (FETCH_SIZE and
        # WRITE_SIZE passes, copy-calibrated), valid while the kernel source is unchanged
        txt = open(tpath).read()
        tj = json.loads(txt.split("```json", 1)[1].split("```", 1)[0])
        if tj.get("source_hash") == src_hash("k_decode.hip", "device_common.h"):
            traffic = tj["traffic_ratio"] * head["gateup_bytes"]
    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded counter-based generator; random-init experts N(0,0.02), x N(0,1))",
        "config": {"workload": "decode MoE layer, bf16, 16 tokens, d 4096, 256 experts resident, I 1024, top-6 "
                               "(router GEMV + top-k + permutation + gate/up/SwiGLU + down + combine); "
                               "64 rotating batches, "
                               + ("HIP graph per batch" if head["graph"] else "eager launches")
                               + (", host-generated inputs" if args.host_inputs else ""),
                   "tokens": 16, "hidden": 4096, "experts": 256, "inter": 1024, "top_k": 6},
        "roofline": {"bound": "hbm", "kernel": "decode_gateup", "achieved": head["gateup_GBps"],
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": head["gateup_GBps"] / HBM_PEAK_GBS,
                     "traffic": traffic, "algorithmic_bytes_per_launch": head["gateup_bytes"],
                     "avg_launch_us": head["gateup_avg_us"],
                     "whole_layer_GBps": head["layer_GBps"], "whole_layer_frac": head["layer_hbm_frac"],
                     "achievable_on_this_gpu": hbm},
        "cpu_baseline": cpu,
        "also": also,
        "headline_detail": head,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
