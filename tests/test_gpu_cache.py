"""GPU tests of the expert-cache mode: split invariance (all-GPU, all-host,
fixed and q* splits agree with the all-resident layer within 1e-5 * RMS),
cache-state invariance (cold, warm, resized), LRU statistics against the
oracle's reference LRU on the same routing, and prefetch_layer."""
import numpy as np
import pytest
import torch

import ecf_synth as syn
import expert_cache_ffn_amd as ecf
import oracle
from expert_cache_ffn_amd.layer import Layer, pack_expert
from gpu_util import say, shape_of

pytestmark = pytest.mark.gpu

SPLIT_TOL = 1e-5


class CachedSetup:
    """L layers over an (optionally aliased) pinned host pool of expert blobs."""

    def __init__(self, cfg, L, n_slots, n_blobs=None, gen_device="cpu"):
        self.cfg, self.L = cfg, L
        self.shape = shape_of(cfg)
        self.slot_bytes = ecf.ecf_expert_bytes(self.shape)
        E = cfg.experts
        self.n_blobs = n_blobs or L * E
        self.host = torch.empty((self.n_blobs, self.slot_bytes), dtype=torch.uint8).pin_memory()
        self.dev_blobs = torch.empty((self.n_blobs, self.slot_bytes), dtype=torch.uint8, device="cuda")
        for b in range(self.n_blobs):
            ex = syn.expert_weights(cfg, b // E, b % E, device=gen_device)
            pack_expert(self.shape, {k: v.to("cuda") for k, v in ex.items()}, self.dev_blobs[b])
        self.host.copy_(self.dev_blobs.cpu())
        self.slots = torch.empty((max(n_slots, 1), self.slot_bytes), dtype=torch.uint8, device="cuda")
        hbase, dbase = self.host.data_ptr(), self.dev_blobs.data_ptr()
        self.blob_of = lambda l, e: (l * E + e) % self.n_blobs
        self.h_pool = [hbase + self.blob_of(l, e) * self.slot_bytes for l in range(L) for e in range(E)]
        self.resident_ptrs = [torch.tensor([dbase + self.blob_of(l, e) * self.slot_bytes for e in range(E)],
                                           dtype=torch.int64, device="cuda") for l in range(L)]
        self.cache = ecf.ecf_cache_create(L, E, n_slots, max(n_slots, 1), self.slot_bytes, self.slots.data_ptr(),
                                          self.h_pool, host_threads=4)

    def close(self):
        ecf.ecf_cache_destroy(self.cache)


def _run(layer_obj, a, x, T, d):
    out = torch.full((T, d), float("nan"), dtype=torch.float32, device="cuda")
    st = layer_obj.forward(a, x, out)
    torch.cuda.synchronize()
    return out.cpu().numpy(), st


@pytest.mark.parametrize("w_dtype", ["bf16", "mxfp4"])
@pytest.mark.parametrize("mode,q_fixed", [(ecf.ECF_Q_ALL_GPU, 0), (ecf.ECF_Q_ALL_HOST, 0), (ecf.ECF_Q_FIXED, 2),
                                          (ecf.ECF_Q_AUTO, 0)])
def test_split_invariance_small(mode, q_fixed, w_dtype):
    cfg = syn.gen.Config(100, "cs", (4,), 512, 16, 256, 4, w_dtype, "bf16", "zipf", layers=3)
    L, T, d = 3, 4, cfg.hidden
    cs = CachedSetup(cfg, L, n_slots=10)
    lay = Layer(cs.shape, T)
    cstream = torch.cuda.Stream()
    ref_lru = oracle.LRURef(10, cfg.experts)
    rule = {ecf.ECF_Q_ALL_GPU: lambda m: m, ecf.ECF_Q_ALL_HOST: lambda m: 0,
            ecf.ECF_Q_FIXED: lambda m: min(q_fixed, m), ecf.ECF_Q_AUTO: lambda m: oracle.qstar(m, 0.4, 1.0)}[mode]
    try:
        for step in range(9):
            l = step % L
            x = syn.activations(cfg, T, layer=l, batch=step, device="cuda")
            lg = syn.router_logits(cfg, T, layer=l, step=step, device="cuda")
            ref, _ = _run(lay, lay.args(layer=l, router_logits=lg, expert_ptrs=cs.resident_ptrs[l]), x, T, d)
            a = lay.args(layer=l, router_logits=lg, cache=cs.cache, b_p=0.4, b_h=1.0, q_mode=mode,
                         q_fixed=q_fixed, copy_stream=cstream)
            got, st = _run(lay, a, x, T, d)
            rms = np.sqrt(np.mean(ref ** 2))
            err = np.max(np.abs(got - ref)) / rms
            say(f"step {step} layer {l} mode {mode}: m={st['misses']} q={st['q']} host={st['host']} "
                f"err/RMS={err:.2e}")
            assert err <= SPLIT_TOL, f"split changed the output: {err:.3e}"
            # LRU bookkeeping against the reference on the oracle's routing
            idx, _ = oracle.route(lg.cpu().numpy(), cfg.top_k)
            rows = {}
            for e in idx.ravel():
                rows[int(e)] = rows.get(int(e), 0) + 1
            plan = ref_lru.step(l, rows, rule)
            assert (st["hits"], st["misses"], st["q"]) == (len(plan["hits"]), plan["m"], plan["q"])
        stats = ecf.ecf_cache_get_stats(cs.cache)
        assert {k: stats[k] for k in ref_lru.stats} == ref_lru.stats
    finally:
        cs.close()


@pytest.mark.parametrize("w_dtype", ["bf16", "mxfp4"])
def test_split_invariance_many_tokens(w_dtype):
    """100 tokens (past the decode/prefill switch of the all-resident mode): cache
    mode still runs the GEMVs, so every split agrees with the resident decode
    path within 1e-5; an explicit PREFILL request in cache mode is refused."""
    cfg = syn.gen.Config(102, "cs", (100,), 512, 16, 256, 4, w_dtype, "bf16", "zipf", layers=1)
    T, d = 100, cfg.hidden
    cs = CachedSetup(cfg, 1, n_slots=6)
    lay = Layer(cs.shape, T)
    cstream = torch.cuda.Stream()
    try:
        x = syn.activations(cfg, T, device="cuda")
        lg = syn.router_logits(cfg, T, device="cuda")
        ref, st_ref = _run(lay, lay.args(router_logits=lg, expert_ptrs=cs.resident_ptrs[0], path=ecf.ECF_PATH_DECODE),
                           x, T, d)
        rms = np.sqrt(np.mean(ref ** 2))
        for mode, qf in [(ecf.ECF_Q_ALL_HOST, 0), (ecf.ECF_Q_FIXED, 3), (ecf.ECF_Q_ALL_GPU, 0), (ecf.ECF_Q_AUTO, 0)]:
            got, st = _run(lay, lay.args(router_logits=lg, cache=cs.cache, q_mode=mode, q_fixed=qf,
                                         copy_stream=cstream), x, T, d)
            err = np.max(np.abs(got - ref)) / rms
            say(f"T=100 {w_dtype} mode {mode}: path={st['path']} m={st['misses']} q={st['q']} host={st['host']} "
                f"err/RMS={err:.2e}")
            assert st["path"] == ecf.ECF_PATH_DECODE
            assert err <= SPLIT_TOL
        with pytest.raises(ecf.EcfError) as ei:
            _run(lay, lay.args(router_logits=lg, cache=cs.cache, path=ecf.ECF_PATH_PREFILL), x, T, d)
        assert ei.value.code == ecf.ECF_EUNSUPPORTED
    finally:
        cs.close()


def test_cache_state_invariance_and_resize():
    cfg = syn.gen.Config(101, "cs", (8,), 512, 16, 256, 4, "bf16", "bf16", "zipf", layers=2)
    L, T, d = 2, 8, cfg.hidden
    cs = CachedSetup(cfg, L, n_slots=24)
    lay = Layer(cs.shape, T)
    try:
        x = syn.activations(cfg, T, layer=0, device="cuda")
        lg = syn.router_logits(cfg, T, layer=0, step=0, device="cuda")
        ref, _ = _run(lay, lay.args(layer=0, router_logits=lg, expert_ptrs=cs.resident_ptrs[0]), x, T, d)
        a = lay.args(layer=0, router_logits=lg, cache=cs.cache, q_mode=ecf.ECF_Q_ALL_GPU)
        cold, st0 = _run(lay, a, x, T, d)
        warm, st1 = _run(lay, a, x, T, d)
        assert st0["hits"] == 0 and st1["misses"] == 0
        ecf.ecf_cache_resize(cs.cache, 3)
        shrunk, st2 = _run(lay, lay.args(layer=0, router_logits=lg, cache=cs.cache, q_mode=ecf.ECF_Q_AUTO), x, T, d)
        ecf.ecf_cache_resize(cs.cache, 0)
        none, st3 = _run(lay, lay.args(layer=0, router_logits=lg, cache=cs.cache, q_mode=ecf.ECF_Q_AUTO), x, T, d)
        assert st3["q"] == 0 and st3["host"] == st3["n_unique"]
        rms = np.sqrt(np.mean(ref ** 2))
        for name, o in [("cold", cold), ("warm", warm), ("shrunk", shrunk), ("no slots", none)]:
            err = np.max(np.abs(o - ref)) / rms
            say(f"{name}: err/RMS = {err:.2e}")
            assert err <= SPLIT_TOL
        assert np.array_equal(cold, warm)
    finally:
        cs.close()


def test_cached_decode_full_shape_two_layers():
    """d 4096, 256 experts, I 1024, top-6, T 16, slots = 37% of the (2-layer)
    pool, Zipf(1.1) routing, q* at B_P/B_H = 0.4; host blobs aliased 32 ways."""
    base = syn.CONFIGS["cached"]
    L, T, d = 2, 16, base.hidden
    n_slots = int(0.37 * L * base.experts)
    say(f"case: cached decode full shape, {n_slots} slots")
    cs = CachedSetup(base, L, n_slots=n_slots, n_blobs=32, gen_device="cuda")
    lay = Layer(cs.shape, T)
    cstream = torch.cuda.Stream()
    try:
        for step in range(6):
            l = step % L
            x = syn.activations(base, T, layer=l, batch=step, device="cuda")
            lg = syn.router_logits(base, T, layer=l, step=step, device="cuda")
            ref, _ = _run(lay, lay.args(layer=l, router_logits=lg, expert_ptrs=cs.resident_ptrs[l]), x, T, d)
            got, st = _run(lay, lay.args(layer=l, router_logits=lg, cache=cs.cache, b_p=0.4, b_h=1.0,
                                         copy_stream=cstream), x, T, d)
            err = np.max(np.abs(got - ref)) / np.sqrt(np.mean(ref ** 2))
            say(f"step {step}: unique={st['n_unique']} hits={st['hits']} m={st['misses']} q={st['q']} "
                f"host={st['host']} wait={st['ms_wait_route']:.2f}ms host_ffn={st['ms_host_ffn']:.2f}ms "
                f"err/RMS={err:.2e}")
            assert st["q"] == ecf.qstar_split(st["misses"], 0.4, 1.0)
            assert err <= SPLIT_TOL
    finally:
        cs.close()


def test_residual_stack_and_activation_copy():
    cfg = syn.gen.Config(102, "cs", (4,), 512, 8, 256, 2, "bf16", "bf16", "zipf", layers=2)
    cs = CachedSetup(cfg, 2, n_slots=4)
    T, d = 4, cfg.hidden
    lay = Layer(cs.shape, T)
    try:
        x = syn.activations(cfg, T, device="cuda")
        res = torch.randn(T, d, device="cuda")
        act = torch.empty(T, d, dtype=torch.bfloat16, device="cuda")
        lg = syn.router_logits(cfg, T, layer=0, device="cuda")
        out = torch.empty(T, d, dtype=torch.float32, device="cuda")
        a = lay.args(layer=0, router_logits=lg, cache=cs.cache, residual=res, out_act=act)
        lay.forward(a, x, out)
        plain = torch.empty_like(out)
        lay.forward(lay.args(layer=0, router_logits=lg, expert_ptrs=cs.resident_ptrs[0]), x, plain)
        torch.cuda.synchronize()
        assert torch.allclose(out, plain + res, atol=1e-5 * float(plain.abs().max()) + 1e-6)
        assert torch.equal(act, out.to(torch.bfloat16))
    finally:
        cs.close()


def test_prefetch_layer_copies_and_signals():
    n = 64 << 20
    h = torch.randint(0, 255, (n,), dtype=torch.uint8).pin_memory()
    dbuf = torch.zeros(2 * n, dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    ev = torch.cuda.Event()
    ev.record(s)  # creates the underlying hipEvent
    ecf.prefetch_layer(h.data_ptr(), dbuf.data_ptr() + n, n, n, s.cuda_stream, ev.cuda_event)
    ev.synchronize()
    assert torch.equal(dbuf[n:].cpu(), h)
    with pytest.raises(ecf.EcfError) as ei:
        ecf.prefetch_layer(h.data_ptr(), dbuf.data_ptr(), n, n - 1, s.cuda_stream, ev.cuda_event)
    assert ei.value.code == ecf.ECF_ENOSPC


def test_bandwidth_profile_sane():
    """ecf_bandwidth_profile on a few small pinned blobs: every rate positive,
    b_h the sum of the concurrent rates, and its ratio usable by qstar_split."""
    cfg = syn.Config(90, "bw", (1,), 1024, 8, 512, 2, "bf16", "bf16", "router")
    shape = shape_of(cfg)
    S = ecf.ecf_expert_bytes(shape)
    n = 6
    host = torch.zeros((n, S), dtype=torch.uint8).pin_memory()
    dbuf = torch.empty((4, S), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    say(f"bandwidth profile: {n} blobs of {S} bytes, 0.4 s")
    r = ecf.ecf_bandwidth_profile(shape, [host.data_ptr() + i * S for i in range(n)], dbuf.data_ptr(),
                                  dbuf.numel(), seconds=0.4, host_threads=4)
    say(str(r))
    for key in ("b_p", "b_cpu", "b_read", "b_p_conc", "b_cpu_conc", "b_h"):
        assert r[key] > 0.0 and np.isfinite(r[key]), key
    assert r["b_h"] == pytest.approx(r["b_p_conc"] + r["b_cpu_conc"], rel=1e-12)
    assert r["host_threads"] == 4
    for m in (0, 1, 7, 40):
        q = ecf.qstar_split(m, r["b_p_conc"], r["b_h"])
        assert 0 <= q <= m
