"""GPU tests of the expert-cache mode: split invariance (all-GPU, all-host,
fixed and q* splits agree with the all-resident layer within 1e-5 * RMS),
cache-state invariance (cold, warm, resized), LRU statistics against the
oracle's reference LRU on the same routing, the whole-layer prefetch into the
slot pool and prefill through it."""
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
    path within 1e-5.  An explicit PREFILL request in cache mode copies every miss
    (no host split), so with 6 slots for ~16 routed experts it is ECF_ENOSPC."""
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
        assert ei.value.code == ecf.ECF_ENOSPC
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


def _layer_experts(cs, cfg, l):
    """CPU tensors of layer l's experts as the cache's host pool holds them (aliased blobs)."""
    E = cfg.experts
    memo = cs.__dict__.setdefault("_cpu_blobs", {})
    out = []
    for e in range(E):
        b = cs.blob_of(l, e)
        if b not in memo:
            memo[b] = {k: v.cpu() for k, v in syn.expert_weights(cfg, b // E, b % E, device="cuda").items()}
        out.append(memo[b])
    return out


@pytest.mark.parametrize("T", [1, 4, 16, 64])
def test_cached_decode_full_shape_two_layers(T):
    """d 4096, 256 experts, I 1024, top-6, slots = 37% of the (2-layer) pool,
    Zipf(1.1) routing, q* at B_P/B_H = 0.4, host blobs aliased 32 ways: every
    step's cache-mode output (GPU experts + host experts + host partial) against
    the oracle within the bf16 bar, routing and counts exact, and against the
    all-resident layer within 1e-5."""
    base = syn.CONFIGS["cached"]
    L, d, k, E = 2, base.hidden, base.top_k, base.experts
    n_slots = int(0.37 * L * base.experts)
    say(f"case: cached decode full shape T={T}, {n_slots} slots")
    cs = CachedSetup(base, L, n_slots=n_slots, n_blobs=32, gen_device="cuda")
    lay = Layer(cs.shape, T)
    cstream = torch.cuda.Stream()
    try:
        host_total = 0
        for step in range(6):
            l = step % L
            x = syn.activations(base, T, layer=l, batch=step, device="cuda")
            lg = syn.router_logits(base, T, layer=l, step=step, device="cuda")
            ref, _ = _run(lay, lay.args(layer=l, router_logits=lg, expert_ptrs=cs.resident_ptrs[l]), x, T, d)
            idx = torch.full((T * k,), -1, dtype=torch.int32, device="cuda")
            counts = torch.full((E,), -1, dtype=torch.int32, device="cuda")
            got, st = _run(lay, lay.args(layer=l, router_logits=lg, cache=cs.cache, b_p=0.4, b_h=1.0,
                                         copy_stream=cstream, topk_idx=idx, counts=counts), x, T, d)
            host_total += st["host"]
            orc = oracle.moe_layer(x.cpu(), _layer_experts(cs, base, l), k, lg=lg.cpu())
            assert np.array_equal(idx.cpu().numpy().reshape(T, k), orc["idx"])
            assert np.array_equal(counts.cpu().numpy(), orc["counts"])
            rms = np.sqrt(np.mean(orc["out"] ** 2))
            e_orc = np.max(np.abs(got - orc["out"])) / rms
            err = np.max(np.abs(got - ref)) / np.sqrt(np.mean(ref ** 2))
            say(f"step {step}: unique={st['n_unique']} hits={st['hits']} m={st['misses']} q={st['q']} "
                f"host={st['host']} wait={st['ms_wait_route']:.2f}ms host_ffn={st['ms_host_ffn']:.2f}ms "
                f"err/RMS vs resident {err:.2e}, vs oracle {e_orc:.2e}")
            assert st["q"] == ecf.qstar_split(st["misses"], 0.4, 1.0)
            assert err <= SPLIT_TOL
            assert e_orc <= 2e-2
        assert host_total > 0  # the host half of the split ran
    finally:
        cs.close()


def test_stack_three_layers_against_oracle():
    """Three stacked layers in cache mode (q* at 0.4, host experts on): the residual
    stream stays fp32 (out = residual + MoE(x)) and each layer's input is the
    previous output rounded to bf16 (d_out_act).  Layer by layer, the GPU output
    equals the GPU's residual input plus the oracle's layer on the GPU's own bf16
    input, within 2e-2 of that layer's RMS, and the bf16 copy is the output
    rounded to nearest even."""
    cfg = syn.gen.Config(103, "stack", (6,), 512, 16, 256, 4, "bf16", "bf16", "zipf", layers=3)
    L, T, d, k = 3, 6, cfg.hidden, cfg.top_k
    cs = CachedSetup(cfg, L, n_slots=12)
    lay = Layer(cs.shape, T)
    cstream = torch.cuda.Stream()
    try:
        x = syn.activations(cfg, T, device="cuda")
        res_f = x.float().clone()
        act = torch.empty(T, d, dtype=torch.bfloat16, device="cuda")
        for l in range(L):
            lg = syn.router_logits(cfg, T, layer=l, device="cuda")
            x_in, r_in = x.cpu().clone(), res_f.cpu().numpy().copy()
            a = lay.args(layer=l, router_logits=lg, cache=cs.cache, b_p=0.4, b_h=1.0, copy_stream=cstream,
                         residual=res_f, out_act=act)
            st = lay.forward(a, x, res_f)
            torch.cuda.synchronize()
            out = res_f.cpu().numpy()
            moe = oracle.moe_layer(x_in, _layer_experts(cs, cfg, l), k, lg=lg.cpu())["out"]
            rms = np.sqrt(np.mean(moe ** 2))
            err = np.max(np.abs(out - (r_in + moe))) / rms
            say(f"stack layer {l}: m={st['misses']} q={st['q']} host={st['host']} err/RMS {err:.2e}")
            assert err <= 2e-2
            assert torch.equal(act.cpu(), res_f.cpu().to(torch.bfloat16))
            x = act.clone()
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


def test_prefetch_layer_fills_slots_and_signals():
    """prefetch_layer binds every expert of a layer to cache slots and copies each
    host blob in (consecutive slots and host blobs as one copy); the slots then
    hold the blobs byte for byte, a second prefetch of the pending layer adds
    nothing, and bad arguments are refused."""
    cfg = syn.gen.Config(104, "pf", (8,), 512, 8, 256, 2, "bf16", "bf16", "uniform", layers=2)
    cs = CachedSetup(cfg, 2, n_slots=16)
    s = torch.cuda.Stream()
    ev = torch.cuda.Event()
    ev.record(s)  # creates the underlying hipEvent
    try:
        blob = ecf.ecf_expert_bytes(cs.shape)
        assert ecf.prefetch_layer(cs.cache, 1, blob, s.cuda_stream, ev.cuda_event) == (8, 0)
        ev.synchronize()
        for e in range(8):
            sl = ecf.ecf_cache_slot_of(cs.cache, 1, e)
            assert sl == e  # lowest free slots, ascending expert id
            assert torch.equal(cs.slots[sl].cpu(), cs.host[cs.blob_of(1, e)])
        assert ecf.prefetch_layer(cs.cache, 1, blob, s.cuda_stream) == (0, 0)
        with pytest.raises(ecf.EcfError) as ei:
            ecf.prefetch_layer(cs.cache, 2, blob, s.cuda_stream)
        assert ei.value.code == ecf.ECF_EINVAL
        with pytest.raises(ecf.EcfError) as ei:
            ecf.prefetch_layer(cs.cache, 0, cs.slot_bytes + 1, s.cuda_stream)
        assert ei.value.code == ecf.ECF_EINVAL
        assert ecf.ecf_cache_get_stats(cs.cache)["inserts"] == 8
    finally:
        cs.close()


def _rows_of(lg, k):
    idx, _ = oracle.route(lg.cpu().numpy(), k)
    rows = {}
    for e in idx.ravel():
        rows[int(e)] = rows.get(int(e), 0) + 1
    return rows


@pytest.mark.parametrize("w_dtype,layers_of_slots", [("bf16", 2.0), ("mxfp4", 2.0), ("bf16", 1.5)])
def test_streamed_prefill_through_slot_pool(w_dtype, layers_of_slots):
    """Prefill over 3 stacked layers with layer l+1 prefetched into the shared slot
    pool while layer l computes (no host sync between layers): each layer's
    output equals the all-resident prefill layer bit for bit and the oracle
    within the bar; with 1.5 layers of slots part of each prefetch does not fit
    and the forward call fills the rest on demand.  Afterwards the cache state
    (every (layer, expert) slot, the LRU counters) equals the reference LRU run
    through the same prefetches and steps, and a decode step on the last layer
    finds its experts resident."""
    E, L, T, k = 16, 3, 300, 4
    cfg = syn.gen.Config(105, "pf", (T,), 512, E, 256, k, w_dtype, "bf16", "uniform", layers=L)
    d = cfg.hidden
    n_slots = int(layers_of_slots * E)
    say(f"case: streamed prefill {w_dtype}, {n_slots} slots for {E}-expert layers")
    cs = CachedSetup(cfg, L, n_slots=n_slots)
    lay = Layer(cs.shape, T)
    cstream = torch.cuda.Stream()
    ref_lru = oracle.LRURef(n_slots, E)
    blob = ecf.ecf_expert_bytes(cs.shape)
    tol = 5e-2 if w_dtype == "mxfp4" else 2e-2
    try:
        xs = [syn.activations(cfg, T, layer=l, device="cuda") for l in range(L)]
        lgs = [syn.router_logits(cfg, T, layer=l, device="cuda") for l in range(L)]
        outs = [torch.full((T, d), float("nan"), dtype=torch.float32, device="cuda") for _ in range(L)]
        torch.cuda.synchronize()
        pf = [ecf.prefetch_layer(cs.cache, 0, blob, cstream.cuda_stream)]
        sts = []
        for l in range(L):
            if l + 1 < L:
                pf.append(ecf.prefetch_layer(cs.cache, l + 1, blob, cstream.cuda_stream))
            a = lay.args(layer=l, router_logits=lgs[l], cache=cs.cache, path=ecf.ECF_PATH_PREFILL,
                         copy_stream=cstream)
            sts.append(lay.forward(a, xs[l], outs[l]))
        torch.cuda.synchronize()
        for l in range(L):
            r = ref_lru.prefetch(l) if l == 0 else None
            if l + 1 < L:
                r1 = ref_lru.prefetch(l + 1)
                assert (len(r1["copied"]), r1["missing"]) == pf[l + 1], (l, r1, pf[l + 1])
            if r is not None:
                assert (len(r["copied"]), r["missing"]) == pf[0]
            plan = ref_lru.step(l, _rows_of(lgs[l], k), lambda m: m, prefill=True)
            st = sts[l]
            say(f"layer {l}: prefetch copied/missing {pf[l]}, step hits={st['hits']} m={st['misses']} q={st['q']}")
            assert st["path"] == ecf.ECF_PATH_PREFILL and st["host"] == 0
            assert (st["hits"], st["misses"], st["q"]) == (len(plan["hits"]), plan["m"], plan["q"])
            ref, _ = _run(lay, lay.args(layer=l, router_logits=lgs[l], expert_ptrs=cs.resident_ptrs[l],
                                        path=ecf.ECF_PATH_PREFILL), xs[l], T, d)
            got = outs[l].cpu().numpy()
            assert np.array_equal(got, ref), f"layer {l}: slot-pool prefill differs from the resident layer"
            toks = np.arange(0, T, 5)
            orc = oracle.moe_layer(xs[l].cpu(), _layer_experts(cs, cfg, l), k, lg=lgs[l].cpu(), w_dtype=w_dtype,
                                   tokens=toks)
            err = np.max(np.abs(got[toks] - orc["out"])) / np.sqrt(np.mean(orc["out"] ** 2))
            say(f"layer {l}: err/RMS vs oracle {err:.2e} on {len(toks)} tokens")
            assert err <= tol
        if layers_of_slots < 2:
            assert any(m > 0 for _, m in pf)  # part of a prefetch did not fit
        for l in range(L):
            for e in range(E):
                want = ref_lru.resident(l, e)
                assert ecf.ecf_cache_slot_of(cs.cache, l, e) == (-1 if want is None else want), (l, e)
        stats = ecf.ecf_cache_get_stats(cs.cache)
        assert {n: stats[n] for n in ref_lru.stats} == ref_lru.stats
        # survivors warm decode
        x = syn.activations(cfg, 4, layer=L - 1, batch=7, device="cuda")
        lg = syn.router_logits(cfg, 4, layer=L - 1, step=7, device="cuda")
        _, st = _run(lay, lay.args(layer=L - 1, router_logits=lg, cache=cs.cache), x, 4, d)
        say(f"decode after prefill: unique={st['n_unique']} hits={st['hits']}")
        assert st["hits"] > 0
        if layers_of_slots >= 2:
            assert st["hits"] == st["n_unique"]
    finally:
        cs.close()


def test_prefetch_holds_against_decode_and_resize():
    """A pending whole-layer prefetch next to decode steps of other layers: its
    entries are held (a decode step copying every miss never evicts them, and
    fewer slots are then available to it), a second prefetch of the layer adds
    nothing, the layer's own step ends the hold, and a resize waits for pending
    copies and drops the holds.  Every step's output matches the all-resident
    layer within 1e-5, and the cache state follows the reference LRU."""
    E, L, T, k = 8, 3, 4, 2
    cfg = syn.gen.Config(107, "ph", (T,), 512, E, 256, k, "bf16", "bf16", "zipf", layers=L)
    d = cfg.hidden
    n_slots = 12
    cs = CachedSetup(cfg, L, n_slots=n_slots)
    lay = Layer(cs.shape, T)
    cstream = torch.cuda.Stream()
    ref = oracle.LRURef(n_slots, E)
    blob = ecf.ecf_expert_bytes(cs.shape)

    def step(l, s, q_mode=ecf.ECF_Q_ALL_GPU):
        x = syn.activations(cfg, T, layer=l, batch=s, device="cuda")
        lg = syn.router_logits(cfg, T, layer=l, step=s, device="cuda")
        got, st = _run(lay, lay.args(layer=l, router_logits=lg, cache=cs.cache, q_mode=q_mode, copy_stream=cstream),
                       x, T, d)
        want, _ = _run(lay, lay.args(layer=l, router_logits=lg, expert_ptrs=cs.resident_ptrs[l]), x, T, d)
        err = np.max(np.abs(got - want)) / np.sqrt(np.mean(want ** 2))
        plan = ref.step(l, _rows_of(lg, k), (lambda m: m) if q_mode == ecf.ECF_Q_ALL_GPU else (lambda m: 0))
        assert (st["hits"], st["misses"], st["q"]) == (len(plan["hits"]), plan["m"], plan["q"]), (l, s, st, plan)
        assert err <= SPLIT_TOL
        return st

    def state_matches():
        for l in range(L):
            for e in range(E):
                want = ref.resident(l, e)
                assert ecf.ecf_cache_slot_of(cs.cache, l, e) == (-1 if want is None else want), (l, e)

    try:
        step(0, 0)
        step(2, 1)
        assert ecf.prefetch_layer(cs.cache, 1, blob, cstream.cuda_stream) == (lambda r: (len(r["copied"]), r["missing"]))(
            ref.prefetch(1))
        assert ecf.prefetch_layer(cs.cache, 1, blob, cstream.cuda_stream) == (0, ref.prefetch(1)["missing"])
        state_matches()
        for s_ in range(2, 6):  # decode steps of layers 0 and 2 while layer 1 is held
            step(0 if s_ % 2 == 0 else 2, s_)
            state_matches()
        assert all(ecf.ecf_cache_slot_of(cs.cache, 1, e) >= 0 for e in range(E) if ref.resident(1, e) is not None)
        st = step(1, 6)  # the held layer's own step: its prefetched experts are hits
        assert st["hits"] > 0
        state_matches()
        # a prefetch left pending across a resize: the copies land, the hold ends
        ecf.prefetch_layer(cs.cache, 2, blob, cstream.cuda_stream)
        ref.prefetch(2)
        ecf.ecf_cache_resize(cs.cache, 6)
        ref.resize(6)
        state_matches()
        step(2, 7)
        step(0, 8)
        state_matches()
        stats = ecf.ecf_cache_get_stats(cs.cache)
        assert {n: stats[n] for n in ref.stats} == ref.stats
    finally:
        cs.close()


def _hot_set(cfg, n_slots):
    """The n_slots most popular (layer, expert) pairs of the Zipf recipe."""
    per, extra = divmod(n_slots, cfg.layers)
    return [sorted(int(e) for e in (syn.popularity_rank(cfg, l) <= per + (1 if l < extra else 0)).nonzero().flatten())
            for l in range(cfg.layers)]


@pytest.mark.parametrize("policy,drift", [("static_hot", 0), ("all_pcie", 0), ("static_hot", 3), ("all_pcie", 3)])
def test_policy_ablation_small(policy, drift):
    """The two comparison policies at equal capacity (37% of the pairs), through
    the C ABI: a static hot subset (the most popular pairs bound once with
    expert_cache_lookup / expert_cache_evict and filled, then every miss on the
    host, q = 0) and the shared LRU with every miss copied (q = m).  Each step's
    output matches the oracle and the all-resident layer, and its hit / miss /
    copy counts match a Python reference of the policy (a fixed set for the
    static subset, the reference LRU for all-PCIe).  drift > 0: each layer's
    popularity ranking is redrawn every `drift` steps, while the static subset
    stays the one bound from the first ranking."""
    E, L, T, k = 16, 3, 4, 4
    cfg = syn.gen.Config(106, "pol", (T,), 512, E, 256, k, "bf16", "bf16", "zipf", layers=L, drift_steps=drift)
    d = cfg.hidden
    n_slots = int(0.37 * L * E)
    cs = CachedSetup(cfg, L, n_slots=n_slots)
    lay = Layer(cs.shape, T)
    cstream = torch.cuda.Stream()
    try:
        if policy == "static_hot":
            hot = _hot_set(cfg, n_slots)
            assert sum(len(h) for h in hot) == n_slots
            for l, h in enumerate(hot):
                assert ecf.expert_cache_lookup(cs.cache, l, h) == [-1] * len(h)
                slots, victims = ecf.expert_cache_evict(cs.cache, l, h)
                assert victims == [-1] * len(h)
                for e, sl in zip(h, slots):
                    cs.slots[sl].copy_(cs.dev_blobs[cs.blob_of(l, e)])
            torch.cuda.synchronize()
            q_mode = ecf.ECF_Q_ALL_HOST
        else:
            ref_lru = oracle.LRURef(n_slots, E)
            q_mode = ecf.ECF_Q_ALL_GPU
        for step in range(12):
            l = step % L
            x = syn.activations(cfg, T, layer=l, batch=step, device="cuda")
            lg = syn.router_logits(cfg, T, layer=l, step=step, device="cuda")
            got, st = _run(lay, lay.args(layer=l, router_logits=lg, cache=cs.cache, q_mode=q_mode,
                                         copy_stream=cstream), x, T, d)
            ref, _ = _run(lay, lay.args(layer=l, router_logits=lg, expert_ptrs=cs.resident_ptrs[l]), x, T, d)
            orc = oracle.moe_layer(x.cpu(), _layer_experts(cs, cfg, l), k, lg=lg.cpu())
            rows = _rows_of(lg, k)
            if policy == "static_hot":
                hits = len(set(rows) & set(hot[l]))
                want = (hits, len(rows) - hits, 0, len(rows) - hits)
            else:
                plan = ref_lru.step(l, rows, lambda m: m)
                want = (len(plan["hits"]), plan["m"], plan["q"], len(plan["host"]))
            assert (st["hits"], st["misses"], st["q"], st["host"]) == want, (step, st, want)
            e_res = np.max(np.abs(got - ref)) / np.sqrt(np.mean(ref ** 2))
            e_orc = np.max(np.abs(got - orc["out"])) / np.sqrt(np.mean(orc["out"] ** 2))
            say(f"{policy} step {step}: hits={st['hits']} m={st['misses']} q={st['q']} host={st['host']} "
                f"err/RMS vs resident {e_res:.2e}, vs oracle {e_orc:.2e}")
            assert e_res <= SPLIT_TOL and e_orc <= 2e-2
        if policy == "static_hot":  # the subset never changed
            for l, h in enumerate(hot):
                assert all(ecf.ecf_cache_slot_of(cs.cache, l, e) >= 0 for e in h)
            assert ecf.ecf_cache_get_stats(cs.cache)["evictions"] == 0
    finally:
        cs.close()


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
