"""CPU tests of libecf's host side: exports, layouts, q*, the shared LRU and
the host expert FFN, each against the oracle (no GPU calls)."""
import ctypes
import json
import os
import re

import numpy as np
import pytest
import torch

import ecf_synth as syn
import expert_cache_ffn_amd as ecf
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLD = os.path.join(ROOT, "tests", "golden")


def test_library_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "ecf.h")).read()
    hdr = re.sub(r"/\*.*?\*/", "", hdr, flags=re.S)
    hdr = "\n".join(l for l in hdr.splitlines() if not l.lstrip().startswith("#"))
    declared = set(re.findall(r"\b([A-Za-z_][A-Za-z0-9_]*)\s*\([^;{]*\)\s*;", hdr))
    declared = {n for n in declared if n not in ("if", "while", "sizeof")}
    assert declared == set(ecf.EXPORTS), declared ^ set(ecf.EXPORTS)
    L = ecf.lib()
    for name in declared:
        assert hasattr(L, name), name


def test_expert_blob_sizes():
    bf = ecf.make_shape(4096, 1024, 256, 6, "bf16", "bf16")
    assert ecf.ecf_expert_bytes(bf) == 6 * 4096 * 1024  # 25,165,824
    mx = ecf.make_shape(4096, 2048, 256, 8, "mxfp4", "bf16")
    assert ecf.ecf_expert_bytes(mx) == 13_369_344       # 1.5 d I + 3 d I / 32
    offs = ecf.ecf_expert_layout(mx)
    assert offs[:3] == [0, 4096 * 2048 // 2, 2 * 4096 * 2048 // 2]
    assert all(o % 256 == 0 for o in offs)
    f32 = ecf.make_shape(256, 128, 16, 2, "f32", "f32")
    assert ecf.ecf_expert_bytes(f32) == 12 * 256 * 128


def test_invalid_shapes_rejected():
    for bad in [ecf.make_shape(100, 64, 4, 2), ecf.make_shape(256, 60, 4, 2), ecf.make_shape(256, 64, 4, 5),
                ecf.make_shape(256, 64, 2000, 2), ecf.make_shape(256, 64, 4, 2, "bf16", "f32")]:
        with pytest.raises(ecf.EcfError):
            ecf.ecf_expert_bytes(bad)
    assert ecf.ecf_workspace_bytes(ecf.make_shape(256, 64, 4, 2), 10) > 0


def test_token_count_bound():
    """Row indices are 32-bit: n_tokens * top_k is capped at 2^26, in the
    workspace query and in the forward call (rejected before any device work)."""
    sh = ecf.make_shape(256, 64, 8, 4)
    assert ecf.ecf_workspace_bytes(sh, (1 << 26) // 4) > 0
    with pytest.raises(ecf.EcfError):
        ecf.ecf_workspace_bytes(sh, (1 << 26) // 4 + 1)
    a = ecf.LayerArgs()
    a.shape = sh
    rc = ecf.lib().moe_layer_forward(ctypes.byref(a), None, (1 << 26) // 4 + 1, None, None)
    assert rc == ecf.ECF_EINVAL and b"n_tokens" in ecf.lib().ecf_last_error()
    # the host half alone: the same cap, checked before any row is read
    with pytest.raises(ecf.EcfError):
        ecf.ecf_host_experts(sh, [], [], 0, (1 << 26) // 4 + 1, 0, 1)


# ---- q* -----------------------------------------------------------------------------

def test_qstar_matches_oracle_golden():
    for line in open(os.path.join(GOLD, "qstar_splits.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        bp, bh, m, q = line.split()
        assert ecf.qstar_split(int(m), float(bp), float(bh)) == int(q), line


def test_qstar_matches_oracle_brute_force():
    rng = np.random.default_rng(5)
    for _ in range(4000):
        bh = float(rng.uniform(0.5, 300))
        bp = float(rng.choice([rng.uniform(0, 1), 0.4, 0.5, 0.25, 0.75])) * bh
        m = int(rng.integers(0, 200))
        assert ecf.qstar_split(m, bp, bh) == oracle.qstar(m, bp, bh), (m, bp, bh)
    for m in range(0, 64):
        assert ecf.qstar_split(m, 0.4, 1.0) == oracle.qstar(m, 0.4, 1.0)


def test_qstar_errors_and_edges():
    assert ecf.qstar_split(0, 1, 2) == 0
    assert ecf.qstar_split(5, 0, 2) == 0
    assert ecf.qstar_split(5, 2, 2) == 5
    for bad in [(-1, 1, 2), (3, 1, 0), (3, float("nan"), 1), (3, 1, float("nan"))]:
        with pytest.raises(ecf.EcfError) as ei:
            ecf.qstar_split(*bad)
        assert ei.value.code == ecf.ECF_EINVAL


# ---- shared LRU ---------------------------------------------------------------------

FAKE_SLOTS = 1 << 40  # slot memory is never touched by the metadata calls


def _run_step(cache, ref, layer, rows, q_of_m):
    """Drive one layer-step through the C calls the way the forward call does."""
    U = sorted(rows)
    slots = ecf.expert_cache_lookup(cache, layer, U)
    miss = [e for e, s in zip(U, slots) if s < 0]
    q = min(q_of_m(len(miss)), ecf.ecf_cache_available(cache))
    order = sorted(miss, key=lambda e: (-rows[e], e))
    cs, vs = ecf.expert_cache_evict(cache, layer, order[:q]) if q else ([], [])
    plan = ref.step(layer, rows, q_of_m)
    assert {e: s for e, s in zip(U, slots) if s >= 0} == plan["hits"]
    assert dict(zip(order[:q], cs)) == plan["copied"]
    E = ref.E
    want_v = {e: (None if v is None else v[0] * E + v[1]) for e, v in plan["victims"].items()}
    got_v = {e: (None if v < 0 else v) for e, v in zip(order[:q], vs)}
    assert got_v == want_v
    assert order[q:] == plan["host"]


def test_lru_hand_trace_through_c_api():
    tr = json.load(open(os.path.join(GOLD, "lru_trace.json")))
    E = tr["n_experts"]
    cache = ecf.ecf_cache_create(2, E, tr["n_slots"], tr["n_slots"], 4096, FAKE_SLOTS)
    try:
        ref = oracle.LRURef(tr["n_slots"], E)
        rules = {"all": lambda m: m, "q04": lambda m: ecf.qstar_split(m, 0.4, 1.0)}
        for st in tr["steps"]:
            _run_step(cache, ref, st["layer"], {int(e): n for e, n in st["rows"].items()}, rules[st["q"]])
        s = ecf.ecf_cache_get_stats(cache)
        assert {k: s[k] for k in tr["stats"]} == tr["stats"]
    finally:
        ecf.ecf_cache_destroy(cache)


@pytest.mark.parametrize("n_slots,L,E,k,T", [(37, 5, 32, 4, 4), (8, 3, 16, 2, 3), (200, 43, 64, 6, 16)])
def test_lru_random_trace_against_reference(n_slots, L, E, k, T):
    rng = np.random.default_rng(n_slots + L)
    cache = ecf.ecf_cache_create(L, E, n_slots, n_slots, 4096, FAKE_SLOTS)
    ref = oracle.LRURef(n_slots, E)
    zipf = 1.0 / np.arange(1, E + 1) ** 1.1
    zipf /= zipf.sum()
    rules = [lambda m: m, lambda m: 0, lambda m: ecf.qstar_split(m, 0.4, 1.0),
             lambda m: ecf.qstar_split(m, 0.68, 1.0)]
    try:
        for step in range(300):
            layer = step % L
            rows = {}
            for _ in range(T):
                for e in rng.choice(E, size=k, replace=False, p=zipf):
                    rows[int(e)] = rows.get(int(e), 0) + 1
            _run_step(cache, ref, layer, rows, rules[step % len(rules)])
        assert {k2: v for k2, v in ecf.ecf_cache_get_stats(cache).items() if k2 != "dropped"} == ref.stats
        for l in range(L):
            for e in range(E):
                s = ref.resident(l, e)
                assert ecf.ecf_cache_slot_of(cache, l, e) == (-1 if s is None else s)
    finally:
        ecf.ecf_cache_destroy(cache)


def test_cache_error_paths():
    cache = ecf.ecf_cache_create(2, 8, 2, 4, 4096, FAKE_SLOTS)
    try:
        with pytest.raises(ecf.EcfError) as ei:
            ecf.expert_cache_evict(cache, 0, [1])      # no layer-step open
        assert ei.value.code == ecf.ECF_ESTATE
        ecf.expert_cache_lookup(cache, 0, [1, 2, 3])
        with pytest.raises(ecf.EcfError) as ei:
            ecf.expert_cache_evict(cache, 1, [1])      # other layer
        assert ei.value.code == ecf.ECF_ESTATE
        with pytest.raises(ecf.EcfError) as ei:
            ecf.expert_cache_evict(cache, 0, [1, 2, 3])  # 3 wanted, 2 slots
        assert ei.value.code == ecf.ECF_ENOSPC
        assert ecf.ecf_cache_get_stats(cache)["inserts"] == 0  # no change on failure
        assert ecf.expert_cache_evict(cache, 0, [1, 2])[0] == [0, 1]
        with pytest.raises(ecf.EcfError) as ei:
            ecf.expert_cache_evict(cache, 0, [1])      # already resident
        assert ei.value.code == ecf.ECF_EINVAL
        assert ecf.ecf_cache_available(cache) == 0     # both slots pinned by this step
        ecf.expert_cache_lookup(cache, 0, [4])         # new step: nothing pinned
        assert ecf.ecf_cache_available(cache) == 2
        with pytest.raises(ecf.EcfError):
            ecf.ecf_cache_resize(cache, 5)             # above max_slots
        with pytest.raises(ecf.EcfError):
            ecf.expert_cache_lookup(cache, 2, [0])     # layer out of range
    finally:
        ecf.ecf_cache_destroy(cache)


def test_cache_resize_matches_reference():
    cache = ecf.ecf_cache_create(3, 16, 6, 10, 4096, FAKE_SLOTS)
    ref = oracle.LRURef(6, 16)
    try:
        _run_step(cache, ref, 0, {0: 1, 1: 1, 2: 1, 3: 1, 4: 1, 5: 1}, lambda m: m)
        ecf.ecf_cache_resize(cache, 3)
        ref.resize(3)
        assert ecf.ecf_cache_get_stats(cache)["dropped"] == 3
        for e in range(6):
            s = ref.resident(0, e)
            assert ecf.ecf_cache_slot_of(cache, 0, e) == (-1 if s is None else s)
        ecf.ecf_cache_resize(cache, 10)
        ref.resize(10)
        _run_step(cache, ref, 1, {e: 1 for e in range(8)}, lambda m: m)
        _run_step(cache, ref, 0, {e: 2 for e in range(4, 12)}, lambda m: m)
    finally:
        ecf.ecf_cache_destroy(cache)


# ---- host expert FFN against the oracle -------------------------------------------------

def _blob(shape, tensors):
    nbytes = ecf.ecf_expert_bytes(shape)
    buf = torch.zeros(nbytes, dtype=torch.uint8)
    from expert_cache_ffn_amd.layer import pack_expert
    pack_expert(shape, tensors, buf)
    return buf


@pytest.mark.parametrize("isa", ["native", "avx2", "scalar"])
@pytest.mark.parametrize("w_dtype", ["bf16", "f32", "mxfp4"])
def test_host_experts_against_oracle(w_dtype, isa, monkeypatch):
    """Every host instruction-set path (the widest the CPU has, AVX2, scalar) against the oracle."""
    if isa != "native":
        monkeypatch.setenv("ECF_HOST_ISA", isa)
    a_dtype = "f32" if w_dtype == "f32" else "bf16"
    cfg = syn.gen.Config(93, "t", (6,), 512, 4, 192, 2, w_dtype, a_dtype, "router")
    shape = ecf.make_shape(cfg.hidden, cfg.inter, cfg.experts, cfg.top_k, w_dtype, a_dtype)
    experts = [syn.expert_weights(cfg, 0, e) for e in range(cfg.experts)]
    blobs = [_blob(shape, ex) for ex in experts]
    T, k = 6, cfg.top_k
    x = syn.activations(cfg, T)
    lg = syn.gen.normal(syn.key_of(93, 0, 9), T * cfg.experts).view(T, cfg.experts).float()
    idx, _ = oracle.route(lg, k)
    rows = [[f for f in range(T * k) if idx.reshape(-1)[f] == e] for e in range(cfg.experts)]
    y = torch.full((T * k, cfg.hidden), float("nan"), dtype=torch.float32)
    xc = x.contiguous()
    ecf.ecf_host_experts(shape, [b.data_ptr() for b in blobs], rows, xc.data_ptr(), T, y.data_ptr(), 3)
    ref = np.zeros((T * k, cfg.hidden))
    x64 = xc.double().numpy()
    for e in range(cfg.experts):
        for f in rows[e]:
            ref[f] = oracle.expert_ffn(experts[e], x64[f // k], w_dtype)
    rms = np.sqrt(np.mean(ref ** 2))
    assert np.max(np.abs(y.numpy() - ref)) <= 1e-5 * rms


def test_bandwidth_profile_argument_checks():
    """Every rejection happens before any HIP call (fake pointers are never used)."""
    bf = ecf.make_shape(1024, 512, 8, 2, "bf16", "bf16")
    S = ecf.ecf_expert_bytes(bf)
    fake = [4096, 8192]

    def code(**kw):
        a = dict(shape=bf, blob_ptrs=fake, d_buf=4096, d_buf_bytes=4 * S, seconds=0.5)
        a.update(kw)
        with pytest.raises(ecf.EcfError) as ei:
            ecf.ecf_bandwidth_profile(**a)
        return ei.value.code

    assert code(blob_ptrs=[]) == ecf.ECF_EINVAL
    assert code(blob_ptrs=[4096, 0]) == ecf.ECF_EINVAL
    assert code(d_buf=0) == ecf.ECF_EINVAL
    assert code(seconds=0.0) == ecf.ECF_EINVAL
    assert code(host_threads=-1) == ecf.ECF_EINVAL
    assert code(d_buf_bytes=S - 1) == ecf.ECF_ENOSPC
    assert code(shape=ecf.make_shape(1000, 512, 8, 2, "bf16", "bf16")) == ecf.ECF_EINVAL


@pytest.mark.parametrize("isa", ["native", "avx2", "scalar"])
def test_host_experts_nan_scale_block(isa, monkeypatch):
    """An E8M0 byte of 0xFF is NaN (OCP MX v1.0): every row routed to that expert
    comes out NaN on the host path and in the oracle; the other rows stay exact."""
    if isa != "native":
        monkeypatch.setenv("ECF_HOST_ISA", isa)
    cfg = syn.gen.Config(94, "t", (5,), 256, 4, 128, 2, "mxfp4", "bf16", "router")
    shape = ecf.make_shape(cfg.hidden, cfg.inter, cfg.experts, cfg.top_k, "mxfp4", "bf16")
    experts = [syn.expert_weights(cfg, 0, e) for e in range(cfg.experts)]
    experts[2]["s_gate"][5, 3] = 255  # one scale group of gate row 5
    blobs = [_blob(shape, ex) for ex in experts]
    T, k = 5, cfg.top_k
    x = syn.activations(cfg, T).contiguous()
    idx, _ = oracle.route(syn.gen.normal(syn.key_of(94, 0, 9), T * 4).view(T, 4).float(), k)
    rows = [[f for f in range(T * k) if idx.reshape(-1)[f] == e] for e in range(4)]
    assert rows[2], "the test needs rows routed to expert 2"
    y = torch.full((T * k, cfg.hidden), 7.0, dtype=torch.float32)
    ecf.ecf_host_experts(shape, [b.data_ptr() for b in blobs], rows, x.data_ptr(), T, y.data_ptr(), 2)
    x64 = x.double().numpy()
    for e in range(4):
        for f in rows[e]:
            ref = oracle.expert_ffn(experts[e], x64[f // k], "mxfp4")
            got = y[f].numpy()
            assert np.array_equal(np.isnan(got), np.isnan(ref)), (e, f)
            if e == 2:
                assert np.isnan(ref).all()
            else:
                assert np.max(np.abs(got - ref)) <= 1e-5 * np.sqrt(np.mean(ref ** 2))


def test_stream_read_argument_checks():
    """Rejected before any HIP call: unaligned buffer, size not a multiple of 16, NULL sink."""
    for buf, n, sink in ((4096 + 4, 64, 8192), (4096, 60, 8192), (4096, 64, 0), (0, 64, 8192)):
        with pytest.raises(ecf.EcfError) as ei:
            ecf.ecf_stream_read(buf, n, sink)
        assert ei.value.code == ecf.ECF_EINVAL



def test_mfma_rate_argument_checks():
    """The MFMA-rate yardstick rejects bad arguments before touching a GPU."""
    for iters, bpc, sink in ((0, 1, 64), (-5, 1, 64), (10, 0, 64), (10, 9, 64), (10, 1, 0)):
        with pytest.raises(ecf.EcfError) as e:
            ecf.ecf_mfma_rate(iters, bpc, sink)
        assert e.value.code == ecf.ECF_EINVAL

def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus above 1 exits with status 2 and says so,
    before anything touches a GPU."""
    import subprocess
    import sys
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stdout


def test_drifting_zipf_phases():
    """The drifting trace's popularity: phase 0 is the stationary ranking, a
    phase keeps one ranking for drift_steps steps, and the next phase draws
    another one (a permutation of the same ranks)."""
    import dataclasses
    base = syn.CONFIGS["cached"]
    cfg = dataclasses.replace(base, drift_steps=4)
    assert [syn.phase_of(cfg, s) for s in (0, 3, 4, 7, 8)] == [0, 0, 1, 1, 2]
    assert [syn.phase_of(base, s) for s in (0, 5, 500)] == [0, 0, 0]
    r0 = syn.popularity_rank(base, 3)
    assert torch.equal(syn.popularity_rank(cfg, 3, phase=0), r0)
    r1 = syn.popularity_rank(cfg, 3, phase=1)
    assert not torch.equal(r1, r0)
    assert torch.equal(torch.sort(r1).values, torch.arange(1, cfg.experts + 1, dtype=torch.float64))
    assert torch.equal(syn.router_logits(cfg, 2, layer=3, step=2), syn.router_logits(base, 2, layer=3, step=2))
    # step 5 lies in phase 1: its logits add the same Gumbel draws to the phase-1 law
    g = syn.router_logits(base, 2, layer=3, step=5) - syn.router_logits(cfg, 2, layer=3, step=5)
    assert not torch.allclose(g, torch.zeros_like(g))


def test_lru_on_drifting_trace_against_reference():
    """The C-ABI LRU on the drifting Zipf trace (rankings redrawn every 8 steps)
    makes the reference LRU's decisions; on such a trace the LRU ends with fewer
    misses than a subset fixed from the first phase's law at equal capacity."""
    import dataclasses
    cfg = dataclasses.replace(syn.CONFIGS["cached"], experts=64, layers=4, drift_steps=8)
    L, E, k, T = cfg.layers, cfg.experts, cfg.top_k, 16
    n_slots = int(0.37 * L * E)
    per, extra = divmod(n_slots, L)
    hot = [set(int(e) for e in (syn.popularity_rank(cfg, l) <= per + (1 if l < extra else 0)).nonzero().flatten())
           for l in range(L)]
    cache = ecf.ecf_cache_create(L, E, n_slots, n_slots, 4096, FAKE_SLOTS)
    ref = oracle.LRURef(n_slots, E)
    miss_lru = miss_static = 0
    try:
        for step in range(48):
            for layer in range(L):
                idx, _ = oracle.route(syn.router_logits(cfg, T, layer=layer, step=step).numpy(), k)
                rows = {}
                for e in idx.ravel():
                    rows[int(e)] = rows.get(int(e), 0) + 1
                m0 = ref.stats["misses"]
                _run_step(cache, ref, layer, rows, lambda m: ecf.qstar_split(m, 0.4, 1.0))
                if step >= 8:
                    miss_lru += ref.stats["misses"] - m0
                    miss_static += sum(1 for e in rows if e not in hot[layer])
        assert {k2: v for k2, v in ecf.ecf_cache_get_stats(cache).items() if k2 != "dropped"} == ref.stats
        for l in range(L):
            for e in range(E):
                s = ref.resident(l, e)
                assert ecf.ecf_cache_slot_of(cache, l, e) == (-1 if s is None else s)
        print(f"drifting trace: LRU {miss_lru} misses, first-phase static subset {miss_static}")
        assert miss_lru < miss_static, (miss_lru, miss_static)
    finally:
        ecf.ecf_cache_destroy(cache)
