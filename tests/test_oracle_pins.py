"""Pins of the oracle to facts outside itself (CPU only).

Each test checks the oracle against something it does not compute itself: a
table from the OCP MX specification, a brute-force sort, a library softmax or
matmul, a closed form, an invariant, or a hand-worked trace.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import softmax

import ecf_synth as syn
import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed=0):
    return np.random.default_rng(seed)


def _bf16(a):
    return torch.from_numpy(np.asarray(a, np.float64)).to(torch.float32).to(torch.bfloat16)


# ---- element decoding ----------------------------------------------------------

def test_e2m1_matches_ocp_table():
    rows = [l.split() for l in open(os.path.join(GOLD, "ocp_e2m1.txt")) if l.strip() and not l.startswith("#")]
    assert len(rows) == 16
    for code, val in rows:
        got = oracle.e2m1(int(code))
        assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val)) or float(val) == 0


def test_e8m0_values():
    assert oracle.e8m0(127) == 1.0
    assert oracle.e8m0(128) == 2.0
    assert oracle.e8m0(0) == 2.0 ** -127
    assert oracle.e8m0(254) == 2.0 ** 127
    assert math.isnan(oracle.e8m0(255))


def test_mxfp4_weight_decode_by_hand():
    # one row of 64 elements: block 0 scale 2^-1 (126), block 1 scale 2^3 (130)
    nib = np.zeros(64, np.uint8)
    nib[0], nib[1], nib[2], nib[31] = 0x7, 0x9, 0x3, 0xF     # 6, -0.5, 1.5, -6
    nib[32], nib[33], nib[63] = 0x5, 0xC, 0x1                # 3, -2, 0.5
    packed = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)[None, :]
    scales = np.array([[126, 130]], np.uint8)
    L = oracle.lib()
    get = lambda c: L.orc_weight(oracle.ORC_MXFP4, packed.ctypes.data, scales.ctypes.data, 0, c, 64)
    assert [get(c) for c in (0, 1, 2, 31, 5)] == [3.0, -0.25, 0.75, -3.0, 0.0]
    assert [get(c) for c in (32, 33, 63)] == [24.0, -16.0, 4.0]


def test_mxfp4_generator_roundtrip_bound():
    # data-prep sanity: with X = floor(log2 amax) - 2 the scaled block lies in (-8, 8);
    # rounding errs by at most half a grid step (1 * 2^X below 4, 1 * 2^X in [4, 6])
    # and saturation of [6, 8) at 6 by less than 2 * 2^X
    w = torch.from_numpy(_rng(1).normal(0, 0.02, (8, 128))).to(torch.float32)
    q, s = syn.quantize_mxfp4(w)
    table = np.array([float(l.split()[1]) for l in open(os.path.join(GOLD, "ocp_e2m1.txt"))
                      if l.strip() and not l.startswith("#")])
    qn = q.numpy()
    nib = np.stack([qn & 15, qn >> 4], axis=2).reshape(8, 128)
    scale = 2.0 ** (s.numpy().astype(np.int64) - 127)
    deq = table[nib] * np.repeat(scale, 32, axis=1)
    err = np.abs(deq - w.double().numpy())
    assert np.all(err < np.repeat(scale, 32, axis=1) * 2.0)
    # the block maximum maps into the top binade of E2M1 ([4, 6]) or saturates at 6
    amax_code = np.abs(table[nib]).reshape(8, 4, 32).max(axis=2)
    assert np.all(amax_code >= 4.0)


def test_mxfp4_as_bf16_by_hand_and_exact():
    # the hand row of test_mxfp4_weight_decode_by_hand, re-encoded: bf16 bits of
    # 3, -0.25, 0.75, -3, 0 and 24, -16, 4 (exact binary fractions)
    nib = np.zeros(64, np.uint8)
    nib[0], nib[1], nib[2], nib[31] = 0x7, 0x9, 0x3, 0xF
    nib[32], nib[33], nib[63] = 0x5, 0xC, 0x1
    packed = (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)[None, :]
    sc = np.array([[126, 130]], np.uint8)
    ex = {n: torch.from_numpy(packed.copy()) for n in ("w_gate", "w_up", "w_down")}
    ex.update({n: torch.from_numpy(sc.copy()) for n in ("s_gate", "s_up", "s_down")})
    bits = oracle.mxfp4_as_bf16(ex)["w_gate"][0]
    as_f = lambda b: float(torch.tensor([int(b)], dtype=torch.int32).to(torch.int16).view(torch.bfloat16).float())
    assert [as_f(bits[c]) for c in (0, 1, 2, 31, 5, 32, 33, 63)] == [3.0, -0.25, 0.75, -3.0, 0.0, 24.0, -16.0, 4.0]
    # a scale of 2^126 with element 6 (1.5 * 2^128) does not fit bf16: refused
    big = dict(ex, s_up=torch.full((1, 2), 253, dtype=torch.uint8))
    with pytest.raises(ValueError):
        oracle.mxfp4_as_bf16(big)


def test_mxfp4_layer_equals_its_bf16_reencoding():
    # the layer on MXFP4 experts and on their exact bf16 re-encoding: the same
    # fp64 values in the same order, so the outputs are identical bit for bit
    cfg = syn.gen.Config(93, "t", (9,), 256, 4, 128, 2, "mxfp4", "bf16", "normal_t", temperature=0.5)
    experts = [syn.expert_weights(cfg, 0, e) for e in range(4)]
    re = [oracle.mxfp4_as_bf16(ex) for ex in experts]
    x = syn.activations(cfg, 9)
    lg = syn.router_logits(cfg, 9)
    a = oracle.moe_layer(x, experts, 2, lg=lg, w_dtype="mxfp4")
    b = oracle.moe_layer(x, re, 2, lg=lg, w_dtype="bf16")
    assert np.array_equal(a["out"], b["out"])
    for nm in ("w_gate", "w_down"):
        dense = _mx_dense(experts[1][nm], experts[1]["s" + nm[1:]]).numpy()
        got = torch.from_numpy(re[1][nm].view(np.int16)).view(torch.bfloat16).double().numpy()
        assert np.array_equal(got, dense)


# ---- router ---------------------------------------------------------------------

def test_logits_bf16_against_fp64_matmul():
    x = _bf16(_rng(2).normal(0, 1, (9, 256)))
    wr = _bf16(_rng(3).normal(0, 0.02, (16, 256)))
    ref = (x.double() @ wr.double().T).to(torch.float32).numpy()
    got = oracle.logits(x, wr)
    # both are exact products summed in fp64 and rounded once; sums in another
    # order may land one fp32 ulp apart only next to a rounding midpoint
    ulp = np.spacing(np.abs(ref).astype(np.float32))
    assert np.all(np.abs(got - ref) <= ulp)
    assert np.mean(got == ref) > 0.99


def test_logits_fp32_inputs():
    x = torch.from_numpy(_rng(4).normal(0, 1, (5, 64)).astype(np.float32))
    wr = torch.from_numpy(_rng(5).normal(0, 0.02, (7, 64)).astype(np.float32))
    ref = (x.double() @ wr.double().T).to(torch.float32).numpy()
    got = oracle.logits(x, wr)
    assert np.all(np.abs(got - ref) <= np.spacing(np.abs(ref)))


@pytest.mark.parametrize("E,k", [(16, 2), (8, 8), (256, 6), (5, 1), (64, 8)])
def test_topk_against_full_sort(E, k):
    rng = _rng(E * 10 + k)
    T = 40
    # coarse values force many ties
    lg = np.round(rng.normal(0, 1, (T, E)) * 4) / 4
    lg = lg.astype(np.float32)
    idx, _ = oracle.route(lg, k)
    for t in range(T):
        order = np.lexsort((np.arange(E), -lg[t].astype(np.float64)))  # value desc, id asc
        assert list(idx[t]) == list(order[:k])


def test_special_logits_hand_derived():
    """NaN ranks as -inf in the order and the softmax, -0 ties with +0 (lower id
    first), -inf is selectable after every finite logit; values derived by hand."""
    nan, inf = np.float32(np.nan), np.float32(np.inf)
    lg = np.array([[nan, 1.0, 0.5, nan, -inf, -0.0, 0.0, -2.0]], np.float32)
    idx, g = oracle.route(lg, 8, renorm=True)
    # 1, 0.5, -0 (id 5) and +0 (id 6) tie -> 5 first, -2, then -inf, NaN, NaN as -inf in id order
    assert list(idx[0]) == [1, 2, 5, 6, 7, 0, 3, 4]
    z = 1.0 + np.exp(-0.5) + 2 * np.exp(-1.0) + np.exp(-3.0)
    want = np.array([1.0, np.exp(-0.5), np.exp(-1.0), np.exp(-1.0), np.exp(-3.0), 0, 0, 0]) / z
    assert np.allclose(g[0], want, rtol=1e-15, atol=0)
    # renorm=0: the NaN entries add nothing to the full softmax either
    idx2, g2 = oracle.route(lg, 2, renorm=False)
    assert list(idx2[0]) == [1, 2]
    assert np.allclose(g2[0], [1.0 / z, np.exp(-0.5) / z], rtol=1e-15, atol=0)


def test_gates_against_library_softmax():
    rng = _rng(7)
    lg = rng.normal(0, 2, (30, 32)).astype(np.float32)
    for k in (1, 3, 8):
        idx, g = oracle.route(lg, k, renorm=True)
        for t in range(30):
            ref = softmax(lg[t, idx[t]].astype(np.float64))
            assert np.allclose(g[t], ref, rtol=1e-14, atol=0)
        assert np.allclose(g.sum(1), 1.0, rtol=1e-14)
        if k == 1:
            assert np.all(g == 1.0)
        idx0, g0 = oracle.route(lg, k, renorm=False)
        assert np.array_equal(idx0, idx)
        full = softmax(lg.astype(np.float64), axis=1)
        assert np.allclose(g0, np.take_along_axis(full, idx0, 1), rtol=1e-13, atol=0)


def test_gates_monotone_and_positive():
    lg = _rng(8).normal(0, 1, (20, 64)).astype(np.float32)
    idx, g = oracle.route(lg, 6)
    assert np.all(g > 0)
    assert np.all(np.diff(g, axis=1) <= 0)


# ---- permutation ------------------------------------------------------------------

@pytest.mark.parametrize("T,k,E", [(64, 2, 16), (1, 6, 256), (37, 8, 32), (0, 4, 8), (100, 1, 1)])
def test_permute_against_stable_argsort(T, k, E):
    idx = _rng(T + k + E).integers(0, E, (T, k)).astype(np.int32)
    counts, offsets, perm, pos = oracle.permute(idx, E)
    flat = idx.ravel()
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    assert np.array_equal(perm, np.argsort(flat, kind="stable"))
    assert np.array_equal(pos[perm], np.arange(T * k))
    assert counts.sum() == T * k


# ---- experts and combine -------------------------------------------------------------

def _dense_swiglu(x64, wg, wu, wd):
    """torch fp64 matmuls of the dense FFN (library routine)."""
    a = x64 @ wg.T
    b = x64 @ wu.T
    h = torch.nn.functional.silu(a) * b
    return h @ wd.T


def _mx_dense(q, s):
    table = np.array([float(l.split()[1]) for l in open(os.path.join(GOLD, "ocp_e2m1.txt"))
                      if l.strip() and not l.startswith("#")])
    qn, sn = q.numpy(), s.numpy().astype(np.int64)
    nib = np.stack([qn & 15, qn >> 4], axis=2).reshape(qn.shape[0], qn.shape[1] * 2)
    return torch.from_numpy(table[nib] * np.repeat(2.0 ** (sn - 127), 32, axis=1))


@pytest.mark.parametrize("w_dtype", ["f32", "bf16", "mxfp4"])
def test_single_expert_reduces_to_dense_ffn(w_dtype):
    cfg = syn.gen.Config(90, "t", (8,), 128, 1, 64, 1, w_dtype, "bf16" if w_dtype != "f32" else "f32", "router")
    ex = syn.expert_weights(cfg, 0, 0)
    x = syn.activations(cfg, 11)
    lg = np.zeros((11, 1), np.float32)
    res = oracle.moe_layer(x, [ex], 1, lg=lg, w_dtype=w_dtype)
    assert np.all(res["idx"] == 0) and np.all(res["gates"] == 1.0)
    if w_dtype == "mxfp4":
        wg, wu, wd = (_mx_dense(ex[n], ex["s" + n[1:]]) for n in ("w_gate", "w_up", "w_down"))
    else:
        wg, wu, wd = (ex[n].double() for n in ("w_gate", "w_up", "w_down"))
    ref = _dense_swiglu(x.double(), wg, wu, wd).numpy()
    assert np.allclose(res["out"], ref, rtol=1e-12, atol=1e-15)


def test_swiglu_closed_form():
    # d=4, I=1: gate row picks 2*x0, up row picks -3*x1, down column is (1, 0.5, 0, -2)
    ex = dict(w_gate=torch.tensor([[2.0, 0, 0, 0]], dtype=torch.float32),
              w_up=torch.tensor([[0, -3.0, 0, 0]], dtype=torch.float32),
              w_down=torch.tensor([[1.0], [0.5], [0.0], [-2.0]], dtype=torch.float32))
    v = np.array([0.7, -1.1, 5.0, 9.0])
    y = oracle.expert_ffn(ex, v, "f32")
    a, b = 2 * 0.7, -3 * -1.1
    h = a / (1 + math.exp(-a)) * b
    assert np.allclose(y, [h, 0.5 * h, 0.0, -2 * h], rtol=1e-15, atol=0)


def test_identical_experts_combine_to_one_ffn():
    # k experts holding the same tensors: the renormalised gates sum to one, so the
    # layer equals the dense FFN -- catches a dropped gate or a wrong combine
    cfg = syn.gen.Config(91, "t", (6,), 64, 4, 32, 3, "bf16", "bf16", "router")
    ex = syn.expert_weights(cfg, 0, 0)
    x = syn.activations(cfg, 6)
    lg = _rng(9).normal(0, 1, (6, 4)).astype(np.float32)
    res = oracle.moe_layer(x, [ex] * 4, 3, lg=lg)
    ref = _dense_swiglu(x.double(), *(ex[n].double() for n in ("w_gate", "w_up", "w_down"))).numpy()
    assert np.allclose(res["out"], ref, rtol=1e-12, atol=1e-15)


def test_combine_weights_by_gate():
    # two experts with w_down differing by a factor 2: out = (g0*c0 + g1*c1) * FFN
    cfg = syn.gen.Config(92, "t", (5,), 64, 2, 32, 2, "bf16", "bf16", "router")
    ex0 = syn.expert_weights(cfg, 0, 0)
    ex1 = dict(ex0, w_down=(ex0["w_down"].float() * 2).to(torch.bfloat16))
    x = syn.activations(cfg, 5)
    lg = _rng(10).normal(0, 1, (5, 2)).astype(np.float32)
    res = oracle.moe_layer(x, [ex0, ex1], 2, lg=lg)
    base = _dense_swiglu(x.double(), *(ex0[n].double() for n in ("w_gate", "w_up", "w_down"))).numpy()
    g = res["gates"]
    scale = np.where(res["idx"] == 1, 2.0, 1.0)
    assert np.allclose(res["out"], base * (g * scale).sum(1, keepdims=True), rtol=1e-12, atol=1e-15)


def test_token_order_invariance():
    cfg = syn.CONFIGS["tiny"]
    experts = [syn.expert_weights(cfg, 0, e) for e in range(cfg.experts)]
    wr = syn.router_weights(cfg)
    x = syn.activations(cfg, 24)
    a = oracle.moe_layer(x, experts, cfg.top_k, wr=wr, w_dtype="f32")
    p = np.random.default_rng(11).permutation(24)
    b = oracle.moe_layer(x[torch.from_numpy(p)], experts, cfg.top_k, wr=wr, w_dtype="f32")
    assert np.array_equal(b["logits"], a["logits"][p])
    assert np.array_equal(b["idx"], a["idx"][p])
    assert np.array_equal(b["gates"], a["gates"][p])
    assert np.array_equal(b["counts"], a["counts"])
    assert np.array_equal(b["out"], a["out"][p])


# ---- q* ---------------------------------------------------------------------------

def test_qstar_golden_hand_derived():
    for line in open(os.path.join(GOLD, "qstar_splits.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        bp, bh, m, q = line.split()
        assert oracle.qstar(int(m), float(bp), float(bh)) == int(q), line


def test_qstar_brackets_closed_form():
    rng = _rng(12)
    for _ in range(3000):
        bh = float(rng.uniform(1, 200))
        bp = float(rng.uniform(0.01, 0.999)) * bh
        m = int(rng.integers(0, 300))
        q = oracle.qstar(m, bp, bh)
        x = oracle.qstar_closed_form(m, bp, bh)
        assert math.floor(x) <= q <= math.ceil(x)


def test_qstar_edges():
    assert oracle.qstar(0, 10, 20) == 0
    assert oracle.qstar(7, 0.0, 20) == 0
    assert oracle.qstar(7, -1.0, 20) == 0
    assert oracle.qstar(7, 20.0, 20.0) == 7
    assert oracle.qstar(7, 30.0, 20.0) == 7
    for bad in [(-1, 1, 2), (3, 1, 0), (3, 1, -2), (3, float("nan"), 2), (3, 1, float("nan"))]:
        with pytest.raises(ValueError):
            oracle.qstar(*bad)


# ---- shared LRU ---------------------------------------------------------------------

def test_lru_hand_trace():
    tr = json.load(open(os.path.join(GOLD, "lru_trace.json")))
    c = oracle.LRURef(tr["n_slots"], tr["n_experts"])
    rules = {"all": lambda m: m, "q04": lambda m: oracle.qstar(m, 0.4, 1.0)}
    for st in tr["steps"]:
        rows = {int(e): n for e, n in st["rows"].items()}
        plan = c.step(st["layer"], rows, rules[st["q"]])
        assert plan["hits"] == {int(e): s for e, s in st["hits"].items()}
        assert plan["copied"] == {int(e): s for e, s in st["copied"].items()}
        assert plan["host"] == st["host"]
        assert plan["victims"] == {int(e): (tuple(v) if v else None) for e, v in st["victims"].items()}
    assert c.stats == tr["stats"]


def test_lru_resize_keeps_low_slots():
    c = oracle.LRURef(4, 8)
    c.step(0, {0: 1, 1: 1, 2: 1, 3: 1}, lambda m: m)
    c.resize(2)
    assert c.resident(0, 0) == 0 and c.resident(0, 1) == 1
    assert c.resident(0, 2) is None and c.resident(0, 3) is None
    c.resize(3)
    plan = c.step(1, {5: 1}, lambda m: m)
    assert plan["copied"] == {5: 2}


def test_lru_prefetch_hand_trace():
    # whole-layer prefetches held until their layer's step, a prefetch that does
    # not fit (its missing expert reserved and filled by the step on demand), and
    # the prefill path copying every miss: a hand-worked trace
    tr = json.load(open(os.path.join(GOLD, "lru_prefetch_trace.json")))
    c = oracle.LRURef(tr["n_slots"], tr["n_experts"])
    for op in tr["ops"]:
        if op["op"] == "prefetch":
            assert c.prefetch(op["layer"]) == op["expect"]
        else:
            rows = {int(e): n for e, n in op["rows"].items()}
            plan = c.step(op["layer"], rows, lambda m: m, prefill=op["prefill"])
            assert sorted(plan["hits"]) == op["expect"]["hits"]
            assert plan["copied"] == {int(e): s for e, s in op["expect"]["copied"].items()}
    assert [[l, e, s] for (l, e), s in c.od.items()] == tr["final_lru_order"]
    assert c.stats == tr["final_stats"]
    assert c.held == {} and c.reserve == 0


def test_lru_prefetch_never_starves_a_held_layer():
    # capacity of one and a half layers: each prefetch places what the reserve
    # allows, and every prefill step, in prefetch order, can copy what is missing
    E = 8
    c = oracle.LRURef(12, E)
    c.prefetch(0)
    for l in range(6):
        nxt = c.prefetch(l + 1)
        assert nxt["missing"] > 0
        plan = c.step(l, {e: 1 for e in range(E)}, lambda m: m, prefill=True)
        assert len(plan["hits"]) + len(plan["copied"]) == E
    with pytest.raises(ValueError):  # one slot short of a whole layer
        small = oracle.LRURef(E - 1, E)
        small.step(0, {e: 1 for e in range(E)}, lambda m: m, prefill=True)
