"""Python face of the oracle (TEST INFRASTRUCTURE ONLY).

* The layer itself (router logits, top-k and gates, permutation, expert FFNs,
  combine) is the C definition in moe_oracle.c, called through ctypes.
* The two policy pieces of the method that have their own algorithm are
  written here in plain Python:
    - qstar: the integer optimum of the pages' bandwidth balance, by brute
      force over every q in 0..m;
    - LRURef: one least-recently-used cache over (layer, expert) pairs,
      shared by every layer, as an OrderedDict.

Sources (page title, section):
  techfeed summary of "Meet FreeToken" (MarkTechPost), "Bandwidth-adaptive
  execution (q* policy)": PCIe copies and CPU expert execution draw on the
  same host memory; PCIe uses B_P of the host bandwidth B_H and the CPU
  computes with the remaining B_H - B_P; of the m experts missed in a step,
  about m * B_P / B_H are copied into the GPU cache and the rest run on the
  CPU; partial sums are added at the end.
  Same page, "Semantic-aware caching": during decode one LRU expert cache
  spans all MoE layers and follows the router.
  FreeToken paper explainer (ta-paperlens), "Design: two-tier expert memory":
  the host pool is the source of truth; one cache slot holds every tensor of a
  (layer, expert) pair; the GPU cache affects performance, never results.
"""
from __future__ import annotations

import ctypes
import math
import os
from collections import OrderedDict

import numpy as np

from . import build as _build

ORC_F32, ORC_BF16, ORC_MXFP4 = 0, 1, 2
_DT = {"f32": ORC_F32, "bf16": ORC_BF16, "mxfp4": ORC_MXFP4}

_lib = None


def lib():
    """Load (compiling first if absent or stale) the oracle's C library."""
    global _lib
    if _lib is None:
        path = _build.build(force=False)
        L = ctypes.CDLL(path)
        P, I32, D, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_float
        L.orc_e2m1.argtypes, L.orc_e2m1.restype = [ctypes.c_uint], D
        L.orc_e8m0.argtypes, L.orc_e8m0.restype = [ctypes.c_uint8], D
        L.orc_weight.argtypes = [I32, P, P, ctypes.c_long, ctypes.c_long, ctypes.c_long]
        L.orc_weight.restype = D
        L.orc_logits.argtypes = [I32, P, P, I32, I32, I32, P]
        L.orc_route.argtypes = [P, I32, I32, I32, I32, P, P]
        L.orc_permute.argtypes = [P, I32, I32, I32, P, P, P, P]
        L.orc_expert_ffn.argtypes = [I32, P, P, P, P, P, P, I32, I32, P, P]
        L.orc_moe_tokens.argtypes = [I32, I32, P, I32, I32, I32, P, P, P, P, P, P, P, P, P, I32, P]
        L.orc_mxfp4_to_bf16.argtypes = [P, P, ctypes.c_long, ctypes.c_long, P]
        L.orc_mxfp4_to_bf16.restype = ctypes.c_long
        for f in ("orc_logits", "orc_route", "orc_permute", "orc_expert_ffn", "orc_moe_tokens"):
            getattr(L, f).restype = None
        _ = F
        _lib = L
    return _lib


def _np(a, dtype=None):
    """torch tensor (CPU) or numpy array -> contiguous numpy array (bf16 -> uint16 bits)."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().contiguous()
            if a.dtype == torch.bfloat16:
                a = a.view(torch.int16).numpy().view(np.uint16)
            else:
                a = a.numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(a)
    if dtype is not None:
        a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _adt(a) -> int:
    return ORC_BF16 if a.dtype == np.uint16 else ORC_F32


# ---- exact element decoding (exposed for pins) ---------------------------------

def e2m1(nib: int) -> float:
    return lib().orc_e2m1(nib)


def e8m0(s: int) -> float:
    return lib().orc_e8m0(s)


# ---- the layer -----------------------------------------------------------------

def logits(x, wr) -> np.ndarray:
    """Router logits [T, E] fp32 (fp64 sums of exact products, one rounding)."""
    x, wr = _np(x), _np(wr)
    assert _adt(x) == _adt(wr)
    T, d = x.shape
    E = wr.shape[0]
    out = np.zeros((T, E), np.float32)
    lib().orc_logits(_adt(x), _ptr(x), _ptr(wr), T, d, E, _ptr(out))
    return out


def route(lg, k: int, renorm: bool = True):
    """(idx int32 [T, k], gates fp64 [T, k]) from fp32 logits [T, E]."""
    lg = _np(lg, np.float32)
    T, E = lg.shape
    idx = np.zeros((T, k), np.int32)
    g = np.zeros((T, k), np.float64)
    lib().orc_route(_ptr(lg), T, E, k, int(bool(renorm)), _ptr(idx), _ptr(g))
    return idx, g


def permute(idx, E: int):
    """(counts [E], offsets [E+1], perm [R], pos [R]) of the stable counting sort."""
    idx = _np(idx, np.int32)
    T, k = idx.shape
    R = T * k
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    perm = np.zeros(R, np.int32)
    pos = np.zeros(R, np.int32)
    lib().orc_permute(_ptr(idx), T, k, E, _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(pos))
    return counts, offsets, perm, pos


class _ExpertTable:
    """Keeps numpy copies alive and exposes the C pointer arrays."""

    def __init__(self, experts, w_dtype: str):
        self.arrs = []
        names = ["w_gate", "w_up", "w_down"] + (["s_gate", "s_up", "s_down"] if w_dtype == "mxfp4" else [])
        self.tables = {}
        for nm in names:
            ptrs = (ctypes.c_void_p * len(experts))()
            cache = {}
            for e, ex in enumerate(experts):
                t = ex[nm]
                key = id(t)
                if key not in cache:
                    a = _np(t)
                    self.arrs.append(a)
                    cache[key] = a.ctypes.data
                ptrs[e] = cache[key]
            self.tables[nm] = ptrs

    def get(self, nm):
        return self.tables.get(nm)


def moe_tokens(x, experts, idx, gates, tokens=None, w_dtype: str = "bf16"):
    """out [len(tokens), d] fp64: sum_j gates[t,j] * FFN_{idx[t,j]}(x[t]).

    experts: list (index = expert id) of dicts with w_gate [I,d], w_up [I,d],
    w_down [d,I] (and s_gate, s_up, s_down for MXFP4), as made by ecf_synth.
    Several entries may share tensors (aliased host blobs)."""
    x = _np(x)
    idx = _np(idx, np.int32)
    gates = _np(gates, np.float64)
    T, d = x.shape
    k = idx.shape[1]
    if tokens is None:
        tokens = np.arange(T, dtype=np.int32)
    tokens = _np(tokens, np.int32)
    ex0 = experts[next(i for i, e in enumerate(experts) if e is not None)]
    I = ex0["w_gate"].shape[0]
    # unused experts may be None; give them any valid entry (never read)
    experts = [e if e is not None else ex0 for e in experts]
    tab = _ExpertTable(experts, w_dtype)
    out = np.zeros((len(tokens), d), np.float64)
    sg = tab.get("s_gate")
    lib().orc_moe_tokens(_DT[w_dtype], _adt(x), _ptr(x), d, I, k, tab.get("w_gate"), tab.get("w_up"),
                         tab.get("w_down"), sg, tab.get("s_up"), tab.get("s_down"), _ptr(idx),
                         _ptr(gates), _ptr(tokens), len(tokens), _ptr(out))
    return out


def mxfp4_as_bf16(ex) -> dict:
    """One MXFP4 expert (nibbles + E8M0 scales) as bf16 bit patterns (uint16
    arrays w_gate [I,d], w_up [I,d], w_down [d,I]) holding exactly the values
    the oracle's MXFP4 decoding gives, so moe_tokens(..., "bf16") on them
    computes the MXFP4 layer fp64 for fp64 without decoding every element per
    token.  Raises if a value does not fit bf16 exactly (scale byte above 252)."""
    out = {}
    for nm, sn in (("w_gate", "s_gate"), ("w_up", "s_up"), ("w_down", "s_down")):
        w, sc = _np(ex[nm]), _np(ex[sn])
        rows, cols = w.shape[0], w.shape[1] * 2
        assert sc.shape == (rows, cols // 32)
        o = np.empty((rows, cols), np.uint16)
        bad = lib().orc_mxfp4_to_bf16(_ptr(w), _ptr(sc), rows, cols, _ptr(o))
        if bad:
            raise ValueError(f"{nm}: {bad} MXFP4 values do not fit bf16 exactly")
        out[nm] = o
    return out


def expert_ffn(ex, v, w_dtype: str = "bf16"):
    """One expert applied to one fp64 vector v [d] -> y [d] fp64."""
    v = _np(v, np.float64)
    d = v.shape[0]
    I = ex["w_gate"].shape[0]
    arrs = {nm: _np(t) for nm, t in ex.items()}
    y = np.zeros(d, np.float64)
    sp = [(_ptr(arrs[n]) if n in arrs else None) for n in ("s_gate", "s_up", "s_down")]
    lib().orc_expert_ffn(_DT[w_dtype], _ptr(arrs["w_gate"]), _ptr(arrs["w_up"]), _ptr(arrs["w_down"]),
                         sp[0], sp[1], sp[2], d, I, _ptr(v), _ptr(y))
    return y


def moe_layer(x, experts, k: int, wr=None, lg=None, renorm: bool = True, w_dtype: str = "bf16",
              tokens=None):
    """Whole layer: routing for every token, outputs for `tokens` (default all)."""
    if lg is None:
        lg = logits(x, wr)
    lg = _np(lg, np.float32)
    idx, g = route(lg, k, renorm)
    counts, offsets, perm, pos = permute(idx, lg.shape[1])
    out = moe_tokens(x, experts, idx, g, tokens, w_dtype)
    return dict(logits=lg, idx=idx, gates=g, counts=counts, offsets=offsets, perm=perm, pos=pos, out=out)


# ---- q* (bandwidth-adaptive split) -------------------------------------------------

def qstar_closed_form(m: int, b_p: float, b_h: float) -> float:
    """The pages' real-valued split m * B_P / B_H."""
    return m * b_p / b_h


def qstar(m: int, b_p: float, b_h: float) -> int:
    """Integer optimum of the balance, by brute force.

    Copying q experts over PCIe takes q*S/B_P; the CPU computing the other m-q
    (each reading S bytes of host memory) takes (m-q)*S/(B_H-B_P); both run at
    once, so a step's miss time is the larger of the two.  Return the q in
    0..m minimising it; equal times (relative 1e-12) go to the larger q.
    B_P <= 0: nothing can be copied -> 0.  B_P >= B_H: the CPU has no
    bandwidth left -> m.  m < 0, B_H <= 0 or NaN inputs -> ValueError."""
    if m < 0 or not (b_h > 0) or math.isnan(b_p):
        raise ValueError("invalid q* arguments")
    if m == 0 or b_p <= 0:
        return 0
    if b_p >= b_h:
        return m
    best_q, best_t = None, None
    for q in range(m + 1):
        t = max(q / b_p, (m - q) / (b_h - b_p))
        if best_t is None or t < best_t * (1 - 1e-12) or abs(t - best_t) <= 1e-12 * max(t, best_t):
            best_q, best_t = q, t
    return best_q


# ---- shared LRU over (layer, expert) ------------------------------------------------

class LRURef:
    """Textbook LRU over (layer, expert) keys, one for all layers.

    Per layer-step (the policy readings, where the pages are silent):
      * the step's hits are touched in ascending expert id;
      * the misses to copy are the first q of the misses ordered by
        (routed rows descending, expert id ascending);
      * a copied miss takes the lowest free slot, else the slot of the least
        recently used entry that this layer-step does not use and no pending
        prefetch holds;
      * misses computed on the host are not inserted;
      * q is cut to the slots that can be had (see available());
      * on the prefill path every miss is copied (q = m), and more misses
        than available slots is an error.

    Whole-layer prefetch (FreeToken paper explainer, "Prefill: full-layer
    double buffer and semantic anchors": the next layer streams into the slot
    pool while the current one computes, and what stays resident warms
    decode), with the readings taken for it:
      * in ascending expert id, a resident entry is touched and a missing one
        is inserted (most recent) while slots can be had;
      * the layer's resident entries are then held -- no insertion evicts
        them -- until that layer's next step, which ends the hold first;
      * the experts that did not fit are counted as reserved: a later
        prefetch places at most available() minus the reserve, so the held
        layers' steps can still copy them.
    """

    def __init__(self, n_slots: int, n_experts: int):
        self.n_slots = n_slots
        self.E = n_experts
        self.od: "OrderedDict[tuple, int]" = OrderedDict()
        self.free = list(range(n_slots))
        self.held = {}  # layer -> [set of held keys, experts that did not fit]
        self.reserve = 0
        self.stats = dict(lookups=0, hits=0, misses=0, inserts=0, evictions=0)

    def resident(self, layer: int, expert: int):
        return self.od.get((layer, expert))

    def _held_keys(self):
        return set().union(*(h[0] for h in self.held.values())) if self.held else set()

    def available(self, pinned=frozenset()) -> int:
        """Free slots plus entries neither pinned by the step nor held."""
        held = self._held_keys()
        return len(self.free) + sum(1 for key, s in self.od.items() if s not in pinned and key not in held)

    def _insert(self, key, pinned=frozenset()):
        """Lowest free slot, else the least recently used entry neither pinned nor held."""
        if self.free:
            s = min(self.free)
            self.free.remove(s)
            victim = None
        else:
            held = self._held_keys()
            victim = next(k for k, sl in self.od.items() if sl not in pinned and k not in held)
            s = self.od.pop(victim)
            self.stats["evictions"] += 1
        self.od[key] = s
        self.stats["inserts"] += 1
        return s, victim

    def prefetch(self, layer: int):
        """Whole-layer prefetch; returns {copied: [experts], missing: count}."""
        if layer in self.held:
            return dict(copied=[], missing=self.held[layer][1])
        keys = {(layer, e) for e in range(self.E) if (layer, e) in self.od}
        self.held[layer] = [keys, 0]
        budget = self.available() - self.reserve
        copied, missing = [], 0
        for e in range(self.E):
            key = (layer, e)
            if key in self.od:
                self.od.move_to_end(key)
            elif budget > 0:
                self._insert(key)
                keys.add(key)
                copied.append(e)
                budget -= 1
            else:
                missing += 1
        self.held[layer][1] = missing
        self.reserve += missing
        return dict(copied=copied, missing=missing)

    def step(self, layer: int, rows: dict, q_of_m, prefill: bool = False):
        """rows: expert -> routed row count (> 0).  Returns a plan dict."""
        if layer in self.held:
            self.reserve -= self.held.pop(layer)[1]
        U = sorted(rows)
        pinned = set()
        hits = {}
        misses = []
        for e in U:
            self.stats["lookups"] += 1
            s = self.od.get((layer, e))
            if s is None:
                misses.append(e)
                self.stats["misses"] += 1
            else:
                self.od.move_to_end((layer, e))
                pinned.add(s)
                hits[e] = s
                self.stats["hits"] += 1
        m = len(misses)
        avail = self.available(pinned)
        if prefill:
            q = m
            if q > avail:
                raise ValueError(f"prefill step: {q} misses, {avail} slots available")
        else:
            q = min(q_of_m(m), avail)
        order = sorted(misses, key=lambda e: (-rows[e], e))
        copied, victims = {}, {}
        for e in order[:q]:
            s, victims[e] = self._insert((layer, e), pinned)
            pinned.add(s)
            copied[e] = s
        host = order[q:]
        return dict(hits=hits, copied=copied, host=host, victims=victims, m=m, q=q)

    def resize(self, n_slots: int):
        """Keep the entries in slots below n_slots (slot memory is fixed per id);
        pending prefetch holds end (a resize is a safe point)."""
        self.held.clear()
        self.reserve = 0
        for key, s in list(self.od.items()):
            if s >= n_slots:
                del self.od[key]
        self.free = sorted(set(s for s in self.free if s < n_slots)
                           | set(range(self.n_slots, n_slots)))
        self.n_slots = n_slots
