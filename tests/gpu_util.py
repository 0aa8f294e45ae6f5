"""Helpers shared by the GPU parity tests: build a layer's inputs once (seeded,
from ecf_synth), run libecf through the C ABI, run the oracle on the same
bytes, and compare."""
from __future__ import annotations

import sys

import numpy as np
import torch

import ecf_synth as syn
import expert_cache_ffn_amd as ecf
import oracle
from expert_cache_ffn_amd.layer import ExpertPool, Layer


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def shape_of(cfg, renorm=1):
    return ecf.make_shape(cfg.hidden, cfg.inter, cfg.experts, cfg.top_k, cfg.w_dtype, cfg.a_dtype, renorm)


class Case:
    """Experts (device pool + lazily copied host tensors), router input, x."""

    def __init__(self, cfg, T, layer=0, batch=0, gen_device="cpu", renorm=1, logits=None):
        self.cfg, self.T = cfg, T
        self.shape = shape_of(cfg, renorm)
        self.renorm = renorm
        self.gen_device = gen_device
        self.pool = ExpertPool(self.shape, "cuda")
        self.host_experts = {}
        for e in range(cfg.experts):
            ex = syn.expert_weights(cfg, layer, e, device=gen_device)
            self.pool.load(e, {k: v.to("cuda") for k, v in ex.items()})
            if gen_device == "cpu":
                self.host_experts[e] = ex
        self.layer_id = layer
        self.x = syn.activations(cfg, T, layer=layer, batch=batch, device=gen_device)
        self.router_w = None
        if logits is not None:
            self.logits = logits.to(gen_device)
        elif cfg.logits == "router":
            self.router_w = syn.router_weights(cfg, layer, device=gen_device)
            self.logits = None
        else:
            self.logits = syn.router_logits(cfg, T, layer=layer, step=batch, device=gen_device)

    def host_expert(self, e):
        if e not in self.host_experts:
            ex = {k: v.detach().cpu() for k, v in syn.expert_weights(self.cfg, self.layer_id, e,
                                                                       device="cuda").items()}
            self.host_experts[e] = ex
        return self.host_experts[e]

    def run(self, path=ecf.ECF_PATH_AUTO, residual=None, want_logits=True, layer=None):
        T, k, E = self.T, self.cfg.top_k, self.cfg.experts
        L = Layer(self.shape, max(T, 1))
        dev = lambda t: None if t is None else t.to("cuda").contiguous()
        x = dev(self.x)
        out = torch.full((T, self.cfg.hidden), float("nan"), dtype=torch.float32, device="cuda")
        idx = torch.full((max(T * k, 1),), -7, dtype=torch.int32, device="cuda")
        gate = torch.zeros(max(T * k, 1), dtype=torch.float32, device="cuda")
        counts = torch.zeros(E, dtype=torch.int32, device="cuda")
        perm = torch.full((max(T * k, 1),), -7, dtype=torch.int32, device="cuda")
        lg_out = torch.zeros((max(T, 1), E), dtype=torch.float32, device="cuda") if self.router_w is not None else None
        rw, lg = dev(self.router_w), dev(self.logits)  # held: LayerArgs keeps raw addresses only
        a = L.args(router_w=rw, router_logits=lg, expert_ptrs=self.pool.ptrs,
                   path=path, residual=residual, topk_idx=idx, topk_gate=gate, counts=counts, perm=perm,
                   logits_out=lg_out)
        st = L.forward(a, x, out)
        torch.cuda.synchronize()
        res = dict(out=out.cpu().numpy(), idx=idx.cpu().numpy()[:T * k].reshape(T, k),
                   gate=gate.cpu().numpy()[:T * k].reshape(T, k), counts=counts.cpu().numpy(),
                   perm=perm.cpu().numpy()[:T * k], stats=st)
        if lg_out is not None:
            res["logits"] = lg_out.cpu().numpy()[:T]
        return res

    def oracle(self, tokens=None):
        """Oracle routing for every token and outputs for `tokens` (default all)."""
        x = self.x.detach().cpu()
        if self.logits is not None:
            lg = self.logits.detach().cpu().numpy()
        else:
            lg = oracle.logits(x, self.router_w.detach().cpu())
        idx, g = oracle.route(lg, self.cfg.top_k, bool(self.renorm))
        counts, offsets, perm, pos = oracle.permute(idx, self.cfg.experts)
        toks = np.arange(self.T) if tokens is None else np.asarray(tokens, dtype=np.int64)
        need = sorted(set(int(e) for e in idx[toks].ravel()))
        experts = [None] * self.cfg.experts
        for e in need:
            experts[e] = self.host_expert(e)
        out = oracle.moe_tokens(x, experts, idx, g, toks, self.cfg.w_dtype) if len(toks) else np.zeros((0, self.cfg.hidden))
        return dict(logits=lg, idx=idx, gates=g, counts=counts, perm=perm, out=out, tokens=toks,
                    renorm=bool(self.renorm), reoracle=self.reoracle)

    def reoracle(self, tokens, idx, gates):
        """Oracle outputs of `tokens` under the given routing (all tokens' idx/gates)."""
        need = sorted(set(int(e) for e in idx[np.asarray(tokens)].ravel()))
        experts = [None] * self.cfg.experts
        for e in need:
            experts[e] = self.host_expert(e)
        return oracle.moe_tokens(self.x.detach().cpu(), experts, idx, gates, tokens, self.cfg.w_dtype)


def max_1ulp_rows(T):
    """How many tokens may have router logits one ulp off the oracle's: fp64 sums
    taken in another order round to the same fp32 except in rare ties, so a few
    per hundred tokens at most; anything more is a router regression."""
    return max(2, T // 100)


def compare(res, ref, tol_rel, label="", reoracle=None):
    """Routing bit-exact, gates close, outputs within tol_rel * RMS(oracle output).

    Router logits must agree with the oracle's within one ulp.  Tokens whose
    logits differ (at most max_1ulp_rows) are routed again by the oracle on the
    GPU's own logits, and the GPU's indices, gates, counts and permutation must
    then equal the oracle's exactly on every token; such a token whose experts
    changed has its oracle output recomputed with `reoracle(tokens, idx, gates)`
    when given, else it is left out of the output check (and counted).  Returns
    the measured max error / RMS."""
    T = res["idx"].shape[0]
    reoracle = reoracle or ref.get("reoracle")
    idx_ref, gate_ref = ref["idx"].copy(), ref["gates"].copy()
    want = ref["out"]
    toks = np.asarray(ref["tokens"])
    keep = np.ones(len(toks), bool)
    if "logits" in res:
        gl, ol = res["logits"], ref["logits"]
        ulp = np.spacing(np.abs(ol).astype(np.float32))
        assert np.all((np.abs(gl - ol) <= ulp) | (np.isnan(gl) & np.isnan(ol))), \
            f"{label}: router logits beyond 1 ulp"
        diff = ~np.all((gl == ol) | (np.isnan(gl) & np.isnan(ol)), axis=1)
        n_diff = int(diff.sum())
        assert n_diff <= max_1ulp_rows(T), f"{label}: {n_diff} tokens with 1-ulp logit differences"
        if n_diff:
            rows = np.nonzero(diff)[0]
            i2, g2 = oracle.route(gl[rows], res["idx"].shape[1], bool(ref.get("renorm", True)))
            moved = rows[np.any(i2 != idx_ref[rows], axis=1)]
            idx_ref[rows], gate_ref[rows] = i2, g2
            say(f"{label}: {n_diff} token(s) with 1-ulp logit differences, routed again on the GPU's "
                f"logits; {len(moved)} changed experts")
            if len(moved):
                at = np.isin(toks, moved)
                if reoracle is not None and at.any():
                    want = want.copy()
                    want[at] = reoracle(toks[at], idx_ref, gate_ref)
                else:
                    keep &= ~at
    assert np.array_equal(res["idx"], idx_ref), f"{label}: top-k indices differ"
    assert np.allclose(res["gate"], gate_ref, rtol=2e-6, atol=1e-7), f"{label}: gates differ"
    counts, _, perm, _ = oracle.permute(idx_ref, len(ref["counts"]))
    assert np.array_equal(res["counts"], counts), f"{label}: counts differ"
    assert np.array_equal(res["perm"], perm), f"{label}: permutation differs"
    got = res["out"][toks][keep]
    want = want[keep]
    if (~keep).any():
        say(f"{label}: {int((~keep).sum())} token(s) left out of the output check (experts changed)")
    rms = float(np.sqrt(np.mean(want ** 2))) if want.size else 1.0
    err = float(np.max(np.abs(got - want))) / rms if want.size else 0.0
    say(f"{label}: max|err|/RMS = {err:.3e} over {len(got)} tokens (tolerance {tol_rel:g}), RMS = {rms:.4g}")
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    assert err <= tol_rel, f"{label}: max|err|/RMS {err:.3e} > {tol_rel}"
    return err


def stratified_tokens(idx, counts, top_k, min_tokens=1024, block=32, seed=0):
    """Tokens whose routed rows cover every expert and every `block`-row block of
    each expert's rows in the expert-sorted order (so every row block of every
    prefill GEMM tile), topped up with random tokens to min_tokens.  Uses the
    oracle's stable counting sort: row f = t*k + j sits at position
    pos[f] - offsets[e] among expert e's rows."""
    T = idx.shape[0]
    _, offsets, _, pos = oracle.permute(idx, len(counts))
    flat = idx.reshape(-1)
    key = flat.astype(np.int64) * 4096 + (pos - offsets[flat]) // block
    rng = np.random.default_rng(seed)
    covered, chosen = set(), []
    for t in rng.permutation(T):
        ks = set(int(v) for v in key[t * top_k:(t + 1) * top_k])
        if not ks <= covered:
            covered |= ks
            chosen.append(int(t))
    need = set(int(v) for v in np.unique(key))
    assert covered == need
    rest = np.setdiff1d(np.arange(T), chosen)
    extra = rng.choice(rest, max(0, min(len(rest), min_tokens - len(chosen))), replace=False)
    toks = np.sort(np.concatenate([np.asarray(chosen, np.int64), extra.astype(np.int64)]))
    return toks, len(need)

