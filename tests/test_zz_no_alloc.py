"""moe_layer_forward_noalloc (workspace in the library's own device array)
against moe_layer_forward (caller's workspace) through the C ABI: two calls in
a row on the same GPU, the second with fewer tokens, must give the same
routing, counts, permutation and outputs bit for bit (the same kernels run in
the same order), and the first call's oracle parity is checked as well."""
import ctypes

import numpy as np
import pytest
import torch

import ecf_synth as syn
import expert_cache_ffn_amd as ecf
from expert_cache_ffn_amd.layer import Layer
from gpu_util import Case, compare, say

pytestmark = pytest.mark.gpu


def _outs(T, k, E, d):
    return dict(out=torch.full((T, d), float("nan"), dtype=torch.float32, device="cuda"),
                idx=torch.full((T * k,), -7, dtype=torch.int32, device="cuda"),
                gate=torch.zeros(T * k, dtype=torch.float32, device="cuda"),
                counts=torch.full((E,), -7, dtype=torch.int32, device="cuda"),
                perm=torch.full((T * k,), -7, dtype=torch.int32, device="cuda"))


def _call(fn, case, lay, T, path):
    cfg = case.cfg
    o = _outs(T, cfg.top_k, cfg.experts, cfg.hidden)
    x = case.x[:T].to("cuda").contiguous()
    wr = case.router_w.to("cuda").contiguous()
    a = lay.args(router_w=wr, expert_ptrs=case.pool.ptrs, path=path, topk_idx=o["idx"], topk_gate=o["gate"],
                 counts=o["counts"], perm=o["perm"])
    st = fn(a, x.data_ptr(), T, o["out"].data_ptr())
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in o.items()}, st


@pytest.mark.parametrize("path,T1,T2", [(ecf.ECF_PATH_DECODE, 48, 5), (ecf.ECF_PATH_PREFILL, 300, 97)])
def test_noalloc_matches_workspace_entry(path, T1, T2):
    cfg = syn.gen.Config(170 + path, "noalloc", (T1,), 1024, 16, 256, 4, "bf16", "bf16", "router")
    say(f"case: noalloc vs workspace entry, path {path}, T {T1} then {T2}")
    case = Case(cfg, T1)
    assert ecf.ecf_workspace_bytes(case.shape, T1) <= ecf.ecf_noalloc_scratch_bytes()
    lay = Layer(case.shape, T1)
    for T in (T1, T2):
        ref, st_ref = _call(ecf.moe_layer_forward, case, lay, T, path)
        got, st = _call(ecf.moe_layer_forward_noalloc, case, lay, T, path)
        assert st["path"] == st_ref["path"] == path
        for key in ("idx", "counts", "perm"):
            assert np.array_equal(got[key], ref[key]), f"T={T}: {key} differs"
        assert np.array_equal(got["gate"], ref["gate"]), f"T={T}: gates differ"
        assert np.array_equal(got["out"], ref["out"]), f"T={T}: outputs differ"
        say(f"T={T}: noalloc output equals the workspace entry's bit for bit")
    # the noalloc call's last batch also meets the oracle bar
    res = dict(out=got["out"], idx=got["idx"].reshape(T2, -1), gate=got["gate"].reshape(T2, -1),
               counts=got["counts"], perm=got["perm"])
    small = Case(cfg, T2)
    small.x = case.x[:T2]  # the rows both entry points ran
    compare(res, small.oracle(), 2e-2, f"noalloc T={T2}")


def test_noalloc_refuses_oversize_and_cache_mode():
    cfg = syn.gen.Config(175, "noalloc", (8,), 4096, 256, 1024, 6, "bf16", "bf16", "router")
    shape = ecf.make_shape(cfg.hidden, cfg.inter, cfg.experts, cfg.top_k)
    cap = ecf.ecf_noalloc_scratch_bytes()
    T_big = next(T for T in range(64, 4096, 8) if ecf.ecf_workspace_bytes(shape, T) > cap)
    a = ecf.LayerArgs()
    a.shape = shape
    a.d_router_logits = 256  # never read: the size check comes first
    a.d_expert_ptrs = 256
    with pytest.raises(ecf.EcfError) as ei:
        ecf.moe_layer_forward_noalloc(a, 256, T_big, 256)
    assert ei.value.code == ecf.ECF_ENOSPC
    a.d_expert_ptrs = None
    a.cache = ctypes.c_void_p(1).value  # any non-NULL handle is refused before use
    with pytest.raises(ecf.EcfError) as ei:
        ecf.moe_layer_forward_noalloc(a, 256, 4, 256)
    assert ei.value.code == ecf.ECF_EUNSUPPORTED
    say(f"noalloc: {T_big} decode-shape tokens exceed the {cap}-byte scratch; cache mode refused")


def test_noalloc_one_token_mxfp4_and_graph_capture():
    """The allocation-free call on one MXFP4 token (the fused down + combine
    kernel) equals moe_layer_forward bit for bit, and captured in a HIP graph it
    gives the eager result on every replay, with eager work in between."""
    cfg = syn.gen.Config(176, "noalloc", (1,), 1024, 16, 256, 6, "mxfp4", "bf16", "router")
    say("case: noalloc, one MXFP4 token, eager and graph replays")
    case = Case(cfg, 1)
    lay = Layer(case.shape, 1)
    ref, _ = _call(ecf.moe_layer_forward, case, lay, 1, ecf.ECF_PATH_AUTO)
    got, st = _call(ecf.moe_layer_forward_noalloc, case, lay, 1, ecf.ECF_PATH_AUTO)
    assert st["path"] == ecf.ECF_PATH_DECODE
    for key in ("idx", "gate", "counts", "perm", "out"):
        assert np.array_equal(got[key], ref[key]), key
    s = torch.cuda.Stream()
    x = case.x.to("cuda").contiguous()
    wr = case.router_w.to("cuda").contiguous()
    out = torch.zeros((1, cfg.hidden), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        a = lay.args(router_w=wr, expert_ptrs=case.pool.ptrs, stream=s)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            rc = ecf.lib().moe_layer_forward_noalloc(a, x.data_ptr(), 1, out.data_ptr(), None)
        assert rc == 0
    for rep in range(4):
        out.fill_(float("nan"))
        junk = torch.randn(1000, 1000, device="cuda") @ torch.randn(1000, 1000, device="cuda")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), ref["out"]), f"replay {rep} differs"
        del junk
