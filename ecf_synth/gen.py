"""Counter-based synthetic input generator (inputs only, no layer arithmetic).

Recipe
------
* Every tensor has a 64-bit key built from (config id, layer, tensor id,
  expert).  Element n of the tensor draws from splitmix64 at counter n of
  that key, so a tensor (or one expert of one layer) can be regenerated alone.
* splitmix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014): state_n = key + (n + 1) * 0x9E3779B97F4A7C15,
  then the published xor-shift-multiply finaliser.
* uniform: top 53 bits of the output, u = (b + 0.5) * 2^-53, so u lies in
  (0, 1) and log(u) is finite.
* normal: Box-Muller in fp64 from counters 2n and 2n+1, first output only.
* bf16 cast: fp64 -> fp32 (round to nearest even) -> bf16 (round to nearest
  even), done in two explicit steps so CPU and GPU round identically.
* MXFP4 (OCP Microscaling Formats v1.0, E2M1 elements, E8M0 shared scale per
  32 consecutive elements along the reduction dimension): the OCP conversion
  rule, shared exponent X = floor(log2(amax)) - 2, element = RNE(v / 2^X) on
  the E2M1 grid, saturating at +-6.  Element 2i goes to the low nibble of
  byte i.  This is data preparation: both sides read the same bytes.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

# tensor ids used in keys
T_X, T_WR, T_WG, T_WU, T_WD, T_LOGITS, T_PERM = 0, 1, 2, 3, 4, 5, 6

_MASK64 = (1 << 64) - 1
_GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB


def _s64(v: int) -> int:
    """Unsigned 64-bit integer -> the int64 with the same bits."""
    v &= _MASK64
    return v - (1 << 64) if v >= (1 << 63) else v


def _mix_py(z: int) -> int:
    z &= _MASK64
    z = ((z ^ (z >> 30)) * _M1) & _MASK64
    z = ((z ^ (z >> 27)) * _M2) & _MASK64
    return z ^ (z >> 31)


def key_of(config: int, layer: int, tensor: int, expert: int = 0, extra: int = 0) -> int:
    """64-bit key of one tensor; the fields are mixed so nearby ids decorrelate."""
    k = 0x243F6A8885A308D3  # seed 0 of the recipe, offset by a fixed constant
    for f in (config, layer, tensor, expert, extra):
        k = _mix_py(k ^ ((f + 1) * _GAMMA))
    return k


def _lsr(z: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of int64 bits."""
    return (z >> s) & ((1 << (64 - s)) - 1)


def _splitmix(key: int, start: int, n: int, device) -> torch.Tensor:
    ctr = torch.arange(start + 1, start + n + 1, dtype=torch.int64, device=device)
    z = ctr * _s64(_GAMMA) + _s64(key)
    z = (z ^ _lsr(z, 30)) * _s64(_M1)
    z = (z ^ _lsr(z, 27)) * _s64(_M2)
    return z ^ _lsr(z, 31)


def uniform(key: int, n: int, device="cpu", start: int = 0) -> torch.Tensor:
    """n uniforms in (0, 1), fp64, from counters start..start+n-1."""
    bits = _lsr(_splitmix(key, start, n, device), 11)
    return (bits.to(torch.float64) + 0.5) * (2.0 ** -53)


def normal(key: int, n: int, std: float = 1.0, device="cpu", chunk: int = 1 << 24) -> torch.Tensor:
    """n N(0, std^2) samples as fp64 (Box-Muller, counters 2i and 2i+1)."""
    out = torch.empty(n, dtype=torch.float64, device=device)
    for s in range(0, n, chunk):
        m = min(chunk, n - s)
        u = uniform(key, 2 * m, device, start=2 * s).view(m, 2)
        r = torch.sqrt(-2.0 * torch.log(u[:, 0]))
        out[s:s + m] = r * torch.cos((2.0 * math.pi) * u[:, 1]) * std
    return out


def to_bf16(v: torch.Tensor) -> torch.Tensor:
    return v.to(torch.float32).to(torch.bfloat16)


def _normal_tensor(key, shape, std, dtype, device):
    n = 1
    for s in shape:
        n *= s
    v = normal(key, n, std, device).view(*shape)
    if dtype == "f32":
        return v.to(torch.float32)
    if dtype == "bf16":
        return to_bf16(v)
    if dtype == "f64":
        return v
    raise ValueError(dtype)


# --- MXFP4 encoding (OCP MX v1.0) -------------------------------------------

def quantize_mxfp4(w: torch.Tensor):
    """Encode w [N, K] (K % 32 == 0) as (nibbles uint8 [N, K/2], scales uint8 [N, K/32])."""
    N, K = w.shape
    assert K % 32 == 0
    v = w.to(torch.float32).view(N, K // 32, 32)
    amax = v.abs().amax(dim=2)
    _, e = torch.frexp(amax)                      # amax = m * 2^e, m in [0.5, 1)
    X = (e - 1 - 2).to(torch.int32)               # floor(log2 amax) - emax(E2M1)=2
    X = torch.where(amax > 0, X, torch.zeros_like(X))
    X = X.clamp(-127, 127)
    q = torch.ldexp(v, (-X).to(torch.float32).unsqueeze(2))  # exact scaling by 2^-X
    a = q.abs()
    code = ((a > 0.25).to(torch.int32) + (a >= 0.75) + (a > 1.25) + (a >= 1.75)
            + (a > 2.5) + (a >= 3.5) + (a > 5.0))
    sign = ((q < 0) & (code > 0)).to(torch.int32) << 3
    nib = (code | sign).to(torch.uint8).view(N, K)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).contiguous()
    scales = (X + 127).to(torch.uint8).contiguous()
    return packed, scales


# --- configurations ------------------------------------------------------------

@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    tokens: tuple
    hidden: int
    experts: int
    inter: int
    top_k: int
    w_dtype: str          # "f32" | "bf16" | "mxfp4"
    a_dtype: str          # "f32" | "bf16"
    logits: str           # "router" | "zipf" | "uniform" | "normal_t"
    w_std: float = 0.02
    layers: int = 1
    temperature: float = 1.0
    zipf_s: float = 1.1
    # "zipf" logits: 0 keeps one popularity law per layer for the whole trace;
    # n > 0 draws a new ranking of each layer's experts every n steps (phase
    # step // n), a trace whose hot set moves, as the working set of a served
    # session does between turns
    drift_steps: int = 0


CONFIGS = {
    "tiny": Config(0, "tiny", (64,), 256, 16, 128, 2, "f32", "f32", "router"),
    "decode": Config(1, "decode", (1, 4, 16), 4096, 256, 1024, 6, "bf16", "bf16", "router"),
    "cached": Config(2, "cached", (1, 4, 16), 4096, 256, 1024, 6, "bf16", "bf16", "zipf", layers=43),
    "prefill": Config(3, "prefill", (4096,), 4096, 256, 1024, 6, "bf16", "bf16", "uniform", layers=8),
    "prefill_fp4": Config(4, "prefill_fp4", (8192,), 4096, 256, 2048, 8, "mxfp4", "bf16", "normal_t",
                          temperature=0.5),
}


def activations(cfg: Config, T: int, layer: int = 0, batch: int = 0, device="cpu", dtype=None):
    """x [T, d] ~ N(0, 1) in the config's activation dtype."""
    return _normal_tensor(key_of(cfg.cid, layer, T_X, 0, batch * 65536 + T), (T, cfg.hidden), 1.0,
                          dtype or cfg.a_dtype, device)


def router_weights(cfg: Config, layer: int = 0, device="cpu"):
    """W_r [E, d] ~ N(0, 0.02^2), row = expert, in the activation dtype."""
    return _normal_tensor(key_of(cfg.cid, layer, T_WR), (cfg.experts, cfg.hidden), cfg.w_std,
                          cfg.a_dtype, device)


def expert_weights(cfg: Config, layer: int, expert: int, device="cpu", dtype=None):
    """One expert's tensors.

    Returns a dict with w_gate [I, d], w_up [I, d], w_down [d, I] (row-major,
    reduction dim contiguous).  For MXFP4 the values are the encoded nibbles
    ([rows, cols/2] uint8) and s_gate / s_up / s_down hold the E8M0 scales
    ([rows, cols/32] uint8).
    """
    d, I = cfg.hidden, cfg.inter
    dt = dtype or cfg.w_dtype
    shapes = {"w_gate": (T_WG, (I, d)), "w_up": (T_WU, (I, d)), "w_down": (T_WD, (d, I))}
    out = {}
    for name, (tid, shape) in shapes.items():
        key = key_of(cfg.cid, layer, tid, expert)
        if dt == "mxfp4":
            w = _normal_tensor(key, shape, cfg.w_std, "f32", device)
            q, s = quantize_mxfp4(w)
            out[name] = q
            out["s" + name[1:]] = s
        else:
            out[name] = _normal_tensor(key, shape, cfg.w_std, dt, device)
    return out


def popularity_rank(cfg: Config, layer: int, device="cpu", phase: int = 0) -> torch.Tensor:
    """Rank (1 = most popular) of each expert of `layer` in the Zipf recipe, fp64 [E].
    `phase` selects the ranking of a drifting trace (phase 0 is the stationary one)."""
    E = cfg.experts
    u = uniform(key_of(cfg.cid, layer, T_PERM, 0, phase), E, device)
    rank = torch.empty(E, dtype=torch.float64, device=device)
    rank[torch.argsort(u, stable=True)] = torch.arange(1, E + 1, dtype=torch.float64, device=device)
    return rank


def phase_of(cfg: Config, step: int) -> int:
    """Popularity phase of a step: 0 throughout unless cfg.drift_steps > 0."""
    return step // cfg.drift_steps if cfg.drift_steps > 0 else 0


def zipf_gumbel_logits(cfg: Config, layer: int, step: int, T: int, device="cpu"):
    """Logits whose top-k is a Zipf(s)-weighted draw without replacement.

    Layer l ranks its experts by a seeded permutation; the expert of rank r
    (1-based) has popularity p_r proportional to r^-s.  Each (step, token,
    expert) adds an independent Gumbel(0, 1) draw to log p, so the k largest
    logits are a sample of k experts without replacement with weights p
    (the Gumbel-top-k construction of Kool, van Hoof and Welling, ICML 2019).
    With cfg.drift_steps = n > 0 the ranking is redrawn every n steps.
    """
    E = cfg.experts
    rank = popularity_rank(cfg, layer, device, phase_of(cfg, step))
    logp = -cfg.zipf_s * torch.log(rank)
    logp = logp - torch.logsumexp(logp, 0)
    g = uniform(key_of(cfg.cid, layer, T_LOGITS, 0, step), T * E, device).view(T, E)
    gumbel = -torch.log(-torch.log(g))
    return (logp.unsqueeze(0) + gumbel).to(torch.float32)


def router_logits(cfg: Config, T: int, layer: int = 0, step: int = 0, device="cpu"):
    """Synthetic router logits [T, E] fp32 for the configs that supply them."""
    E = cfg.experts
    key = key_of(cfg.cid, layer, T_LOGITS, 0, step)
    if cfg.logits == "uniform":
        return uniform(key, T * E, device).view(T, E).to(torch.float32)
    if cfg.logits == "normal_t":
        return (normal(key, T * E, 1.0, device) / cfg.temperature).view(T, E).to(torch.float32)
    if cfg.logits == "zipf":
        return zipf_gumbel_logits(cfg, layer, step, T, device)
    raise ValueError(f"config {cfg.name} computes logits with its router")
