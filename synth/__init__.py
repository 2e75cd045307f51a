"""Seeded synthetic inputs for the Beam-1.0 MoE block.

This module only *makes inputs*: token activations, router weights and expert
weights, with the shapes and value distributions of the workloads described for
the Beam-1.0 mixture-of-experts layer ("Welcome Beam: a 501B open model you can
own, customize, and scale", section "Mixture of Experts": hidden size 5,120,
256 SwiGLU experts of intermediate size 2,560, 8 groups of 32).  It holds none
of the layer's arithmetic; the CPU oracle and the HIP library both consume what
it produces, and neither is imported here.

Random numbers come from a counter-based generator, so any element of any
tensor can be produced independently, on the CPU or on a GPU, with identical
bits:

* ``mix32`` is the "lowbias32" integer hash from Chris Wellons' hash-prospector
  (xorshift-multiply, constants 0x7feb352d and 0x846ca68b).
* An approximately standard normal draw for element ``n`` of a stream is the
  Irwin-Hall sum of four 16-bit uniforms taken from two chained hashes of ``n``,
  centred and scaled to unit variance (bounded at +-2*sqrt(3)).  Integer work is
  exact; the only float operation is one fp32 multiply by an fp32 constant,
  followed by round-to-nearest-even to bf16 where the tensor is bf16.  Both are
  IEEE-defined, so CPU and GPU results agree bit for bit.

Everything is done with torch integer tensors (int64 holding 32-bit values,
products kept below 2**63) so the same code runs on ``cpu`` and ``cuda``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

M32 = 0xFFFFFFFF

# Stream tags: one independent stream per kind of tensor.
TAG_X = 0
TAG_ROUTER = 1
TAG_GATE_UP = 2
TAG_DOWN = 3
TAG_HOT = 4
TAG_MIX = 5
TAG_BIAS = 6
TAG_LORA = 7


# ---------------------------------------------------------------------------
# counter-based generator
# ---------------------------------------------------------------------------
def mix32_int(x: int) -> int:
    """lowbias32 on a Python int (used for stream keys and small draws)."""
    x &= M32
    x ^= x >> 16
    x = (x * 0x7FEB352D) & M32
    x ^= x >> 15
    x = (x * 0x846CA68B) & M32
    x ^= x >> 16
    return x


def _mul32(x: torch.Tensor, c: int) -> torch.Tensor:
    # (x * c) mod 2**32 for 0 <= x < 2**32, split so every product is < 2**49
    lo, hi = c & 0xFFFF, c >> 16
    return (x * lo + (((x * hi) & 0xFFFF) << 16)) & M32


def mix32(x: torch.Tensor) -> torch.Tensor:
    """lowbias32 on an int64 tensor of 32-bit values."""
    x = x ^ (x >> 16)
    x = _mul32(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32(x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


def stream_key(seed: int, tag: int, index: int = 0) -> int:
    """32-bit key of stream (seed, tag, index)."""
    k = mix32_int(seed ^ 0x243F6A88)
    k = mix32_int(k ^ (tag * 0x9E3779B9 & M32))
    k = mix32_int(k ^ ((index + 1) * 0x85EBCA6B & M32))
    return k


_IH_CENTER = 2 * 0xFFFF  # mean of a sum of four uniforms on {0..65535}
_IH_UNIT = math.sqrt(3.0) / 65536.0  # 1 / std of that sum (std = 65536/sqrt(3) to 1e-9)


def counter_normal(key: int, n: int, std: float = 1.0, start: int = 0,
                   device="cpu", chunk: int = 1 << 24) -> torch.Tensor:
    """``n`` approximately N(0, std**2) fp32 values of stream ``key``.

    Element j uses counter ``start + j`` (must stay below 2**32).
    """
    if start + n > (1 << 32):
        raise ValueError("counter_normal: stream longer than 2**32 elements")
    k1 = key & M32
    k2 = mix32_int(key ^ 0x9E3779B9)
    scale = torch.tensor(_IH_UNIT * std, dtype=torch.float32, device=device)
    out = torch.empty(n, dtype=torch.float32, device=device)
    for c0 in range(0, n, chunk):
        c1 = min(n, c0 + chunk)
        ctr = torch.arange(start + c0, start + c1, dtype=torch.int64, device=device)
        h1 = mix32(ctr ^ k1)
        h2 = mix32(h1 ^ k2)
        s = (h1 & 0xFFFF) + (h1 >> 16) + (h2 & 0xFFFF) + (h2 >> 16) - _IH_CENTER
        out[c0:c1] = s.to(torch.float32) * scale
    return out


def counter_uint(key: int, n: int, device="cpu") -> torch.Tensor:
    """``n`` 32-bit uniform integers (int64 tensor) of stream ``key``."""
    ctr = torch.arange(0, n, dtype=torch.int64, device=device)
    return mix32(mix32(ctr ^ (key & M32)) ^ mix32_int(key ^ 0x7F4A7C15))


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    """Shape and value recipe of one synthetic MoE-layer call."""
    name: str
    T: int                 # tokens in the call
    H: int                 # hidden size
    I: int                 # SwiGLU intermediate size
    E: int = 256           # routed experts
    G: int = 8             # expert groups
    KG: int = 4            # groups kept per token
    K: int = 8             # experts per token
    router_std: float = 0.02
    expert_std: float = 0.02
    x_std: float = 1.0
    skew: bool = False     # mixture input favouring 16 hot experts
    notes: str = field(default="", compare=False)


WORKLOADS = {
    "tiny": Workload("tiny", T=128, H=256, I=128,
                     notes="oracle-sized check of the full layer"),
    "decode": Workload("decode", T=32, H=5120, I=2560,
                       notes="decode batch; weight streaming"),
    "mid": Workload("mid", T=512, H=5120, I=2560,
                    notes="~16 tokens per expert"),
    "prefill": Workload("prefill", T=4096, H=5120, I=2560,
                        notes="prefill chunk; ~128 tokens per expert"),
    "skew": Workload("skew", T=16384, H=5120, I=2560, skew=True,
                     notes="mixture input; 16 hot experts get +2.0 logit"),
}


def workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    if overrides:
        d = dict(w.__dict__)
        d.update(overrides)
        w = Workload(**d)
    return w


def make_router(w: Workload, seed: int = 0, device="cpu") -> torch.Tensor:
    """Router weight, fp32 [E, H] (one row per expert), ~N(0, router_std**2)."""
    key = stream_key(seed, TAG_ROUTER)
    return counter_normal(key, w.E * w.H, w.router_std, device=device).view(w.E, w.H)


def make_expert(w: Workload, e: int, seed: int = 0, device="cpu"):
    """Expert ``e``'s weights: gate/up bf16 [2I, H] (gate rows first), down bf16 [H, I]."""
    gu = counter_normal(stream_key(seed, TAG_GATE_UP, e), 2 * w.I * w.H, w.expert_std,
                        device=device).to(torch.bfloat16).view(2 * w.I, w.H)
    dn = counter_normal(stream_key(seed, TAG_DOWN, e), w.H * w.I, w.expert_std,
                        device=device).to(torch.bfloat16).view(w.H, w.I)
    return gu, dn


def make_experts(w: Workload, seed: int = 0, device="cpu"):
    """All experts: gate/up bf16 [E, 2I, H] and down bf16 [E, H, I]."""
    w_gu = torch.empty(w.E, 2 * w.I, w.H, dtype=torch.bfloat16, device=device)
    w_dn = torch.empty(w.E, w.H, w.I, dtype=torch.bfloat16, device=device)
    for e in range(w.E):
        gu, dn = make_expert(w, e, seed, device)
        w_gu[e].copy_(gu)
        w_dn[e].copy_(dn)
    return w_gu, w_dn


def hot_experts(w: Workload, seed: int = 0) -> list[int]:
    """The 16 hot experts of the skewed workload: 6, 5 and 5 experts from three
    distinct groups, all chosen by hash rank (deterministic, seeded)."""
    key = stream_key(seed, TAG_HOT)
    per_group = w.E // w.G
    groups = sorted(range(w.G), key=lambda g: (mix32_int(key ^ (0x1000 + g)), g))[:3]
    hot = []
    for g, take in zip(groups, (6, 5, 5)):
        members = range(g * per_group, (g + 1) * per_group)
        hot += sorted(members, key=lambda e: (mix32_int(key ^ (0x2000 + e)), e))[:take]
    return sorted(hot)


def skew_shift(w_router: torch.Tensor, hot: list[int], delta: float = 2.0) -> torch.Tensor:
    """Minimum-norm input shift that adds exactly ``delta`` to the hot experts'
    logits and 0 to all others: W^T (W W^T)^-1 (delta * 1_hot), in fp64."""
    W = w_router.detach().to("cpu", torch.float64)
    b = torch.zeros(W.shape[0], dtype=torch.float64)
    b[hot] = delta
    return W.T @ torch.linalg.solve(W @ W.T, b)


def make_x(w: Workload, seed: int = 0, device="cpu", w_router: torch.Tensor | None = None,
           ncomp: int = 16, mix: float = 0.9) -> torch.Tensor:
    """Token activations, bf16 [T, H].

    Plain workloads: ~N(0, x_std**2).  Skewed workload: a mixture
    x_t = bf16(mix * mu_{c_t} + sqrt(1 - mix**2) * z_t + shift), with ``ncomp``
    component means mu_c ~ N(0,1)^H, c_t drawn uniformly per token, z_t ~ N(0,1)^H,
    and ``shift`` from :func:`skew_shift` (+2.0 on the 16 hot experts' logits).
    """
    if not w.skew:
        return counter_normal(stream_key(seed, TAG_X), w.T * w.H, w.x_std,
                              device=device).to(torch.bfloat16).view(w.T, w.H)
    if w_router is None:
        w_router = make_router(w, seed, device="cpu")
    shift = skew_shift(w_router, hot_experts(w, seed)).to(device=device, dtype=torch.float32)
    mu = counter_normal(stream_key(seed, TAG_MIX, 0), ncomp * w.H, device=device).view(ncomp, w.H)
    comp = counter_uint(stream_key(seed, TAG_MIX, 1), w.T, device=device) % ncomp
    z = counter_normal(stream_key(seed, TAG_MIX, 2), w.T * w.H, device=device).view(w.T, w.H)
    a = torch.tensor(mix, dtype=torch.float32, device=device)
    b = torch.tensor(math.sqrt(1.0 - mix * mix), dtype=torch.float32, device=device)
    x = mu[comp] * a
    x = x + z * b
    x = x + shift
    return x.to(torch.bfloat16)


def make_sel_bias(w: Workload, seed: int = 0, std: float = 0.05, device="cpu") -> torch.Tensor:
    """Optional per-expert selection bias, fp32 [E] (off unless asked for)."""
    return counter_normal(stream_key(seed, TAG_BIAS), w.E, std, device=device)


def make_lora(w: Workload, seed: int = 0, device="cpu", rank: int = 16, std: float = 0.02):
    """Synthetic expert adapters, bf16 and ~N(0, std**2) (nonzero B, unlike a
    fresh adapter, so that the adapter term is visible): a_gate_up [E, r, H],
    b_gate_up [E, 2I, r], a_down [E, r, I], b_down [E, H, r]."""
    shapes = [(w.E, rank, w.H), (w.E, 2 * w.I, rank), (w.E, rank, w.I), (w.E, w.H, rank)]
    out = []
    for j, shp in enumerate(shapes):
        n = shp[0] * shp[1] * shp[2]
        out.append(counter_normal(stream_key(seed, TAG_LORA, j), n, std, device=device)
                   .to(torch.bfloat16).view(*shp))
    return tuple(out)


def make_inputs(name: str | Workload, seed: int = 0, device="cpu", experts: bool = True,
                **overrides) -> dict:
    """All inputs of one workload as a dict of tensors on ``device``."""
    w = name if isinstance(name, Workload) else workload(name, **overrides)
    w_router = make_router(w, seed, device)
    x = make_x(w, seed, device, w_router=w_router)
    out = {"workload": w, "x": x, "w_router": w_router}
    if experts:
        out["w_gate_up"], out["w_down"] = make_experts(w, seed, device)
    return out
