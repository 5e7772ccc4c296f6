"""Seeded synthetic workloads for the KDA forward pass.

This module only draws random inputs with the shapes, value distributions and
packing structure of the benchmark workloads and rounds them to their storage
dtypes.  It holds none of the method's arithmetic, so both the HIP path and the
fp64 oracle can be fed from it.

Recipe (all draws from one torch.Generator seeded with 1234 + workload id):
  q, k  ~ N(0, 1), L2-normalised per (token, head) in fp32, stored bf16
          (fp32 when dtype="fp32");
  v     ~ N(0, 1), stored bf16 (fp32 when dtype="fp32");
  g     = -exp(u), u ~ U(ln g_lo, ln g_hi) per (token, head, channel), fp32
          (the log of the per-channel decay, so alpha = exp(g) in (0, 1));
  beta  = sigmoid(N(0, 1)) per (token, head), fp32;
  initial states ~ N(0, 0.02^2) (0.02 is the standard deviation), in the
          workload's state dtype, or absent;
  varlen lengths: n draws exp(U(ln 256, ln 16384)), rescaled to the packed
          total and rounded by largest remainder (every length >= 1, not
          aligned to the chunk size).
The softmax scale 1/sqrt(d_k) is passed as `scale`, never folded into q.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

D = 128  # head dimension d_k = d_v of every workload


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    B: int
    T: int                      # tokens per batch row (packed total when varlen)
    H: int
    n_seqs: int = 0             # > 0: varlen packing of that many sequences, B == 1
    g_lo: float = 1e-3
    g_hi: float = 0.5
    init_state: str | None = None   # None, "bf16" or "fp32"
    final_state: str | None = "fp32"
    dtype: str = "bf16"         # storage dtype of q/k/v (the kernel's I/O is bf16)
    notes: str = field(default="", compare=False)

    @property
    def seed(self) -> int:
        return 1234 + self.wid

    @property
    def tokens(self) -> int:
        return self.B * self.T

    @property
    def num_states(self) -> int:
        return self.n_seqs if self.n_seqs else self.B


WORKLOADS = {
    0: Workload(0, "tiny T=256 H=1", B=1, T=256, H=1, dtype="fp32",
                notes="oracle self-test size; the GPU run rounds q/k/v to bf16"),
    1: Workload(1, "prefill T=8192 H=32", B=1, T=8192, H=32),
    2: Workload(2, "varlen 16 seqs 65536 tokens H=32", B=1, T=65536, H=32, n_seqs=16,
                init_state="bf16", final_state="bf16"),
    3: Workload(3, "continuation B=4 T=32768 H=32", B=4, T=32768, H=32,
                init_state="fp32", final_state="fp32"),
    4: Workload(4, "long context T=1048576 H=32", B=1, T=1048576, H=32, g_lo=1e-4, g_hi=0.1),
}


def varlen_lengths(n: int, total: int, gen: torch.Generator, lo: float = 256.0,
                   hi: float = 16384.0) -> list[int]:
    """n log-uniform lengths in [lo, hi], rescaled to sum exactly to `total`."""
    u = torch.rand(n, generator=gen, dtype=torch.float64, device=gen.device).cpu()
    raw = torch.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))
    target = raw * (total / float(raw.sum()))
    base = torch.clamp(torch.floor(target), min=1).to(torch.int64)
    rest = total - int(base.sum())
    if rest > 0:   # hand the remainder to the largest fractional parts
        order = torch.argsort(target - torch.floor(target), descending=True)
        for i in range(rest):
            base[order[i % n]] += 1
    while int(base.sum()) > total:   # only reachable when clamping to 1 added tokens
        j = int(torch.argmax(base))
        base[j] -= 1
    return [int(x) for x in base]


def cu_from_lengths(lengths, device="cpu") -> torch.Tensor:
    cu = [0]
    for L in lengths:
        cu.append(cu[-1] + int(L))
    return torch.tensor(cu, dtype=torch.int32, device=device)


def _store(x: torch.Tensor, dtype: str) -> torch.Tensor:
    return x.to(torch.bfloat16) if dtype == "bf16" else x.to(torch.float32)


def random_inputs(B: int, T: int, H: int, DK: int = D, DV: int = D, *, seed: int,
                  device="cpu", dtype: str = "bf16", g_lo: float = 1e-3, g_hi: float = 0.5,
                  init_state: str | None = None, n_states: int | None = None,
                  lengths: list[int] | None = None) -> dict:
    """Draw one workload's tensors (see the module docstring for the recipe).

    Returns a dict with q, k, v ([B, T, H, DK|DV]), g ([B, T, H, DK] fp32),
    beta ([B, T, H] fp32), initial_state ([N, H, DK, DV] or None), cu_seqlens
    (int32 [N+1] or None) and scale = 1/sqrt(DK).
    """
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out: dict = {}
    cu = None
    if lengths is not None:
        if B != 1 or sum(lengths) != T:
            raise ValueError("varlen packing needs B == 1 and sum(lengths) == T")
        cu = cu_from_lengths(lengths, device)
    for name, dim in (("q", DK), ("k", DK)):
        x = torch.randn(B, T, H, dim, generator=gen, device=device, dtype=torch.float32)
        x = x / torch.linalg.vector_norm(x, dim=-1, keepdim=True).clamp_min(1e-12)
        out[name] = _store(x, dtype)
        del x
    out["v"] = _store(torch.randn(B, T, H, DV, generator=gen, device=device,
                                  dtype=torch.float32), dtype)
    u = torch.rand(B, T, H, DK, generator=gen, device=device, dtype=torch.float32)
    u.mul_(math.log(g_hi) - math.log(g_lo)).add_(math.log(g_lo))
    out["g"] = torch.exp(u).neg_()
    del u
    out["beta"] = torch.sigmoid(torch.randn(B, T, H, generator=gen, device=device,
                                            dtype=torch.float32))
    N = n_states if n_states is not None else (len(lengths) if lengths is not None else B)
    if init_state is None:
        out["initial_state"] = None
    else:
        s = 0.02 * torch.randn(N, H, DK, DV, generator=gen, device=device, dtype=torch.float32)
        out["initial_state"] = _store(s, init_state)
    out["cu_seqlens"] = cu
    out["scale"] = 1.0 / math.sqrt(DK)
    return out


def make_inputs(wid: int, device="cpu", dtype: str | None = None) -> dict:
    """The tensors of workload `wid` (0..4), drawn on `device`."""
    w = WORKLOADS[wid]
    lengths = None
    if w.n_seqs:
        lgen = torch.Generator(device="cpu")
        lgen.manual_seed(w.seed)
        lengths = varlen_lengths(w.n_seqs, w.T, lgen)
    x = random_inputs(w.B, w.T, w.H, seed=w.seed + 7919, device=device,
                      dtype=dtype or w.dtype, g_lo=w.g_lo, g_hi=w.g_hi,
                      init_state=w.init_state, lengths=lengths)
    x["workload"] = w
    x["lengths"] = lengths if lengths is not None else [w.T] * w.B
    return x


def sample_heads(wid: int, count: int = 4) -> list[int]:
    """`count` distinct heads chosen with the workload's seed (sampled checks)."""
    w = WORKLOADS[wid]
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed + 17)
    return sorted(int(h) for h in torch.randperm(w.H, generator=gen)[:count])
