"""GPU parity of the scalar-gate (Gated DeltaNet) entry points against the fp64
scalar-gate oracle, through the C ABI.

The gate is one log-decay per token and head; the inputs reuse the KDA recipe
and take the first channel of its per-channel gate as the scalar gate (same
distribution).  Bar: max|x - x_ref| / max|x_ref| <= 1e-2 for outputs and final
states, and per (sequence, head) for the 64K varlen workload.  One case also
checks that the scalar-gate path gives bit-identical results to kda_fwd fed the
same gate on every channel (the kernels after the gate load are shared).
"""
import sys

import numpy as np
import pytest
import torch

from linear_attention_kda_amd import binding
from linear_attention_kda_amd.workloads import random_inputs
from oracle import oracle

pytestmark = pytest.mark.gpu

TOL = 1e-2
DEV = "cuda"


def announce(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def rel_err(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max()
    num = np.abs(x - ref).max()
    return num if den == 0.0 else num / den


def host(t):
    return t.detach().float().cpu().numpy()


@pytest.fixture(autouse=True)
def _gpu_required():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    binding.load_library()


def gdn_inputs(B, T, H, seed, state="fp32", lengths=None):
    x = random_inputs(B, T, H, seed=seed, device=DEV, init_state=state, lengths=lengths)
    x["gs"] = x["g"][..., 0].contiguous()
    return x


def run_gdn(x, final_dtype=torch.float32):
    N = (x["cu_seqlens"].numel() - 1) if x["cu_seqlens"] is not None else x["q"].shape[0]
    H = x["q"].shape[2]
    if x["initial_state"] is not None:
        final_dtype = x["initial_state"].dtype
    fin = torch.empty(N, H, 128, 128, dtype=final_dtype, device=DEV)
    out, fin = binding.gdn_fwd(x["q"], x["k"], x["v"], x["gs"], x["beta"], x["scale"],
                               initial_state=x["initial_state"], final_state=fin,
                               cu_seqlens=x["cu_seqlens"])
    torch.cuda.synchronize()
    return out, fin


def check_gdn(x, out, fin, heads=None):
    sel = (lambda t: t) if heads is None else (lambda t: t[:, :, heads])
    selS = (lambda t: t) if heads is None else (lambda t: t[:, heads])
    init = x["initial_state"]
    o_ref, S_ref = oracle.gdn_fwd(sel(x["q"]).cpu(), sel(x["k"]).cpu(), sel(x["v"]).cpu(),
                                  sel(x["gs"]).cpu(), sel(x["beta"]).cpu(), x["scale"],
                                  None if init is None else selS(init).cpu(),
                                  cu_seqlens=None if x["cu_seqlens"] is None else x["cu_seqlens"].cpu())
    e_o = rel_err(host(sel(out)), o_ref)
    e_s = rel_err(host(selS(fin)), S_ref)
    print(f"    out rel err {e_o:.3e}, state rel err {e_s:.3e}", flush=True)
    assert e_o <= TOL and e_s <= TOL


@pytest.mark.parametrize("B,T,H,state", [(2, 300, 3, "fp32"), (1, 129, 2, "bf16"),
                                          (1, 64, 1, None), (3, 1, 2, "fp32")])
def test_gdn_matches_oracle(B, T, H, state):
    announce(f"gdn B={B} T={T} H={H} state={state}")
    x = gdn_inputs(B, T, H, seed=50 + T, state=state)
    out, fin = run_gdn(x)
    check_gdn(x, out, fin)


def test_gdn_varlen():
    lengths = [1, 64, 65, 200, 0, 33]
    announce(f"gdn varlen {lengths}")
    x = gdn_inputs(1, sum(lengths), 2, seed=60, lengths=lengths)
    out, fin = run_gdn(x)
    check_gdn(x, out, fin)


def test_gdn_split_long_sequence(monkeypatch):
    monkeypatch.setenv("KDA_SEG_MIN", "3")
    announce("gdn split B=1 T=1000 H=4 seg_min=3")
    x = gdn_inputs(1, 1000, 4, seed=61)
    out, fin = run_gdn(x)
    check_gdn(x, out, fin)


@pytest.mark.parametrize("seg_min", [None, "3"])
def test_gdn_is_kda_with_the_gate_on_every_channel(monkeypatch, seg_min):
    if seg_min is not None:
        monkeypatch.setenv("KDA_SEG_MIN", seg_min)
    announce(f"gdn vs kda with repeated gate, seg_min={seg_min}")
    x = gdn_inputs(1, 700, 3, seed=62)
    out_g, fin_g = run_gdn(x)
    check_gdn(x, out_g, fin_g)
    g_rep = x["gs"][..., None].expand(-1, -1, -1, 128).contiguous()
    fin_k = torch.empty_like(fin_g)
    out_k, fin_k = binding.fwd(x["q"], x["k"], x["v"], g_rep, x["beta"], x["scale"],
                               initial_state=x["initial_state"], final_state=fin_k)
    torch.cuda.synchronize()
    assert torch.equal(out_g, out_k)
    assert torch.equal(fin_g, fin_k)


def test_gdn_strong_decay():
    """Scalar gate down to -5 per token: the chunk's decay reaches ~300 (natural log),
    so the 16-row block references carry the tile products."""
    announce("gdn strong decay g in [-5, -1e-4]")
    x = random_inputs(1, 640, 2, seed=64, device=DEV, g_lo=1e-4, g_hi=5.0, init_state="fp32")
    x["gs"] = x["g"][..., 0].contiguous()
    out, fin = run_gdn(x)
    check_gdn(x, out, fin)


def test_gdn_varlen_workload_all_heads():
    """The scalar-gate bench workload: 16 packed sequences, 65,536 tokens, H = 32, bf16
    states, every head, with the per-(sequence, head) bar."""
    from linear_attention_kda_amd.workloads import make_inputs
    announce("gdn 64K varlen workload, all heads")
    x = make_inputs(2, DEV)
    x["gs"] = x["g"][..., 0].contiguous()
    out, fin = run_gdn(x)
    check_gdn(x, out, fin)
    o_ref, S_ref = oracle.gdn_fwd(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), x["gs"].cpu(),
                                  x["beta"].cpu(), x["scale"], x["initial_state"].cpu(),
                                  cu_seqlens=x["cu_seqlens"].cpu())
    o = host(out)
    cu = [int(c) for c in x["cu_seqlens"].cpu()]
    worst = 0.0
    for n in range(len(cu) - 1):
        a, b = cu[n], cu[n + 1]
        if b <= a:
            continue
        num = np.abs(o[0, a:b] - o_ref[0, a:b]).max(axis=(0, 2))
        den = np.abs(o_ref[0, a:b]).max(axis=(0, 2))
        worst = max(worst, float((num / np.maximum(den, 1e-30)).max()))
    f = host(fin)
    ws = float((np.abs(f - S_ref).max(axis=(2, 3)) / np.maximum(np.abs(S_ref).max(axis=(2, 3)), 1e-30)).max())
    print(f"    worst per-(sequence, head): out {worst:.3e}, state {ws:.3e}", flush=True)
    assert worst <= TOL and ws <= TOL


def test_gdn_full_size_sampled_heads():
    B, T, H = 1, 8192, 32
    heads = [3, 29]
    announce(f"gdn B={B} T={T} H={H}, oracle on heads {heads}")
    x = gdn_inputs(B, T, H, seed=63, state="bf16")
    out, fin = run_gdn(x)
    check_gdn(x, out, fin, heads=heads)


@pytest.mark.parametrize("state", ["fp32", "bf16"])
def test_gdn_decode_chained_steps(state):
    N, H, T = 5, 3, 12
    announce(f"gdn decode {T} chained steps N={N} H={H} state={state}")
    x = gdn_inputs(N, T, H, seed=64, state=state)
    o_ref, S_ref = oracle.gdn_fwd(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), x["gs"].cpu(),
                                  x["beta"].cpu(), x["scale"], x["initial_state"].cpu())
    S = x["initial_state"].clone()
    outs = []
    for t in range(T):
        sl = lambda a: a[:, t].contiguous()  # noqa: E731
        outs.append(binding.gdn_decode(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["gs"]),
                                       sl(x["beta"]), S, scale=x["scale"]))
    torch.cuda.synchronize()
    e_o = rel_err(host(torch.stack(outs, dim=1)), o_ref)
    e_s = rel_err(host(S), S_ref)
    print(f"    out rel err {e_o:.3e}, state rel err {e_s:.3e}", flush=True)
    assert e_o <= TOL and e_s <= TOL


def test_gdn_decode_continues_a_prefill():
    H, T = 4, 257
    announce(f"gdn prefill {T} tokens then decode one, H={H}")
    x = gdn_inputs(1, T + 1, H, seed=65)
    pre = {k: x[k][:, :T].contiguous() for k in ("q", "k", "v", "gs", "beta")}
    _, S = binding.gdn_fwd(pre["q"], pre["k"], pre["v"], pre["gs"], pre["beta"], x["scale"],
                           initial_state=x["initial_state"], output_final_state=True)
    last = lambda a: a[:, T].contiguous()  # noqa: E731
    out = binding.gdn_decode(last(x["q"]), last(x["k"]), last(x["v"]), last(x["gs"]),
                             last(x["beta"]), S, scale=x["scale"])
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.gdn_fwd(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), x["gs"].cpu(),
                                  x["beta"].cpu(), x["scale"], x["initial_state"].cpu())
    e_o = rel_err(host(out), o_ref[:, T])
    e_s = rel_err(host(S), S_ref)
    print(f"    out rel err {e_o:.3e}, state rel err {e_s:.3e}", flush=True)
    assert e_o <= TOL and e_s <= TOL
