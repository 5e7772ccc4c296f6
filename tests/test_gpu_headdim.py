"""GPU parity of the head-dimension 64 and 256 forward path (kda_fwd and
kda_gdn_fwd with K = V = d, through the C ABI) against the fp64 oracle.

The oracle is head-dimension generic (the recurrence has no size of its own), so
the same bar applies as at d = 128: max|x - x_ref| / max|x_ref| <= 1e-2 for the
output and, separately, the final state.  Cases span several chunks with ragged
tails, varlen packing with empty and one-token sequences, both state dtypes and
no state, an aliased state, strong decay, the scalar gate, a call without tokens,
and the 64K varlen workload at H = 32 on sampled heads.
"""
import sys

import numpy as np
import pytest
import torch

from linear_attention_kda_amd import binding
from linear_attention_kda_amd.workloads import WORKLOADS, random_inputs, sample_heads, varlen_lengths
from oracle import oracle

pytestmark = pytest.mark.gpu

TOL = 1e-2
DEV = "cuda"
DIMS = [64, 256]


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


def inputs(D, B, T, H, seed, state="fp32", lengths=None, **kw):
    return random_inputs(B, T, H, D, D, seed=seed, device=DEV, init_state=state,
                         lengths=lengths, **kw)


def run(x, final_dtype=torch.float32, scalar_gate=False, final=None):
    q = x["q"]
    N = (x["cu_seqlens"].numel() - 1) if x["cu_seqlens"] is not None else q.shape[0]
    H, D = q.shape[2], q.shape[3]
    if final is None and final_dtype is not None:
        final = torch.empty(N, H, D, D, dtype=final_dtype, device=DEV)
    g = x["g"][..., 0].contiguous() if scalar_gate else x["g"]
    entry = binding.gdn_fwd if scalar_gate else binding.fwd
    res = entry(q, x["k"], x["v"], g, x["beta"], x["scale"], initial_state=x["initial_state"],
                final_state=final, cu_seqlens=x["cu_seqlens"])
    torch.cuda.synchronize()
    return res if final is not None else (res, None)


def reference(x, scalar_gate=False, heads=None):
    cpu = lambda t: None if t is None else t.cpu()  # noqa: E731
    s0 = cpu(x["initial_state"])
    if scalar_gate:
        return oracle.gdn_fwd(cpu(x["q"]), cpu(x["k"]), cpu(x["v"]), cpu(x["g"][..., 0]),
                              cpu(x["beta"]), x["scale"], s0, cpu(x["cu_seqlens"]))
    return oracle.fwd(cpu(x["q"]), cpu(x["k"]), cpu(x["v"]), cpu(x["g"]), cpu(x["beta"]),
                      x["scale"], s0, cpu(x["cu_seqlens"]), heads=heads, col_block=16)


def check(o, f, o_ref, f_ref, what):
    e_o = rel_err(host(o), o_ref)
    msg = f"    {what}: out rel err {e_o:.3e}"
    ok = e_o <= TOL
    if f is not None:
        e_s = rel_err(host(f), f_ref)
        msg += f", state rel err {e_s:.3e}"
        ok = ok and e_s <= TOL
    print(msg, flush=True)
    assert ok, msg


@pytest.mark.parametrize("D", DIMS)
@pytest.mark.parametrize("state", ["fp32", "bf16", None])
def test_fixed_length_ragged(D, state):
    B, T, H = 2, 200, 3
    announce(f"d={D} fixed length B={B} T={T} H={H} state={state}")
    x = inputs(D, B, T, H, seed=500 + D, state=state)
    fd = {"fp32": torch.float32, "bf16": torch.bfloat16, None: torch.float32}[state]
    o, f = run(x, final_dtype=fd)
    o_ref, f_ref = reference(x)
    check(o, f, o_ref, f_ref, "fixed length")


@pytest.mark.parametrize("D", DIMS)
def test_varlen_with_empty_and_short_sequences(D):
    lengths = [0, 1, 130, 64, 0, 257, 65]
    T, H = sum(lengths), 2
    announce(f"d={D} varlen {lengths} H={H}")
    x = inputs(D, 1, T, H, seed=510 + D, lengths=lengths)
    o, f = run(x)
    o_ref, f_ref = reference(x)
    check(o, f, o_ref, f_ref, "varlen")
    # the empty sequences return their initial state unchanged
    for n in (0, 4):
        assert torch.equal(f[n], x["initial_state"][n])


@pytest.mark.parametrize("D", DIMS)
def test_single_token(D):
    announce(f"d={D} T=1")
    x = inputs(D, 3, 1, 2, seed=520 + D)
    o, f = run(x)
    o_ref, f_ref = reference(x)
    check(o, f, o_ref, f_ref, "single token")


@pytest.mark.parametrize("D", DIMS)
def test_strong_decay(D):
    announce(f"d={D} strong decay g in [-5, -1e-4]")
    x = inputs(D, 1, 320, 2, seed=530 + D, g_lo=1e-4, g_hi=5.0)
    o, f = run(x)
    o_ref, f_ref = reference(x)
    check(o, f, o_ref, f_ref, "strong decay")


@pytest.mark.parametrize("D", DIMS)
def test_in_place_state(D):
    announce(f"d={D} initial state == final state tensor")
    x = inputs(D, 2, 150, 2, seed=540 + D)
    o_ref, f_ref = reference(x)
    s = x["initial_state"].clone()
    x2 = dict(x, initial_state=s)
    o, f = run(x2, final=s)
    check(o, f, o_ref, f_ref, "aliased state")


@pytest.mark.parametrize("D", DIMS)
def test_scalar_gate(D):
    lengths = [70, 0, 190, 3]
    announce(f"d={D} scalar gate varlen {lengths}")
    x = inputs(D, 1, sum(lengths), 2, seed=550 + D, lengths=lengths)
    o, f = run(x, scalar_gate=True)
    o_ref, f_ref = reference(x, scalar_gate=True)
    check(o, f, o_ref, f_ref, "scalar gate")


@pytest.mark.parametrize("state", ["fp32", "bf16"])
def test_d64_split_sequences(monkeypatch, state):
    """d = 64 with sequences split into segments of 3 chunks (KDA_SEG_MIN=3): segment
    0 from the true initial state, zero- and identity-start runs of the later segments,
    the segment scan and the output fix-ups, at head dimension 64 (fixed length)."""
    monkeypatch.setenv("KDA_SEG_MIN", "3")
    B, T, H = 1, 1500, 2
    announce(f"d=64 split B={B} T={T} H={H} state={state}, seg_min=3")
    x = inputs(64, B, T, H, seed=570 + len(state), state=state)
    fd = {"fp32": torch.float32, "bf16": torch.bfloat16}[state]
    o, f = run(x, final_dtype=fd)
    o_ref, f_ref = reference(x)
    check(o, f, o_ref, f_ref, "split fixed length")


@pytest.mark.parametrize("scalar_gate", [False, True])
def test_d64_split_varlen(monkeypatch, scalar_gate):
    """d = 64, varlen with an empty and a short sequence among split ones, both gates."""
    monkeypatch.setenv("KDA_SEG_MIN", "3")
    lengths = [900, 0, 1300, 5, 64, 451]
    announce(f"d=64 split varlen {lengths} H=3 scalar_gate={scalar_gate}, seg_min=3")
    x = inputs(64, 1, sum(lengths), 3, seed=580 + scalar_gate, lengths=lengths)
    o, f = run(x, scalar_gate=scalar_gate)
    o_ref, f_ref = reference(x, scalar_gate=scalar_gate)
    check(o, f, o_ref, f_ref, "split varlen")
    assert torch.equal(f[1], x["initial_state"][1])


@pytest.mark.parametrize("D", DIMS)
def test_no_tokens_copies_the_state(D):
    announce(f"d={D} T=0")
    x = inputs(D, 2, 0, 2, seed=560 + D, state="bf16")
    o, f = run(x, final_dtype=torch.bfloat16)
    assert o.shape == (2, 0, 2, D)
    assert torch.equal(f, x["initial_state"])


@pytest.mark.parametrize("D", DIMS)
def test_full_size_varlen_sampled_heads(D):
    """The 64K-token varlen workload (16 sequences, H = 32, bf16 states) at head
    dimension D in the launch configuration the benchmark times (at d = 64 the long
    sequences split into segments); two seeded heads are compared with the oracle in
    full."""
    w = WORKLOADS[2]
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed)
    lengths = varlen_lengths(w.n_seqs, w.T, gen)   # the benchmark workload's lengths
    announce(f"d={D} {w.name} sampled heads")
    x = random_inputs(1, w.T, w.H, D, D, seed=w.seed + 7919 + D, device=DEV,
                      init_state=w.init_state, lengths=lengths)
    o, f = run(x, final_dtype=torch.bfloat16)
    heads = sample_heads(2, 2)
    if D == 64:  # every head, with the per-(sequence, head) bar as well
        heads = list(range(w.H))
    sub = {k: (x[k][:, :, heads].contiguous() if k in ("q", "k", "v", "g", "beta") else x[k])
           for k in x}
    sub["initial_state"] = x["initial_state"][:, heads].contiguous()
    o_ref, f_ref = reference(sub)
    check(o[:, :, heads], f[:, heads], o_ref, f_ref, f"heads {heads[0]}..{heads[-1]}")
    if D == 64:
        oh, fh = host(o[:, :, heads]), host(f[:, heads])
        cu = [int(c) for c in x["cu_seqlens"].cpu()]
        worst_o = worst_s = 0.0
        for n in range(len(cu) - 1):
            a, b = cu[n], cu[n + 1]
            if b > a:
                num = np.abs(oh[0, a:b] - o_ref[0, a:b]).max(axis=(0, 2))
                den = np.abs(o_ref[0, a:b]).max(axis=(0, 2))
                worst_o = max(worst_o, float((num / np.maximum(den, 1e-30)).max()))
            num = np.abs(fh[n] - f_ref[n]).max(axis=(1, 2))
            den = np.abs(f_ref[n]).max(axis=(1, 2))
            worst_s = max(worst_s, float((num / np.maximum(den, 1e-30)).max()))
        print(f"    worst per-(sequence, head): out {worst_o:.3e}, state {worst_s:.3e}", flush=True)
        assert worst_o <= TOL and worst_s <= TOL
