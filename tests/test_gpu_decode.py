"""GPU parity of the decode step (kda_decode through the C ABI) against the fp64 oracle.

A decode step is the recurrence's single-token step, so the oracle is its
forward pass over one token per sequence (cu_seqlens = 0, 1, ..., N) from the
same start states; chained steps compare with the oracle over as many tokens.
Bar: max|x - x_ref| / max|x_ref| <= 1e-2 for the outputs and the updated states.
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


def step_inputs(N, H, seed, T=1, state="fp32", D=128):
    """T tokens for each of N sequences, packed as [N, T, H, .] rows, and start states."""
    x = random_inputs(N, T, H, D, D, seed=seed, device=DEV, init_state=state)
    return x


def oracle_steps(x):
    """Oracle over the T tokens of each of the N sequences (batch rows)."""
    o, S = oracle.fwd(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), x["g"].cpu(), x["beta"].cpu(),
                      x["scale"], x["initial_state"].cpu(), col_block=16)
    return o, S


@pytest.mark.parametrize("D", [128, 64, 256])
@pytest.mark.parametrize("state", ["fp32", "bf16"])
def test_decode_single_step(state, D):
    N, H = 12, 4
    announce(f"decode single step N={N} H={H} state={state} d={D}")
    x = step_inputs(N, H, seed=40, state=state, D=D)
    o_ref, S_ref = oracle_steps(x)
    S = x["initial_state"].clone()
    out = binding.decode(x["q"][:, 0].contiguous(), x["k"][:, 0].contiguous(),
                         x["v"][:, 0].contiguous(), x["g"][:, 0].contiguous(),
                         x["beta"][:, 0].contiguous(), S, scale=x["scale"])
    torch.cuda.synchronize()
    e_o = rel_err(host(out), o_ref[:, 0])
    e_s = rel_err(host(S), S_ref)
    print(f"    out rel err {e_o:.3e}, state rel err {e_s:.3e}", flush=True)
    assert e_o <= TOL and e_s <= TOL


@pytest.mark.parametrize("D", [128, 64, 256])
def test_decode_chained_steps(D):
    N, H, T = 6, 3, 24
    announce(f"decode {T} chained steps N={N} H={H} d={D}")
    x = step_inputs(N, H, seed=41, T=T, D=D)
    o_ref, S_ref = oracle_steps(x)
    S = x["initial_state"].clone()
    outs = []
    for t in range(T):
        sl = lambda a: a[:, t].contiguous()  # noqa: E731
        outs.append(binding.decode(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["g"]), sl(x["beta"]),
                                   S, scale=x["scale"]))
    torch.cuda.synchronize()
    out = torch.stack(outs, dim=1)
    e_o = rel_err(host(out), o_ref)
    e_s = rel_err(host(S), S_ref)
    print(f"    out rel err {e_o:.3e}, state rel err {e_s:.3e}", flush=True)
    assert e_o <= TOL and e_s <= TOL


def test_decode_state_indices_and_skip():
    N, H, slots = 5, 2, 9
    announce(f"decode with slot indices N={N} slots={slots}")
    x = step_inputs(N, H, seed=42)
    o_ref, S_ref = oracle_steps(x)
    gen = torch.Generator().manual_seed(43)
    pool = (0.02 * torch.randn(slots, H, 128, 128, generator=gen)).to(DEV)
    idx = torch.tensor([7, 2, -1, 0, 5], dtype=torch.int32, device=DEV)
    for n in range(N):
        if idx[n] >= 0:
            pool[int(idx[n])] = x["initial_state"][n]
    before = pool.clone()
    out = torch.full((N, H, 128), 3.0, dtype=torch.bfloat16, device=DEV)
    binding.decode(x["q"][:, 0].contiguous(), x["k"][:, 0].contiguous(), x["v"][:, 0].contiguous(),
                   x["g"][:, 0].contiguous(), x["beta"][:, 0].contiguous(), pool,
                   scale=x["scale"], state_indices=idx, out=out)
    torch.cuda.synchronize()
    for n in range(N):
        s = int(idx[n])
        if s < 0:
            assert torch.all(out[n] == 3.0), "a skipped sequence's output row is untouched"
            continue
        assert rel_err(host(out[n]), o_ref[n, 0]) <= TOL
        assert rel_err(host(pool[s]), S_ref[n]) <= TOL
    untouched = [s for s in range(slots) if s not in [int(i) for i in idx if i >= 0]]
    assert torch.equal(pool[untouched], before[untouched])


@pytest.mark.parametrize("D", [128, 64, 256])
def test_decode_continues_a_prefill(D):
    """kda_fwd over T tokens, then kda_decode of token T+1 == kda_fwd over T+1 tokens."""
    H, T = 4, 300
    announce(f"prefill {T} tokens then decode one, H={H} d={D}")
    x = random_inputs(1, T + 1, H, D, D, seed=44, device=DEV, init_state="fp32")
    pre = {k: x[k][:, :T].contiguous() for k in ("q", "k", "v", "g", "beta")}
    _, S = binding.fwd(pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], x["scale"],
                       initial_state=x["initial_state"], output_final_state=True)
    last = lambda a: a[:, T].contiguous()  # noqa: E731
    out = binding.decode(last(x["q"]), last(x["k"]), last(x["v"]), last(x["g"]), last(x["beta"]),
                         S, scale=x["scale"])
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.fwd(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), x["g"].cpu(),
                              x["beta"].cpu(), x["scale"], x["initial_state"].cpu(), col_block=16)
    e_o = rel_err(host(out), o_ref[:, T])
    e_s = rel_err(host(S), S_ref)
    print(f"    out rel err {e_o:.3e}, state rel err {e_s:.3e}", flush=True)
    assert e_o <= TOL and e_s <= TOL


def test_decode_zero_sequences_is_a_noop():
    x = torch.zeros(0, 2, 128, dtype=torch.bfloat16, device=DEV)
    S = torch.zeros(1, 2, 128, 128, device=DEV)
    out = binding.decode(x, x, x, x.float(), torch.zeros(0, 2, device=DEV), S)
    assert out.shape == (0, 2, 128)
