"""kda_fwd_noalloc (the entry point that allocates nothing) against kda_fwd.

Two calls in a row through the C ABI, the second on a smaller input, each
compared with kda_fwd on the same inputs to the parity bar (1e-2 relative for
the output and the final state).  The first call is the 4 x 32K continuation
workload (fp32 states): its segment plan is bound by the static scratch, so
it runs with longer segments than kda_fwd picks.  The second, a small varlen
call that splits its sequences, fits the scratch as kda_fwd's plan does, so the
two entry points run the same kernels on the same plan and agree bit for bit.
Both entry points are also checked against the fp64 oracle (two seeded heads
of the large call, every head of the small ones).  Head dimension 64 takes the
records path from the scratch; a head-256 call whose records exceed the
scratch is rejected before any launch.
"""
import sys

import numpy as np
import pytest
import torch

from linear_attention_kda_amd import binding
from linear_attention_kda_amd.workloads import make_inputs, random_inputs, sample_heads
from oracle import oracle

pytestmark = pytest.mark.gpu

TOL = 1e-2
DEV = "cuda"
ERR_WORKSPACE = -9


def announce(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def rel_err(x, ref):
    x = x.detach().double().cpu().numpy()
    ref = ref.detach().double().cpu().numpy()
    den = np.abs(ref).max()
    num = np.abs(x - ref).max()
    return num if den == 0.0 else num / den


@pytest.fixture(autouse=True)
def _gpu_required(monkeypatch):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    for var in ("KDA_VSPLIT", "KDA_SEQSPLIT", "KDA_SEG_MIN"):
        monkeypatch.delenv(var, raising=False)
    binding.load_library()


def run(fn, x, final_dtype):
    N = (x["cu_seqlens"].numel() - 1) if x["cu_seqlens"] is not None else x["q"].shape[0]
    H, d = x["q"].shape[2], x["q"].shape[3]
    fin = torch.empty(N, H, d, d, dtype=final_dtype, device=DEV)
    out = fn(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"],
             initial_state=x["initial_state"], final_state=fin, cu_seqlens=x["cu_seqlens"])
    torch.cuda.synchronize()
    return out[0], fin


def oracle_err(x, o, f, heads):
    """Worst of the output and final-state errors against the oracle on `heads`."""
    sel = (lambda t: t) if heads is None else (lambda t: t[:, :, heads])  # noqa: E731
    selS = (lambda t: t) if heads is None else (lambda t: t[:, heads])  # noqa: E731
    init = x["initial_state"]
    cu = x["cu_seqlens"]
    o_ref, s_ref = oracle.fwd(sel(x["q"]).cpu(), sel(x["k"]).cpu(), sel(x["v"]).cpu(),
                              sel(x["g"]).cpu(), sel(x["beta"]).cpu(), x["scale"],
                              None if init is None else selS(init).cpu(),
                              cu_seqlens=None if cu is None else cu.cpu(), col_block=16)
    err = lambda a, r: np.abs(a - r).max() / max(np.abs(r).max(), 1e-30)  # noqa: E731
    return max(err(sel(o).double().cpu().numpy(), o_ref), err(selS(f).double().cpu().numpy(), s_ref))


def compare(x, final_dtype, label, heads=None):
    o_ref, f_ref = run(binding.fwd, x, final_dtype)
    o, f = run(binding.fwd_noalloc, x, final_dtype)
    e_o, e_s = rel_err(o, o_ref), rel_err(f, f_ref)
    same = torch.equal(o, o_ref) and torch.equal(f, f_ref)
    e_a, e_b = oracle_err(x, o_ref, f_ref, heads), oracle_err(x, o, f, heads)
    print(f"    {label}: vs kda_fwd out rel err {e_o:.3e}, state rel err {e_s:.3e}, "
          f"bit-identical {same}; vs oracle kda_fwd {e_a:.3e}, kda_fwd_noalloc {e_b:.3e}",
          flush=True)
    assert e_o <= TOL and e_s <= TOL
    assert e_a <= TOL and e_b <= TOL
    return same


def test_noalloc_matches_kda_fwd_two_calls():
    free0 = torch.cuda.mem_get_info()[0]
    announce("no-alloc call 1: 4 x 32K continuation workload, H=32, fp32 states")
    x = make_inputs(3, DEV)
    binding.plan(4, 32768, 32)  # library loaded; the plan of kda_fwd splits this workload
    compare(x, torch.float32, "call 1", heads=sample_heads(3, 2))
    free1 = torch.cuda.mem_get_info()[0]
    print(f"    device memory free before / after the first calls: {free0 / 2**20:.0f} / "
          f"{free1 / 2**20:.0f} MiB", flush=True)
    del x
    announce("no-alloc call 2: varlen [1500, 40, 900, 0, 333], H=4, bf16 states")
    lengths = [1500, 40, 900, 0, 333]
    x = random_inputs(1, sum(lengths), 4, seed=77, device=DEV, init_state="bf16", lengths=lengths)
    assert binding.plan(len(lengths), sum(lengths), 4, varlen=True)[2] > 0
    assert compare(x, torch.bfloat16, "call 2"), "same plan, same kernels: bit-identical"


def test_noalloc_head_dim_64_and_rejection():
    announce("no-alloc d=64: varlen [700, 64, 1], H=3, fp32 states")
    lengths = [700, 64, 1]
    x = random_inputs(1, sum(lengths), 3, 64, 64, seed=78, device=DEV, init_state="fp32",
                      lengths=lengths)
    assert compare(x, torch.float32, "d=64"), "same kernels on the same records: bit-identical"
    announce("no-alloc d=256: records beyond the static scratch are rejected")
    x = random_inputs(1, 8192, 32, 256, 256, seed=79, device=DEV)
    assert binding.dim_workspace_bytes(1, 8192, 32, 256) > (256 << 20)
    out = torch.full_like(x["v"], 7.0)
    with pytest.raises(binding.KdaError) as e:
        binding.fwd_noalloc(x["q"], x["k"], x["v"], x["g"], x["beta"], out=out)
    assert e.value.status == ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "a rejected call touches no output"
