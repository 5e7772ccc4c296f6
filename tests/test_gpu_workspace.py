"""GPU tests of the workspaces the library keeps between calls (one per stream):
calls on several streams, queued back to back without host synchronisation,
with sizes that make a kept buffer grow and with more streams than kept
buffers, give the same bytes as the same calls run one at a time with the kept
buffers released in between; a call after kda_release_workspaces still runs.
The kernels are deterministic (a repeated call is bit-identical), so any
overlap of two calls on one buffer would show as a difference.
"""
import sys

import pytest
import torch

from linear_attention_kda_amd import binding
from linear_attention_kda_amd.workloads import random_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"


def announce(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _gpu_required():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    binding.load_library()


def fwd(x, out, final):
    binding.fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["scale"],
                initial_state=x["initial_state"], final_state=final, out=out)


# (T, H, seed): every case splits its sequence (a workspace is taken), and the
# sizes rise and fall so that kept buffers are reused and grown.
CASES = [(4096, 4, 31), (8192, 8, 32), (2048, 4, 33), (8192, 4, 34), (4096, 8, 35)]


def test_kept_workspaces_two_streams_match_serial_calls():
    announce("kept workspaces: two streams back to back vs serial calls")
    xs = [random_inputs(1, T, H, seed=s, device=DEV, init_state="fp32") for T, H, s in CASES]
    for T, H, _ in CASES:
        assert binding.plan(1, T, H)[2] > 0, "case must take a workspace"

    def buffers():
        return [(torch.empty_like(x["v"]),
                 torch.empty(1, x["q"].shape[2], 128, 128, dtype=torch.float32, device=DEV))
                for x in xs]

    # serial reference: one call at a time, kept buffers released in between
    ref = buffers()
    for x, (o, f) in zip(xs, ref):
        fwd(x, o, f)
        torch.cuda.synchronize()
        binding.release_workspaces()

    # two streams, no host synchronisation between the calls, repeated twice
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(2):
        got = buffers()
        torch.cuda.synchronize()
        for i, (x, (o, f)) in enumerate(zip(xs, got)):
            with torch.cuda.stream(streams[(i + rep) % 2]):
                fwd(x, o, f)
        torch.cuda.synchronize()
        for i, ((o, f), (ro, rf)) in enumerate(zip(got, ref)):
            assert torch.equal(o, ro), f"rep {rep} case {CASES[i]}: output differs"
            assert torch.equal(f, rf), f"rep {rep} case {CASES[i]}: final state differs"

    # after a release the next call allocates again
    binding.release_workspaces()
    o, f = buffers()[0]
    fwd(xs[0], o, f)
    torch.cuda.synchronize()
    assert torch.equal(o, ref[0][0]) and torch.equal(f, ref[0][1])


def test_more_streams_than_kept_buffers():
    announce("kept workspaces: six streams, four kept buffers")
    x = random_inputs(1, 4096, 4, seed=36, device=DEV, init_state="fp32")
    ref_o = torch.empty_like(x["v"])
    ref_f = torch.empty(1, 4, 128, 128, dtype=torch.float32, device=DEV)
    fwd(x, ref_o, ref_f)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(6)]
    outs = [(torch.empty_like(ref_o), torch.empty_like(ref_f)) for _ in range(12)]
    torch.cuda.synchronize()
    for i, (o, f) in enumerate(outs):
        with torch.cuda.stream(streams[i % 6]):
            fwd(x, o, f)
    torch.cuda.synchronize()
    for i, (o, f) in enumerate(outs):
        assert torch.equal(o, ref_o) and torch.equal(f, ref_f), f"call {i} differs"


def test_kept_workspace_shared_by_forward_and_backward():
    announce("kept workspaces: backward on one stream beside a forward on another")
    x = random_inputs(1, 1024, 2, seed=41, device=DEV, init_state="fp32")
    xf = random_inputs(1, 4096, 4, seed=42, device=DEV, init_state="fp32")
    gen = torch.Generator(device=DEV)
    gen.manual_seed(43)
    do = torch.randn(x["v"].shape, generator=gen, device=DEV).to(torch.bfloat16)

    def bwd():
        return binding.bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], do, x["scale"],
                           initial_state=x["initial_state"])

    ref_b = bwd()
    ref_o = torch.empty_like(xf["v"])
    ref_f = torch.empty(1, 4, 128, 128, dtype=torch.float32, device=DEV)
    fwd(xf, ref_o, ref_f)
    torch.cuda.synchronize()
    binding.release_workspaces()

    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    o = torch.empty_like(xf["v"])
    f = torch.empty_like(ref_f)
    with torch.cuda.stream(s1):
        got_b = bwd()
    with torch.cuda.stream(s2):
        fwd(xf, o, f)
    torch.cuda.synchronize()
    for k in ("dq", "dk", "dv", "dg", "dbeta"):
        assert torch.equal(got_b[k], ref_b[k]), f"{k} differs"
    assert torch.equal(o, ref_o) and torch.equal(f, ref_f)
