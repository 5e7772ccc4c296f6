"""CPU tests of the C ABI boundary: the library loads, exports what the header
declares, and rejects invalid arguments with the documented status codes
before touching any device (no compute calls without a GPU)."""
import ctypes
import os
import re

import pytest

from linear_attention_kda_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, ERR_NULL, ERR_HEAD_DIM, ERR_VARLEN_BATCH, ERR_STATE_DTYPE, ERR_DTYPE, ERR_SHAPE, ERR_ALIGN = (
    0, -1, -2, -3, -4, -5, -6, -7)

# fake, never dereferenced, 16-byte aligned addresses
P = 0x10000


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(kda_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.library_path()):
        pytest.fail("libkda.so is not built (run python -m linear_attention_kda_amd.build)")
    return binding.load_library()


def test_header_declares_expected_entry_points():
    assert header_functions() == ["kda_bwd", "kda_bwd_check", "kda_bwd_workspace_bytes",
                                  "kda_decode", "kda_decode_check", "kda_dim_workspace_bytes",
                                  "kda_fwd", "kda_fwd_check", "kda_fwd_noalloc",
                                  "kda_gdn_decode", "kda_gdn_decode_check", "kda_gdn_fwd",
                                  "kda_gdn_fwd_check", "kda_last_error", "kda_plan",
                                  "kda_release_workspaces", "kda_status_string"]


def test_library_exports_every_header_symbol(lib):
    cdll = ctypes.CDLL(binding.library_path())
    for name in header_functions():
        assert hasattr(cdll, name), name


def ok_args(**over):
    a = dict(B=1, T=256, H=4, K=128, V=128, q=P, k=P + 0x1000, v=P + 0x2000, g=P + 0x3000,
             beta=P + 0x4000, out=P + 0x5000)
    a.update(over)
    return a


def test_check_accepts_valid_arguments(lib):
    assert binding.fwd_check(**ok_args()) == OK
    assert binding.fwd_check(**ok_args(K=64, V=64)) == OK
    assert binding.fwd_check(**ok_args(K=256, V=256)) == OK
    assert binding.gdn_fwd_check(**ok_args(K=256, V=256, g=P + 4)) == OK
    assert binding.fwd_check(**ok_args(initial_state=P, initial_dtype=0, final_state=P,
                                       final_dtype=0)) == OK
    assert binding.fwd_check(**ok_args(cu_seqlens=P, num_seqs=3)) == OK
    assert binding.fwd_check(**ok_args(T=0, q=0, k=0, v=0, g=0, beta=0, out=0)) == OK


@pytest.mark.parametrize("over,status", [
    (dict(K=64), ERR_HEAD_DIM),
    (dict(V=256), ERR_HEAD_DIM),
    (dict(K=96, V=96), ERR_HEAD_DIM),
    (dict(K=512, V=512), ERR_HEAD_DIM),
    (dict(B=2, cu_seqlens=P, num_seqs=2), ERR_VARLEN_BATCH),
    (dict(cu_seqlens=P, num_seqs=0), ERR_SHAPE),
    (dict(initial_state=P, initial_dtype=0, final_state=P + 64, final_dtype=1), ERR_STATE_DTYPE),
    (dict(initial_state=P, initial_dtype=2), ERR_DTYPE),
    (dict(final_state=P, final_dtype=-1), ERR_DTYPE),
    (dict(B=0), ERR_SHAPE),
    (dict(H=0), ERR_SHAPE),
    (dict(T=-1), ERR_SHAPE),
    (dict(H=32769), ERR_SHAPE),
    (dict(q=0), ERR_NULL),
    (dict(beta=0), ERR_NULL),
    (dict(out=0), ERR_NULL),
    (dict(k=P + 8), ERR_ALIGN),
    (dict(g=P + 4), ERR_ALIGN),
    (dict(beta=P + 2), ERR_ALIGN),
    (dict(initial_state=P + 8, initial_dtype=1), ERR_ALIGN),
])
def test_check_rejections(lib, over, status):
    assert binding.fwd_check(**ok_args(**over)) == status
    assert lib.kda_last_error().decode() != ""
    assert lib.kda_status_string(status).decode() not in ("", "unknown status")


def dec_args(**over):
    a = dict(N=8, H=4, K=128, V=128, q=P, k=P + 0x1000, v=P + 0x2000, g=P + 0x3000,
             beta=P + 0x4000, out=P + 0x5000, state=P + 0x10000, state_dtype=1)
    a.update(over)
    return a


def test_decode_check_accepts_valid_arguments(lib):
    assert binding.decode_check(**dec_args()) == OK
    assert binding.decode_check(**dec_args(K=64, V=64)) == OK
    assert binding.decode_check(**dec_args(K=256, V=256)) == OK
    assert binding.decode_check(**dec_args(state_dtype=0, state_indices=P + 0x8000)) == OK
    assert binding.decode_check(**dec_args(N=0, q=0, k=0, v=0, g=0, beta=0, out=0, state=0)) == OK


@pytest.mark.parametrize("over,status", [
    (dict(K=64), ERR_HEAD_DIM),
    (dict(V=256), ERR_HEAD_DIM),
    (dict(K=96, V=96), ERR_HEAD_DIM),
    (dict(N=-1), ERR_SHAPE),
    (dict(H=0), ERR_SHAPE),
    (dict(state_dtype=2), ERR_DTYPE),
    (dict(state=0), ERR_NULL),
    (dict(q=0), ERR_NULL),
    (dict(out=0), ERR_NULL),
    (dict(v=P + 8), ERR_ALIGN),
    (dict(state=P + 8), ERR_ALIGN),
    (dict(beta=P + 2), ERR_ALIGN),
    (dict(state_indices=P + 2), ERR_ALIGN),
])
def test_decode_check_rejections(lib, over, status):
    assert binding.decode_check(**dec_args(**over)) == status
    assert lib.kda_last_error().decode() != ""


def test_gdn_checks_take_a_scalar_gate(lib):
    """The scalar-gate entry points validate like the KDA ones, except that g holds
    one fp32 per token and head and needs only 4-byte alignment."""
    assert binding.gdn_fwd_check(**ok_args(g=P + 4)) == OK
    assert binding.fwd_check(**ok_args(g=P + 4)) == ERR_ALIGN
    assert binding.gdn_fwd_check(**ok_args(g=P + 2)) == ERR_ALIGN
    assert binding.gdn_fwd_check(**ok_args(K=64)) == ERR_HEAD_DIM
    assert binding.gdn_fwd_check(**ok_args(B=2, cu_seqlens=P, num_seqs=2)) == ERR_VARLEN_BATCH
    assert binding.gdn_fwd_check(**ok_args(g=0)) == ERR_NULL
    assert binding.gdn_decode_check(**dec_args(g=P + 4)) == OK
    assert binding.decode_check(**dec_args(g=P + 4)) == ERR_ALIGN
    assert binding.gdn_decode_check(**dec_args(g=P + 2)) == ERR_ALIGN
    assert binding.gdn_decode_check(**dec_args(state_dtype=2)) == ERR_DTYPE
    assert binding.gdn_decode_check(**dec_args(N=0, q=0, k=0, v=0, g=0, beta=0, out=0, state=0)) == OK


def bwd_args(**over):
    a = dict(B=1, T=256, H=4, K=128, V=128, q=P, k=P + 0x1000, v=P + 0x2000, g=P + 0x3000,
             beta=P + 0x4000, d_out=P + 0x5000, dq=P + 0x6000, dk=P + 0x7000, dv=P + 0x8000,
             dg=P + 0x9000, dbeta=P + 0xa000)
    a.update(over)
    return a


def test_bwd_check(lib):
    assert binding.bwd_check(**bwd_args()) == OK
    assert binding.bwd_check(**bwd_args(initial_state=P, initial_dtype=0, d_final_state=P + 0x100,
                                        d_final_dtype=1, d_initial_state=P + 0x200)) == OK
    assert binding.bwd_check(**bwd_args(cu_seqlens=P, num_seqs=3)) == OK
    assert binding.bwd_check(**bwd_args(T=0, q=0, k=0, v=0, g=0, beta=0, d_out=0, dq=0, dk=0,
                                        dv=0, dg=0, dbeta=0)) == OK
    assert binding.bwd_check(**bwd_args(K=64)) == ERR_HEAD_DIM
    assert binding.bwd_check(**bwd_args(K=64, V=64)) == ERR_HEAD_DIM
    assert binding.bwd_check(**bwd_args(d_out=0)) == ERR_NULL
    assert binding.bwd_check(**bwd_args(dg=0)) == ERR_NULL
    assert binding.bwd_check(**bwd_args(dq=P + 8)) == ERR_ALIGN
    assert binding.bwd_check(**bwd_args(dbeta=P + 2)) == ERR_ALIGN
    assert binding.bwd_check(**bwd_args(d_final_state=P, d_final_dtype=3)) == ERR_DTYPE
    assert binding.bwd_check(**bwd_args(B=2, cu_seqlens=P, num_seqs=2)) == ERR_VARLEN_BATCH


def bwd_ws_formula(N, rows, H, g=None):
    # s = N + ceil(rows / 64) + 1 slots; one group of g slots holds every head's
    # per-chunk tiles, the checkpoints cover every slot, two carries when g < s
    per = (14 * 64 * 128 + 6 * 64 * 64 + 128 * 64 + 2 * 128 * 128 + 64 + 2 * 128 + 1) * 4
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    s = N + (rows + 63) // 64 + 1
    if g is None:
        g = (8 << 30) // (H * per)
    g = max(1, min(g, s))
    return (up(g * H * per) + up(s * H * 128 * 128 * 4) + (up(2 * H * 128 * 128 * 4) if g < s else 0)
            + up(rows * H * 128 * 2))


def test_bwd_workspace_bytes(lib, monkeypatch):
    monkeypatch.delenv("KDA_BWD_GROUP_SLOTS", raising=False)
    assert binding.bwd_workspace_bytes(1, 8192, 32) == bwd_ws_formula(1, 8192, 32)
    assert binding.bwd_workspace_bytes(1, 8192, 32) == 3344007424        # one group
    assert binding.bwd_workspace_bytes(1, 1 << 20, 32) == bwd_ws_formula(1, 1 << 20, 32)
    assert binding.bwd_workspace_bytes(1, 1 << 20, 32) < 52 * 10**9      # 45 groups
    assert binding.bwd_workspace_bytes(16, 65536, 32) == bwd_ws_formula(16, 65536, 32)
    assert binding.bwd_workspace_bytes(0, 8192, 32) == -1
    # the group size knob: read at each call, clamped to [1, slots]
    for g in (1, 7, 130, 10**6):
        monkeypatch.setenv("KDA_BWD_GROUP_SLOTS", str(g))
        assert binding.bwd_workspace_bytes(1, 8192, 32) == bwd_ws_formula(1, 8192, 32, g), g
    monkeypatch.setenv("KDA_BWD_GROUP_SLOTS", "0")   # not >= 1: the default
    assert binding.bwd_workspace_bytes(1, 8192, 32) == bwd_ws_formula(1, 8192, 32)


def test_dim_workspace_bytes(lib):
    # d = 256: one record per (chunk slot, head); slots: N + ceil(rows / 64) + 1.  A
    # record holds kg, qg (64 rows of d + 4 bf16), kp^T (d rows of 68 bf16), three
    # tiles of 64 rows of 68 bf16 and d fp32.  d = 64 runs on the fused kernel: none.
    d = 256
    rec = 2 * 64 * (d + 4) * 2 + d * 68 * 2 + 3 * 64 * 68 * 2 + d * 4
    assert rec == 128512
    assert binding.dim_workspace_bytes(16, 65536, 32, d) == (16 + 1024 + 1) * 32 * rec
    assert binding.dim_workspace_bytes(1, 65, 2, d) == (1 + 2 + 1) * 2 * rec
    assert binding.dim_workspace_bytes(3, 0, 2, d) == 0
    assert binding.dim_workspace_bytes(16, 65536, 32, 64) == 0
    assert binding.dim_workspace_bytes(1, 64, 1, 128) == -1
    assert binding.dim_workspace_bytes(0, 64, 1, 64) == -1


def test_state_dtype_ignored_for_absent_state(lib):
    assert binding.fwd_check(**ok_args(initial_dtype=7)) == OK


def _split_workspace(units, H, emax):
    """Fix-up output blocks (64 x 128 bf16 per unit), then the fp32 segment states,
    maps and end states, then their bf16 fix-up copies, then one int32 per (state
    slot, head): the counter through which the scan publishes each start state."""
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    return (up(units * 64 * 128 * 2) + up(3 * emax * H * 128 * 128 * 4) + up(emax * H * 128 * 128 * 2)
            + up(emax * H * 4))


def test_plan_value_split(lib, monkeypatch):
    monkeypatch.delenv("KDA_SEQSPLIT", raising=False)
    monkeypatch.delenv("KDA_SEG_MIN", raising=False)
    monkeypatch.delenv("KDA_VSPLIT", raising=False)
    # short sequences (4 chunks <= 8): no splitting; fewer (sequence, head) pairs
    # than CUs -> two value slices per pair
    assert binding.plan(1, 256, 32, False, 256) == (64, 2, 0)
    assert binding.plan(16, 256, 32, False, 256) == (512, 1, 0)
    assert binding.plan(4, 256, 32, False, 256) == (256, 2, 0)
    assert binding.plan(3, 256, 3, False, 256) == (32, 2, 0)   # 9 pairs padded to 16, times 2
    # H >= CUs: never split
    assert binding.plan(1, 8192, 256, False, 256) == (256, 1, 0)
    # one 8K sequence (128 chunks), 32 heads: the host evaluates the device's rule,
    # 32 (128 + (128 - M)) <= 0.95 * 256 M  ->  M = 30, i.e. 5 segments: 4 state slots
    # and 98 chunks past the first segment per head (3136 fix-up units); the grid
    # covers the sequence plus two runs per extra segment
    assert binding.plan(1, 8192, 32, False, 256) == ((1 + 8) * 32, 1, _split_workspace(3136, 32, 4))
    # 16 equal sequences of 128 chunks on 256 CUs: 512 pairs already fill the CUs
    assert binding.plan(16, 8192, 32, False, 256) == (512, 1, 0)
    # varlen: the lengths live on the device, so the plan allows splitting with
    # 256/32 + 1 = 9 state slots and a fix-up block for every chunk that could need
    # one (65536 / 64 + 16 chunks per head)
    assert binding.plan(16, 65536, 32, True, 256) == ((16 + 18) * 32, 1,
                                                      _split_workspace(1040 * 32, 32, 9))
    with pytest.raises(binding.KdaError):
        binding.plan(0, 256, 32, False, 256)


def test_plan_split_switches(lib, monkeypatch):
    monkeypatch.setenv("KDA_SEQSPLIT", "0")
    assert binding.plan(1, 8192, 32, False, 256) == (64, 2, 0)
    monkeypatch.delenv("KDA_SEQSPLIT")
    monkeypatch.setenv("KDA_VSPLIT", "2")
    assert binding.plan(1, 8192, 32, False, 256) == (64, 2, 0)
    monkeypatch.delenv("KDA_VSPLIT")
    monkeypatch.setenv("KDA_SEG_MIN", "200")
    assert binding.plan(1, 8192, 32, False, 256) == (64, 2, 0)   # 128 chunks <= 200


def test_binding_rejects_host_tensors(lib):
    import torch
    x = torch.zeros(1, 4, 1, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        binding.fwd(x, x, x, x.float(), torch.zeros(1, 4, 1))


def test_product_path_never_touches_the_oracle():
    """The package (Python and native sources) must not import, load or call oracle/."""
    pkg = os.path.join(ROOT, "linear_attention_kda_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert not re.search(r"(from\s+oracle|import\s+oracle|oracle\.\w+\(|kda_oracle)",
                                     text), f"{f} reaches into oracle/"
    for f in os.listdir(os.path.join(ROOT, "include")):
        assert "oracle" not in open(os.path.join(ROOT, "include", f)).read()
