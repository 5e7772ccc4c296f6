"""Algorithmic traffic and work of the KDA forward pass (for roofline figures).

Bytes are the compulsory HBM traffic of one forward pass: every input read
once and every output written once, nothing else.  Per (token, head):
q, k, v and o in bf16 (4 x 128 x 2 B), g in fp32 (128 x 4 B) and beta in fp32
(4 B): 1540 B.  With the scalar gate (Gated DeltaNet) g is one fp32 per token
and head: 1032 B.  Per (sequence, head) state: 128 x 128 elements read if an
initial state is given and written if a final state is wanted.

Work follows the pages' cost model for one head,
6 T d^2 + 3 T C d + T C^2 FLOPs [core.today "Kimi Linear 특집", ch.4,
"연산량 비교" (cost comparison)], with d = 128 and C = 64.
"""
from __future__ import annotations

D = 128
C = 64
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s


def bytes_per_token_head(d: int = D, scalar_gate: bool = False) -> int:
    return 4 * d * 2 + (4 if scalar_gate else d * 4) + 4


def flops_per_head(T: int, d: int = D, chunk: int = C) -> float:
    return 6.0 * T * d * d + 3.0 * T * chunk * d + T * chunk * chunk


def state_bytes(n_states: int, H: int, dtype_bytes: int, d: int = D) -> int:
    return n_states * H * d * d * dtype_bytes


def workload_bytes(tokens: int, H: int, n_states: int, init_bytes: int | None,
                   final_bytes: int | None, scalar_gate: bool = False, d: int = D) -> int:
    """Compulsory bytes of one pass over `tokens` packed tokens with H heads of size d."""
    b = tokens * H * bytes_per_token_head(d, scalar_gate=scalar_gate)
    if init_bytes:
        b += state_bytes(n_states, H, init_bytes, d)
    if final_bytes:
        b += state_bytes(n_states, H, final_bytes, d)
    return b


def workload_flops(tokens: int, H: int) -> float:
    return H * flops_per_head(tokens)
