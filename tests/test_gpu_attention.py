"""Causal attention with the algebraic score (appendix G) on the GPU against the fp64 oracle.

Bar: relative Frobenius error of each head's output <= 5e-3 (bf16).  The kernel
rounds P to bf16 for the value product (<= 2^-9 relative per weight) and O once;
scores and softmax statistics are fp32.  Bitwise run-to-run reproducible.
"""
import numpy as np
import pytest

import gemm_qalg_forward_amd as Q
import synth
from gpu_common import say, to_dev, to_f64, torch_cuda
from oracle import qalg_oracle as O
from qalg_check import BF16_TOL

pytestmark = pytest.mark.gpu

ATTN_SHAPES = [
    # Hq, Hkv, S, d, q, L
    (4, 4, 256, 128, 4, 0),
    (8, 2, 300, 128, 8, 0),     # GQA, ragged S (300 = 8 * 37 + 4)
    (2, 2, 1000, 64, 4, 0),
    (4, 1, 513, 128, 1, 0),     # q = 1: ordinary causal attention
    (2, 2, 777, 128, 4, 2),     # the recursive law Q_2^(x)2
    (2, 2, 64, 64, 2, 1),       # L = 1 is Q_2
    (3, 3, 1, 128, 4, 0),       # one position
    (2, 1, 129, 64, 4, 0),
]


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.mark.parametrize("shape", ATTN_SHAPES, ids=[f"H{s[0]}kv{s[1]}S{s[2]}d{s[3]}q{s[4]}L{s[5]}" for s in ATTN_SHAPES])
def test_attention_forward_matches_oracle(shape):
    torch = torch_cuda()
    Hq, Hkv, S, d, q, L = shape
    say(f"[attn] Hq={Hq} Hkv={Hkv} S={S} d={d} q={q} L={L}")
    Qo = synth.normal_operand(9600 + S, (Hq, S, d), 1.0, "bf16")
    Ko = synth.normal_operand(9700 + S, (Hkv, S, d), 1.0, "bf16")
    Vo = synth.normal_operand(9800 + S, (Hkv, S, d), 1.0, "bf16")
    flags = Q.QALG_FLAG_LAW_TENSOR if L else 0
    Qd, Kd, Vd = to_dev(Qo), to_dev(Ko), to_dev(Vo)
    Og = Q.qalg_attention_forward(Qd, Kd, Vd, q, flags=flags)
    Og2 = Q.qalg_attention_forward(Qd, Kd, Vd, q, flags=flags)
    torch.cuda.synchronize()
    assert torch.equal(Og, Og2), "not bitwise reproducible"
    tau = np.arange(S) % q
    Or = O.algebraic_attention(Qo.f64, Ko.f64, Vo.f64, tau, q, L)
    got = to_f64(Og)
    errs = [_rel(got[h], Or[h]) for h in range(Hq)]
    say(f"    max rel err over heads {max(errs):.2e}")
    assert max(errs) <= BF16_TOL, errs
