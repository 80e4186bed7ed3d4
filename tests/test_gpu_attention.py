"""Causal attention with the algebraic score (appendix G) on the GPU against the fp64 oracle:
the prefill forward, the cached decode, and the gradients.

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


OFFSET_SHAPES = [
    # Hq, Hkv, S, d, q, L, first position
    (4, 2, 300, 128, 4, 0, 5),
    (2, 2, 257, 64, 4, 0, 4099),
    (2, 1, 200, 128, 4, 2, 3),     # the recursive law at an offset
    (2, 2, 37, 128, 4, 0, 2),
    (2, 2, 100, 128, 1, 0, 7),     # q = 1: the offset changes nothing
]


@pytest.mark.parametrize("shape", OFFSET_SHAPES, ids=[f"H{s[0]}kv{s[1]}S{s[2]}d{s[3]}q{s[4]}L{s[5]}p{s[6]}" for s in OFFSET_SHAPES])
def test_attention_forward_at_offset_matches_oracle(shape):
    """A prefill chunk whose first row sits at absolute position p0: types (p0 + s) mod q."""
    torch = torch_cuda()
    Hq, Hkv, S, d, q, L, p0 = shape
    say(f"[attn offset] Hq={Hq} Hkv={Hkv} S={S} d={d} q={q} L={L} p0={p0}")
    Qo = synth.normal_operand(9610 + S, (Hq, S, d), 1.0, "bf16")
    Ko = synth.normal_operand(9710 + S, (Hkv, S, d), 1.0, "bf16")
    Vo = synth.normal_operand(9810 + S, (Hkv, S, d), 1.0, "bf16")
    flags = Q.QALG_FLAG_LAW_TENSOR if L else 0
    Qd, Kd, Vd = to_dev(Qo), to_dev(Ko), to_dev(Vo)
    Og = Q.qalg_attention_forward_at(Qd, Kd, Vd, q, p0, flags=flags)
    Og2 = Q.qalg_attention_forward_at(Qd, Kd, Vd, q, p0, flags=flags)
    torch.cuda.synchronize()
    assert torch.equal(Og, Og2), "not bitwise reproducible"
    pos = p0 + np.arange(S)
    Or = O.algebraic_attention(Qo.f64, Ko.f64, Vo.f64, pos % q, q, L, positions=pos)
    got = to_f64(Og)
    errs = [_rel(got[h], Or[h]) for h in range(Hq)]
    say(f"    max rel err over heads {max(errs):.2e}")
    assert max(errs) <= BF16_TOL, errs
    if q > 1 and p0 % q:
        # the offset changes the pairs: not the zero-offset result
        O0 = to_f64(Q.qalg_attention_forward(Qd, Kd, Vd, q, flags=flags))
        assert not np.allclose(O0, got)


def _decode_case(B, Hq, Hkv, N, d, q, L, kind, period, lens, p0s, seed, holes=0, future=0):
    """Caches of N slots: sequence b holds positions p0s[b] .. p0s[b] + lens[b] - 1 in a shuffled slot
    order, `holes` of them emptied (-1) and `future` positions after the query added; the new row
    sits at the last position p0s[b] + lens[b] - 1."""
    g = np.random.Generator(np.random.PCG64(seed))
    key_pos = np.full((B, N), -1, np.int64)
    q_pos = np.zeros(B, np.int64)
    for b in range(B):
        n = lens[b]
        pos = p0s[b] + np.arange(n)
        q_pos[b] = pos[-1]
        slots = g.permutation(N)[:n]
        key_pos[b, slots] = pos
        free = np.setdiff1d(np.arange(N), slots)
        if holes and n > 1:
            key_pos[b, g.choice(slots, size=min(holes, n - 1), replace=False)] = -1
        if future and free.size:
            key_pos[b, free[:future]] = q_pos[b] + 1 + np.arange(min(future, free.size))
    Qo = synth.normal_operand(seed + 1, (B, Hq, d), 1.0, "bf16")
    Ko = synth.normal_operand(seed + 2, (B, Hkv, N, d), 1.0, "bf16")
    Vo = synth.normal_operand(seed + 3, (B, Hkv, N, d), 1.0, "bf16")
    return Qo, Ko, Vo, q_pos, key_pos


DECODE_CASES = [
    # B, Hq, Hkv, N, d, q, L, kind, period, lens, first positions, holes, future keys
    (2, 4, 1, 1, 128, 4, 0, 0, 0, [1, 1], [3, 6], 0, 0),                 # S = 1: one cached key
    (3, 8, 2, 37, 128, 4, 0, 0, 0, [37, 20, 5], [5, 0, 101], 3, 2),     # S = 37, offsets, holes, future keys
    (2, 32, 8, 4096, 128, 4, 0, 0, 0, [4096, 3000], [3, 17], 0, 0),     # S = 4096 (several chunks), GQA 4
    (2, 8, 1, 700, 64, 8, 0, 0, 0, [700, 513], [1, 9], 5, 3),           # d = 64, q = 8, GQA 8
    (2, 4, 2, 300, 128, 4, 2, 0, 0, [300, 299], [2, 7], 4, 0),          # the recursive law
    (2, 4, 4, 600, 128, 4, 0, 1, 768, [600, 450], [100, 700], 0, 1),    # the interval schedule
    (1, 4, 4, 512, 128, 1, 0, 0, 0, [512], [0], 0, 0),                  # q = 1: ordinary decode
    (2, 2, 2, 260, 128, 16, 0, 0, 0, [260, 3], [1, 2], 2, 0),           # q = 16 (groups of 8 features)
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[f"B{c[0]}H{c[1]}kv{c[2]}N{c[3]}d{c[4]}q{c[5]}L{c[6]}k{c[7]}"
                                                    for c in DECODE_CASES])
def test_attention_decode_matches_oracle(case):
    torch = torch_cuda()
    B, Hq, Hkv, N, d, q, L, kind, period, lens, p0s, holes, future = case
    say(f"[decode] B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} q={q} L={L} kind={kind} lens={lens} p0={p0s}")
    Qo, Ko, Vo, q_pos, key_pos = _decode_case(B, Hq, Hkv, N, d, q, L, kind, period, lens, p0s, 9950 + N + q,
                                              holes, future)
    Qd, Kd, Vd = to_dev(Qo), to_dev(Ko), to_dev(Vo)
    qp, kp = torch.from_numpy(q_pos).to("cuda"), torch.from_numpy(key_pos).to("cuda")
    flags = Q.QALG_FLAG_LAW_TENSOR if L else 0
    Og = Q.qalg_attention_decode(Qd, Kd, Vd, qp, kp, q, kind, period, flags=flags)
    Og2 = Q.qalg_attention_decode(Qd, Kd, Vd, qp, kp, q, kind, period, flags=flags)
    torch.cuda.synchronize()
    assert torch.equal(Og, Og2), "not bitwise reproducible"
    sched = "cyclic" if kind == 0 else "interval"
    Or = O.algebraic_attention_decode(Qo.f64, Ko.f64, Vo.f64, q_pos, key_pos, q, L, sched, period)
    got = to_f64(Og)
    errs = [_rel(got[b, h], Or[b, h]) for b in range(B) for h in range(Hq)]
    say(f"    max rel err over rows {max(errs):.2e}")
    assert max(errs) <= BF16_TOL, errs


def test_attention_decode_empty_rows_are_zero():
    """A new row with no allowed cached slot (all empty, or all after it) gets a zero output."""
    torch = torch_cuda()
    B, Hq, Hkv, N, d, q = 3, 4, 2, 300, 128, 4
    Qo, Ko, Vo, _, _ = _decode_case(B, Hq, Hkv, N, d, q, 0, 0, 0, [1, 1, 1], [0, 0, 0], 9990)
    key_pos = np.full((B, N), -1, np.int64)
    key_pos[1, 10:20] = 50 + np.arange(10)   # every key after the query
    key_pos[2, 5] = 7                        # one allowed key
    q_pos = np.array([9, 9, 9], np.int64)
    Og = Q.qalg_attention_decode(to_dev(Qo), to_dev(Ko), to_dev(Vo), torch.from_numpy(q_pos).to("cuda"),
                                 torch.from_numpy(key_pos).to("cuda"), q)
    torch.cuda.synchronize()
    got = to_f64(Og)
    assert not got[0].any() and not got[1].any()
    Or = O.algebraic_attention_decode(Qo.f64, Ko.f64, Vo.f64, q_pos, key_pos, q)
    assert _rel(got[2], Or[2]) <= BF16_TOL


BWD_SHAPES = [
    # Hq, Hkv, S, d, q, L, first position
    (4, 2, 300, 128, 4, 0, 0),     # GQA 2, ragged S (several 64-row blocks per type, a partial one)
    (2, 2, 257, 64, 4, 0, 5),      # d = 64 at an offset
    (2, 1, 200, 128, 4, 2, 3),     # the recursive law Q_2^(x)2 at an offset, GQA 2
    (4, 4, 390, 128, 8, 0, 0),     # q = 8: groups of 16 features, half a 32-feature block
    (2, 2, 160, 128, 2, 1, 1),     # L = 1 is Q_2
    (2, 2, 100, 128, 1, 0, 0),     # q = 1: ordinary causal attention
    (3, 3, 1, 128, 4, 0, 0),       # one position
    (8, 2, 1100, 128, 4, 0, 2),    # GQA 4, more than one 128-key block per type
]


@pytest.mark.parametrize("shape", BWD_SHAPES, ids=[f"H{s[0]}kv{s[1]}S{s[2]}d{s[3]}q{s[4]}L{s[5]}p{s[6]}" for s in BWD_SHAPES])
def test_attention_backward_matches_oracle(shape):
    """Algorithm 2, step 9 on the GPU (the training forward's O and lse, then dQ, dK, dV) against the
    oracle's fp64 gradients on the same bf16 inputs.  Bar: relative Frobenius error of each head's
    gradient <= 5e-3 (BF16_TOL).  Each gradient is an fp32 sum of products in which one factor was
    rounded to bf16 (P for dV; dS for dQ and dK, whose own error adds the rounding of O in
    D = <dO, O>), i.e. relative errors of at most 2^-9 per term that do not line up in sign; the
    measured errors (2.3e-3 to 2.8e-3) are printed by the test.  Where the exact gradient is zero
    (one position: the softmax over one key is constant, so dQ = dK = 0), the bar is an absolute
    1e-3 on the largest element (the GPU leaves the fp32 rounding of dP - D)."""
    torch = torch_cuda()
    Hq, Hkv, S, d, q, L, p0 = shape
    say(f"[attn bwd] Hq={Hq} Hkv={Hkv} S={S} d={d} q={q} L={L} p0={p0}")
    Qo = synth.normal_operand(9620 + S, (Hq, S, d), 1.0, "bf16")
    Ko = synth.normal_operand(9720 + S, (Hkv, S, d), 1.0, "bf16")
    Vo = synth.normal_operand(9820 + S, (Hkv, S, d), 1.0, "bf16")
    dOo = synth.normal_operand(9920 + S, (Hq, S, d), 1.0, "bf16")
    flags = Q.QALG_FLAG_LAW_TENSOR if L else 0
    Qd, Kd, Vd, dOd = to_dev(Qo), to_dev(Ko), to_dev(Vo), to_dev(dOo)
    Og, lse = Q.qalg_attention_forward_train(Qd, Kd, Vd, q, p0, flags=flags)
    Oa = Q.qalg_attention_forward_at(Qd, Kd, Vd, q, p0, flags=flags)
    g1 = Q.qalg_attention_backward(Qd, Kd, Vd, Og, dOd, lse, q, p0, flags=flags)
    g2 = Q.qalg_attention_backward(Qd, Kd, Vd, Og, dOd, lse, q, p0, flags=flags)
    torch.cuda.synchronize()
    assert torch.equal(Og, Oa), "the training forward's O differs from the forward's"
    for a, b in zip(g1, g2):
        assert torch.equal(a, b), "not bitwise reproducible"
    pos = p0 + np.arange(S)
    want = O.algebraic_attention_backward(Qo.f64, Ko.f64, Vo.f64, dOo.f64, pos % q, q, L, positions=pos)
    worst = {}
    for name, got, ref in zip(("dQ", "dK", "dV"), g1, want):
        got = to_f64(got)
        assert np.isfinite(got).all(), name
        errs = []
        for h in range(ref.shape[0]):
            if np.linalg.norm(ref[h]) == 0.0:
                assert np.abs(got[h]).max() <= 1e-3, (name, h, np.abs(got[h]).max())
            else:
                errs.append(_rel(got[h], ref[h]))
        worst[name] = max(errs, default=0.0)
    say("    max rel err over heads " + ", ".join(f"{k} {v:.2e}" for k, v in worst.items()))
    assert max(worst.values()) <= BF16_TOL, worst


def test_attention_backward_full_size_one_group():
    """The bench's attention shape (32 query heads over 8 key/value heads, S = 4096, d = 128, q = 4):
    the GPU computes every head; the oracle recomputes the gradients of key/value head 0 and of the
    4 query heads that read it (which depend on nothing else), whole, to the same bar."""
    torch = torch_cuda()
    Hq, Hkv, S, d, q = 32, 8, 4096, 128, 4
    say(f"[attn bwd full] Hq={Hq} Hkv={Hkv} S={S} d={d} q={q}")
    Qo = synth.normal_operand(9631, (Hq, S, d), 1.0, "bf16")
    Ko = synth.normal_operand(9731, (Hkv, S, d), 1.0, "bf16")
    Vo = synth.normal_operand(9831, (Hkv, S, d), 1.0, "bf16")
    dOo = synth.normal_operand(9931, (Hq, S, d), 1.0, "bf16")
    Qd, Kd, Vd, dOd = to_dev(Qo), to_dev(Ko), to_dev(Vo), to_dev(dOo)
    Og, lse = Q.qalg_attention_forward_train(Qd, Kd, Vd, q)
    dQ, dK, dV = Q.qalg_attention_backward(Qd, Kd, Vd, Og, dOd, lse, q)
    torch.cuda.synchronize()
    G = Hq // Hkv
    tau = np.arange(S) % q
    want = O.algebraic_attention_backward(Qo.f64[:G], Ko.f64[:1], Vo.f64[:1], dOo.f64[:G], tau, q)
    worst = {}
    for name, got, ref in zip(("dQ", "dK", "dV"), (to_f64(dQ)[:G], to_f64(dK)[:1], to_f64(dV)[:1]), want):
        worst[name] = max(_rel(got[h], ref[h]) for h in range(ref.shape[0]))
    say("    max rel err over heads " + ", ".join(f"{k} {v:.2e}" for k, v in worst.items()))
    assert max(worst.values()) <= BF16_TOL, worst
