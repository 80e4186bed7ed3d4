"""Planted mistakes in the oracle (on the CPU) must each trip at least one pin.

Each mutant replaces one oracle function with a plausibly wrong version (a
dropped term, a wrong index, a transposed operand, a sign flip, an unstable
index) for the duration of one test; the pins of oracle_pins.py then run and
at least one of them has to fail.
"""
import numpy as np
import pytest

from oracle import qalg_oracle as O
from oracle_pins import ALL_PINS

_real_table = O.structure_table
_real_fwd = O.row_typed_forward
_real_bwd = O.row_typed_backward
_real_index = O.type_index
_real_silu = O.silu
_real_gated = O.gated_forward
_real_silu_grad = O.silu_grad
_real_tensor = O.tensor_power_table
_real_attn = O.algebraic_attention
_real_support = O.score_support
_real_swiglu_bwd = O.swiglu_backward
_real_decode = O.algebraic_attention_decode
_real_decode_macs = O.attention_decode_macs
_real_attn_bwd = O.algebraic_attention_backward


def table_with_edge_edge(q, edges=None):
    """Mistake: keeps edge*edge products (this is ordinary block matmul)."""
    t = list(_real_table(q, edges))
    slots = O.graph_slots(q, edges)
    for (a, b) in slots:
        for (c, d) in slots:
            if b == c and a != b and c != d and (a, d) in slots:
                t.append(((a, b), (c, d), (a, d)))
    return t


def table_without_right_vertex(q, edges=None):
    """Mistake: drops a_ij e_j (the x_ij W_jj term)."""
    return [(x, w, z) for (x, w, z) in _real_table(q, edges) if not (x[0] != x[1] and w[0] == w[1])]


def table_wrong_result(q, edges=None):
    """Mistake: writes the product to the right factor's slot instead of (a, d)."""
    return [(x, w, w) for (x, w, z) in _real_table(q, edges)]


def table_transposed_weight(q, edges=None):
    """Mistake: uses weight block (d, b) instead of (b, d)."""
    return [(x, (w[1], w[0]), z) for (x, w, z) in _real_table(q, edges)]


def fwd_sign_flip(X, W, tau, q, in_widths=None, out_widths=None, edges=None, table=None):
    """Mistake: subtracts the off-diagonal endpoint product."""
    Y = _real_fwd(X, W, tau, q, in_widths, out_widths, edges, table)
    X = np.asarray(X, float)
    W = np.asarray(W, float)
    kb = O.group_bounds(X.shape[1], q, in_widths)
    nb = O.group_bounds(W.shape[1], q, out_widths)
    for m in range(X.shape[0]):
        i = int(tau[m])
        if not 0 <= i < q:
            continue
        for j in range(q):
            if j != i:
                Y[m, nb[j][0]:nb[j][1]] -= 2 * X[m, kb[i][0]:kb[i][1]] @ W[kb[i][0]:kb[i][1], nb[j][0]:nb[j][1]]
    return Y


def bwd_dw_all_rows(X, W, dY, tau, q, in_widths=None, out_widths=None, edges=None, table=None):
    """Mistake: off-diagonal weight gradients summed over every row, not just type-i rows."""
    dX, dW = _real_bwd(X, W, dY, tau, q, in_widths, out_widths, edges, table)
    X = np.asarray(X, float)
    dY = np.asarray(dY, float)
    kb = O.group_bounds(X.shape[1], q, in_widths)
    nb = O.group_bounds(dY.shape[1], q, out_widths)
    for b in range(q):
        for j in range(q):
            if b != j:
                dW[kb[b][0]:kb[b][1], nb[j][0]:nb[j][1]] = X[:, kb[b][0]:kb[b][1]].T @ dY[:, nb[j][0]:nb[j][1]]
    return dX, dW


def bwd_dx_drops_eq32(X, W, dY, tau, q, in_widths=None, out_widths=None, edges=None, table=None):
    """Mistake: activation gradient keeps only the source-row terms (drops eq 32)."""
    dX, dW = _real_bwd(X, W, dY, tau, q, in_widths, out_widths, edges, table)
    X = np.asarray(X, float)
    kb = O.group_bounds(X.shape[1], q, in_widths)
    for m in range(X.shape[0]):
        i = int(tau[m])
        for a in range(q):
            if a != i:
                dX[m, kb[a][0]:kb[a][1]] = 0.0
    return dX, dW


def bwd_dx_untransposed(X, W, dY, tau, q, in_widths=None, out_widths=None, edges=None, table=None):
    """Mistake: multiplies by W_bj instead of its transpose (square blocks, so shapes still fit)."""
    X = np.asarray(X, float)
    W = np.asarray(W, float)
    dY = np.asarray(dY, float)
    kb = O.group_bounds(X.shape[1], q, in_widths)
    nb = O.group_bounds(W.shape[1], q, out_widths)
    dX, dW = _real_bwd(X, W, dY, tau, q, in_widths, out_widths, edges, table)
    dX[:] = 0.0
    for m in range(X.shape[0]):
        i = int(tau[m])
        for (xa, xb), (wa, wd), (ya, yd) in (O.structure_table(q, edges) if table is None else table):
            if xa != i:
                continue
            blk = W[kb[wa][0]:kb[wa][1], nb[wd][0]:nb[wd][1]]
            if blk.shape[0] != blk.shape[1]:
                blk = blk.T
            dX[m, kb[xb][0]:kb[xb][1]] += dY[m, nb[yd][0]:nb[yd][1]] @ blk
    return dX, dW


def index_unstable(tau, q):
    """Mistake: rows of each type listed in descending order."""
    counts, offsets, rows, bad = _real_index(tau, q)
    rows = rows.copy()
    for i in range(q):
        rows[offsets[i]:offsets[i + 1]] = rows[offsets[i]:offsets[i + 1]][::-1]
    return counts, offsets, rows, bad


def index_drops_bad_count(tau, q):
    """Mistake: rows with out-of-range types are not counted."""
    counts, offsets, rows, _bad = _real_index(tau, q)
    return counts, offsets, rows, 0


def schedule_one_based(positions, q, kind="cyclic", period=0):
    """Mistake: keeps the page's 1-based types without shifting to 0-based."""
    p = np.asarray(positions, dtype=np.int64)
    if kind == "cyclic":
        return (1 + ((p - 1) % q)).astype(np.int32)
    return ((p % period) // (period // q)).astype(np.int32)


def silu_wrong_sign(z):
    """Mistake: x * sigmoid(-x)."""
    z = np.asarray(z, float)
    return z / (1.0 + np.exp(z))


def gated_swapped(X, Wg, Wu, tau, q):
    """Mistake: the activation applied to the up product instead of the gate."""
    return O.row_typed_forward(X, Wg, tau, q) * _real_silu(O.row_typed_forward(X, Wu, tau, q))


def gated_dense_gate(X, Wg, Wu, tau, q):
    """Mistake: the gate product ignores the row types (plain X W_gate)."""
    return _real_silu(np.asarray(X, float) @ np.asarray(Wg, float)) * O.row_typed_forward(X, Wu, tau, q)


def silu_grad_drops_term(z):
    """Mistake: silu' taken as sigmoid(z) alone (the product rule's second term dropped)."""
    z = np.asarray(z, float)
    return 1.0 / (1.0 + np.exp(-z))


def swiglu_bwd_swapped(G, U, dH):
    """Mistake: the gate and up gradients exchanged."""
    dG, dU = _real_swiglu_bwd(G, U, dH)
    return dU, dG


def swiglu_bwd_no_up(G, U, dH):
    """Mistake: the gate gradient misses the factor U."""
    dH = np.asarray(dH, float)
    return dH * _real_silu_grad(G), dH * _real_silu(G)


def tensor_msb_lsb_mixed(L):
    """Mistake: the levels combined with inconsistent bit order for the two factors' slots."""
    t = _real_tensor(L)
    if L < 2:
        return t
    def swap(v):
        return ((v & 1) << 1) | ((v >> 1) & 1) if L == 2 else v
    return [((swap(x[0]), x[1]), (w[0], w[1]), (swap(z[0]), z[1])) for (x, w, z) in t]


def tensor_drops_far_terms(L):
    """Mistake: only one intermediate group per level pair (the Q_q-like {alpha, delta} support)."""
    return [(x, w, z) for (x, w, z) in _real_tensor(L) if w[0] in (x[0], z[1])]


def tensor_edge_edge(L):
    """Mistake: a level keeps edge * edge (plain block matmul on that level)."""
    t = list(_real_tensor(L))
    q = 2 ** L
    have = {(x, w) for x, w, _ in t}
    for a in range(q):
        for b in range(q):
            for d in range(q):
                if ((a, b), (b, d)) not in have:
                    t.append(((a, b), (b, d), (a, d)))
                    return t
    return t


def attn_dense_scale(Q, K, V, tau, q, L=0, positions=None):
    """Mistake: the dense scale: queries shrunk by sqrt(m / d), so that an equal-type pair is
    scaled by 1/sqrt(d) as in ordinary attention instead of 1/sqrt(m)."""
    d = np.asarray(Q).shape[2]
    return _real_attn(np.asarray(Q, float) * np.sqrt((d // q) / d), K, V, tau, q, L, positions)


def support_own_group_only(i, j, q, L=0):
    """Mistake: a pair compares only the query's own group."""
    return [i]


def attn_kv_head_modulo(Q, K, V, tau, q, L=0, positions=None):
    """Mistake: query head h uses key/value head h mod Hkv."""
    Q = np.asarray(Q, float)
    K = np.asarray(K, float)
    V = np.asarray(V, float)
    Hq, Hkv = Q.shape[0], K.shape[0]
    idx = [h % Hkv for h in range(Hq)]
    return _real_attn(Q, K[idx], V[idx], tau, q, L, positions)


def attn_anticausal(Q, K, V, tau, q, L=0, positions=None):
    """Mistake: the mask admits keys at or after the query."""
    S = np.asarray(Q).shape[1]
    pos = np.arange(S) if positions is None else np.asarray(positions)
    return _real_attn(Q, K, V, tau, q, L, -pos)


def _decode_variant(Qn, Kc, Vc, q_pos, key_pos, q, L, kind, period, key_types, allowed):
    """Algorithm 3 with the key types and the allowed slots supplied by a mutant."""
    Qn, Kc, Vc = (np.asarray(a, float) for a in (Qn, Kc, Vc))
    B, Hq, d = Qn.shape
    Hkv = Kc.shape[1]
    m = d // q
    out = np.zeros(Qn.shape)
    for b in range(B):
        i = int(O.type_schedule(np.array([q_pos[b]]), q, kind, period)[0])
        slots = np.where(allowed(b))[0]
        if slots.size == 0:
            continue
        js = key_types(b)[slots]
        for h in range(Hq):
            kv = h // (Hq // Hkv)
            s_ = np.array([sum(Kc[b, kv, u, a * m:(a + 1) * m] @ Qn[b, h, a * m:(a + 1) * m]
                               for a in O.score_support(i, int(j), q, L)) / np.sqrt(len(O.score_support(i, int(j), q, L)) * m)
                           for u, j in zip(slots, js)])
            w = np.exp(s_ - s_.max())
            out[b, h] = (w / w.sum()) @ Vc[b, kv][slots]
    return out


def decode_type_from_slot(Qn, Kc, Vc, q_pos, key_pos, q, L=0, kind="cyclic", period=0):
    """Mistake: a cached key's type is taken from its slot index, not from its position."""
    kp = np.asarray(key_pos)
    return _decode_variant(Qn, Kc, Vc, q_pos, key_pos, q, L, kind, period,
                           key_types=lambda b: O.type_schedule(np.arange(kp.shape[1]), q, kind, period),
                           allowed=lambda b: (kp[b] >= 0) & (kp[b] <= q_pos[b]))


def decode_admits_future(Qn, Kc, Vc, q_pos, key_pos, q, L=0, kind="cyclic", period=0):
    """Mistake: every non-empty slot is attended, including keys after the query's position."""
    kp = np.asarray(key_pos)
    return _decode_variant(Qn, Kc, Vc, q_pos, key_pos, q, L, kind, period,
                           key_types=lambda b: O.type_schedule(np.maximum(kp[b], 0), q, kind, period),
                           allowed=lambda b: kp[b] >= 0)


def decode_dense_scale(Qn, Kc, Vc, q_pos, key_pos, q, L=0, kind="cyclic", period=0):
    """Mistake: scores scaled by 1/sqrt(d) as in dense attention instead of 1/sqrt(|F| m)."""
    d = np.asarray(Qn).shape[2]
    return _real_decode(np.asarray(Qn, float) * np.sqrt((d // q) / d), Kc, Vc, q_pos, key_pos, q, L, kind, period)


def decode_macs_full_keys(p, key_pos, q, d, L=0, kind="cyclic", period=0):
    """Mistake: every cached key costs d score MACs (the dense count)."""
    sm, vm = _real_decode_macs(p, key_pos, q, d, L, kind, period)
    return vm, vm



def _attn_bwd_variant(Q, K, V, dO, tau, q, L, positions, row_term=True, all_groups=False, assign_heads=False):
    """The attention gradients with one step replaced by a mutant's choice."""
    Q, K, V, dO = (np.asarray(a, float) for a in (Q, K, V, dO))
    Hq, S, d = Q.shape
    Hkv = K.shape[0]
    m = d // q
    tau = np.asarray(tau)
    pos = np.arange(S) if positions is None else np.asarray(positions)
    sel = np.zeros((q, S, S), dtype=bool)
    for i in range(q):
        for j in range(q):
            for a in O.score_support(i, j, q, L):
                sel[a][np.ix_(tau == i, tau == j)] = True
    k_pair = np.maximum(sel.sum(axis=0) * m, 1)
    dQ, dK, dV = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    for h in range(Hq):
        kv = h // (Hq // Hkv)
        r = sum(np.where(sel[a], Q[h][:, a * m:(a + 1) * m] @ K[kv][:, a * m:(a + 1) * m].T, 0.0) for a in range(q))
        sc = np.where(pos[None, :] <= pos[:, None], r / np.sqrt(k_pair), -np.inf)
        P = np.exp(sc - sc.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        dP = dO[h] @ V[kv].T
        dS = P * (dP - (P * dP).sum(axis=1, keepdims=True)) if row_term else P * dP
        dR = dS / np.sqrt(k_pair)
        if assign_heads:
            dV[kv] = P.T @ dO[h]
            dK[kv] = 0.0
        else:
            dV[kv] += P.T @ dO[h]
        for a in range(q):
            ga = slice(a * m, (a + 1) * m)
            dRa = dR if all_groups else np.where(sel[a], dR, 0.0)
            dQ[h][:, ga] += dRa @ K[kv][:, ga]
            dK[kv][:, ga] += dRa.T @ Q[h][:, ga]
    return dQ, dK, dV


def attn_bwd_drops_row_term(Q, K, V, dO, tau, q, L=0, positions=None):
    """Mistake: the softmax VJP without its row term (dS = P dP)."""
    return _attn_bwd_variant(Q, K, V, dO, tau, q, L, positions, row_term=False)


def attn_bwd_all_groups(Q, K, V, dO, tau, q, L=0, positions=None):
    """Mistake: the score gradient reaches every feature group, not only the compared ones."""
    return _attn_bwd_variant(Q, K, V, dO, tau, q, L, positions, all_groups=True)


def attn_bwd_last_head_wins(Q, K, V, dO, tau, q, L=0, positions=None):
    """Mistake: a key/value head keeps the gradient of its last query head only (no GQA sum)."""
    return _attn_bwd_variant(Q, K, V, dO, tau, q, L, positions, assign_heads=True)


def attn_bwd_swaps_dk_dv(Q, K, V, dO, tau, q, L=0, positions=None):
    """Mistake: dK and dV returned in each other's place."""
    dQ, dK, dV = _real_attn_bwd(Q, K, V, dO, tau, q, L, positions)
    return dQ, dV, dK


MUTANTS = [
    ("structure_table", table_with_edge_edge),
    ("structure_table", table_without_right_vertex),
    ("structure_table", table_wrong_result),
    ("structure_table", table_transposed_weight),
    ("row_typed_forward", fwd_sign_flip),
    ("row_typed_backward", bwd_dw_all_rows),
    ("row_typed_backward", bwd_dx_drops_eq32),
    ("row_typed_backward", bwd_dx_untransposed),
    ("type_index", index_unstable),
    ("type_index", index_drops_bad_count),
    ("type_schedule", schedule_one_based),
    ("silu", silu_wrong_sign),
    ("gated_forward", gated_swapped),
    ("gated_forward", gated_dense_gate),
    ("silu_grad", silu_grad_drops_term),
    ("swiglu_backward", swiglu_bwd_swapped),
    ("swiglu_backward", swiglu_bwd_no_up),
    ("tensor_power_table", tensor_msb_lsb_mixed),
    ("tensor_power_table", tensor_drops_far_terms),
    ("tensor_power_table", tensor_edge_edge),
    ("algebraic_attention", attn_dense_scale),
    ("score_support", support_own_group_only),
    ("algebraic_attention", attn_kv_head_modulo),
    ("algebraic_attention", attn_anticausal),
    ("algebraic_attention_decode", decode_type_from_slot),
    ("algebraic_attention_decode", decode_admits_future),
    ("algebraic_attention_decode", decode_dense_scale),
    ("attention_decode_macs", decode_macs_full_keys),
    ("algebraic_attention_backward", attn_bwd_drops_row_term),
    ("algebraic_attention_backward", attn_bwd_all_groups),
    ("algebraic_attention_backward", attn_bwd_last_head_wins),
    ("algebraic_attention_backward", attn_bwd_swaps_dk_dv),
]


@pytest.mark.parametrize("name,mutant", MUTANTS, ids=[m.__name__ for _, m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, name, mutant):
    monkeypatch.setattr(O, name, mutant)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(O)
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {mutant.__name__}"
