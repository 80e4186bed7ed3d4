"""fp64 CPU oracle for the row-typed associative-algebra projection Y = X *_{Q_q} W.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or link
this module: only the tests, the smoke check and the bench's CPU-baseline leg
use it.  It shares no code with the HIP library or its Python binding.

Source: arXiv 2609.32814, "Change the Product, Keep the Parameters: Associative
Algebra Layers for Transformers".  Every function names the passage it follows.

What is computed, plainly:

* The graph algebra Q_G (section 3.1, eq 9) has one basis element per vertex
  slot (a, a) and per directed-edge slot (a, b).  Its only nonzero basis
  products are  vertex*vertex = vertex,  vertex*edge = edge,  edge*vertex =
  edge  when the inner indices agree; every other product is zero.
  `structure_table` writes those structure constants out as a list of
  (left slot, right slot, result slot) triples (eq 5 with c = 1 on each triple).
* Lifted to matrix blocks, each triple is one block GEMM (section 1: a
  product of two blocks in the table is an ordinary GEMM).  `square_product` sums the
  block GEMMs of every triple (eq 10-11, eq 13-14 for the complete graph Q_q).
* The row-typed projection (section 4, eq 16-17; section 6.1, eq 27 and
  Algorithm 1) gives each token row m the type i = tau[m]; the row uses the
  triples whose left slot lies in block-row i.  `row_typed_forward` runs
  Algorithm 1 with the support read off the table.
* The vector-Jacobian products (appendix B, eq 31-35) are the same triples
  with the GEMMs transposed: `row_typed_backward`.
* `type_index` forms the row sets I_i = {m : tau[m] = i} (Algorithm 1, the
  step that builds I_i), `type_schedule` the position-type schedule (section 4,
  the cyclic tau; appendix D.5, the interval schedule of the pilot).
* `mac_count` counts the multiply-accumulates the row-typed evaluator executes
  (eq 18-19; eq 24 for equal groups).
* `tensor_power_table` lists the triples of the recursive law Q_2^{(x)L}
  (appendix C): bit-string slots, one Q_2 triple per level, 6^L triples; the
  evaluators take any law's triples through their `table` argument, so a row
  of type alpha sums x_beta W_beta,delta over the beta whose bits each come
  from alpha or delta (eq 36's support; section 6.1's B(i, j) for this law).
* `algebraic_attention` is appendix G's causal attention with the algebraic
  score: a query of type i and a key of type j compare only the feature groups
  F(i, j) ({i} or {i, j}, eq 38; eq 42 for the recursive law), scaled by
  1 / sqrt(|F| m) (eq 41), then the causal softmax and a dense PV (eq 43-44);
  `attention_score_macs` counts its score and value MACs (eq 45);
  `algebraic_attention_backward` gives its gradients (Algorithm 2, step 9):
  the softmax and value-sum VJPs, and the score's gradient routed to the
  compared groups only.
* `algebraic_attention_decode` is appendix G's cached decoding (Algorithm 3,
  the loop over cached positions and the softmax / value sum): one new query
  row per sequence against that sequence's full-key cache, each key's type
  recovered from its absolute position (G.2); `attention_decode_macs` counts
  its score and value MACs (eq 57-58 for Q_q, eq 61 for the recursive law).
* `gated_forward` is the gate/up half of a gated (SwiGLU) FFN: both D x F
  projections are row-typed exactly like any other projection, while gates
  and pointwise activations are left as they are (section 4), combined as silu(X *_{Q_q} W_gate) * (X *_{Q_q} W_up), silu
  being x * sigmoid(x) (the pilot's bias-free SwiGLU, appendix D; SwiGLU
  x * sigma(beta x) with beta = 1).
* `gated_ffn_forward` / `gated_ffn_backward` are the whole gated FFN
  (gate, up, down; section 4) and its training step: the projections' VJPs
  from appendix B and the chain rule through silu(G) * U
  (`swiglu_backward`, with silu' = sigmoid (1 + x (1 - sigmoid))).

All arithmetic is float64; block products are numpy.matmul (a library
primitive standing for one block GEMM).  The oracle itself rounds nothing.

Readings where the pages leave a step open:
* types are 0-based: the page's 1 + ((p-1) mod q) with 1-based p is the same
  cycle as p mod q with 0-based p;
* B(i, i) = {i} is a set: the j = i output group gets the single term x_i W_ii;
* group widths default to equal (K/q, N/q); unequal widths are accepted;
* a row whose tau lies outside [0, q) belongs to no type: it contributes to
  nothing and its output row is zero (it is counted by `type_index`).

Every function here is pinned by tests against closed forms or independent
formulas from the pages (worked q=2 example, unit and associativity laws,
product counts, appendix A's (d, n) form, masked-dense and brute-force forms,
autograd of the masked-dense form for the VJPs).
"""
from __future__ import annotations

from typing import Iterable, Sequence

import numpy as np

Slot = tuple[int, int]
Triple = tuple[Slot, Slot, Slot]

__all__ = [
    "complete_graph_edges",
    "graph_slots",
    "structure_table",
    "tensor_power_table",
    "group_bounds",
    "square_product",
    "row_typed_forward",
    "row_typed_backward",
    "row_typed_forward_batched",
    "type_index",
    "type_schedule",
    "mac_count",
    "dense_equivalent_macs",
    "silu",
    "gated_forward",
    "score_support",
    "algebraic_attention",
    "algebraic_attention_backward",
    "attention_score_macs",
    "algebraic_attention_decode",
    "attention_decode_macs",
]


# ----------------------------------------------------------------------------
# The algebra: section 3.1 (eq 9-11) and section 3.2 (eq 13-15)
# ----------------------------------------------------------------------------

def complete_graph_edges(q: int) -> list[Slot]:
    """Directed edges of the complete graph on q vertices (section 3.2: Q_q)."""
    return [(a, b) for a in range(q) for b in range(q) if a != b]


def graph_slots(q: int, edges: Iterable[Slot] | None = None) -> list[Slot]:
    """Slots of Q_G: vertices (a, a) and edges (a, b) (section 3.1).

    `edges=None` means the complete graph, i.e. Q_q.
    """
    e = complete_graph_edges(q) if edges is None else [tuple(x) for x in edges]
    for a, b in e:
        if a == b or not (0 <= a < q and 0 <= b < q):
            raise ValueError(f"bad edge {(a, b)} for q={q}")
    return [(a, a) for a in range(q)] + sorted(set(e))


def structure_table(q: int, edges: Iterable[Slot] | None = None) -> list[Triple]:
    """Nonzero structure constants of Q_G as (left, right, result) slot triples.

    Basis rule (eq 9): e_i e_i = e_i, e_i a_ij = a_ij, a_ij e_j = a_ij, and all
    other basis products vanish.  In slot terms: (a, b) * (c, d) is nonzero only
    when b == c and at least one factor is a vertex; the result is slot (a, d).
    """
    slots = graph_slots(q, edges)
    slot_set = set(slots)
    table: list[Triple] = []
    for left in slots:
        a, b = left
        for right in slots:
            c, d = right
            if b != c:
                continue                      # inner indices must meet
            if a != b and c != d:
                continue                      # edge * edge = 0
            out = (a, d)
            assert out in slot_set            # vertex*x and x*vertex return x
            table.append((left, right, out))
    return table


def tensor_power_table(L: int) -> list[Triple]:
    """Nonzero structure constants of the recursive law Q_2^{(x)L} (appendix C).

    Basis elements of a tensor product are tensors of basis elements, and
    their product is the tensor of the factors' products, so a triple of the
    L-fold power is one Q_2 triple per level.  Slots are pairs of L-bit
    strings (a, b); level 1 is the most significant bit (the first split of
    the recursion).  L = 1 is Q_2 itself.
    """
    if L < 1:
        raise ValueError("L >= 1")
    base = structure_table(2)
    table = base
    for _ in range(L - 1):
        table = [((2 * l[0] + l2[0], 2 * l[1] + l2[1]),
                  (2 * r[0] + r2[0], 2 * r[1] + r2[1]),
                  (2 * o[0] + o2[0], 2 * o[1] + o2[1]))
                 for (l, r, o) in table for (l2, r2, o2) in base]
    return table


# ----------------------------------------------------------------------------
# Block bookkeeping
# ----------------------------------------------------------------------------

def group_bounds(total: int, q: int, widths: Sequence[int] | None = None) -> list[tuple[int, int]]:
    """[start, end) of each feature group; equal widths total/q unless given (section 4)."""
    if widths is None:
        if total % q:
            raise ValueError(f"q={q} does not divide width {total}")
        widths = [total // q] * q
    if len(widths) != q or sum(widths) != total or min(widths) < 0:
        raise ValueError(f"widths {widths} do not partition {total} into {q} groups")
    out, s = [], 0
    for w in widths:
        out.append((s, s + w))
        s += w
    return out


# ----------------------------------------------------------------------------
# Square form: Z = X * W over block arrays (eq 10-11; eq 13-14; eq 3 at q = 2)
# ----------------------------------------------------------------------------

def square_product(X: np.ndarray, W: np.ndarray, q: int,
                   row_heights: Sequence[int] | None = None,
                   mid_widths: Sequence[int] | None = None,
                   out_widths: Sequence[int] | None = None,
                   edges: Iterable[Slot] | None = None,
                   table: Sequence[Triple] | None = None) -> np.ndarray:
    """Block-array product Z = X *_{Q_G} W (or of the law whose triples `table` lists).

    X is split into q x q blocks (block-row heights `row_heights`, block-column
    widths `mid_widths`), W into q x q blocks (heights `mid_widths`, widths
    `out_widths`).  For every structure-constant triple (a,b)*(b,d) -> (a,d) the
    block GEMM X_ab W_bd is added to Z_ad (eq 5 lifted to blocks).  Slots that
    are not in the algebra (non-complete G) must hold zero blocks in X and W;
    they are ignored.
    """
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    rb = group_bounds(X.shape[0], q, row_heights)
    mb = group_bounds(X.shape[1], q, mid_widths)
    if W.shape[0] != X.shape[1]:
        raise ValueError("inner dimensions differ")
    ob = group_bounds(W.shape[1], q, out_widths)
    Z = np.zeros((X.shape[0], W.shape[1]), dtype=np.float64)
    for (a, b), (_, d), (za, zd) in (structure_table(q, edges) if table is None else table):
        xa = X[rb[a][0]:rb[a][1], mb[b][0]:mb[b][1]]
        wb = W[mb[b][0]:mb[b][1], ob[d][0]:ob[d][1]]
        Z[rb[za][0]:rb[za][1], ob[zd][0]:ob[zd][1]] += xa @ wb
    return Z


# ----------------------------------------------------------------------------
# Type schedule and type index: section 4 (tau), Algorithm 1 (I_i), App D.5
# ----------------------------------------------------------------------------

def type_schedule(positions: np.ndarray, q: int, kind: str = "cyclic",
                  period: int = 0) -> np.ndarray:
    """Row types from absolute positions.

    * "cyclic": tau(p) = p mod q (section 4, 0-based form of 1 + ((p-1) mod q)).
    * "interval": tau(p) = floor((p mod period) / (period / q)) (appendix D.5,
      the pilot's schedule floor((p mod 768) / 192) with period 768, q = 4).
    """
    p = np.asarray(positions, dtype=np.int64)
    if kind == "cyclic":
        return (p % q).astype(np.int32)
    if kind == "interval":
        if period <= 0 or period % q:
            raise ValueError("interval schedule needs q | period > 0")
        return ((p % period) // (period // q)).astype(np.int32)
    raise ValueError(kind)


def type_index(tau: np.ndarray, q: int):
    """Row sets I_i = {m : tau[m] = i} (Algorithm 1).

    Returns (counts[q], offsets[q+1], rows[sum counts], bad) where rows lists
    the members of I_0, then I_1, ..., each in ascending row order, offsets are
    the running sums of counts, and `bad` counts rows whose tau lies outside
    [0, q) (they belong to no I_i).
    """
    tau = np.asarray(tau, dtype=np.int64)
    counts = np.zeros(q, dtype=np.int64)
    members: list[list[int]] = [[] for _ in range(q)]
    bad = 0
    for m, t in enumerate(tau.tolist()):
        if 0 <= t < q:
            members[t].append(m)
            counts[t] += 1
        else:
            bad += 1
    offsets = np.zeros(q + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    rows = np.array([m for grp in members for m in grp], dtype=np.int64)
    return counts, offsets, rows, bad


# ----------------------------------------------------------------------------
# Row-typed projection: section 4 (eq 16-17), section 6.1 (eq 27, Algorithm 1)
# ----------------------------------------------------------------------------

def _row_sets(tau: np.ndarray, q: int) -> list[np.ndarray]:
    counts, offsets, rows, _ = type_index(tau, q)
    return [rows[offsets[i]:offsets[i + 1]] for i in range(q)]


def row_typed_forward(X: np.ndarray, W: np.ndarray, tau: np.ndarray, q: int,
                      in_widths: Sequence[int] | None = None,
                      out_widths: Sequence[int] | None = None,
                      edges: Iterable[Slot] | None = None,
                      table: Sequence[Triple] | None = None) -> np.ndarray:
    """Y = X *_{Q_G} W with row types tau (Algorithm 1); `table` gives another law's triples.

    Y <- 0; for each type i with rows I_i, for each structure-constant triple
    (i, b) * (b, j) -> (i, j) whose left slot is in block-row i:
        Y[I_i, g_j] += X[I_i, g_b] W[g_b, g_j].
    For the complete graph that is y_i = x_i W_ii and y_j = x_i W_ij + x_j W_jj
    (eq 16-17; support B(i, j) = {i, j} of eq 27).
    """
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    M, K = X.shape
    if W.shape[0] != K:
        raise ValueError("X and W inner widths differ")
    N = W.shape[1]
    kb = group_bounds(K, q, in_widths)
    nb = group_bounds(N, q, out_widths)
    if table is None:
        table = structure_table(q, edges)
    Y = np.zeros((M, N), dtype=np.float64)
    for i, rows in enumerate(_row_sets(tau, q)):
        if rows.size == 0:
            continue
        Xi = X[rows]
        Yi = np.zeros((rows.size, N), dtype=np.float64)
        for (xa, xb), (wa, wd), (ya, yd) in table:
            if xa != i:
                continue                      # the row of type i supplies slots (i, *)
            assert ya == i
            xs, xe = kb[xb]
            ws, we = kb[wa]
            ns, ne = nb[wd]
            Yi[:, nb[yd][0]:nb[yd][1]] += Xi[:, xs:xe] @ W[ws:we, ns:ne]
        Y[rows] = Yi
    return Y


def row_typed_backward(X: np.ndarray, W: np.ndarray, dY: np.ndarray, tau: np.ndarray, q: int,
                       in_widths: Sequence[int] | None = None,
                       out_widths: Sequence[int] | None = None,
                       edges: Iterable[Slot] | None = None,
                       table: Sequence[Triple] | None = None):
    """(dX, dW) of Y = X *_{Q_G} W (appendix B, eq 31-35); `table` as in the forward.

    Each forward block GEMM Y[I_i, g_j] += X[I_i, g_b] W[g_b, g_j] contributes
        dX[I_i, g_b] += dY[I_i, g_j] W[g_b, g_j]^T      (eq 31-32)
        dW[g_b, g_j] += X[I_i, g_b]^T dY[I_i, g_j]      (eq 33-35)
    summed over all types; blocks no type reaches stay zero.
    """
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    dY = np.asarray(dY, dtype=np.float64)
    M, K = X.shape
    N = W.shape[1]
    if dY.shape != (M, N):
        raise ValueError("dY shape")
    kb = group_bounds(K, q, in_widths)
    nb = group_bounds(N, q, out_widths)
    if table is None:
        table = structure_table(q, edges)
    dX = np.zeros((M, K), dtype=np.float64)
    dW = np.zeros((K, N), dtype=np.float64)
    for i, rows in enumerate(_row_sets(tau, q)):
        if rows.size == 0:
            continue
        Xi = X[rows]
        dYi = dY[rows]
        dXi = np.zeros((rows.size, K), dtype=np.float64)
        for (xa, xb), (wa, wd), (ya, yd) in table:
            if xa != i:
                continue
            assert ya == i
            xs, xe = kb[xb]
            ws, we = kb[wa]
            ns, ne = nb[wd]
            ys, ye = nb[yd]
            dXi[:, xs:xe] += dYi[:, ys:ye] @ W[ws:we, ns:ne].T
            dW[ws:we, ns:ne] += Xi[:, xs:xe].T @ dYi[:, ys:ye]
        dX[rows] = dXi
    return dX, dW


def row_typed_forward_batched(X: np.ndarray, W: np.ndarray, tau: np.ndarray, q: int) -> np.ndarray:
    """E independent projections (one weight bank per expert): X[E,M,K], W[E,K,N], tau[E,M]."""
    return np.stack([row_typed_forward(X[e], W[e], tau[e], q) for e in range(X.shape[0])])


# ----------------------------------------------------------------------------
# Cost: eq 18-19 (rectangular cost), eq 21 / eq 24 (equal groups)
# ----------------------------------------------------------------------------

def mac_count(tau: np.ndarray, q: int, K: int, N: int,
              in_widths: Sequence[int] | None = None,
              out_widths: Sequence[int] | None = None,
              edges: Iterable[Slot] | None = None,
              table: Sequence[Triple] | None = None) -> tuple[int, int]:
    """(block GEMMs executed, MACs executed) by `row_typed_forward` on these types.

    Counts, for every type i with M_i > 0, each triple with left slot in
    block-row i as one block GEMM of M_i * s_b * r_j MACs.
    """
    kb = group_bounds(K, q, in_widths)
    nb = group_bounds(N, q, out_widths)
    counts, _, _, _ = type_index(tau, q)
    gemms = 0
    macs = 0
    for (xa, _xb), (wa, wd), _out in (structure_table(q, edges) if table is None else table):
        Mi = int(counts[xa])
        if Mi == 0:
            continue
        gemms += 1
        macs += Mi * (kb[wa][1] - kb[wa][0]) * (nb[wd][1] - nb[wd][0])
    return gemms, macs


def dense_equivalent_macs(M: int, K: int, N: int) -> int:
    """MACs of the ordinary product X W (the dense control)."""
    return M * K * N


# ----------------------------------------------------------------------------
# Gated FFN: section 4 (gated FFN shapes, the same row law for each
# projection), the pilot's bias-free SwiGLU (appendix D), table 9
# ----------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    """x * sigmoid(x) (SwiGLU's swish with beta = 1), evaluated in float64."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def gated_forward(X: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, tau: np.ndarray, q: int,
                  table: Sequence[Triple] | None = None) -> np.ndarray:
    """H = silu(X *_{Q_q} W_gate) * (X *_{Q_q} W_up), both products row-typed with the same tau.

    The activation applies to the gate product, elementwise, after both
    endpoint sums of each product are complete (the same Algorithm 1 for
    both D x F weights).
    """
    G = row_typed_forward(X, Wg, tau, q, table=table)
    U = row_typed_forward(X, Wu, tau, q, table=table)
    return silu(G) * U


def silu_grad(z: np.ndarray) -> np.ndarray:
    """d silu / dz = sigmoid(z) (1 + z (1 - sigmoid(z))), evaluated in float64."""
    z = np.asarray(z, dtype=np.float64)
    sg = 1.0 / (1.0 + np.exp(-z))
    return sg * (1.0 + z * (1.0 - sg))


def swiglu(G: np.ndarray, U: np.ndarray) -> np.ndarray:
    """The pointwise gate of a SwiGLU FFN: silu(G) * U (appendix D; beta = 1)."""
    return silu(G) * np.asarray(U, dtype=np.float64)


def swiglu_backward(G: np.ndarray, U: np.ndarray, dH: np.ndarray):
    """(dG, dU) of H = silu(G) * U: dG = dH * U * silu'(G), dU = dH * silu(G)."""
    dH = np.asarray(dH, dtype=np.float64)
    return dH * np.asarray(U, dtype=np.float64) * silu_grad(G), dH * silu(G)


def gated_ffn_forward(X, Wg, Wu, Wd, tau, q, table=None):
    """Y = (silu(X *_Q W_gate) * (X *_Q W_up)) *_Q W_down, each projection row-typed with the
    same tau (section 4: all three gated-FFN weights are row-typed projections).

    Returns Y and the intermediates (G, U, H) that the backward pass uses.
    """
    G = row_typed_forward(X, Wg, tau, q, table=table)
    U = row_typed_forward(X, Wu, tau, q, table=table)
    H = swiglu(G, U)
    return row_typed_forward(H, Wd, tau, q, table=table), (G, U, H)


def gated_ffn_backward(X, Wg, Wu, Wd, dY, tau, q, table=None):
    """(dX, dW_gate, dW_up, dW_down) of `gated_ffn_forward`.

    Each projection's VJP is appendix B's (eq 31-35) with the same support as
    its forward; the activation's is the chain rule of silu(G) * U.  Six
    projection-shaped products against the forward's three: the 9 B D F ->
    9 rho B D F training count of section 6.2.
    """
    _, (G, U, H) = gated_ffn_forward(X, Wg, Wu, Wd, tau, q, table)
    dH, dWd = row_typed_backward(H, Wd, dY, tau, q, table=table)
    dG, dU = swiglu_backward(G, U, dH)
    dXg, dWg = row_typed_backward(X, Wg, dG, tau, q, table=table)
    dXu, dWu = row_typed_backward(X, Wu, dU, tau, q, table=table)
    return dXg + dXu, dWg, dWu, dWd


# ----------------------------------------------------------------------------
# Algebraic attention scores: appendix G (eq 38-46), Algorithm 2
# ----------------------------------------------------------------------------

def score_support(i: int, j: int, q: int, L: int = 0) -> list[int]:
    """Feature groups a query of type i and a key of type j compare (eq 38 for Q_q: {i} or
    {i, j}; eq 42 for the recursive law Q_2^(x)L, L >= 1: every b whose bits each come from i or j)."""
    if L == 0:
        return [i] if i == j else [i, j]
    return [b for b in range(q) if all(((b >> k) & 1) in (((i >> k) & 1), ((j >> k) & 1)) for k in range(L))]


def algebraic_attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, tau: np.ndarray, q: int,
                        L: int = 0, positions: np.ndarray | None = None) -> np.ndarray:
    """Causal attention with the algebraic score (appendix G, Algorithm 2, steps 3-7).

    Q: [Hq, S, d], K and V: [Hkv, S, d] with Hkv dividing Hq (query head h uses key/value head
    h // (Hq / Hkv), the GQA convention of appendix G); tau: [S] types of the S positions;
    positions: [S] absolute positions for the causal mask (default 0..S-1).  Each head's d
    features form q groups of width m = d / q.  For a query at p (type i) and a key at u (type j):
        r_pu = sum over a in F(i, j) of <Q_p^(a), K_u^(a)>          (eq 39)
        s_pu = r_pu / sqrt(|F(i, j)| m)                              (eq 40-41)
        P_p  = softmax over u with position(u) <= position(p)        (eq 43-44)
        O_p  = sum_u P_pu V_u                                         (dense PV)
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Hq, S, d = Q.shape
    Hkv = K.shape[0]
    if d % q or Hq % Hkv or K.shape[1:] != (S, d) or V.shape != K.shape:
        raise ValueError("shapes")
    m = d // q
    tau = np.asarray(tau)
    pos = np.arange(S) if positions is None else np.asarray(positions)
    allowed = pos[None, :] <= pos[:, None]                       # [p, u]
    # selection of group a for each (p, u) pair and the support size k_ij = |F| m
    sel = np.zeros((q, S, S), dtype=bool)
    for i in range(q):
        for j in range(q):
            pi = tau == i
            uj = tau == j
            for a in score_support(i, j, q, L):
                sel[a][np.ix_(pi, uj)] = True
    k_pair = sel.sum(axis=0) * m
    O = np.zeros((Hq, S, d))
    for h in range(Hq):
        kv = h // (Hq // Hkv)
        r = np.zeros((S, S))
        for a in range(q):
            g = Q[h][:, a * m:(a + 1) * m] @ K[kv][:, a * m:(a + 1) * m].T
            r += np.where(sel[a], g, 0.0)
        s = np.where(allowed, r / np.sqrt(np.maximum(k_pair, 1)), -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        P = np.exp(s)
        P /= P.sum(axis=1, keepdims=True)
        O[h] = P @ V[kv]
    return O



def algebraic_attention_backward(Q: np.ndarray, K: np.ndarray, V: np.ndarray, dO: np.ndarray,
                                 tau: np.ndarray, q: int, L: int = 0,
                                 positions: np.ndarray | None = None):
    """Gradients of `algebraic_attention` (Algorithm 2, step 9: backpropagation through steps
    3-7), returned as (dQ, dK, dV) with the shapes of Q, K, V.

    With r, s, P as in the forward (eq 39-44) and the incoming gradient dO of the outputs, per
    query head (chain rule through each step, last step first):
        dV_u     = sum_p P_pu dO_p                                (the dense PV, transposed)
        dP_pu    = <dO_p, V_u>
        dS_pu    = P_pu (dP_pu - sum_u' P_pu' dP_pu')             (the row softmax)
        dR_pu    = dS_pu / sqrt(|F(i, j)| m)                      (eq 41's scale)
        dQ_p^(a) = sum_u dR_pu K_u^(a),  dK_u^(a) = sum_p dR_pu Q_p^(a),  for a in F(i, j) only
                                                                  (eq 39: r is bilinear in the
                                                                   compared groups)
    Masked pairs (eq 43) have P = 0 and contribute nothing.  A key/value head's dK and dV sum
    over the query heads that read it (GQA).
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    Hq, S, d = Q.shape
    Hkv = K.shape[0]
    if d % q or Hq % Hkv or K.shape[1:] != (S, d) or V.shape != K.shape or dO.shape != Q.shape:
        raise ValueError("shapes")
    m = d // q
    tau = np.asarray(tau)
    pos = np.arange(S) if positions is None else np.asarray(positions)
    allowed = pos[None, :] <= pos[:, None]
    sel = np.zeros((q, S, S), dtype=bool)
    for i in range(q):
        for j in range(q):
            for a in score_support(i, j, q, L):
                sel[a][np.ix_(tau == i, tau == j)] = True
    k_pair = np.maximum(sel.sum(axis=0) * m, 1)
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    for h in range(Hq):
        kv = h // (Hq // Hkv)
        # forward again: scores over the compared groups, scale, causal softmax
        r = np.zeros((S, S))
        for a in range(q):
            g = Q[h][:, a * m:(a + 1) * m] @ K[kv][:, a * m:(a + 1) * m].T
            r += np.where(sel[a], g, 0.0)
        s = np.where(allowed, r / np.sqrt(k_pair), -np.inf)
        P = np.exp(s - s.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        # backward, step by step
        dV[kv] += P.T @ dO[h]
        dP = dO[h] @ V[kv].T
        dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
        dR = dS / np.sqrt(k_pair)
        for a in range(q):
            ga = slice(a * m, (a + 1) * m)
            dRa = np.where(sel[a], dR, 0.0)
            dQ[h][:, ga] += dRa @ K[kv][:, ga]
            dK[kv][:, ga] += dRa.T @ Q[h][:, ga]
    return dQ, dK, dV


def attention_score_macs(tau: np.ndarray, q: int, d: int, L: int = 0,
                         positions: np.ndarray | None = None) -> tuple[int, int]:
    """(score MACs, value MACs) of one head over the allowed pairs: sum of |F(i, j)| m per pair
    for the structured QK^T, d per pair for the dense PV (appendix G, eq 45)."""
    tau = np.asarray(tau)
    S = tau.size
    pos = np.arange(S) if positions is None else np.asarray(positions)
    m = d // q
    score = 0
    pairs = 0
    for p in range(S):
        for u in range(S):
            if pos[u] <= pos[p]:
                pairs += 1
                score += len(score_support(int(tau[p]), int(tau[u]), q, L)) * m
    return score, pairs * d


def algebraic_attention_decode(Qn: np.ndarray, Kc: np.ndarray, Vc: np.ndarray, q_pos: np.ndarray,
                               key_pos: np.ndarray, q: int, L: int = 0, kind: str = "cyclic",
                               period: int = 0) -> np.ndarray:
    """Cached decoding with the algebraic score (appendix G, Algorithm 3: the loop over the
    allowed cached positions, then the softmax and the value sum; G.2 for the cache).

    Qn: [B, Hq, d], the new row's queries of each of B sequences; Kc, Vc: [B, Hkv, N, d], each
    sequence's cache of N slots (full keys and values, Hkv dividing Hq: query head h reads
    key/value head h // (Hq / Hkv)); q_pos: [B] absolute position p of the new row; key_pos:
    [B, N] absolute position u of each cached slot, negative for an empty slot.  The query's type
    is i = tau(p), a cached key's j = tau(u), tau the position schedule (`type_schedule`).  For
    every slot with 0 <= u <= p:
        r_pu = sum over a in F(i, j) of <Q_p^(a), K_u^(a)>        (eq 39)
        s_pu = r_pu / sqrt(|F(i, j)| m),  m = d / q                 (eq 41)
    P_p = softmax over those slots, O_p = sum_u P_pu V_u (dense).  A row with no allowed slot
    is written as zeros (the softmax of an empty set is not defined).
    """
    Qn = np.asarray(Qn, dtype=np.float64)
    Kc = np.asarray(Kc, dtype=np.float64)
    Vc = np.asarray(Vc, dtype=np.float64)
    B, Hq, d = Qn.shape
    Hkv, N = Kc.shape[1], Kc.shape[2]
    if Kc.shape != (B, Hkv, N, d) or Vc.shape != Kc.shape or Hq % Hkv or d % q:
        raise ValueError("shapes")
    q_pos = np.asarray(q_pos, dtype=np.int64)
    key_pos = np.asarray(key_pos, dtype=np.int64)
    m = d // q
    O = np.zeros((B, Hq, d))
    for b in range(B):
        p = int(q_pos[b])
        i = int(type_schedule(np.array([p]), q, kind, period)[0])
        slots = np.where((key_pos[b] >= 0) & (key_pos[b] <= p))[0]
        if slots.size == 0:
            continue
        js = type_schedule(key_pos[b][slots], q, kind, period)
        # sel[a, k]: group a is compared for the k-th allowed slot
        sel = np.zeros((q, slots.size), dtype=bool)
        for k, j in enumerate(js):
            sel[score_support(i, int(j), q, L), k] = True
        k_pair = sel.sum(axis=0) * m
        for h in range(Hq):
            kv = h // (Hq // Hkv)
            K = Kc[b, kv][slots]
            r = np.zeros(slots.size)
            for a in range(q):
                r += np.where(sel[a], K[:, a * m:(a + 1) * m] @ Qn[b, h, a * m:(a + 1) * m], 0.0)
            s = r / np.sqrt(k_pair)
            w = np.exp(s - s.max())
            O[b, h] = (w / w.sum()) @ Vc[b, kv][slots]
    return O


def attention_decode_macs(p: int, key_pos: np.ndarray, q: int, d: int, L: int = 0, kind: str = "cyclic",
                          period: int = 0) -> tuple[int, int]:
    """(score MACs, value MACs) of one query head decoding position p against one cache
    (appendix G.2): each allowed key of type j costs |F(tau(p), j)| m score MACs, so for Q_q with
    n_j allowed keys of type j the score cost is m (2 N_p - n_i) (eq 57), and for the recursive
    law m sum_j 2^h(i, j) n_j (eq 61); the dense value sum costs N_p d."""
    key_pos = np.asarray(key_pos, dtype=np.int64)
    allowed = key_pos[(key_pos >= 0) & (key_pos <= p)]
    i = int(type_schedule(np.array([p]), q, kind, period)[0])
    js = type_schedule(allowed, q, kind, period)
    m = d // q
    score = sum(len(score_support(i, int(j), q, L)) * m for j in js)
    return score, allowed.size * d
