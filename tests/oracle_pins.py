"""Pins of the fp64 oracle against what the paper fixes, independent of the oracle's own code.

Each `pin_*` function raises AssertionError when the oracle module `O` disagrees
with a value, closed form or independent formula from arXiv 2609.32814.  They
are run against the real oracle (test_oracle_pins.py) and against oracles with
planted mistakes (test_oracle_mutations.py), which must each trip at least one pin.
"""
from __future__ import annotations

import itertools
import pathlib
from fractions import Fraction

import math

import numpy as np

GOLDEN = pathlib.Path(__file__).resolve().parent / "golden"


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _ints(g, shape, lo=-4, hi=5):
    return g.integers(lo, hi, size=shape).astype(np.float64)


def _bounds(widths):
    out, s = [], 0
    for w in widths:
        out.append((s, s + w))
        s += w
    return out


# --------------------------------------------------------------------------
# golden: the q = 2 law as printed (section 1, eq 1-3)
# --------------------------------------------------------------------------

def load_q2_products():
    rows = []
    for line in (GOLDEN / "q2_products.txt").read_text().splitlines():
        if not line.strip() or line.startswith("#"):
            continue
        xs, ws, zs, _name = line.split()
        rows.append(tuple(tuple(int(v) for v in t.split(",")) for t in (xs, ws, zs)))
    return rows


def load_q2_scalar():
    vals = {}
    for line in (GOLDEN / "q2_scalar_example.txt").read_text().splitlines():
        if not line.strip() or line.startswith("#"):
            continue
        key, *nums = line.split()
        vals[key] = np.array([float(v) for v in nums]).reshape(2, 2)
    return vals


def load_product_counts():
    out = []
    for line in (GOLDEN / "product_counts.txt").read_text().splitlines():
        if not line.strip() or line.startswith("#"):
            continue
        out.append(tuple(int(v) for v in line.split()))
    return out


def pin_q2_table(O):
    """The q=2 structure table is exactly the six products of eq (3)."""
    assert sorted(O.structure_table(2)) == sorted(load_q2_products())


def pin_q2_scalar_example(O):
    """Hand evaluation of eq (3) at small integers, square and row-typed forms."""
    v = load_q2_scalar()
    Z = O.square_product(v["X"], v["W"], 2)
    np.testing.assert_array_equal(Z, v["Q2"])
    # each token row uses one row of the table (section 1 / section 4)
    Y = O.row_typed_forward(v["X"], v["W"], np.array([0, 1]), 2)
    np.testing.assert_array_equal(Y, v["Q2"])
    # eq (2) differs exactly by the two removed cycle terms U W_v and V W_u
    diff = v["DENSE"] - v["Q2"]
    X, W = v["X"], v["W"]
    np.testing.assert_array_equal(diff, np.array([[X[0, 1] * W[1, 0], 0], [0, X[1, 0] * W[0, 1]]]))


def pin_eq3_rectangular_blocks(O, seed=11):
    """eq (3) with random rectangular blocks of unequal sizes equals the table-driven square form."""
    g = _rng(seed)
    m0, m1, k0, k1, n0, n1 = 3, 5, 4, 2, 6, 3
    A, U = g.standard_normal((m0, k0)), g.standard_normal((m0, k1))
    V, D = g.standard_normal((m1, k0)), g.standard_normal((m1, k1))
    Wa, Wu = g.standard_normal((k0, n0)), g.standard_normal((k0, n1))
    Wv, Wd = g.standard_normal((k1, n0)), g.standard_normal((k1, n1))
    X = np.block([[A, U], [V, D]])
    W = np.block([[Wa, Wu], [Wv, Wd]])
    want = np.block([[A @ Wa, A @ Wu + U @ Wd], [V @ Wa + D @ Wv, D @ Wd]])
    Z = O.square_product(X, W, 2, row_heights=[m0, m1], mid_widths=[k0, k1], out_widths=[n0, n1])
    np.testing.assert_allclose(Z, want, rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# eq 13-14 entry rule of Q_q; eq 15 counts; eq 12 for general graphs
# --------------------------------------------------------------------------

def pin_eq13_14(O, qs=(3, 4, 5), seed=12):
    """(A*B)_ii = A_ii B_ii ; (A*B)_ij = A_ii B_ij + A_ij B_jj, blockwise with unequal widths."""
    g = _rng(seed)
    for q in qs:
        hs = list(g.integers(1, 4, size=q))
        ks = list(g.integers(1, 4, size=q))
        ns = list(g.integers(1, 4, size=q))
        A = g.standard_normal((sum(hs), sum(ks)))
        B = g.standard_normal((sum(ks), sum(ns)))
        hb, kb, nb = _bounds(hs), _bounds(ks), _bounds(ns)
        Ab = lambda a, b: A[hb[a][0]:hb[a][1], kb[b][0]:kb[b][1]]
        Bb = lambda a, b: B[kb[a][0]:kb[a][1], nb[b][0]:nb[b][1]]
        want = np.zeros((sum(hs), sum(ns)))
        for i in range(q):
            for j in range(q):
                blk = Ab(i, i) @ Bb(i, j) if i == j else Ab(i, i) @ Bb(i, j) + Ab(i, j) @ Bb(j, j)
                want[hb[i][0]:hb[i][1], nb[j][0]:nb[j][1]] = blk
        Z = O.square_product(A, B, q, row_heights=hs, mid_widths=ks, out_widths=ns)
        np.testing.assert_allclose(Z, want, rtol=1e-12, atol=1e-12)


def pin_product_counts(O):
    """R(Q_q) = 2q^2 - q block GEMMs (eq 15), 2q - 1 per row, rho_q = (2q-1)/q^2 (eq 21)."""
    for q, total, per_row, rn, rd in load_product_counts():
        t = O.structure_table(q)
        assert len(t) == total == 2 * q * q - q
        for i in range(q):
            assert sum(1 for (x, _w, _z) in t if x[0] == i) == per_row == 2 * q - 1
        assert Fraction(per_row, q) / q == Fraction(rn, rd)
        # every slot of the algebra is a result at least once and dim = q^2 (eq 15)
        assert len({z for (_x, _w, z) in t}) == q * q
        # each product pairs matching inner indices: a juxtaposition is one block GEMM
        for x, w, z in t:
            assert x[1] == w[0] and z == (x[0], w[1])


def pin_graph_counts(O, seed=13):
    """R(Q_G) = |V| + 2|E| explicit products for random digraphs (eq 12, section 3.1)."""
    g = _rng(seed)
    for q in (1, 2, 3, 5, 7):
        all_e = [(a, b) for a in range(q) for b in range(q) if a != b]
        for _ in range(4):
            keep = [e for e in all_e if g.random() < 0.5]
            t = O.structure_table(q, keep)
            assert len(t) == q + 2 * len(keep)
            # eq 10-11: vertex i gets x_i w_i; edge ij gets x_i w_ij + x_ij w_j
            for (a, b) in keep:
                terms = sorted((x, w) for (x, w, z) in t if z == (a, b))
                assert terms == sorted([((a, a), (a, b)), ((a, b), (b, b))])
            for a in range(q):
                assert [(x, w) for (x, w, z) in t if z == (a, a)] == [((a, a), (a, a))]


# --------------------------------------------------------------------------
# appendix A (d, n) form; associativity; unit (eq 4, eq 6, eq 30, prop 3.1)
# --------------------------------------------------------------------------

def _scalar_square(O, d, n):
    """Element (d, n) of Q_q as a q x q array with d on the diagonal."""
    return np.diag(d) + n


def pin_appendix_a(O, seed=14):
    """(d,n)*(d',n') = (dd', dn' + nd') with (dn')_ij = d_i n'_ij, (nd')_ij = n_ij d'_j (eq 30)."""
    g = _rng(seed)
    for q in (1, 2, 3, 4, 5):
        off = 1.0 - np.eye(q)
        for _ in range(5):
            d, d2 = _ints(g, q), _ints(g, q)
            n, n2 = _ints(g, (q, q)) * off, _ints(g, (q, q)) * off
            Z = O.square_product(_scalar_square(O, d, n), _scalar_square(O, d2, n2), q)
            want_d = d * d2
            want_n = d[:, None] * n2 + n * d2[None, :]
            np.testing.assert_array_equal(np.diag(Z), want_d)
            np.testing.assert_array_equal(Z * off, want_n)


def _basis(q, slot):
    e = np.zeros((q, q))
    e[slot] = 1.0
    return e


def pin_associativity(O, seed=15):
    """(x*y)*z = x*(y*z): every basis triple for q <= 4, random integer elements for q <= 5 (eq 4, eq 30)."""
    for q in (1, 2, 3, 4):
        slots = [(a, b) for a in range(q) for b in range(q)]
        prod = {}
        for s1 in slots:
            for s2 in slots:
                prod[s1, s2] = O.square_product(_basis(q, s1), _basis(q, s2), q)
        for s1, s2, s3 in itertools.product(slots, repeat=3):
            left = O.square_product(prod[s1, s2], _basis(q, s3), q)
            right = O.square_product(_basis(q, s1), prod[s2, s3], q)
            np.testing.assert_array_equal(left, right)
    g = _rng(seed)
    for q in (2, 3, 5):
        for _ in range(3):
            x, y, z = (_ints(g, (2 * q, 2 * q)) for _ in range(3))
            np.testing.assert_array_equal(O.square_product(O.square_product(x, y, q), z, q),
                                          O.square_product(x, O.square_product(y, z, q), q))


def pin_row_typed_composition(O, seed=16):
    """Phi_{W2}(Phi_{W1}(X)) = Phi_{W1 * W2}(X) for the row-typed maps (eq 4, eq 6; section 4)."""
    g = _rng(seed)
    for q in (1, 2, 3, 4):
        s = 2
        K = q * s
        M = 7
        X = _ints(g, (M, K))
        W1, W2 = _ints(g, (K, K)), _ints(g, (K, K))
        tau = g.integers(0, q, size=M)
        lhs = O.row_typed_forward(O.row_typed_forward(X, W1, tau, q), W2, tau, q)
        rhs = O.row_typed_forward(X, O.square_product(W1, W2, q), tau, q)
        np.testing.assert_array_equal(lhs, rhs)


def pin_unit_laws(O, seed=17):
    """E = block identity: X*E = X and E*W = W (section 1, prop 3.1); row-typed identity bank (section 4)."""
    g = _rng(seed)
    for q in (1, 2, 3, 4, 6):
        n = 2 * q
        X, W = g.standard_normal((n, n)), g.standard_normal((n, n))
        E = np.eye(n)
        np.testing.assert_array_equal(O.square_product(X, E, q), X)
        np.testing.assert_array_equal(O.square_product(E, W, q), W)
        # row-typed: a diagonal bank of identity maps is the identity projection
        M = 9
        Xr = g.standard_normal((M, n))
        tau = g.integers(0, q, size=M)
        np.testing.assert_array_equal(O.row_typed_forward(Xr, E, tau, q), Xr)
        # and feeding the identity's rows with interval types floor(m / s) returns W (Phi_w(1) = w)
        s = n // q
        tau_i = np.arange(n) // s
        np.testing.assert_array_equal(O.row_typed_forward(E, W, tau_i, q), W)


# --------------------------------------------------------------------------
# row-typed form (section 4, eq 16-17; eq 27; Algorithm 1)
# --------------------------------------------------------------------------

def brute_force_row_typed(X, W, tau, q, kw, nw):
    """Scalar loops over eq 16-17 directly: y_i = x_i W_ii, y_j = x_i W_ij + x_j W_jj."""
    kb, nb = _bounds(kw), _bounds(nw)
    M = X.shape[0]
    Y = np.zeros((M, W.shape[1]))
    for m in range(M):
        i = int(tau[m])
        if not 0 <= i < q:
            continue
        for j in range(q):
            for c in range(nb[j][0], nb[j][1]):
                acc = 0.0
                for k in range(kb[i][0], kb[i][1]):
                    acc += X[m, k] * W[k, c]
                if j != i:
                    for k in range(kb[j][0], kb[j][1]):
                        acc += X[m, k] * W[k, c]
                Y[m, c] = acc
    return Y


def pin_brute_force(O, seed=18):
    """Table-driven Algorithm 1 equals scalar eq 16-17 (unequal widths, absent and invalid types)."""
    g = _rng(seed)
    for q in (1, 2, 3, 4):
        kw = list(g.integers(1, 4, size=q))
        nw = list(g.integers(1, 4, size=q))
        M = 11
        X = g.standard_normal((M, sum(kw)))
        W = g.standard_normal((sum(kw), sum(nw)))
        tau = g.integers(0, q, size=M)
        tau[3] = q          # out of range: no type, zero row
        tau[5] = -1
        Y = O.row_typed_forward(X, W, tau, q, in_widths=kw, out_widths=nw)
        np.testing.assert_allclose(Y, brute_force_row_typed(X, W, tau, q, kw, nw), rtol=1e-12, atol=1e-12)


def masked_bank(W, i, q):
    """T_i(W): W with every block (a, b), a != i and a != b, set to zero.

    Generalises the slide deck's teaching matrix T_1(W) = [[W11, W12], [0, W22]]
    (derived there from eq 16-17): a type-i row sees its own block row and the diagonal.
    """
    K, N = W.shape
    s, r = K // q, N // q
    T = W.copy()
    for a in range(q):
        for b in range(q):
            if a != i and a != b:
                T[a * s:(a + 1) * s, b * r:(b + 1) * r] = 0.0
    return T


def pin_teaching_matrix(O):
    """q=2: T_1(W) = [[W11, W12], [0, W22]] and T_2(W) = [[W11, 0], [W21, W22]]."""
    W = np.array([[5.0, 6.0], [7.0, 8.0]])
    np.testing.assert_array_equal(masked_bank(W, 0, 2), [[5, 6], [0, 8]])
    np.testing.assert_array_equal(masked_bank(W, 1, 2), [[5, 0], [7, 8]])
    for i in range(2):
        x = np.array([[1.0 + 2 * i, 2.0 + 2 * i]])
        np.testing.assert_array_equal(O.row_typed_forward(x, W, np.array([i]), 2), x @ masked_bank(W, i, 2))


def pin_masked_dense(O, seed=19):
    """Y[I_i] = X[I_i] T_i(W) by plain matmul: an independent formula, like the paper's checks."""
    g = _rng(seed)
    for q, M, s, r in ((2, 10, 3, 4), (3, 13, 2, 5), (4, 17, 3, 2), (5, 9, 1, 1)):
        X = g.standard_normal((M, q * s))
        W = g.standard_normal((q * s, q * r))
        tau = g.integers(0, q, size=M)
        Y = O.row_typed_forward(X, W, tau, q)
        for m in range(M):
            want = X[m] @ masked_bank(W, int(tau[m]), q)
            np.testing.assert_allclose(Y[m], want, rtol=1e-12, atol=1e-13)


def pin_graph_masked_dense(O, seed=41):
    """Q_G rows by plain matmul (section 3.1, eq 10-11): a type-i row sees block (i, i), and for
    each edge (i, b) the blocks (i, b) and (b, b); every other block of W is masked to zero."""
    g = _rng(seed)
    for q, M, s, r in ((3, 11, 2, 3), (4, 15, 3, 2), (5, 12, 1, 2)):
        X = g.standard_normal((M, q * s))
        W = g.standard_normal((q * s, q * r))
        tau = g.integers(0, q, size=M)
        edges = [(a, b) for a in range(q) for b in range(q) if a != b and g.random() < 0.5]
        Y = O.row_typed_forward(X, W, tau, q, edges=edges)
        for m in range(M):
            i = int(tau[m])
            T = np.zeros_like(W)
            T[i * s:(i + 1) * s, i * r:(i + 1) * r] = W[i * s:(i + 1) * s, i * r:(i + 1) * r]
            for b in range(q):
                if (i, b) in edges:
                    T[i * s:(i + 1) * s, b * r:(b + 1) * r] = W[i * s:(i + 1) * s, b * r:(b + 1) * r]
                    T[b * s:(b + 1) * s, b * r:(b + 1) * r] = W[b * s:(b + 1) * s, b * r:(b + 1) * r]
            np.testing.assert_allclose(Y[m], X[m] @ T, rtol=1e-12, atol=1e-13)


def pin_row_typed_is_square_rows(O, seed=20):
    """Rows grouped by type form the square form's block rows (section 1: one row of the table per token)."""
    g = _rng(seed)
    for q, M in ((2, 9), (3, 14), (4, 6)):
        s, r = 2, 3
        X = g.standard_normal((M, q * s))
        W = g.standard_normal((q * s, q * r))
        tau = g.integers(0, q, size=M)
        order = np.argsort(tau, kind="stable")
        heights = [int((tau == i).sum()) for i in range(q)]
        Z = O.square_product(X[order], W, q, row_heights=heights)
        Y = np.empty_like(Z)
        Y[order] = Z
        np.testing.assert_allclose(O.row_typed_forward(X, W, tau, q), Y, rtol=1e-13, atol=1e-13)


def pin_q1_is_matmul(O, seed=21):
    """Q_1 is the ground field: one group, the projection is X W (eq 13 at q = 1)."""
    g = _rng(seed)
    X, W = g.standard_normal((7, 6)), g.standard_normal((6, 5))
    np.testing.assert_allclose(O.row_typed_forward(X, W, np.zeros(7, np.int32), 1), X @ W, rtol=1e-14, atol=1e-14)


def pin_block_diagonal(O, seed=22):
    """With W_ij = 0 for i != j every type computes X W (eq 16-17 lose their cross terms)."""
    g = _rng(seed)
    q, s, r, M = 4, 3, 2, 15
    X = g.standard_normal((M, q * s))
    W = np.zeros((q * s, q * r))
    for a in range(q):
        W[a * s:(a + 1) * s, a * r:(a + 1) * r] = g.standard_normal((s, r))
    tau = g.integers(0, q, size=M)
    np.testing.assert_allclose(O.row_typed_forward(X, W, tau, q), X @ W, rtol=1e-13, atol=1e-14)


def pin_coverage(O, seed=23):
    """A weight in block (a, b) reaches rows of every type if a == b, else only type a, in group b only (section 4)."""
    g = _rng(seed)
    q, s, r, M = 3, 2, 2, 12
    X = g.standard_normal((M, q * s)) + 3.0       # no zero entries
    tau = np.arange(M) % q
    for a in range(q):
        for b in range(q):
            W = np.zeros((q * s, q * r))
            k0, c0 = a * s + 1, b * r + 1
            W[k0, c0] = 1.0
            Y = O.row_typed_forward(X, W, tau, q)
            nz = Y != 0
            want = np.zeros_like(nz)
            for m in range(M):
                if a == b or tau[m] == a:
                    want[m, c0] = True
            np.testing.assert_array_equal(nz, want)
            np.testing.assert_array_equal(Y[want], X[want[:, c0], k0])


# --------------------------------------------------------------------------
# VJPs (appendix B, eq 31-35)
# --------------------------------------------------------------------------

def pin_vjp_scalar_eq31_35(O, seed=24):
    """Per-token accumulation of eq 31-35 written out, versus the oracle's transposed table."""
    g = _rng(seed)
    for q, M, s, r in ((2, 5, 2, 3), (3, 7, 2, 2), (4, 9, 1, 2)):
        X = g.standard_normal((M, q * s))
        W = g.standard_normal((q * s, q * r))
        dY = g.standard_normal((M, q * r))
        tau = g.integers(0, q, size=M)
        dX_w = np.zeros_like(X)
        dW_w = np.zeros_like(W)
        xs = lambda m, a: X[m, a * s:(a + 1) * s]
        ys = lambda m, a: dY[m, a * r:(a + 1) * r]
        Wb = lambda a, b: W[a * s:(a + 1) * s, b * r:(b + 1) * r]
        for m in range(M):
            i = int(tau[m])
            dX_w[m, i * s:(i + 1) * s] += ys(m, i) @ Wb(i, i).T          # eq 31, first term
            for j in range(q):
                if j == i:
                    continue
                dX_w[m, i * s:(i + 1) * s] += ys(m, j) @ Wb(i, j).T      # eq 31, sum over j != i
                dX_w[m, j * s:(j + 1) * s] += ys(m, j) @ Wb(j, j).T      # eq 32
                dW_w[i * s:(i + 1) * s, j * r:(j + 1) * r] += np.outer(xs(m, i), ys(m, j))   # eq 34
                dW_w[j * s:(j + 1) * s, j * r:(j + 1) * r] += np.outer(xs(m, j), ys(m, j))   # eq 35
            dW_w[i * s:(i + 1) * s, i * r:(i + 1) * r] += np.outer(xs(m, i), ys(m, i))       # eq 33
        dX, dW = O.row_typed_backward(X, W, dY, tau, q)
        np.testing.assert_allclose(dX, dX_w, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dW, dW_w, rtol=1e-12, atol=1e-12)


def pin_vjp_autograd(O, seed=25):
    """float64 torch autograd of the masked-dense form equals the oracle's dX and dW."""
    import torch
    g = _rng(seed)
    for q, M, s, r in ((2, 12, 3, 2), (3, 10, 2, 4), (5, 16, 2, 1)):
        Xn = g.standard_normal((M, q * s))
        Wn = g.standard_normal((q * s, q * r))
        dYn = g.standard_normal((M, q * r))
        tau = g.integers(0, q, size=M)
        X = torch.tensor(Xn, requires_grad=True)
        W = torch.tensor(Wn, requires_grad=True)
        rows = []
        for m in range(M):
            i = int(tau[m])
            mask = torch.tensor(masked_bank(np.ones_like(Wn), i, q))
            rows.append(X[m:m + 1] @ (W * mask))
        Y = torch.cat(rows)
        (Y * torch.tensor(dYn)).sum().backward()
        dX, dW = O.row_typed_backward(Xn, Wn, dYn, tau, q)
        np.testing.assert_allclose(dX, X.grad.numpy(), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dW, W.grad.numpy(), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(O.row_typed_forward(Xn, Wn, tau, q), Y.detach().numpy(), rtol=1e-12, atol=1e-12)


def _graph_mask(q, s, r, i, edges):
    """Ones where a type-i row reads W under Q_G (section 3.1, eq 10-11), zeros elsewhere."""
    T = np.zeros((q * s, q * r))
    T[i * s:(i + 1) * s, i * r:(i + 1) * r] = 1.0
    for b in range(q):
        if (i, b) in edges:
            T[i * s:(i + 1) * s, b * r:(b + 1) * r] = 1.0
            T[b * s:(b + 1) * s, b * r:(b + 1) * r] = 1.0
    return T


def pin_graph_vjp_autograd(O, seed=42):
    """float64 torch autograd of the Q_G masked-dense rows equals the oracle's graph dX and dW."""
    import torch
    g = _rng(seed)
    for q, M, s, r in ((3, 14, 2, 3), (4, 17, 3, 2), (5, 11, 1, 2)):
        Xn = g.standard_normal((M, q * s))
        Wn = g.standard_normal((q * s, q * r))
        dYn = g.standard_normal((M, q * r))
        tau = g.integers(0, q, size=M)
        edges = [(a, b) for a in range(q) for b in range(q) if a != b and g.random() < 0.5]
        X = torch.tensor(Xn, requires_grad=True)
        W = torch.tensor(Wn, requires_grad=True)
        Y = torch.cat([X[m:m + 1] @ (W * torch.tensor(_graph_mask(q, s, r, int(tau[m]), edges)))
                       for m in range(M)])
        (Y * torch.tensor(dYn)).sum().backward()
        dX, dW = O.row_typed_backward(Xn, Wn, dYn, tau, q, edges=edges)
        np.testing.assert_allclose(dX, X.grad.numpy(), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dW, W.grad.numpy(), rtol=1e-12, atol=1e-12)


def pin_widths_vjp_autograd(O, seed=43):
    """Unequal widths (eq 18): float64 autograd of the masked-dense rows equals the oracle's dX, dW."""
    import torch
    g = _rng(seed)
    for kw, nw, M in (([2, 5, 1], [3, 1, 4], 13), ([4, 1], [2, 6], 9), ([1, 3, 2, 2], [2, 2, 5, 1], 15)):
        q = len(kw)
        kb, nb = _bounds(kw), _bounds(nw)
        Xn = g.standard_normal((M, sum(kw)))
        Wn = g.standard_normal((sum(kw), sum(nw)))
        dYn = g.standard_normal((M, sum(nw)))
        tau = g.integers(0, q, size=M)
        X = torch.tensor(Xn, requires_grad=True)
        W = torch.tensor(Wn, requires_grad=True)
        rows = []
        for m in range(M):
            i = int(tau[m])
            T = np.zeros_like(Wn)
            for a in range(q):
                for b in range(q):
                    if a == i or a == b:
                        T[kb[a][0]:kb[a][1], nb[b][0]:nb[b][1]] = 1.0
            rows.append(X[m:m + 1] @ (W * torch.tensor(T)))
        (torch.cat(rows) * torch.tensor(dYn)).sum().backward()
        dX, dW = O.row_typed_backward(Xn, Wn, dYn, tau, q, in_widths=kw, out_widths=nw)
        np.testing.assert_allclose(dX, X.grad.numpy(), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dW, W.grad.numpy(), rtol=1e-12, atol=1e-12)


def pin_vjp_adjoint(O, seed=26):
    """Bilinearity: <dY, Y> = <dX, X> = <dW, W>; dW blocks with no contributing rows are zero."""
    g = _rng(seed)
    q, M, s, r = 4, 6, 3, 2
    X = g.standard_normal((M, q * s))
    W = g.standard_normal((q * s, q * r))
    dY = g.standard_normal((M, q * r))
    tau = np.array([0, 0, 2, 2, 0, 2])          # types 1 and 3 absent
    Y = O.row_typed_forward(X, W, tau, q)
    dX, dW = O.row_typed_backward(X, W, dY, tau, q)
    a = float((dY * Y).sum())
    np.testing.assert_allclose(float((dX * X).sum()), a, rtol=1e-12)
    np.testing.assert_allclose(float((dW * W).sum()), a, rtol=1e-12)
    for b in range(q):
        for j in range(q):
            blk = dW[b * s:(b + 1) * s, j * r:(j + 1) * r]
            if b != j and b in (1, 3):
                assert not blk.any()                 # off-diagonal rows of absent types
            else:
                assert blk.any()


# --------------------------------------------------------------------------
# cost (eq 18-19, 21, 24) and index / schedule (section 4, Algorithm 1, App D.5)
# --------------------------------------------------------------------------

def pin_mac_count(O, seed=27):
    """MACs = rho_q M K N for equal groups (eq 24); sum_i M_i C_i with C_i of eq 18 in general."""
    g = _rng(seed)
    for q in (1, 2, 3, 4, 8):
        M, s, r = 37, 2 * q, 3
        tau = g.integers(0, q, size=M)
        gemms, macs = O.mac_count(tau, q, q * s, q * r)
        assert Fraction(macs) == Fraction(2 * q - 1, q * q) * M * (q * s) * (q * r)
        assert gemms == (2 * q - 1) * len(set(tau.tolist()))
    q = 3
    kw, nw = [2, 5, 1], [4, 1, 3]
    K, N = sum(kw), sum(nw)
    tau = np.array([0, 2, 2, 1, 0, 0, 2])
    Ddiag = sum(a * b for a, b in zip(kw, nw))
    want = sum(int((tau == i).sum()) * (Ddiag + kw[i] * (N - nw[i])) for i in range(q))
    assert O.mac_count(tau, q, K, N, kw, nw)[1] == want


def pin_type_index(O, seed=28):
    """Cyclic types with any offset give arithmetic row progressions; arbitrary types a stable partition."""
    for q in (1, 2, 3, 4, 8):
        for M in (0, 1, 5, 16, 37):
            for o in (0, 1, q - 1, 5):
                tau = (np.arange(M) + o) % q
                counts, offsets, rows, bad = O.type_index(tau, q)
                assert bad == 0
                for i in range(q):
                    start = (i - o) % q
                    cnt = max(0, -(-(M - start) // q))
                    assert counts[i] == cnt
                    np.testing.assert_array_equal(rows[offsets[i]:offsets[i + 1]], start + q * np.arange(cnt))
    g = _rng(seed)
    for q in (1, 3, 7):
        tau = g.integers(-1, q + 1, size=50)
        counts, offsets, rows, bad = O.type_index(tau, q)
        assert bad == int(((tau < 0) | (tau >= q)).sum())
        assert offsets[0] == 0 and offsets[-1] == 50 - bad
        for i in range(q):
            seg = rows[offsets[i]:offsets[i + 1]]
            np.testing.assert_array_equal(seg, np.flatnonzero(tau == i))


def pin_type_schedule(O):
    """Section 4's 1 + ((p-1) mod q) with 1-based p is p mod q 0-based; App D.5's floor((p mod 768)/192)."""
    p1 = np.arange(1, 200)
    for q in (1, 2, 3, 8):
        paper = 1 + ((p1 - 1) % q)
        np.testing.assert_array_equal(O.type_schedule(p1 - 1, q) + 1, paper)
    p = np.array([0, 191, 192, 383, 384, 575, 576, 767, 768, 959, 1535, 1536])
    np.testing.assert_array_equal(O.type_schedule(p, 4, "interval", 768), [0, 0, 1, 1, 2, 2, 3, 3, 0, 0, 3, 0])


# --------------------------------------------------------------------------
# gated FFN (section 4; appendix D's SwiGLU)
# --------------------------------------------------------------------------

def pin_silu_values(O):
    """silu(0) = 0, silu(x) - silu(-x) = x (sigmoid(x) + sigmoid(-x) = 1), silu(x) -> x and -> 0 at the tails,
    and silu(1) = 1 / (1 + 1/e) written out."""
    x = np.linspace(-30.0, 30.0, 121)
    np.testing.assert_allclose(O.silu(x) - O.silu(-x), x, rtol=1e-14, atol=1e-14)
    assert O.silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(O.silu(np.array([40.0])), [40.0], rtol=1e-15)
    assert abs(O.silu(np.array([-40.0]))[0]) < 1e-15
    np.testing.assert_allclose(O.silu(np.array([1.0])), [1.0 / (1.0 + np.exp(-1.0))], rtol=1e-15)


def pin_gated_masked_dense(O, seed=31):
    """Each gated row is silu(x T_i(W_gate)) * (x T_i(W_up)) with the masked banks, scalar silu per element."""
    g = _rng(seed)
    for q, M, s, r in ((2, 7, 3, 2), (3, 9, 2, 3), (1, 5, 4, 3)):
        X = g.standard_normal((M, q * s))
        Wg = g.standard_normal((q * s, q * r))
        Wu = g.standard_normal((q * s, q * r))
        tau = g.integers(0, q, size=M)
        H = O.gated_forward(X, Wg, Wu, tau, q)
        for m in range(M):
            i = int(tau[m])
            gv = X[m] @ masked_bank(Wg, i, q)
            uv = X[m] @ masked_bank(Wu, i, q)
            for n in range(q * r):
                want = gv[n] / (1.0 + math.exp(-gv[n])) * uv[n]
                assert abs(H[m, n] - want) <= 1e-12 * (1.0 + abs(want)), (q, m, n)


def pin_silu_grad(O):
    """silu' from central differences of silu (error O(h^2)), silu'(0) = 1/2, and
    silu'(x) + silu'(-x) = 1 (the derivative of silu(x) - silu(-x) = x)."""
    x = np.linspace(-12.0, 12.0, 97)
    h = 1e-5
    fd = (O.silu(x + h) - O.silu(x - h)) / (2 * h)
    np.testing.assert_allclose(O.silu_grad(x), fd, rtol=1e-8, atol=1e-9)
    assert O.silu_grad(np.array([0.0]))[0] == 0.5
    np.testing.assert_allclose(O.silu_grad(x) + O.silu_grad(-x), np.ones_like(x), rtol=1e-14, atol=1e-14)


def pin_gated_ffn_autograd(O, seed=33):
    """float64 torch autograd of the masked-dense gated FFN, silu(x T_i(W_g)) * (x T_i(W_u)) then
    T_i(W_d), equals the oracle's forward and its (dX, dW_gate, dW_up, dW_down)."""
    import torch
    g = _rng(seed)
    for q, M, s, r in ((2, 9, 3, 2), (3, 8, 2, 3), (4, 11, 1, 2)):
        D, F = q * s, q * r
        Xn = g.standard_normal((M, D))
        Wgn = g.standard_normal((D, F))
        Wun = g.standard_normal((D, F))
        Wdn = g.standard_normal((F, D))
        dYn = g.standard_normal((M, D))
        tau = g.integers(0, q, size=M)
        X, Wg, Wu, Wd = (torch.tensor(a, requires_grad=True) for a in (Xn, Wgn, Wun, Wdn))
        rows = []
        for m in range(M):
            i = int(tau[m])
            mk = lambda W: torch.tensor(masked_bank(np.ones(W.shape), i, q))  # noqa: E731
            h = torch.nn.functional.silu(X[m:m + 1] @ (Wg * mk(Wgn))) * (X[m:m + 1] @ (Wu * mk(Wun)))
            rows.append(h @ (Wd * mk(Wdn)))
        Y = torch.cat(rows)
        (Y * torch.tensor(dYn)).sum().backward()
        Yo, _ = O.gated_ffn_forward(Xn, Wgn, Wun, Wdn, tau, q)
        np.testing.assert_allclose(Yo, Y.detach().numpy(), rtol=1e-12, atol=1e-12)
        got = O.gated_ffn_backward(Xn, Wgn, Wun, Wdn, dYn, tau, q)
        for a, t in zip(got, (X, Wg, Wu, Wd)):
            np.testing.assert_allclose(a, t.grad.numpy(), rtol=1e-11, atol=1e-11)


# --------------------------------------------------------------------------
# the recursive law Q_2^{(x)L} (appendix C; section 6.1's B(i, j) for it)
# --------------------------------------------------------------------------

def _bits_support(a, d, L):
    """eq 36's index set: the beta whose every bit equals alpha's or delta's bit."""
    return {b for b in range(2 ** L) if all(((b >> k) & 1) in (((a >> k) & 1), ((d >> k) & 1)) for k in range(L))}


def tensor_masked_bank(W, a, L):
    """W with block (beta, delta) zeroed unless beta's bits each come from alpha or delta."""
    q = 2 ** L
    K, N = W.shape
    s, r = K // q, N // q
    T = W.copy()
    for b in range(q):
        for d in range(q):
            if b not in _bits_support(a, d, L):
                T[b * s:(b + 1) * s, d * r:(d + 1) * r] = 0.0
    return T


def pin_tensor_counts(O):
    """6^L triples (the recursive algorithm's 6^L products, appendix C.1); L = 1 is Q_2; at L = 2 the
    4 * 1 + 8 * 2 + 4 * 4 = 36 split by Hamming distance of the endpoints."""
    for L in (1, 2, 3):
        assert len(O.tensor_power_table(L)) == 6 ** L
    assert sorted(O.tensor_power_table(1)) == sorted(O.structure_table(2))
    per_pair = {}
    for (a, b), (_, d), out in O.tensor_power_table(2):
        assert out == (a, d)
        per_pair[(a, d)] = per_pair.get((a, d), 0) + 1
    hist = {}
    for (a, d), n in per_pair.items():
        h = bin(a ^ d).count("1")
        assert n == 2 ** h
        hist[h] = hist.get(h, 0) + 1
    assert hist == {0: 4, 1: 8, 2: 4}


def pin_tensor_support(O):
    """For every (alpha, delta), the intermediate groups of the table are eq 36's set."""
    for L in (1, 2, 3):
        got = {}
        for (a, b), (b2, d), _ in O.tensor_power_table(L):
            assert b == b2
            got.setdefault((a, d), set()).add(b)
        for a in range(2 ** L):
            for d in range(2 ** L):
                assert got.get((a, d), set()) == _bits_support(a, d, L), (L, a, d)


def pin_tensor_associativity(O):
    """The tensor power is associative (all basis triples at L = 2), and unlike Q_4 its radical (slots
    with a != b) does not square to zero (appendix C: J (x) J is nonzero)."""
    L = 2
    prod = {}
    for x, y, z in O.tensor_power_table(L):
        prod[(x, y)] = z
    slots = [(a, b) for a in range(4) for b in range(4)]

    def mul(x, y):
        return None if x is None or y is None else prod.get((x, y))

    for x in slots:
        for y in slots:
            for z in slots:
                assert mul(mul(x, y), z) == mul(x, mul(y, z)), (x, y, z)
    rad = [x for x in slots if x[0] != x[1]]
    assert any(mul(x, y) is not None for x in rad for y in rad)
    q4 = {(x, y) for x, y, _ in O.structure_table(4)}
    assert not any((x, y) in q4 for x in rad for y in rad)


def pin_tensor_masked_dense(O, seed=41):
    """Row-typed evaluation with the tensor table equals x T_alpha(W) with the bit-rule mask."""
    g = _rng(seed)
    for L, M, s, r in ((1, 7, 2, 3), (2, 12, 2, 2), (3, 10, 1, 2)):
        q = 2 ** L
        X = g.standard_normal((M, q * s))
        W = g.standard_normal((q * s, q * r))
        tau = g.integers(0, q, size=M)
        Y = O.row_typed_forward(X, W, tau, q, table=O.tensor_power_table(L))
        for m in range(M):
            want = X[m] @ tensor_masked_bank(W, int(tau[m]), L)
            np.testing.assert_allclose(Y[m], want, rtol=1e-12, atol=1e-12)


def pin_tensor_cost(O, seed=42):
    """eq 36 per type on unequal widths; equal widths and uniform types give (3/4)^L of dense (C.1)."""
    g = _rng(seed)
    L = 2
    q = 4
    sw = [3, 1, 4, 2]
    rw = [2, 5, 1, 3]
    tau = np.array([0, 1, 1, 2, 3, 3, 3])
    _, macs = O.mac_count(tau, q, sum(sw), sum(rw), sw, rw, table=O.tensor_power_table(L))
    want = 0
    for a in range(q):
        Ma = int(np.sum(tau == a))
        for d in range(q):
            for b in _bits_support(a, d, L):
                want += Ma * sw[b] * rw[d]
    assert macs == want
    for L in (1, 2, 3):
        q = 2 ** L
        tau = np.repeat(np.arange(q), 3)
        K, N = 2 * q, 3 * q
        _, macs = O.mac_count(tau, q, K, N, table=O.tensor_power_table(L))
        assert macs * 4 ** L == 3 ** L * tau.size * K * N
    del g


def pin_tensor_vjp_autograd(O, seed=43):
    """float64 torch autograd of the tensor law's masked-dense form equals the table-driven VJPs."""
    import torch
    g = _rng(seed)
    for L, M, s, r in ((2, 11, 2, 3), (3, 9, 1, 1)):
        q = 2 ** L
        Xn = g.standard_normal((M, q * s))
        Wn = g.standard_normal((q * s, q * r))
        dYn = g.standard_normal((M, q * r))
        tau = g.integers(0, q, size=M)
        X = torch.tensor(Xn, requires_grad=True)
        W = torch.tensor(Wn, requires_grad=True)
        rows = [X[m:m + 1] @ (W * torch.tensor(tensor_masked_bank(np.ones_like(Wn), int(tau[m]), L)))
                for m in range(M)]
        (torch.cat(rows) * torch.tensor(dYn)).sum().backward()
        dX, dW = O.row_typed_backward(Xn, Wn, dYn, tau, q, table=O.tensor_power_table(L))
        np.testing.assert_allclose(dX, X.grad.numpy(), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dW, W.grad.numpy(), rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# algebraic attention scores (appendix G)
# --------------------------------------------------------------------------

def pin_attention_q1_is_sdpa(O, seed=51):
    """q = 1 is ordinary causal attention with 1/sqrt(d): fp64 torch scaled_dot_product_attention."""
    import torch
    g = _rng(seed)
    Q = g.standard_normal((4, 13, 8))
    K = g.standard_normal((2, 13, 8))
    V = g.standard_normal((2, 13, 8))
    got = O.algebraic_attention(Q, K, V, np.zeros(13, int), 1)
    Kx = torch.tensor(np.repeat(K, 2, axis=0))
    Vx = torch.tensor(np.repeat(V, 2, axis=0))
    want = torch.nn.functional.scaled_dot_product_attention(torch.tensor(Q), Kx, Vx, is_causal=True).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def _softmax_rows(s):
    s = s - s.max(axis=1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=1, keepdims=True)


def pin_attention_scores_are_typed_product(O, seed=52):
    """Before normalisation the score matrix is Q *_{Q_q} K^T with keys grouped by type (appendix G:
    the block S_ij = Q_ii K_ji^T + Q_ij K_jj^T): the row-typed projection of Q with the bank K^T
    (columns sorted by key type), scaled per pair by 1/sqrt(|F| m), then the causal softmax and PV."""
    g = _rng(seed)
    for q, S, d in ((4, 12, 8), (2, 10, 6), (3, 9, 6)):
        Q = g.standard_normal((1, S, d))
        K = g.standard_normal((1, S, d))
        V = g.standard_normal((1, S, d))
        tau = np.arange(S) % q
        perm = np.argsort(tau, kind="stable")
        Z = O.row_typed_forward(Q[0], K[0][perm].T, tau, q)
        r = np.empty_like(Z)
        r[:, perm] = Z
        m = d // q
        k = np.where(tau[:, None] == tau[None, :], m, 2 * m)
        s = np.where(np.tri(S, dtype=bool), r / np.sqrt(k), -np.inf)
        want = _softmax_rows(s) @ V[0]
        np.testing.assert_allclose(O.algebraic_attention(Q, K, V, tau, q)[0], want, rtol=1e-12, atol=1e-12)


def pin_attention_scale_and_mask(O):
    """With all-ones Q and K the score is sqrt(|F| m) (eq 41); V = I reads P back: P_pu is
    proportional to exp(sqrt(m)) for equal types and exp(sqrt(2m)) otherwise, zero for u > p."""
    q, S = 4, 8
    d = S
    m = d // q
    tau = np.arange(S) % q
    P = O.algebraic_attention(np.ones((1, S, d)), np.ones((1, S, d)), np.eye(S)[None], tau, q)[0]
    for p in range(S):
        w = np.array([np.exp(np.sqrt(m if tau[u] == tau[p] else 2 * m)) if u <= p else 0.0 for u in range(S)])
        np.testing.assert_allclose(P[p], w / w.sum(), rtol=1e-13, atol=1e-15)


def pin_attention_causality(O, seed=53):
    """Proposition G.1: keys and values after position p do not change O_p."""
    g = _rng(seed)
    Q = g.standard_normal((2, 16, 8))
    K = g.standard_normal((2, 16, 8))
    V = g.standard_normal((2, 16, 8))
    tau = np.arange(16) % 4
    a = O.algebraic_attention(Q, K, V, tau, 4)
    K2, V2 = K.copy(), V.copy()
    K2[:, 9:] += 5.0
    V2[:, 9:] -= 3.0
    b = O.algebraic_attention(Q, K2, V2, tau, 4)
    assert np.array_equal(a[:, :9], b[:, :9])
    assert not np.allclose(a[:, 9:], b[:, 9:])


def pin_attention_gqa(O, seed=54):
    """Query head h uses key/value head h // (Hq / Hkv): the same as repeating each K/V head."""
    g = _rng(seed)
    Q = g.standard_normal((6, 10, 8))
    K = g.standard_normal((2, 10, 8))
    V = g.standard_normal((2, 10, 8))
    tau = np.arange(10) % 2
    a = O.algebraic_attention(Q, K, V, tau, 2)
    b = O.algebraic_attention(Q, np.repeat(K, 3, axis=0), np.repeat(V, 3, axis=0), tau, 2)
    np.testing.assert_allclose(a, b, rtol=0, atol=0)


def pin_attention_laws_and_counts(O):
    """eq 38 and eq 42 supports; L = 1 is Q_2; score MACs are (2M - M_eq) m (eq 45) over the allowed
    pairs, value MACs M d."""
    assert O.score_support(2, 2, 4) == [2] and O.score_support(3, 1, 4) == [3, 1]
    for L in (1, 2, 3):
        q = 2 ** L
        for i in range(q):
            for j in range(q):
                assert set(O.score_support(i, j, q, L)) == _bits_support(i, j, L)
    for i in range(2):
        for j in range(2):
            assert sorted(O.score_support(i, j, 2, 1)) == sorted(O.score_support(i, j, 2))
    for q, S, d in ((4, 37, 8), (3, 20, 6), (1, 9, 4)):
        tau = np.arange(S) % q
        sm, vm = O.attention_score_macs(tau, q, d)
        Mp = S * (S + 1) // 2
        Meq = sum(1 for p in range(S) for u in range(p + 1) if tau[u] == tau[p])
        assert sm == (2 * Mp - Meq) * (d // q) and vm == Mp * d


def pin_attention_type_offset(O, seed=55):
    """A sequence chunk starting at absolute position p0 has types (p0 + s) mod q: its scores are
    Q *_{Q_q} K^T under those types (the typed-product closed form of the block S_ij, with the
    key columns sorted by type), and for p0 not a multiple of q they differ from p0 = 0 (the
    offset changes which F(i, j) each pair uses)."""
    g = _rng(seed)
    for q, S, d, p0 in ((4, 12, 8, 5), (3, 9, 6, 7), (2, 10, 4, 3)):
        Q = g.standard_normal((1, S, d))
        K = g.standard_normal((1, S, d))
        V = g.standard_normal((1, S, d))
        pos = p0 + np.arange(S)
        tau = pos % q
        perm = np.argsort(tau, kind="stable")
        Z = O.row_typed_forward(Q[0], K[0][perm].T, tau, q)
        r = np.empty_like(Z)
        r[:, perm] = Z
        m = d // q
        k = np.where(tau[:, None] == tau[None, :], m, 2 * m)
        s_ = np.where(pos[None, :] <= pos[:, None], r / np.sqrt(k), -np.inf)
        want = _softmax_rows(s_) @ V[0]
        got = O.algebraic_attention(Q, K, V, tau, q, positions=pos)
        np.testing.assert_allclose(got[0], want, rtol=1e-12, atol=1e-12)
        assert not np.allclose(got, O.algebraic_attention(Q, K, V, np.arange(S) % q, q))


def pin_decode_is_prefill_row(O, seed=56):
    """Algorithm 3 gives the row Algorithm 2 gives (appendix G: each pair score depends only on the
    query, one key and their types, so a cached key serves every later query): decoding row t of a
    chunk at positions p0 .. p0 + S - 1 against the whole cache (later keys masked by position)
    equals row t of the parallel computation; the cache's slot order and empty slots do not
    matter.  Q_q and the recursive law, cyclic and interval schedules, GQA."""
    g = _rng(seed)
    for q, L, S, d, p0, kind, period in ((4, 0, 11, 8, 5, "cyclic", 0), (3, 0, 9, 6, 4, "cyclic", 0),
                                         (4, 2, 10, 8, 2, "cyclic", 0), (4, 0, 13, 8, 1, "interval", 8)):
        Hq, Hkv = 4, 2
        Q = g.standard_normal((Hq, S, d))
        K = g.standard_normal((Hkv, S, d))
        V = g.standard_normal((Hkv, S, d))
        pos = p0 + np.arange(S)
        tau = O.type_schedule(pos, q, kind, period)
        want = O.algebraic_attention(Q, K, V, tau, q, L, positions=pos)
        # the cache: the S keys in a shuffled slot order, with two empty slots
        order = g.permutation(S)
        slot_pos = np.concatenate([pos[order], [-1, -1]])
        Kc = np.concatenate([K[:, order], g.standard_normal((Hkv, 2, d))], axis=1)
        Vc = np.concatenate([V[:, order], g.standard_normal((Hkv, 2, d))], axis=1)
        B = S
        got = O.algebraic_attention_decode(Q.transpose(1, 0, 2), np.repeat(Kc[None], B, 0), np.repeat(Vc[None], B, 0),
                                           pos, np.repeat(slot_pos[None], B, 0), q, L, kind, period)
        np.testing.assert_allclose(got, want.transpose(1, 0, 2), rtol=1e-12, atol=1e-12)


def pin_decode_q1_is_sdpa(O, seed=57):
    """q = 1: one query row against its whole cache is ordinary attention with 1/sqrt(d)
    (fp64 torch scaled_dot_product_attention, no mask: every cached key is at or before p)."""
    import torch
    g = _rng(seed)
    B, Hq, Hkv, N, d = 3, 4, 2, 9, 8
    Qn = g.standard_normal((B, Hq, d))
    Kc = g.standard_normal((B, Hkv, N, d))
    Vc = g.standard_normal((B, Hkv, N, d))
    kp = np.tile(np.arange(N), (B, 1))
    got = O.algebraic_attention_decode(Qn, Kc, Vc, np.full(B, N - 1), kp, 1)
    Kx = torch.tensor(np.repeat(Kc, 2, axis=1))
    Vx = torch.tensor(np.repeat(Vc, 2, axis=1))
    want = torch.nn.functional.scaled_dot_product_attention(torch.tensor(Qn)[:, :, None], Kx, Vx)[:, :, 0].numpy()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def pin_decode_cached_key_groups(O):
    """G.2's example, q = 4: a type-3 query reads group 3 of a cached type-3 key and groups {3, 1}
    of a cached type-1 key; a later type-2 query reads groups {2, 1} of that same type-1 key.  With
    Q all ones and key group a holding the constant c_a, r = m sum over F of c_a; V = I reads the
    softmax weights back, exp(r / sqrt(|F| m)) normalised.  Empty slots and keys after p get 0."""
    q, d = 4, 8
    m = d // q
    c = np.array([0.3, -0.2, 0.5, 0.1])
    keyvec = lambda: np.repeat(c, m)  # noqa: E731
    N = 5
    key_pos = np.array([[1, 3, -1, 6, 9]])      # types 1, 3, (empty), 2, 1 (position 9 > p for both queries)
    Kc = np.tile(keyvec(), (1, 1, N, 1))
    Vc = np.eye(N)[None, None, :, :N].repeat(1, 0)
    Vc = np.pad(Vc, ((0, 0), (0, 0), (0, 0), (0, d - N)))
    ones = np.ones((1, 1, d))
    # type-3 query at p = 3: keys at 1 (groups {3, 1}) and 3 (group {3})
    P3 = O.algebraic_attention_decode(ones, Kc, Vc, np.array([3]), key_pos, q)[0, 0, :N]
    w = np.array([np.exp(m * (c[3] + c[1]) / np.sqrt(2 * m)), np.exp(m * c[3] / np.sqrt(m)), 0, 0, 0])
    np.testing.assert_allclose(P3, w / w.sum(), rtol=1e-13, atol=1e-15)
    # type-2 query at p = 6: keys at 1 (groups {2, 1}), 3 (groups {2, 3}) and 6 (group {2})
    P2 = O.algebraic_attention_decode(ones, Kc, Vc, np.array([6]), key_pos, q)[0, 0, :N]
    w = np.array([np.exp(m * (c[2] + c[1]) / np.sqrt(2 * m)), np.exp(m * (c[2] + c[3]) / np.sqrt(2 * m)), 0,
                  np.exp(m * c[2] / np.sqrt(m)), 0])
    np.testing.assert_allclose(P2, w / w.sum(), rtol=1e-13, atol=1e-15)
    # no allowed key: a zero row
    assert not O.algebraic_attention_decode(ones, Kc, Vc, np.array([0]), key_pos, q).any()


def pin_decode_macs(O):
    """eq 57: a type-i query over N_p allowed keys, n_i of its own type, costs m (2 N_p - n_i) score
    MACs; eq 58: a balanced cache gives the fraction rho_q = (2q - 1) / q^2 (7/16 at q = 4); eq 61:
    the recursive law costs m sum_j 2^h(i, j) n_j, 9/16 of dense for a balanced Q_2^(x)2 cache;
    the value sum is N_p d in every case."""
    for q, d, Np, p in ((4, 8, 64, 70), (3, 6, 30, 40), (8, 16, 64, 100)):
        key_pos = np.concatenate([np.arange(Np), [p + 1, -1]])   # one future key, one empty slot
        sm, vm = O.attention_decode_macs(p, key_pos, q, d)
        i = p % q
        n_i = sum(1 for u in range(Np) if u % q == i)
        assert sm == (d // q) * (2 * Np - n_i) and vm == Np * d
        if Np % q == 0:
            assert sm * q * q == (2 * q - 1) * Np * d
    sm, vm = O.attention_decode_macs(63, np.arange(64), 4, 8, L=2)
    assert sm * 16 == 9 * 64 * 8 and vm == 64 * 8
    i = 63 % 4
    want = sum(2 ** bin(i ^ (u % 4)).count("1") for u in range(64)) * 2
    assert sm == want



def _torch_algebraic_attention(Qt, Kt, Vt, tau, q, L, pos):
    """A second, differentiable statement of appendix G's forward (fp64 torch): the compared
    groups written out by hand (Q_q: the query's and the key's own groups; the recursive law:
    the groups whose every bit is the query's or the key's), per pair scale 1/sqrt(|F| m),
    causal mask on positions, softmax, dense PV."""
    import torch
    Hq, S, d = Qt.shape
    Hkv = Kt.shape[0]
    m = d // q
    use = np.zeros((q, S, S))
    for p_ in range(S):
        for u in range(S):
            i, j = int(tau[p_]), int(tau[u])
            if L == 0:
                groups = {i, j}
            else:
                groups = {a for a in range(q) if all((a >> k) & 1 in ((i >> k) & 1, (j >> k) & 1) for k in range(L))}
            for a in groups:
                use[a, p_, u] = 1.0
    use_t = torch.tensor(use, dtype=torch.float64)
    k = use_t.sum(0) * m
    causal = torch.tensor(np.asarray(pos)[None, :] <= np.asarray(pos)[:, None])
    outs = []
    for h in range(Hq):
        kv = h // (Hq // Hkv)
        r = sum(use_t[a] * (Qt[h, :, a * m:(a + 1) * m] @ Kt[kv, :, a * m:(a + 1) * m].T) for a in range(q))
        sc = torch.where(causal, r / torch.sqrt(k), torch.tensor(-float("inf"), dtype=torch.float64))
        outs.append(torch.softmax(sc, dim=1) @ Vt[kv])
    return torch.stack(outs)


def pin_attention_backward_autograd(O, seed=58):
    """Algorithm 2, step 9: the oracle's explicit gradients equal fp64 torch autograd of the
    differentiable statement above, for Q_q with GQA at a position offset, the recursive law,
    and q = 3 with one key/value head."""
    import torch
    g = _rng(seed)
    for Hq, Hkv, S, d, q, L, p0 in ((4, 2, 11, 8, 4, 0, 5), (2, 2, 10, 8, 4, 2, 0), (2, 1, 9, 6, 3, 0, 2)):
        Q = g.standard_normal((Hq, S, d))
        K = g.standard_normal((Hkv, S, d))
        V = g.standard_normal((Hkv, S, d))
        dO = g.standard_normal((Hq, S, d))
        pos = p0 + np.arange(S)
        tau = pos % q
        Qt, Kt, Vt = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
        out = _torch_algebraic_attention(Qt, Kt, Vt, tau, q, L, pos)
        (out * torch.tensor(dO)).sum().backward()
        got = O.algebraic_attention_backward(Q, K, V, dO, tau, q, L, positions=pos)
        for gg, want in zip(got, (Qt.grad, Kt.grad, Vt.grad)):
            np.testing.assert_allclose(gg, want.numpy(), rtol=1e-11, atol=1e-11)


def pin_attention_backward_q1_is_sdpa(O, seed=59):
    """q = 1: the gradients of ordinary causal attention (fp64 torch autograd through
    scaled_dot_product_attention; GQA by repeating the key/value heads, whose gradients then sum)."""
    import torch
    g = _rng(seed)
    Hq, Hkv, S, d = 4, 2, 13, 8
    Q = g.standard_normal((Hq, S, d))
    K = g.standard_normal((Hkv, S, d))
    V = g.standard_normal((Hkv, S, d))
    dO = g.standard_normal((Hq, S, d))
    Qt, Kt, Vt = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
    out = torch.nn.functional.scaled_dot_product_attention(Qt, Kt.repeat_interleave(2, 0), Vt.repeat_interleave(2, 0),
                                                           is_causal=True)
    (out * torch.tensor(dO)).sum().backward()
    got = O.algebraic_attention_backward(Q, K, V, dO, np.zeros(S, int), 1)
    for gg, want in zip(got, (Qt.grad, Kt.grad, Vt.grad)):
        np.testing.assert_allclose(gg, want.numpy(), rtol=1e-11, atol=1e-11)


def pin_attention_backward_finite_differences(O, seed=60):
    """The gradients are the derivative of f = <dO, attention(Q, K, V)>: along a random direction
    (E_Q, E_K, E_V) the central difference of f (the oracle's own forward, eps = 1e-5) equals
    <dQ, E_Q> + <dK, E_K> + <dV, E_V>; Q_q and the recursive law, GQA."""
    g = _rng(seed)
    for Hq, Hkv, S, d, q, L in ((4, 2, 9, 8, 4, 0), (2, 1, 8, 8, 4, 2)):
        Q = g.standard_normal((Hq, S, d))
        K = g.standard_normal((Hkv, S, d))
        V = g.standard_normal((Hkv, S, d))
        dO = g.standard_normal((Hq, S, d))
        E = [g.standard_normal(x.shape) for x in (Q, K, V)]
        tau = np.arange(S) % q
        f = lambda t: float((dO * O.algebraic_attention(Q + t * E[0], K + t * E[1], V + t * E[2], tau, q, L)).sum())  # noqa: E731
        eps = 1e-5
        fd = (f(eps) - f(-eps)) / (2 * eps)
        dQ, dK, dV = O.algebraic_attention_backward(Q, K, V, dO, tau, q, L)
        an = float((dQ * E[0]).sum() + (dK * E[1]).sum() + (dV * E[2]).sum())
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (fd, an)


ALL_PINS = [
    pin_q2_table, pin_q2_scalar_example, pin_eq3_rectangular_blocks, pin_eq13_14,
    pin_product_counts, pin_graph_counts, pin_appendix_a, pin_associativity,
    pin_row_typed_composition, pin_unit_laws, pin_brute_force, pin_teaching_matrix,
    pin_masked_dense, pin_graph_masked_dense, pin_row_typed_is_square_rows, pin_q1_is_matmul, pin_block_diagonal,
    pin_coverage, pin_vjp_scalar_eq31_35, pin_vjp_autograd, pin_graph_vjp_autograd, pin_widths_vjp_autograd, pin_vjp_adjoint,
    pin_mac_count, pin_type_index, pin_type_schedule, pin_silu_values, pin_gated_masked_dense,
    pin_silu_grad, pin_gated_ffn_autograd, pin_tensor_counts, pin_tensor_support,
    pin_tensor_associativity, pin_tensor_masked_dense, pin_tensor_cost, pin_tensor_vjp_autograd,
    pin_attention_q1_is_sdpa, pin_attention_scores_are_typed_product, pin_attention_scale_and_mask,
    pin_attention_causality, pin_attention_gqa, pin_attention_laws_and_counts, pin_attention_type_offset,
    pin_decode_is_prefill_row, pin_decode_q1_is_sdpa, pin_decode_cached_key_groups, pin_decode_macs,
    pin_attention_backward_autograd, pin_attention_backward_q1_is_sdpa, pin_attention_backward_finite_differences,
]
