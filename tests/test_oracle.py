"""Pins for the fp64 CPU oracle (no GPU).

The oracle is checked against things other than itself: library routines
(numpy's FFT through the convolution theorem, scipy's circulant and
block-diagonal constructors, plain matmul), hand-derived examples
(tests/golden/*.json), closed forms, invariants (equivariance, linearity),
the dimension of the space of equivariant maps, and the operation counts the
pages state.  test_mutants_are_caught plants plausible mistakes into a copy of
the oracle's C source and checks that these pins reject every one of them.
"""
import json
import os
import subprocess

import numpy as np
import pytest
import scipy.linalg

import oracle
import synthetic

RNG = np.random.default_rng(1234)


def _rand(*shape):
    return RNG.standard_normal(shape)


def rfft_route(x, w):
    """Convolution theorem with numpy's FFT: y = irfft(sum_i rfft(w) * rfft(x))."""
    N = x.shape[-1]
    X = np.fft.rfft(x, axis=-1)  # [T][C_in][K]
    W = np.fft.rfft(w, axis=-1)  # [C_out][C_in][K]
    Y = np.einsum("oik,tik->tok", W, X)
    return np.fft.irfft(Y, n=N, axis=-1)


def pack_rfft(w):
    """numpy rfft of w[C_out][C_in][N] packed into N planes [N][C_out][C_in]."""
    N = w.shape[-1]
    R = np.fft.rfft(w, axis=-1)
    planes = [R[..., 0].real]
    for k in range(1, (N - 1) // 2 + 1):
        planes += [R[..., k].real, R[..., k].imag]
    if N % 2 == 0:
        planes.append(R[..., N // 2].real)
    return np.stack(planes)


def rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


# ---------------------------------------------------------------------------
# Pin functions (each raises AssertionError on failure; reused by the mutant test)

def pin_hand_examples(orc, golden_dir):
    with open(os.path.join(golden_dir, "cn_hand_examples.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        x = np.array(c["x"], float)
        w = np.array(c["w"], float)
        y = np.array(c["y"], float)
        assert np.array_equal(orc.cn_dense(x, w), y), c["name"]
        assert np.array_equal(orc.cn_direct(x, w), y), c["name"]
    for c in g["weight_dft_cases"]:
        w = np.array(c["w"], float)[None, None, :]
        P = orc.cn_weight_dft(w)[:, 0, 0]
        np.testing.assert_allclose(P, c["planes"], rtol=0, atol=1e-14, err_msg=c["name"])


def pin_rfft_route(orc):
    for N in range(1, 10):
        for (C_in, C_out) in [(1, 1), (2, 3), (3, 2)]:
            for T in (1, 5):
                x, w = _rand(T, C_in, N), _rand(C_out, C_in, N)
                ref = rfft_route(x, w)
                assert rel(orc.cn_dense(x, w), ref) < 1e-13, (N, C_in, C_out, T)
                assert rel(orc.cn_direct(x, w), ref) < 1e-13, (N, C_in, C_out, T)


def pin_weight_dft(orc):
    for N in range(1, 17):
        w = _rand(3, 2, N)
        assert rel(orc.cn_weight_dft(w), pack_rfft(w)) < 1e-14, N


def pin_d8_blockdiag(orc, golden_dir):
    with open(os.path.join(golden_dir, "d8_hand_example.json")) as f:
        g = json.load(f)
    order = ["A1", "A2", "B1", "B2", "E"]
    for c in g["cases"]:
        C = c["C"]
        wb = np.concatenate([np.array(c["blocks"][k], float).ravel() for k in order])
        y = orc.d8_dense(np.array(c["x"], float), wb, C)
        assert np.array_equal(y, np.array(c["y"], float)), c["name"]
    # library routine: scipy's block_diag with W_E placed on both E coordinates
    for (C_in, C_out) in [(8, 16), (16, 8), (24, 24)]:
        shapes = synthetic.d8_block_shapes(C_in, C_out)
        blocks = [_rand(*s) for s in shapes]
        wb = np.concatenate([b.ravel() for b in blocks])
        ref = scipy.linalg.block_diag(*blocks, blocks[4])
        assert np.array_equal(orc.d8_expand(wb, C_in, C_out), ref), (C_in, C_out)
        x = _rand(3, C_in)
        assert rel(orc.d8_dense(x, wb, C_out), x @ ref.T) < 1e-14


def pin_closed_forms(orc):
    N, C_in, C_out, T = 6, 3, 2, 4
    x = _rand(T, C_in, N)
    # weight only at shift 0: the same channel map for every group element
    w = np.zeros((C_out, C_in, N))
    w[..., 0] = _rand(C_out, C_in)
    ref = np.einsum("oi,tig->tog", w[..., 0], x)
    assert rel(orc.cn_dense(x, w), ref) < 1e-14
    # w = delta_{o,i} delta_{m,s}: output is the input rolled by s
    for s in range(N):
        w = np.zeros((C_in, C_in, N))
        for i in range(C_in):
            w[i, i, s] = 1.0
        assert np.array_equal(orc.cn_dense(x, w), np.roll(x, s, axis=-1)), s
    # x constant along the group axis: y[t,o,g] = sum_i (sum_m w[o,i,m]) x[t,i]
    w = _rand(C_out, C_in, N)
    xc = np.repeat(_rand(T, C_in, 1), N, axis=-1)
    ref = np.einsum("oi,ti->to", w.sum(-1), xc[..., 0])[..., None].repeat(N, -1)
    assert rel(orc.cn_dense(xc, w), ref) < 1e-14
    # alternating input (-1)^h: y[g] = (-1)^g * sum_i (sum_m (-1)^m w[o,i,m]) a[t,i]
    sgn = (-1.0) ** np.arange(N)
    a = _rand(T, C_in)
    xa = a[..., None] * sgn
    ref = np.einsum("oi,ti->to", (w * sgn).sum(-1), a)[..., None] * sgn
    assert rel(orc.cn_dense(xa, w), ref) < 1e-14
    # N = 1 is a plain matrix product
    x1, w1 = _rand(T, C_in, 1), _rand(C_out, C_in, 1)
    assert rel(orc.cn_dense(x1, w1)[..., 0], x1[..., 0] @ w1[..., 0].T) < 1e-15
    # one channel in and out: scipy's circulant matrix (first column w)
    for n in (2, 3, 5, 8):
        w11 = _rand(1, 1, n)
        xs = _rand(2, 1, n)
        ref = xs[:, 0, :] @ scipy.linalg.circulant(w11[0, 0]).T
        assert rel(orc.cn_dense(xs, w11)[:, 0, :], ref) < 1e-14


def pin_dense_matrix_structure(orc):
    # the replicated matrix equals the Kronecker-assembled circulant blocks
    N, C_in, C_out = 5, 2, 3
    w = _rand(C_out, C_in, N)
    W = orc.cn_expand(w)
    for o in range(C_out):
        for i in range(C_in):
            blk = W[o * N:(o + 1) * N, i * N:(i + 1) * N]
            assert np.array_equal(blk, scipy.linalg.circulant(w[o, i])), (o, i)


def pin_backward_adjoint(orc):
    """The gradients are the adjoints of the (pinned) forward map:
    <dy, y(x, w)> = <dx(dy, w), x> = <dw(x, dy), w> for every x, w, dy, and the
    direct input gradient equals W_dense^T dy."""
    for N, C_in, C_out, T in [(3, 2, 4, 5), (4, 3, 2, 3), (7, 2, 3, 4), (8, 1, 2, 2), (1, 3, 2, 4)]:
        x, w, dy = _rand(T, C_in, N), _rand(C_out, C_in, N), _rand(T, C_out, N)
        lhs = np.sum(dy * orc.cn_dense(x, w))
        dx = orc.cn_backward_data(dy, w)
        dw = orc.cn_backward_weight(x, dy)
        assert abs(np.sum(dx * x) - lhs) <= 1e-12 * max(1.0, abs(lhs)), (N, C_in, C_out)
        assert abs(np.sum(dw * w) - lhs) <= 1e-12 * max(1.0, abs(lhs)), (N, C_in, C_out)
        assert rel(dx, orc.cn_backward_data_dense(dy, w)) < 1e-14


def pin_backward_closed_forms(orc):
    T, C_in, C_out = 5, 3, 2
    # N = 1: plain matrix products dx = dy w, dw = dy^T x
    x, w, dy = _rand(T, C_in, 1), _rand(C_out, C_in, 1), _rand(T, C_out, 1)
    assert rel(orc.cn_backward_data(dy, w)[..., 0], dy[..., 0] @ w[..., 0]) < 1e-15
    assert rel(orc.cn_backward_weight(x, dy)[..., 0], dy[..., 0].T @ x[..., 0]) < 1e-15
    # convolution theorem with numpy's FFT: dx = irfft(sum_o conj(W) DY),
    # dw = irfft(sum_t DY conj(X)) (cross-correlations along the group axis)
    for N in (3, 4, 6, 7):
        x, w, dy = _rand(T, C_in, N), _rand(C_out, C_in, N), _rand(T, C_out, N)
        X, Wf, DY = (np.fft.rfft(a, axis=-1) for a in (x, w, dy))
        ref_dx = np.fft.irfft(np.einsum("oik,tok->tik", np.conj(Wf), DY), n=N, axis=-1)
        ref_dw = np.fft.irfft(np.einsum("tok,tik->oik", DY, np.conj(X)), n=N, axis=-1)
        assert rel(orc.cn_backward_data(dy, w), ref_dx) < 1e-13, N
        assert rel(orc.cn_backward_weight(x, dy), ref_dw) < 1e-13, N
    # w = delta_{o,i} delta_{m,s} (a roll by s): dx is dy rolled back by s
    N = 5
    dy = _rand(T, C_in, N)
    for s in range(N):
        w = np.zeros((C_in, C_in, N))
        for i in range(C_in):
            w[i, i, s] = 1.0
        assert np.array_equal(orc.cn_backward_data(dy, w), np.roll(dy, -s, axis=-1)), s


def pin_backward_equivariance(orc):
    N, C_in, C_out, T = 6, 2, 3, 4
    x, w, dy = _rand(T, C_in, N), _rand(C_out, C_in, N), _rand(T, C_out, N)
    dx, dw = orc.cn_backward_data(dy, w), orc.cn_backward_weight(x, dy)
    for s in (1, 2, 5):
        assert rel(orc.cn_backward_data(np.roll(dy, s, -1), w), np.roll(dx, s, -1)) < 1e-14
        assert rel(orc.cn_backward_weight(np.roll(x, s, -1), np.roll(dy, s, -1)), dw) < 1e-14


def pin_bias_act(orc):
    """GELU(v) = v Phi(v) with scipy's normal CDF; the odd-part identity
    GELU(v) - GELU(-v) = v; textbook values at +-1; the bias is per output
    channel and constant along the group axis; equivariance survives."""
    import scipy.special
    v = np.linspace(-6.0, 6.0, 97).reshape(1, 1, 97)
    g = orc.bias_act(v, None, 1)
    assert np.max(np.abs(g - v * scipy.special.ndtr(v))) < 1e-15
    assert np.max(np.abs((g - orc.bias_act(-v, None, 1)) - v)) < 1e-14
    # relative accuracy in the far negative tail, where 1 + erf would cancel
    # (scipy's ndtr takes erfc there): GELU(-30) is about -3e-196.  The bound is
    # the rounding of the argument v/sqrt 2 carried through erfc, about 2 z^2 2^-53.
    tail = np.linspace(-30.0, -5.0, 51).reshape(1, 1, 51)
    ref = tail * scipy.special.ndtr(tail)
    assert np.all(np.abs(orc.bias_act(tail, None, 1) - ref) <= 1e-12 * np.abs(ref))
    one = orc.bias_act(np.array([1.0, -1.0, 0.0]).reshape(1, 1, 3), None, 1).ravel()
    assert abs(one[0] - 0.8413447460685429) < 1e-15 and abs(one[1] + 0.15865525393145707) < 1e-15 and one[2] == 0.0
    N, C_in, C_out, T = 5, 3, 4, 6
    x, w, b = _rand(T, C_in, N), _rand(C_out, C_in, N), _rand(C_out)
    y = orc.cn_dense(x, w)
    assert np.array_equal(orc.bias_act(y, b, 0), y + b[None, :, None])
    assert np.array_equal(orc.bias_act(y, None, 0), y)
    yb = orc.cn_dense_bias_act(x, w, b, 1)
    for s in (1, 3):
        assert rel(orc.cn_dense_bias_act(np.roll(x, s, -1), w, b, 1), np.roll(yb, s, -1)) < 1e-14


def _d4_elements():
    """D8 as the square's symmetries, 2 x 2 integer matrices: element q = a + 4b is R^a S^b
    (R a quarter turn, S the mirror y -> -y)."""
    R = np.array([[0, -1], [1, 0]])
    S = np.array([[1, 0], [0, -1]])
    return [np.linalg.matrix_power(R, q % 4) @ (S if q // 4 else np.eye(2, dtype=int)) for q in range(8)]


def _left_regular(g):
    """The left-regular action of g on functions of the group: f -> f(g^-1 .), i.e.
    P[q', q] = 1 where h_q' = g h_q (the group law from the matrices)."""
    E = _d4_elements()
    P = np.zeros((8, 8))
    for q in range(8):
        gq = g @ E[q]
        P[next(i for i in range(8) if np.array_equal(E[i], gq)), q] = 1.0
    return P


def _d8_slots(m, j):
    """Fourier-layout columns of regular channel j (the reading of the layout: A1..B2
    at j, E copies 2j + c in the coordinate-0 and coordinate-1 slabs)."""
    return [j, m + j, 2 * m + j, 3 * m + j, 4 * m + 2 * j, 4 * m + 2 * j + 1, 6 * m + 2 * j, 6 * m + 2 * j + 1]


def pin_d8_fourier(orc):
    """The D8 Fourier matrix: orthonormal rows (Schur orthogonality); the
    identity's column by hand; it intertwines the left-regular action (built
    from the group law) with the layer's feature action on one channel, for both
    generators; the transforms invert each other and follow the layout."""
    F = orc.d8_fourier_matrix()
    assert np.max(np.abs(F @ F.T - np.eye(8))) < 1e-15
    assert np.max(np.abs(F[:, 0] - np.array([8 ** -0.5] * 4 + [0.5, 0.0, 0.0, 0.5]))) < 1e-16
    r, s = d8_action(8)
    E = _d4_elements()
    for g, A in ((E[1], r), (E[4], s)):
        assert np.max(np.abs(F @ _left_regular(g) - A @ F)) < 1e-15
    m = 5
    f = _rand(3, m, 8)
    v = orc.d8_to_fourier(f)
    assert rel(orc.d8_to_regular(v), f) < 1e-15
    for j in (0, 3):
        assert rel(v[:, _d8_slots(m, j)], f[:, j] @ F.T) < 1e-15


def pin_d8_bias_act(orc):
    """The D8 round trip: the identity when no bias and no activation; a bias
    constant over the group elements lands on A1 alone, times sqrt(8); a delta
    at the identity comes back times Phi(1); GELU acts on the regular-domain
    values (scipy's ndtr); the layer followed by the round trip is equivariant."""
    import scipy.special
    m, T = 3, 4
    y = _rand(T, 8 * m)
    assert rel(orc.d8_bias_act(y, None, 0), y) < 1e-15
    b = _rand(m)
    expect = np.zeros_like(y)
    expect[:, :m] = np.sqrt(8.0) * b
    assert np.max(np.abs(orc.d8_bias_act(y, b, 0) - y - expect)) < 1e-14
    v = np.zeros((1, 8 * m))
    col = np.array([8 ** -0.5] * 4 + [0.5, 0.0, 0.0, 0.5])
    v[0, _d8_slots(m, 1)] = col
    expect = np.zeros_like(v)
    expect[0, _d8_slots(m, 1)] = 0.8413447460685429 * col
    assert np.max(np.abs(orc.d8_bias_act(v, None, 1) - expect)) < 1e-15
    fr = orc.d8_to_regular(y) + b[None, :, None]
    assert rel(orc.d8_bias_act(y, b, 1), orc.d8_to_fourier(fr * scipy.special.ndtr(fr))) < 1e-14
    C_in, C_out = 16, 24
    x, wb, bb = _rand(T, C_in), _rand(C_in * C_out // 8), _rand(C_out // 8)
    rin, sin_ = d8_action(C_in)
    rout, sout = d8_action(C_out)
    yb = orc.d8_dense_bias_act(x, wb, C_out, bb, 1)
    assert rel(orc.d8_dense_bias_act(x @ rin.T, wb, C_out, bb, 1), yb @ rout.T) < 1e-13
    assert rel(orc.d8_dense_bias_act(x @ sin_.T, wb, C_out, bb, 1), yb @ sout.T) < 1e-13


def _dn_elements(n):
    """D_n as the regular n-gon's symmetries, 2 x 2 matrices: element q = a + n b is
    R^a S^b (R the turn by 2 pi / n, S the mirror y -> -y)."""
    c, s_ = np.cos(2 * np.pi / n), np.sin(2 * np.pi / n)
    R = np.array([[c, -s_], [s_, c]])
    S = np.diag([1.0, -1.0])
    return [np.linalg.matrix_power(R, q % n) @ (S if q // n else np.eye(2)) for q in range(2 * n)]


def _dn_left_regular(n, g):
    E = _dn_elements(n)
    P = np.zeros((2 * n, 2 * n))
    for q in range(2 * n):
        gq = g @ E[q]
        P[next(i for i in range(2 * n) if np.allclose(E[i], gq, atol=1e-12)), q] = 1.0
    return P


def dn_action(n, C):
    """Generators r, s of D_n acting on Fourier features of width C laid out as the
    layer's: m = C/2n channels per 1-D irrep (A1, A2, and B1, B2 for even n), then
    per E_k (k = 1, 2, ...) a coordinate-0 and a coordinate-1 slab of 2m copies,
    r turning each copy by 2 pi k / n and s = diag(1, -1)."""
    m = C // (2 * n)
    chars = [(1, 1), (1, -1)] + ([(-1, 1), (-1, -1)] if n % 2 == 0 else [])
    n2 = n // 2 - 1 if n % 2 == 0 else (n - 1) // 2
    r, s_ = np.zeros((C, C)), np.zeros((C, C))
    for b, (rv, sv) in enumerate(chars):
        for j in range(m):
            r[b * m + j, b * m + j] = rv
            s_[b * m + j, b * m + j] = sv
    base = len(chars) * m
    for k in range(1, n2 + 1):
        c, sn = np.cos(2 * np.pi * k / n), np.sin(2 * np.pi * k / n)
        e0 = base + 4 * m * (k - 1)
        for cp in range(2 * m):
            a, b = e0 + cp, e0 + 2 * m + cp
            r[a, a], r[a, b], r[b, a], r[b, b] = c, -sn, sn, c
            s_[a, a], s_[b, b] = 1.0, -1.0
    return r, s_


def _dn_slots(n, m, j):
    """Fourier columns of regular channel j (the layout reading: 1-D irreps at j, E_k
    copies 2j + c in its coordinate slabs)."""
    n1 = 4 if n % 2 == 0 else 2
    n2 = n // 2 - 1 if n % 2 == 0 else (n - 1) // 2
    cols = [b * m + j for b in range(n1)]
    for k in range(n2):
        for kk in range(2):
            for c in range(2):
                cols.append(n1 * m + 4 * m * k + 2 * m * kk + 2 * j + c)
    return cols


def pin_dn_fourier(orc):
    """Dihedral groups of the regular n-gon: the feature action is a representation
    with the regular character; the Fourier matrix is orthonormal and intertwines
    the left-regular action (group law of the symmetry matrices) with it; the
    transforms invert each other and follow the layout; n = 4 is the D8 matrix."""
    for n in (2, 3, 5, 6):
        r, s_ = dn_action(n, 2 * n)
        G = 2 * n
        assert np.allclose(np.linalg.matrix_power(r, n), np.eye(G), atol=1e-12)
        assert np.allclose(s_ @ s_, np.eye(G)) and np.allclose(s_ @ r @ s_, np.linalg.matrix_power(r, n - 1), atol=1e-12)
        tr = [np.trace(np.linalg.matrix_power(r, a) @ (s_ if b else np.eye(G))) for b in (0, 1) for a in range(n)]
        assert abs(tr[0] - G) < 1e-12 and max(abs(t) for t in tr[1:]) < 1e-12
        F = orc.dn_fourier_matrix(n)
        assert np.max(np.abs(F @ F.T - np.eye(G))) < 1e-14
        E = _dn_elements(n)
        for g, A in ((E[1], r), (E[n], s_)):
            assert np.max(np.abs(F @ _dn_left_regular(n, g) - A @ F)) < 1e-14
        m = 3
        f = _rand(2, m, G)
        v = orc.dn_to_fourier(n, f)
        assert rel(orc.dn_to_regular(n, v), f) < 1e-14
        assert rel(v[:, _dn_slots(n, m, 1)], f[:, 1] @ F.T) < 1e-14
    assert np.max(np.abs(orc.dn_fourier_matrix(4) - orc.d8_fourier_matrix())) < 1e-15


def pin_dn_layer(orc):
    """The D_n layer: the equivariant maps of its features have dimension C^2/2n and
    the oracle's expansion spans them; n = 4 is the D8 layer; the round trip is the
    identity without bias or activation, puts a bias on A1 times sqrt(2n), and the
    layer followed by the GELU round trip is equivariant."""
    for n in (3, 6):
        C = 2 * n * 2
        r, s_ = dn_action(n, C)
        dim = _commutant_dim([r, s_], [r, s_])
        assert dim == C * C // (2 * n) == orc.dn_params(n, C, C)
        basis = []
        for idx in range(dim):
            e = np.zeros(dim)
            e[idx] = 1.0
            W = orc.dn_expand(n, e, C, C)
            assert np.allclose(r @ W, W @ r, atol=1e-12) and np.allclose(s_ @ W, W @ s_, atol=1e-12)
            basis.append(W.ravel())
        assert np.linalg.matrix_rank(np.array(basis)) == dim
    C_in, C_out, T = 16, 24, 4
    wb = _rand(orc.d8_params(C_in, C_out))
    x = _rand(T, C_in)
    assert np.array_equal(orc.dn_expand(4, wb, C_in, C_out), orc.d8_expand(wb, C_in, C_out))
    y = _rand(T, 24)
    b = _rand(3)
    assert rel(orc.dn_bias_act(4, y, b, 1), orc.d8_bias_act(y, b, 1)) < 1e-14
    for n in (3, 6):
        C_in, C_out = 2 * n * 2, 2 * n * 3
        wb, bb = _rand(orc.dn_params(n, C_in, C_out)), _rand(C_out // (2 * n))
        x = _rand(T, C_in)
        y = orc.dn_dense(n, x, wb, C_out)
        assert rel(orc.dn_bias_act(n, y, None, 0), y) < 1e-14
        d = orc.dn_bias_act(n, y, bb, 0) - y
        expect = np.zeros_like(y)
        expect[:, :C_out // (2 * n)] = np.sqrt(2.0 * n) * bb
        assert np.max(np.abs(d - expect)) < 1e-13
        rin, sin_ = dn_action(n, C_in)
        rout, sout = dn_action(n, C_out)
        yb = orc.dn_dense_bias_act(n, x, wb, C_out, bb, 1)
        assert rel(orc.dn_dense_bias_act(n, x @ rin.T, wb, C_out, bb, 1), yb @ rout.T) < 1e-13
        assert rel(orc.dn_dense_bias_act(n, x @ sin_.T, wb, C_out, bb, 1), yb @ sout.T) < 1e-13


ALL_CN_PINS = [pin_rfft_route, pin_weight_dft, pin_closed_forms, pin_dense_matrix_structure, pin_bias_act,
               pin_backward_adjoint, pin_backward_closed_forms, pin_backward_equivariance]


# ---------------------------------------------------------------------------
# Tests

def test_hand_examples(golden_dir):
    pin_hand_examples(oracle, golden_dir)


def test_rfft_route():
    pin_rfft_route(oracle)


def test_weight_dft_matches_numpy_rfft():
    pin_weight_dft(oracle)


def test_weight_dft_closed_forms():
    for N in range(1, 17):
        d = np.zeros((1, 1, N))
        d[..., 0] = 1.0  # delta -> every bin is 1
        P = oracle.cn_weight_dft(d)[:, 0, 0]
        expect = np.zeros(N)
        expect[0] = 1.0
        for k in range(1, (N - 1) // 2 + 1):
            expect[2 * k - 1] = 1.0
        if N % 2 == 0 and N > 1:
            expect[N - 1] = 1.0
        np.testing.assert_allclose(P, expect, atol=1e-15)
        c = np.full((1, 1, N), 2.5)  # constant -> DC = N*c, everything else 0
        P = oracle.cn_weight_dft(c)[:, 0, 0]
        np.testing.assert_allclose(P, np.r_[2.5 * N, np.zeros(N - 1)], atol=1e-13)


def test_closed_forms():
    pin_closed_forms(oracle)


def test_backward_adjoint_identities():
    pin_backward_adjoint(oracle)


def test_backward_closed_forms():
    pin_backward_closed_forms(oracle)


def test_backward_equivariance():
    pin_backward_equivariance(oracle)


def test_bias_and_gelu():
    pin_bias_act(oracle)


def test_d8_fourier_transform():
    pin_d8_fourier(oracle)


def test_d8_round_trip_bias_and_gelu():
    pin_d8_bias_act(oracle)


def test_dihedral_fourier_transform():
    pin_dn_fourier(oracle)


def test_dihedral_layer_and_round_trip():
    pin_dn_layer(oracle)


def test_dense_matrix_structure():
    pin_dense_matrix_structure(oracle)


def test_d8_block_diagonal(golden_dir):
    pin_d8_blockdiag(oracle, golden_dir)


@pytest.mark.parametrize("N", [3, 4, 7, 8])
def test_equivariance_cyclic_roll(N):
    x, w = _rand(4, 3, N), _rand(2, 3, N)
    y = oracle.cn_direct(x, w)
    for s in range(1, N):
        ys = oracle.cn_direct(np.roll(x, s, axis=-1), w)
        # the direct sum visits the same products in the same order: bitwise
        assert np.array_equal(ys, np.roll(y, s, axis=-1))
        yd = oracle.cn_dense(np.roll(x, s, axis=-1), w)
        assert rel(yd, np.roll(y, s, axis=-1)) < 1e-13


def test_linearity():
    N, C_in, C_out = 5, 3, 2
    x1, x2, w1, w2 = _rand(3, C_in, N), _rand(3, C_in, N), _rand(C_out, C_in, N), _rand(C_out, C_in, N)
    a, b = 0.75, -1.25
    assert rel(oracle.cn_dense(a * x1 + b * x2, w1),
               a * oracle.cn_dense(x1, w1) + b * oracle.cn_dense(x2, w1)) < 1e-13
    assert rel(oracle.cn_dense(x1, a * w1 + b * w2),
               a * oracle.cn_dense(x1, w1) + b * oracle.cn_dense(x1, w2)) < 1e-13


def _commutant_dim(gens_in, gens_out):
    """dim {M : R_out(g) M = M R_in(g) for all generators g} by SVD."""
    n_out, n_in = gens_out[0].shape[0], gens_in[0].shape[0]
    rows = []
    I_in, I_out = np.eye(n_in), np.eye(n_out)
    for Rin, Rout in zip(gens_in, gens_out):
        # vec(R_out M - M R_in) = (I_in (x) R_out - R_in^T (x) I_out) vec(M)  (column-major vec)
        rows.append(np.kron(I_in, Rout) - np.kron(Rin.T, I_out))
    L = np.vstack(rows)
    s = np.linalg.svd(L, compute_uv=False)
    return int(np.sum(s < 1e-9 * max(s.max(), 1.0))) + max(0, L.shape[1] - len(s))


def _cyclic_shift(N, C):
    P = np.roll(np.eye(N), 1, axis=0)  # (P v)[h] = v[h-1]
    return np.kron(np.eye(C), P)


@pytest.mark.parametrize("N,C_in,C_out", [(3, 1, 1), (3, 2, 1), (4, 2, 2), (5, 1, 3)])
def test_cn_commutant_dimension(N, C_in, C_out):
    """Every map that commutes with the cyclic shift is group-circulant, and the
    oracle's replicated matrices fill that space: dimension = N*C_in*C_out."""
    dim = _commutant_dim([_cyclic_shift(N, C_in)], [_cyclic_shift(N, C_out)])
    assert dim == oracle.cn_params(N, C_in, C_out) == N * C_in * C_out
    P_in, P_out = _cyclic_shift(N, C_in), _cyclic_shift(N, C_out)
    basis = []
    for idx in range(N * C_in * C_out):
        e = np.zeros(N * C_in * C_out)
        e[idx] = 1.0
        W = oracle.cn_expand(e.reshape(C_out, C_in, N))
        assert np.array_equal(P_out @ W, W @ P_in)
        basis.append(W.ravel())
    assert np.linalg.matrix_rank(np.array(basis)) == dim


def d8_action(C):
    """Generators r (quarter turn) and s (mirror) acting on D8 Fourier features
    laid out [A1 | A2 | B1 | B2 | E coord 0 | E coord 1], m = C/8 copies of each
    1-D irrep and 2m copies of E.  A1: (r,s)=(1,1), A2: (1,-1), B1: (-1,1),
    B2: (-1,-1); E: r = [[0,-1],[1,0]], s = diag(1,-1) on each copy's
    (coord 0, coord 1) pair."""
    m = C // 8
    r = np.zeros((C, C))
    s = np.zeros((C, C))
    for b, (rv, sv) in enumerate([(1, 1), (1, -1), (-1, 1), (-1, -1)]):
        for j in range(m):
            r[b * m + j, b * m + j] = rv
            s[b * m + j, b * m + j] = sv
    e0, e1 = 4 * m, 6 * m
    for j in range(2 * m):
        a, b = e0 + j, e1 + j
        r[a, b] = -1.0  # new coord0 = -coord1
        r[b, a] = 1.0   # new coord1 = coord0
        s[a, a] = 1.0
        s[b, b] = -1.0
    return r, s


def test_d8_action_is_the_regular_representation():
    """The feature action is a D8 representation whose character is that of
    C/8 copies of the regular representation (8m at the identity, 0 elsewhere)."""
    for C in (8, 16):
        r, s = d8_action(C)
        I = np.eye(C)
        assert np.array_equal(np.linalg.matrix_power(r, 4), I)
        assert np.array_equal(s @ s, I)
        assert np.array_equal(s @ r @ s, np.linalg.matrix_power(r, 3))
        elems = [np.linalg.matrix_power(r, k) @ (s if f else I) for k in range(4) for f in (0, 1)]
        tr = [np.trace(g) for g in elems]
        assert tr[0] == C and all(t == 0 for t in tr[1:])


@pytest.mark.parametrize("C", [8, 16])
def test_d8_commutant_dimension(C):
    """Equivariant maps of the Fourier features are exactly the oracle's block
    matrices: the commutant has dimension C^2/8 (eight times fewer parameters
    than a width-C linear), and the oracle's expansion spans it."""
    r, s = d8_action(C)
    dim = _commutant_dim([r, s], [r, s])
    assert dim == C * C // 8 == oracle.d8_params(C, C)
    basis = []
    for idx in range(C * C // 8):
        e = np.zeros(C * C // 8)
        e[idx] = 1.0
        W = oracle.d8_expand(e, C, C)
        assert np.array_equal(r @ W, W @ r) and np.array_equal(s @ W, W @ s)
        basis.append(W.ravel())
    assert np.linalg.matrix_rank(np.array(basis)) == dim


def test_d8_equivariance_random():
    C_in, C_out = 16, 24
    d = synthetic.d8_inputs(C_in, C_out, 5, synthetic.F32, seed=3)
    x, wb = d["x64"], d["w64"]
    rin, sin_ = d8_action(C_in)
    rout, sout = d8_action(C_out)
    y = oracle.d8_dense(x, wb, C_out)
    assert rel(oracle.d8_dense(x @ rin.T, wb, C_out), y @ rout.T) < 1e-14
    assert rel(oracle.d8_dense(x @ sin_.T, wb, C_out), y @ sout.T) < 1e-14


def test_p4_transform_is_dyadic():
    """For N=4 the forward real-DFT matrix has entries in {0, +-1} and the
    inverse (1/N, doubled non-self-conjugate bins) entries in {0, +-1/4, +-1/2}:
    only adds, subtracts and power-of-two scalings ("Flash EQ-Linear",
    Specialization for p4 Rotation Group)."""
    F = oracle.cn_weight_dft(np.eye(4)[None, :, :])[:, 0, :]  # planes x inputs
    assert set(np.round(F.ravel(), 14)) <= {0.0, 1.0, -1.0}
    # inverse: y = G @ planes; find G from the oracle's layer with delta weights
    G = np.zeros((4, 4))
    for p in range(4):
        # a spectrum with one plane set to 1 -> time signal via numpy irfft
        spec = np.zeros(3, complex)
        if p == 0:
            spec[0] = 1
        elif p == 3:
            spec[2] = 1
        elif p == 1:
            spec[1] = 1
        else:
            spec[1] = 1j
        G[:, p] = np.fft.irfft(spec, n=4)
    assert set(np.round(np.abs(G.ravel()), 14)) <= {0.0, 0.25, 0.5}
    assert np.allclose(G @ F, np.eye(4))


def test_page_counts(golden_dir):
    with open(os.path.join(golden_dir, "page_counts.json")) as f:
        counts = {c["what"][:40]: c for c in json.load(f)["counts"]}
    vals = [c["value"] for c in counts.values()]
    # six real products at N=4 against sixteen for the replicated dense matrix
    assert oracle.cn_real_gemms(4) == vals[0] and 4 * 4 == 16
    assert abs(16 / oracle.cn_real_gemms(4) - 2.67) < 0.005
    # parameter reduction against a non-equivariant layer of the same width = N
    assert (4 * 8) * (4 * 8) // oracle.cn_params(4, 8, 8) == vals[1]
    # MACs per token: R(N) C_in C_out <= 2/N * (N C_in)(N C_out), -> 2/N as N grows
    for N in range(2, 65):
        ratio = oracle.cn_real_gemms(N) / N ** 2
        assert ratio <= vals[2] / N + 1e-12
    assert abs(oracle.cn_real_gemms(64) / 64 ** 2 * 64 / 2 - 1) < 0.02
    # D8: 8x fewer parameters, 5.33x fewer multiplies than a same-width linear
    for C in (8, 64, 1280):
        assert C * C / oracle.d8_params(C, C) == vals[3]
        assert abs(C * C / oracle.d8_mults(C, C) - vals[4]) < 0.005
    # odd and even orders of the benchmark workloads
    assert [oracle.cn_real_gemms(n) for n in (4, 7, 8)] == [6, 13, 14]


# ---------------------------------------------------------------------------
# Mutation check: plausible mistakes planted in a copy of the oracle must fail a pin.

MUTANTS = [
    ("correlation instead of convolution", "int m = ((g - h) % N + N) % N;\n                    W[",
     "int m = ((h - g) % N + N) % N;\n                    W["),
    ("direct sum index sign", "int h = ((g - m) % N + N) % N;\n                        acc += w[",
     "int h = ((g + m) % N + N) % N;\n                        acc += w["),
    ("transposed channel operand", "W[((int64_t)o * N + g) * cols + (int64_t)i * N + h] =\n                        w[((int64_t)o * C_in + i) * N + m];",
     "W[((int64_t)o * N + g) * cols + (int64_t)i * N + h] =\n                        w[((int64_t)i * C_out + o) * N + m];"),
    ("dropped last term", "for (int64_t c = 0; c < cols; ++c) acc += Wr[c] * xt[c];",
     "for (int64_t c = 0; c + 1 < cols; ++c) acc += Wr[c] * xt[c];"),
    ("imaginary sign", "im -= wm[m] * sin(ang);", "im += wm[m] * sin(ang);"),
    ("Nyquist plane slot", "planes[(int64_t)(N - 1) * plane + oi] = re;", "planes[(int64_t)(N - 2) * plane + oi] = re;"),
    ("backward data index sign", "int m = ((g - h) % N + N) % N;\n                        acc += w[((int64_t)o * C_in + i) * N + m] *\n                               dy[",
     "int m = ((h - g) % N + N) % N;\n                        acc += w[((int64_t)o * C_in + i) * N + m] *\n                               dy["),
    ("backward weight index sign", "int h = ((g - m) % N + N) % N;\n                        acc += dy[",
     "int h = ((g + m) % N + N) % N;\n                        acc += dy["),
    ("backward weight transposed channels", "acc += dy[(t * C_out + o) * N + g] * x[(t * C_in + i) * N + h];",
     "acc += dy[(t * C_out + o) * N + g] * x[(t * C_in + (i % C_out) % C_in) * N + h];"),
    ("dense transpose drops a row", "for (int64_t r = 0; r < rows; ++r) acc += W[r * cols + c] * dyt[r];",
     "for (int64_t r = 1; r < rows; ++r) acc += W[r * cols + c] * dyt[r];"),
    ("bias along the group axis", "if (bias) v += bias[o];", "if (bias) v += bias[g % C_out];"),
    ("GELU without the 1/sqrt(2)", "v = 0.5 * v * erfc(-v * rsqrt2);", "v = 0.5 * v * erfc(-v);"),
    ("GELU with Phi of the wrong sign", "v = 0.5 * v * erfc(-v * rsqrt2);", "v = 0.5 * v * erfc(v * rsqrt2);"),
    ("D8 transposed 1-D block", "blk[(int64_t)r * mi + c];\n        blk += (int64_t)mo * mi;\n    }\n    for (int e = 0;",
     "blk[(int64_t)c * mi + r];\n        blk += (int64_t)mo * mi;\n    }\n    for (int e = 0;"),
    ("D_n transposed 1-D block", "blk[(int64_t)r * mi + c];\n        blk += (int64_t)mo * mi;\n    }\n    for (int k = 0;",
     "blk[(int64_t)c * mi + r];\n        blk += (int64_t)mo * mi;\n    }\n    for (int k = 0;"),
    ("D8 E weight on coordinate 0 only", "4 * mi + 2 * e * mi + c] =", "4 * mi + c] ="),
    ("D8 Fourier: E copies taken as rows", "return 4 * (int64_t)m + 2 * (int64_t)m * k + 2 * j + c;",
     "return 4 * (int64_t)m + 2 * (int64_t)m * c + 2 * j + k;"),
    ("D8 Fourier: E rows unnormalised", "n2 = sqrt(2.0 / 8.0);", "n2 = sqrt(1.0 / 8.0);"),
    ("D8 Fourier: quarter turn the other way", "Er[2][2] = {{0.0, -1.0}, {1.0, 0.0}}",
     "Er[2][2] = {{0.0, 1.0}, {-1.0, 0.0}}"),
    ("D8 round trip: bias on one group element", "acc += F[p * 8 + q] * v[p];\n                if (bias) acc += bias[j];",
     "acc += F[p * 8 + q] * v[p];\n                if (bias && q == 0) acc += bias[j];"),
    ("D_n round trip: bias on one group element", "acc += F[p * G + q] * v[p];\n                if (bias) acc += bias[j];",
     "acc += F[p * G + q] * v[p];\n                if (bias && q == 0) acc += bias[j];"),
    ("D_n: E_k turning at the next frequency", "const double c1 = cos(two_pi * k / n), s1 = sin(two_pi * k / n);",
     "const double c1 = cos(two_pi * (k + 1) / n), s1 = sin(two_pi * (k + 1) / n);"),
    ("D_n: E rows unnormalised", "F[(n1 + 4 * (k - 1) + 2 * kk + c) * G + q] = sqrt(2.0 / G) * M[kk][c];",
     "F[(n1 + 4 * (k - 1) + 2 * kk + c) * G + q] = sqrt(1.0 / G) * M[kk][c];"),
    ("D_n: E weight on coordinate 0 only", "n1 * mi + 4 * k * mi + 2 * e * mi + c] =", "n1 * mi + 4 * k * mi + c] ="),
    ("D_n: mirror negates row 1", "M[0][1] = -M[0][1];\n                M[1][1] = -M[1][1];",
     "M[1][0] = -M[1][0];\n                M[1][1] = -M[1][1];"),
]


def _build_mutant(tmp_path, old, new):
    src = open(oracle._SRC).read()
    assert src.count(old) == 1, old
    mdir = tmp_path / "m"
    mdir.mkdir(exist_ok=True)
    msrc = mdir / "eqref.c"
    msrc.write_text(src.replace(old, new))
    out = mdir / ("lib%d.so" % abs(hash(new)))
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", str(msrc),
                    "-o", str(out), "-lm"], check=True)
    return str(out)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutants_are_caught(tmp_path, golden_dir, name, old, new):
    path = _build_mutant(tmp_path, old, new)
    saved = oracle._lib
    try:
        oracle._lib = None
        real_build = oracle.build
        oracle.build = lambda *a, **k: path
        caught = []
        checks = [lambda: pin_hand_examples(oracle, golden_dir),
                  lambda: pin_d8_blockdiag(oracle, golden_dir),
                  lambda: pin_d8_fourier(oracle), lambda: pin_d8_bias_act(oracle),
                  lambda: pin_dn_fourier(oracle), lambda: pin_dn_layer(oracle)] + [
            (lambda f=f: f(oracle)) for f in ALL_CN_PINS]
        for chk in checks:
            try:
                chk()
            except AssertionError:
                caught.append(chk)
        assert caught, f"mutant '{name}' passed every pin"
    finally:
        oracle.build = real_build
        oracle._lib = saved


def _preload_in_use():
    if os.environ.get("LD_PRELOAD"):
        return True
    try:
        return bool(open("/etc/ld.so.preload").read().strip())
    except OSError:
        return False


@pytest.mark.skipif(_preload_in_use(), reason="a preload library is already configured; "
                    "ASan must be loaded first and that library is left alone")
def test_oracle_under_sanitizers(tmp_path):
    """Build the oracle with ASan+UBSan and run a small case in a fresh process."""
    out = oracle.build(sanitize=True, out=str(tmp_path / "libeqref_san.so"))
    code = (
        "import ctypes, numpy as np\n"
        f"lib = ctypes.CDLL({out!r})\n"
        "x = np.random.default_rng(0).standard_normal((3, 2, 5)); w = np.ones((4, 2, 5))\n"
        "y = np.zeros((3, 4, 5)); P = np.zeros((5, 4, 2))\n"
        "p = lambda a: a.ctypes.data_as(ctypes.c_void_p)\n"
        "lib.eqref_cn_dense.argtypes = [ctypes.c_int]*3 + [ctypes.c_int64] + [ctypes.c_void_p]*3\n"
        "assert lib.eqref_cn_dense(5, 2, 4, 3, p(x), p(w), p(y)) == 0\n"
        "lib.eqref_cn_direct.argtypes = lib.eqref_cn_dense.argtypes\n"
        "lib.eqref_cn_direct(5, 2, 4, 3, p(x), p(w), p(y))\n"
        "lib.eqref_cn_weight_dft.argtypes = [ctypes.c_int]*3 + [ctypes.c_void_p]*2\n"
        "lib.eqref_cn_weight_dft(5, 4, 2, p(w), p(P))\n"
        "dx = np.zeros((3, 2, 5)); dw = np.zeros((4, 2, 5))\n"
        "lib.eqref_cn_backward_data.argtypes = lib.eqref_cn_dense.argtypes\n"
        "lib.eqref_cn_backward_data(5, 2, 4, 3, p(y), p(w), p(dx))\n"
        "lib.eqref_cn_backward_weight.argtypes = lib.eqref_cn_dense.argtypes\n"
        "lib.eqref_cn_backward_weight(5, 2, 4, 3, p(x), p(y), p(dw))\n"
        "Wd = np.ones((20, 10)); lib.eqref_apply_dense_t.argtypes = [ctypes.c_int64]*3 + [ctypes.c_void_p]*3\n"
        "lib.eqref_apply_dense_t(3, 20, 10, p(Wd), p(y), p(dx))\n"
        "bb = np.ones(4); lib.eqref_bias_act.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]\n"
        "lib.eqref_bias_act(3, 4, 5, p(bb), 1, p(y))\n"
        "wb = np.ones(16*16//8); xd = np.ones((2, 16)); yd = np.zeros((2, 16))\n"
        "lib.eqref_d8_dense.argtypes = [ctypes.c_int]*2 + [ctypes.c_int64] + [ctypes.c_void_p]*3\n"
        "assert lib.eqref_d8_dense(16, 16, 2, p(xd), p(wb), p(yd)) == 0\n"
        "F = np.zeros(64); lib.eqref_d8_fourier_matrix.argtypes = [ctypes.c_void_p]; lib.eqref_d8_fourier_matrix(p(F))\n"
        "fr = np.zeros((2, 2, 8)); lib.eqref_d8_to_regular.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]\n"
        "lib.eqref_d8_to_regular(2, 2, p(yd), p(fr))\n"
        "lib.eqref_d8_to_fourier.argtypes = lib.eqref_d8_to_regular.argtypes; lib.eqref_d8_to_fourier(2, 2, p(fr), p(yd))\n"
        "b2 = np.ones(2); lib.eqref_d8_bias_act.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]\n"
        "lib.eqref_d8_bias_act(2, 2, p(b2), 1, p(yd))\n"
        "wn = np.ones(12); xn = np.ones((2, 12)); yn = np.zeros((2, 12))  # D_6, width 12: 4 + 2 * 4 weights\n"
        "lib.eqref_dn_dense.argtypes = [ctypes.c_int]*3 + [ctypes.c_int64] + [ctypes.c_void_p]*3\n"
        "assert lib.eqref_dn_dense(6, 12, 12, 2, p(xn), p(wn), p(yn)) == 0\n"
        "Fn = np.zeros(144); lib.eqref_dn_fourier_matrix.argtypes = [ctypes.c_int, ctypes.c_void_p]; lib.eqref_dn_fourier_matrix(6, p(Fn))\n"
        "fn = np.zeros((2, 1, 12)); lib.eqref_dn_to_regular.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]\n"
        "lib.eqref_dn_to_regular(6, 2, 1, p(yn), p(fn)); lib.eqref_dn_to_fourier.argtypes = lib.eqref_dn_to_regular.argtypes\n"
        "lib.eqref_dn_to_fourier(6, 2, 1, p(fn), p(yn))\n"
        "bn = np.ones(1); lib.eqref_dn_bias_act.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]\n"
        "lib.eqref_dn_bias_act(6, 2, 1, p(bn), 1, p(yn))\n"
        "print('SAN-OK')\n"
    )
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run(["python3", "-c", code], capture_output=True, text=True, env=env)
    assert r.returncode == 0 and "SAN-OK" in r.stdout, r.stderr[-2000:]
