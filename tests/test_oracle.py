"""Pins for the fp64 CPU oracle (runs on CPU, no GPU).

Every oracle function is checked against something other than itself:
hand-worked fixtures (tests/golden), library routines that take a different
route (numpy BLAS, scipy.linalg.circulant, numpy.fft, scipy.special.softmax),
closed forms and invariants the pages state (rows of circ(softmax z) sum to 1,
softmax and circ commute, weights depend only on the offset i - j, a BCCB
matrix times a vector is a 2D convolution).  The last block plants plausible
mistakes into copies of the oracle and checks that some pin catches each.
"""
import json
import os

import numpy as np
import pytest
import scipy.linalg
import scipy.special

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def rel(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(b), 1e-300))


# ---------------------------------------------------------------- projection
def test_matmul_small_exact():
    X = np.array([[1.0, 2.0, 3.0], [4.0, 5.0, 6.0]])
    W = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, -1.0]])
    # worked by hand: row 0 -> (1+3, 2-3), row 1 -> (4+6, 5-6)
    np.testing.assert_array_equal(oracle.matmul(X, W), [[4.0, -1.0], [10.0, -1.0]])


@pytest.mark.parametrize("M,K,N", [(1, 1, 1), (7, 5, 3), (33, 64, 48)])
def test_matmul_matches_blas(M, K, N):
    X = RNG.standard_normal((M, K))
    W = RNG.standard_normal((K, N))
    assert rel(oracle.matmul(X, W), X @ W) < 1e-13


def test_matmul_batched_leading_dims():
    X = RNG.standard_normal((2, 5, 6))
    W = RNG.standard_normal((6, 4))
    assert rel(oracle.matmul(X, W), np.einsum("bnd,de->bne", X, W)) < 1e-13


def test_scores_1d_matches_blas():
    X = RNG.standard_normal((3, 11, 8))
    WA = RNG.standard_normal((8, 4))
    z = oracle.scores_1d(X, WA)
    assert z.shape == (3, 4, 11)
    assert rel(z, np.transpose(X @ WA, (0, 2, 1))) < 1e-13


# ---------------------------------------------------------------- softmax
def test_softmax_matches_scipy():
    z = RNG.standard_normal((5, 17)) * 3
    assert rel(oracle.softmax(z), scipy.special.softmax(z, axis=-1)) < 1e-14


def test_softmax_closed_forms():
    L = 9
    np.testing.assert_allclose(oracle.softmax(np.zeros((2, L))), np.full((2, L), 1.0 / L), rtol=1e-15)
    # two entries: softmax(a, b)[0] = 1 / (1 + e^(b - a))
    s = oracle.softmax(np.array([[0.3, -1.2]]))
    np.testing.assert_allclose(s[0, 0], 1.0 / (1.0 + np.exp(-1.5)), rtol=1e-15)


def test_softmax_shift_invariance_and_overflow_safety():
    z = RNG.standard_normal((3, 12))
    base = oracle.softmax(z)
    big = oracle.softmax(z + 5000.0)  # exp would overflow without the max subtraction
    assert np.all(np.isfinite(big))
    np.testing.assert_allclose(big, base, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(base.sum(-1), 1.0, rtol=1e-15)


# ---------------------------------------------------------------- 1D circulant
def test_circulant_1d_golden_digits():
    g = gold("circulant_1d_n3_digits.json")
    w = np.array(g["w"])[None, None, :]
    V = np.array(g["V"])[None]
    np.testing.assert_array_equal(oracle.circulant_1d(w, V)[0], np.array(g["O"]))


@pytest.mark.parametrize("N,H,d", [(1, 1, 1), (2, 1, 3), (5, 2, 2), (8, 3, 4), (17, 2, 3)])
def test_circulant_1d_matches_scipy_circulant(N, H, d):
    B, D = 2, H * d
    w = RNG.standard_normal((B, H, N))
    V = RNG.standard_normal((B, N, D))
    O = oracle.circulant_1d(w, V)
    for b in range(B):
        for h in range(H):
            C = scipy.linalg.circulant(w[b, h])  # C[i, j] = w[(i - j) mod N]
            ref = C @ V[b, :, h * d:(h + 1) * d]
            assert rel(O[b, :, h * d:(h + 1) * d], ref) < 1e-13


@pytest.mark.parametrize("N", [3, 16, 31])
def test_circulant_1d_matches_convolution_theorem(N):
    # The CAT note's formula: circ(w) V = IFFT[FFT(w) . FFT(V)] along tokens.
    H, d = 2, 3
    w = RNG.standard_normal((1, H, N))
    V = RNG.standard_normal((1, N, H * d))
    O = oracle.circulant_1d(w, V)
    for h in range(H):
        ref = np.fft.ifft(np.fft.fft(w[0, h])[:, None] * np.fft.fft(V[0, :, h * d:(h + 1) * d], axis=0),
                          axis=0).real
        assert rel(O[0, :, h * d:(h + 1) * d], ref) < 1e-12


@pytest.mark.parametrize("k", [0, 1, 5, 12])
def test_circulant_1d_one_hot_is_cyclic_shift(k):
    N, H, d = 13, 2, 2
    w = np.zeros((1, H, N))
    w[0, :, k] = 1.0
    V = RNG.standard_normal((1, N, H * d))
    np.testing.assert_array_equal(oracle.circulant_1d(w, V), np.roll(V, k, axis=1))


def test_circulant_1d_token_constant_and_single_token():
    N, H, d = 10, 2, 3
    w = oracle.softmax(RNG.standard_normal((1, H, N)))
    V = np.broadcast_to(RNG.standard_normal((1, 1, H * d)), (1, N, H * d)).copy()
    np.testing.assert_allclose(oracle.circulant_1d(w, V), V, rtol=1e-14)
    w1 = np.array([[[0.7]]])
    V1 = RNG.standard_normal((1, 1, 4))
    np.testing.assert_allclose(oracle.circulant_1d(w1, V1), 0.7 * V1, rtol=1e-15)


def test_circulant_1d_row_subset_equals_full_rows():
    B, N, H, d = 3, 7, 2, 2
    w = RNG.standard_normal((B, H, N))
    V = RNG.standard_normal((B, N, H * d))
    full = oracle.circulant_1d(w, V).reshape(B * N, -1)
    rows = [0, 6, 7, 20, 13]
    np.testing.assert_array_equal(oracle.circulant_1d(w, V, rows=rows), full[rows])


def _materialise_circ(w):
    """circ(w) through the oracle: apply it to the identity (D = N channels)."""
    N = w.shape[-1]
    return oracle.circulant_1d(np.asarray(w)[None, None, :], np.eye(N)[None])[0]


def test_circulant_rows_sum_to_one_after_softmax():
    z = RNG.standard_normal(19) * 4
    C = _materialise_circ(oracle.softmax(z))
    np.testing.assert_allclose(C.sum(axis=1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(C.sum(axis=0), 1.0, rtol=1e-14)
    # every row is a permutation of the same weights: only the offset matters
    for i in range(19):
        np.testing.assert_array_equal(np.sort(C[i]), np.sort(C[0]))
        for j in range(19):
            assert C[i, j] == C[(i + 1) % 19, (j + 1) % 19]


def test_softmax_commutes_with_circ():
    # CAT note: softmax(circ(Z)) == circ(softmax(Z)) (row-wise softmax).
    z = RNG.standard_normal(11) * 3
    lhs = oracle.softmax(scipy.linalg.circulant(z))  # materialised by scipy
    rhs = _materialise_circ(oracle.softmax(z))
    np.testing.assert_allclose(lhs, rhs, rtol=1e-14, atol=1e-16)


# ---------------------------------------------------------------- CAT forward
def _cat_library_route(X, WA, WV):
    B, N, D = X.shape
    H = WA.shape[1]
    d = D // H
    z = np.transpose(X @ WA, (0, 2, 1))
    zs = scipy.special.softmax(z, axis=-1)
    V = X @ WV
    O = np.empty_like(V)
    for b in range(B):
        for h in range(H):
            O[b, :, h * d:(h + 1) * d] = scipy.linalg.circulant(zs[b, h]) @ V[b, :, h * d:(h + 1) * d]
    return O


@pytest.mark.parametrize("B,N,D,H", [(1, 1, 4, 2), (2, 3, 6, 3), (2, 16, 16, 4), (1, 23, 12, 2)])
def test_cat1d_matches_library_route(B, N, D, H):
    X = RNG.standard_normal((B, N, D))
    WA = RNG.standard_normal((D, H)) / np.sqrt(D)
    WV = RNG.standard_normal((D, D)) / np.sqrt(D)
    out = oracle.cat_forward_1d(X, WA, WV)
    assert rel(out["O"], _cat_library_route(X, WA, WV)) < 1e-12


@pytest.mark.parametrize("s", [1, 3, 8])
def test_cat1d_roll_tokens_rolls_output_twice(s):
    # Rolling X by s rolls both Z* and V by s, so O rolls by 2 s: the pin that
    # separates C[i][j] = w[i - j] from the mirrored convention.
    B, N, D, H = 1, 16, 8, 2
    X = RNG.standard_normal((B, N, D))
    WA = RNG.standard_normal((D, H))
    WV = RNG.standard_normal((D, D))
    O = oracle.cat_forward_1d(X, WA, WV)["O"]
    Or = oracle.cat_forward_1d(np.roll(X, s, axis=1), WA, WV)["O"]
    np.testing.assert_allclose(Or, np.roll(O, 2 * s, axis=1), rtol=1e-12, atol=1e-12)


def test_cat1d_one_hot_dominant_score_reproduces_shift():
    B, N, D, H, k = 1, 12, 6, 2, 5
    X = RNG.standard_normal((B, N, D)) * 0.01
    X[0, k, 0] = 60.0
    WA = np.zeros((D, H))
    WA[0, :] = 1.0
    WV = RNG.standard_normal((D, D))
    out = oracle.cat_forward_1d(X, WA, WV)
    np.testing.assert_allclose(out["O"], np.roll(out["V"], k, axis=1), rtol=1e-12, atol=1e-12)


def test_cat1d_uniform_scores_give_token_mean():
    B, N, D, H = 2, 9, 6, 3
    X = RNG.standard_normal((B, N, D))
    WA = np.zeros((D, H))
    WV = RNG.standard_normal((D, D))
    out = oracle.cat_forward_1d(X, WA, WV)
    np.testing.assert_allclose(out["O"], np.broadcast_to(out["V"].mean(axis=1, keepdims=True), out["O"].shape),
                               rtol=1e-13, atol=1e-14)


def test_cat1d_token_constant_input_is_fixed_point():
    B, N, D, H = 1, 7, 4, 2
    X = np.broadcast_to(RNG.standard_normal((B, 1, D)), (B, N, D)).copy()
    WA = RNG.standard_normal((D, H))
    WV = RNG.standard_normal((D, D))
    out = oracle.cat_forward_1d(X, WA, WV)
    np.testing.assert_allclose(out["O"], out["V"], rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------- 2D scores
def test_scores_2d_golden_digits():
    g = gold("scores_2d_2x3_digits.json")
    for case in g["cases"]:
        q = np.array(case["q"])[None]
        k = np.array(case["k"])[None]
        a = oracle.scores_bccb_2d(q, k, g["Hg"], g["Wg"], H=1)
        np.testing.assert_array_equal(a[0, 0], np.array(case["a"]))


@pytest.mark.parametrize("Hg,Wg,H,d", [(3, 4, 2, 3), (2, 3, 1, 4), (4, 4, 3, 2)])
def test_scores_2d_equal_wrapped_diagonal_sums_of_qk(Hg, Wg, H, d):
    # a[s] = (1/sqrt(d)) * sum of (Q K^T)[i, j] over pairs with i - j = s on the grid
    N, D = Hg * Wg, H * d
    Q = RNG.standard_normal((1, N, D))
    K = RNG.standard_normal((1, N, D))
    a = oracle.scores_bccb_2d(Q, K, Hg, Wg, H)
    for h in range(H):
        S = Q[0, :, h * d:(h + 1) * d] @ K[0, :, h * d:(h + 1) * d].T / np.sqrt(d)
        ref = np.zeros((Hg, Wg))
        for i in range(N):
            for j in range(N):
                s1 = (i // Wg - j // Wg) % Hg
                s2 = (i % Wg - j % Wg) % Wg
                ref[s1, s2] += S[i, j]
        assert rel(a[0, h], ref) < 1e-13


def test_scores_2d_matches_fft_correlation():
    Hg, Wg, H, d = 6, 5, 2, 4
    Q = RNG.standard_normal((2, Hg * Wg, H * d))
    K = RNG.standard_normal((2, Hg * Wg, H * d))
    a = oracle.scores_bccb_2d(Q, K, Hg, Wg, H)
    for b in range(2):
        for h in range(H):
            q = Q[b, :, h * d:(h + 1) * d].reshape(Hg, Wg, d)
            k = K[b, :, h * d:(h + 1) * d].reshape(Hg, Wg, d)
            spec = (np.fft.fft2(q, axes=(0, 1)) * np.conj(np.fft.fft2(k, axes=(0, 1)))).sum(-1)
            ref = np.fft.ifft2(spec).real / np.sqrt(d)
            assert rel(a[b, h], ref) < 1e-12


# ---------------------------------------------------------------- 2D BCCB
def test_bccb_2d_golden_digits():
    g = gold("bccb_2d_2x3_digits.json")
    w = np.array(g["w"])[None, None]
    V = np.array(g["V"])[None]
    np.testing.assert_array_equal(oracle.bccb_2d(w, V)[0], np.array(g["O"]))


def _bccb_matrix(w):
    """Block-circulant matrix with circulant blocks: block (i1, j1) is
    circ(w[(i1 - j1) mod Hg]) built with scipy."""
    Hg, Wg = w.shape
    blocks = [scipy.linalg.circulant(w[r]) for r in range(Hg)]
    M = np.zeros((Hg * Wg, Hg * Wg))
    for i1 in range(Hg):
        for j1 in range(Hg):
            M[i1 * Wg:(i1 + 1) * Wg, j1 * Wg:(j1 + 1) * Wg] = blocks[(i1 - j1) % Hg]
    return M


@pytest.mark.parametrize("Hg,Wg", [(1, 1), (1, 5), (4, 1), (3, 4), (5, 6)])
def test_bccb_2d_matches_materialised_bccb_and_fft2(Hg, Wg):
    H, d = 2, 3
    w = RNG.standard_normal((1, H, Hg, Wg))
    V = RNG.standard_normal((1, Hg * Wg, H * d))
    O = oracle.bccb_2d(w, V)
    for h in range(H):
        Vh = V[0, :, h * d:(h + 1) * d]
        assert rel(O[0, :, h * d:(h + 1) * d], _bccb_matrix(w[0, h]) @ Vh) < 1e-13
        conv = np.fft.ifft2(np.fft.fft2(w[0, h])[:, :, None] * np.fft.fft2(Vh.reshape(Hg, Wg, d), axes=(0, 1)),
                            axes=(0, 1)).real.reshape(Hg * Wg, d)
        assert rel(O[0, :, h * d:(h + 1) * d], conv) < 1e-12


def test_bccb_2d_one_hot_is_grid_shift():
    Hg, Wg, H, d = 4, 5, 1, 2
    w = np.zeros((1, H, Hg, Wg))
    w[0, 0, 1, 3] = 1.0
    V = RNG.standard_normal((1, Hg * Wg, d))
    O = oracle.bccb_2d(w, V)
    ref = np.roll(V.reshape(Hg, Wg, d), (1, 3), axis=(0, 1)).reshape(1, Hg * Wg, d)
    np.testing.assert_array_equal(O, ref)


def _ca2d_library_route(X, WQ, WK, WV, Hg, Wg, H):
    B, N, D = X.shape
    d = D // H
    Q, K, V = X @ WQ, X @ WK, X @ WV
    O = np.empty_like(V)
    for b in range(B):
        for h in range(H):
            q = Q[b, :, h * d:(h + 1) * d].reshape(Hg, Wg, d)
            k = K[b, :, h * d:(h + 1) * d].reshape(Hg, Wg, d)
            a = np.fft.ifft2((np.fft.fft2(q, axes=(0, 1)) * np.conj(np.fft.fft2(k, axes=(0, 1)))).sum(-1)).real
            a = scipy.special.softmax(a.reshape(-1) / np.sqrt(d)).reshape(Hg, Wg)
            O[b, :, h * d:(h + 1) * d] = _bccb_matrix(a) @ V[b, :, h * d:(h + 1) * d]
    return O


@pytest.mark.parametrize("B,Hg,Wg,D,H", [(1, 1, 1, 4, 2), (2, 3, 4, 6, 2), (1, 5, 3, 8, 2)])
def test_ca2d_matches_library_route(B, Hg, Wg, D, H):
    X = RNG.standard_normal((B, Hg * Wg, D))
    W = [RNG.standard_normal((D, D)) / np.sqrt(D) for _ in range(3)]
    out = oracle.cat_forward_bccb_2d(X, *W, Hg, Wg, H)
    assert rel(out["O"], _ca2d_library_route(X, *W, Hg, Wg, H)) < 1e-12
    np.testing.assert_allclose(out["astar"].reshape(B, H, -1).sum(-1), 1.0, rtol=1e-14)


@pytest.mark.parametrize("t", [(1, 0), (0, 2), (2, 3)])
def test_ca2d_grid_roll_rolls_output(t):
    # The score map only depends on relative offsets, so shifting the image on
    # the (circular) grid shifts the output by the same amount.
    B, Hg, Wg, D, H = 1, 4, 5, 6, 2
    X = RNG.standard_normal((B, Hg * Wg, D))
    W = [RNG.standard_normal((D, D)) / np.sqrt(D) for _ in range(3)]
    O = oracle.cat_forward_bccb_2d(X, *W, Hg, Wg, H)["O"]
    Xr = np.roll(X.reshape(B, Hg, Wg, D), t, axis=(1, 2)).reshape(B, Hg * Wg, D)
    Or = oracle.cat_forward_bccb_2d(Xr, *W, Hg, Wg, H)["O"]
    ref = np.roll(O.reshape(B, Hg, Wg, D), t, axis=(1, 2)).reshape(B, Hg * Wg, D)
    np.testing.assert_allclose(Or, ref, rtol=1e-12, atol=1e-12)


def test_bccb_2d_row_subset_equals_full_rows():
    B, Hg, Wg, H, d = 2, 3, 4, 2, 2
    w = RNG.standard_normal((B, H, Hg, Wg))
    V = RNG.standard_normal((B, Hg * Wg, H * d))
    full = oracle.bccb_2d(w, V).reshape(B * Hg * Wg, -1)
    rows = [0, 5, 12, 23]
    np.testing.assert_array_equal(oracle.bccb_2d(w, V, rows=rows), full[rows])


# ---------------------------------------------------------------- planted mistakes
# Each mutant is a copy of an oracle step with one plausible mistake; some pin
# above must reject it.  The pins are re-run here against the mutant.

def _mutant_mirrored_circ(w, V):
    N = w.shape[-1]
    return oracle.circulant_1d(w[..., (-np.arange(N)) % N], V)  # C[i][j] = w[j - i]


def _mutant_off_by_one_circ(w, V):
    return oracle.circulant_1d(np.roll(w, 1, axis=-1), V)  # C[i][j] = w[i - j - 1]


def _mutant_softmax_wrong_axis(z):
    return np.swapaxes(oracle.softmax(np.swapaxes(z, -1, -2)), -1, -2)


def test_planted_mirrored_convention_is_caught():
    g = gold("circulant_1d_n3_digits.json")
    out = _mutant_mirrored_circ(np.array(g["w"])[None, None, :], np.array(g["V"])[None])[0]
    assert not np.array_equal(out, np.array(g["O"]))
    # and the roll-by-2s pin fails too
    B, N, D, H = 1, 16, 8, 2
    X = RNG.standard_normal((B, N, D))
    WA, WV = RNG.standard_normal((D, H)), RNG.standard_normal((D, D))

    def fwd(x):
        return _mutant_mirrored_circ(oracle.softmax(oracle.scores_1d(x, WA)), oracle.matmul(x, WV))

    assert not np.allclose(fwd(np.roll(X, 3, axis=1)), np.roll(fwd(X), 6, axis=1), atol=1e-6)


def test_planted_off_by_one_is_caught():
    N, H, d = 13, 1, 2
    w = np.zeros((1, H, N))
    w[0, 0, 4] = 1.0
    V = RNG.standard_normal((1, N, d))
    assert not np.array_equal(_mutant_off_by_one_circ(w, V), np.roll(V, 4, axis=1))


def test_planted_transposed_weight_is_caught():
    B, N, D, H = 2, 5, 6, 2
    X = RNG.standard_normal((B, N, D))
    WA = RNG.standard_normal((D, H))
    WV = RNG.standard_normal((D, D))
    bad = oracle.circulant_1d(oracle.softmax(oracle.scores_1d(X, WA)), oracle.matmul(X, WV.T))
    assert rel(bad, _cat_library_route(X, WA, WV)) > 1e-3


def test_planted_softmax_axis_is_caught():
    z = RNG.standard_normal((4, 6))
    assert not np.allclose(_mutant_softmax_wrong_axis(z), scipy.special.softmax(z, axis=-1))


def test_planted_missing_score_scale_is_caught():
    Hg, Wg, H, d = 3, 4, 1, 4
    Q = RNG.standard_normal((1, Hg * Wg, d))
    K = RNG.standard_normal((1, Hg * Wg, d))
    bad = oracle.scores_bccb_2d(Q, K, Hg, Wg, H, scale=1.0)
    S = Q[0] @ K[0].T / np.sqrt(d)
    ref = np.zeros((Hg, Wg))
    for i in range(Hg * Wg):
        for j in range(Hg * Wg):
            ref[(i // Wg - j // Wg) % Hg, (i % Wg - j % Wg) % Wg] += S[i, j]
    assert rel(bad[0, 0], ref) > 0.5


def test_planted_conjugate_on_wrong_side_is_caught():
    # correlating the other way gives a[-s]; the golden digits reject it
    g = gold("scores_2d_2x3_digits.json")
    case = g["cases"][0]
    q = np.array(case["q"])[None]
    k = np.array(case["k"])[None]
    bad = oracle.scores_bccb_2d(k, q, g["Hg"], g["Wg"], H=1)  # swaps the conjugated side
    assert not np.array_equal(bad[0, 0], np.array(case["a"]))


# ---------------------------------------------------------------- CAT-scored 2D variant
@pytest.mark.parametrize("Hg,Wg", [(1, 7), (5, 1), (1, 12)])
def test_cat_scored_2d_on_a_line_is_cat_1d(Hg, Wg):
    """A 1 x N (or N x 1) grid's BCCB matrix is the circulant of the line, so
    the CAT-scored 2D forward equals the 1D CAT forward there."""
    rng = np.random.default_rng(40 + Hg * Wg)
    B, D, H = 2, 6, 3
    N = Hg * Wg
    X = rng.standard_normal((B, N, D))
    WA, WV = rng.standard_normal((D, H)), rng.standard_normal((D, D))
    got = oracle.cat_scored_forward_2d(X, WA, WV, Hg, Wg)["O"]
    assert np.allclose(got, oracle.cat_forward_1d(X, WA, WV)["O"], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("s1,s2", [(1, 0), (0, 2), (2, 3)])
def test_cat_scored_2d_grid_roll_rolls_output_twice(s1, s2):
    """Scores move with their tokens and so do the values: rolling X on the
    grid by (s1, s2) rolls the output by (2 s1, 2 s2)."""
    rng = np.random.default_rng(7)
    B, Hg, Wg, D, H = 1, 4, 5, 4, 2
    X = rng.standard_normal((B, Hg * Wg, D))
    WA, WV = rng.standard_normal((D, H)), rng.standard_normal((D, D))

    def fwd(x):
        return oracle.cat_scored_forward_2d(x, WA, WV, Hg, Wg)["O"].reshape(B, Hg, Wg, D)

    Xr = np.roll(X.reshape(B, Hg, Wg, D), (s1, s2), axis=(1, 2)).reshape(B, Hg * Wg, D)
    assert np.allclose(fwd(Xr), np.roll(fwd(X), (2 * s1, 2 * s2), axis=(1, 2)), atol=1e-12)


def test_cat_scored_2d_matches_materialised_bccb():
    """Against the BCCB matrix built entry by entry from the softmaxed scores."""
    rng = np.random.default_rng(5)
    B, Hg, Wg, D, H = 1, 3, 4, 4, 2
    N, d = Hg * Wg, D // H
    X = rng.standard_normal((B, N, D))
    WA, WV = rng.standard_normal((D, H)), rng.standard_normal((D, D))
    got = oracle.cat_scored_forward_2d(X, WA, WV, Hg, Wg)["O"]
    z = X[0] @ WA
    zs = np.exp(z - z.max(axis=0)) / np.exp(z - z.max(axis=0)).sum(axis=0)
    V = X[0] @ WV
    for h in range(H):
        C = np.zeros((N, N))
        for i in range(N):
            for j in range(N):
                C[i, j] = zs[((i // Wg - j // Wg) % Hg) * Wg + (i % Wg - j % Wg) % Wg, h]
        assert np.allclose(got[0][:, h * d:(h + 1) * d], C @ V[:, h * d:(h + 1) * d], atol=1e-12)


# ---------------------------------------------------------------- 1D mixing backward
def _mix_loss(z, V, G):
    """The scalar <circ(softmax(z)) V, G> whose gradients the backward gives."""
    return float(np.sum(oracle.circulant_1d(oracle.softmax(z), V) * G))


@pytest.mark.parametrize("B,N,H,d", [(1, 1, 1, 2), (2, 5, 2, 2), (1, 7, 3, 2), (1, 4, 1, 4)])
def test_mix_backward_matches_finite_differences(B, N, H, d):
    """Central differences of the (separately pinned) forward: every logit and
    every value entry, step 1e-5, agreement to ~1e-8 relative."""
    rng = np.random.default_rng(7 + N)
    z = rng.standard_normal((B, H, N)) * 1.5
    V = rng.standard_normal((B, N, H * d))
    G = rng.standard_normal((B, N, H * d))
    got = oracle.mix_backward_1d(z, V, G)
    eps = 1e-5
    num_dz = np.zeros_like(z)
    for idx in np.ndindex(z.shape):
        zp, zm = z.copy(), z.copy()
        zp[idx] += eps
        zm[idx] -= eps
        num_dz[idx] = (_mix_loss(zp, V, G) - _mix_loss(zm, V, G)) / (2 * eps)
    num_dV = np.zeros_like(V)
    for idx in np.ndindex(V.shape):
        Vp, Vm = V.copy(), V.copy()
        Vp[idx] += eps
        Vm[idx] -= eps
        num_dV[idx] = (_mix_loss(z, Vp, G) - _mix_loss(z, Vm, G)) / (2 * eps)
    assert np.allclose(got["dz"], num_dz, rtol=1e-7, atol=1e-9), np.max(np.abs(got["dz"] - num_dz))
    assert np.allclose(got["dV"], num_dV, rtol=1e-7, atol=1e-9), np.max(np.abs(got["dV"] - num_dV))


@pytest.mark.parametrize("N,H,d", [(6, 2, 3), (16, 1, 4), (9, 3, 2)])
def test_mix_backward_matches_library_routes(N, H, d):
    """dV against the materialised scipy circulant's transpose; dz* against the
    FFT cross-correlation summed over the head's channels."""
    rng = np.random.default_rng(100 + N)
    w = rng.random((1, H, N))
    V = rng.standard_normal((1, N, H * d))
    G = rng.standard_normal((1, N, H * d))
    dV = oracle.circulant_1d_transpose(w, G)
    dw = oracle.circulant_1d_grad_w(G, V, H)
    for h in range(H):
        C = scipy.linalg.circulant(w[0, h])  # C[i][j] = w[(i - j) mod N]
        sl = slice(h * d, (h + 1) * d)
        assert np.allclose(dV[0][:, sl], C.T @ G[0][:, sl], rtol=1e-12, atol=1e-12)
        xc = np.fft.ifft(np.sum(np.fft.fft(G[0][:, sl], axis=0) * np.conj(np.fft.fft(V[0][:, sl], axis=0)), axis=1))
        assert np.allclose(dw[0, h], xc.real, rtol=1e-10, atol=1e-10)


def test_mix_backward_logit_gradient_sums_to_zero():
    """Softmax is invariant to adding a constant to a line's logits, so each
    line of dz sums to zero; uniform values (token-constant V) give dz = 0."""
    rng = np.random.default_rng(3)
    B, N, H, d = 2, 11, 2, 2
    z = rng.standard_normal((B, H, N))
    G = rng.standard_normal((B, N, H * d))
    V = rng.standard_normal((B, N, H * d))
    dz = oracle.mix_backward_1d(z, V, G)["dz"]
    assert np.allclose(dz.sum(axis=-1), 0.0, atol=1e-12)
    Vc = np.broadcast_to(rng.standard_normal((B, 1, H * d)), (B, N, H * d))
    assert np.allclose(oracle.mix_backward_1d(z, Vc, G)["dz"], 0.0, atol=1e-12)


def test_cat_backward_matches_finite_differences():
    """Central differences of the whole (pinned) CAT forward, for every entry
    of X, W_A and W_V."""
    rng = np.random.default_rng(21)
    B, N, D, H = 2, 4, 4, 2
    X = rng.standard_normal((B, N, D))
    WA = rng.standard_normal((D, H))
    WV = rng.standard_normal((D, D))
    G = rng.standard_normal((B, N, D))
    got = oracle.cat_backward_1d(X, WA, WV, G)

    def loss(x, wa, wv):
        return float(np.sum(oracle.cat_forward_1d(x, wa, wv)["O"] * G))

    eps = 1e-5
    for name, arr, idx_of in (("dX", X, 0), ("dW_A", WA, 1), ("dW_V", WV, 2)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            args_p = [X.copy(), WA.copy(), WV.copy()]
            args_m = [X.copy(), WA.copy(), WV.copy()]
            args_p[idx_of][idx] += eps
            args_m[idx_of][idx] -= eps
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        assert np.allclose(got[name], num, rtol=1e-7, atol=1e-8), (name, np.max(np.abs(got[name] - num)))


def test_planted_backward_lag_sign_is_caught():
    """A score gradient correlating the wrong way (V[(i + k) mod N]) fails the
    finite-difference pin."""
    rng = np.random.default_rng(11)
    B, N, H, d = 1, 5, 1, 2
    z = rng.standard_normal((B, H, N))
    V = rng.standard_normal((B, N, d))
    G = rng.standard_normal((B, N, d))
    zs = oracle.softmax(z)
    bad = oracle.softmax_backward(zs, oracle.circulant_1d_grad_w(G[:, (-np.arange(N)) % N], V[:, (-np.arange(N)) % N], H))
    eps = 1e-5
    num = np.zeros_like(z)
    for idx in np.ndindex(z.shape):
        zp, zm = z.copy(), z.copy()
        zp[idx] += eps
        zm[idx] -= eps
        num[idx] = (_mix_loss(zp, V, G) - _mix_loss(zm, V, G)) / (2 * eps)
    assert not np.allclose(bad, num, rtol=1e-4, atol=1e-6)


def test_oracle_reports_threads():
    assert oracle.num_threads() >= 1


# ---------------------------------------------------------------- averaged-key variant
def test_avgkey_scores_golden_digits():
    g = gold("avgkey_scores_n3_digits.json")
    z = oracle.avgkey_scores_1d(np.array(g["X"])[None], np.array(g["W_Q"]), np.array(g["W_K"]), g["H"])
    np.testing.assert_array_equal(z[0, 0], np.array(g["z"]))


@pytest.mark.parametrize("H,alpha", [(1, 0.7), (3, -1.3), (4, 2.0)])
def test_avgkey_reduces_to_cat_for_a_one_hot_mean_key(H, alpha):
    """With a token-constant input channel (X[:, :, 0] = 1) and W_K whose only
    nonzero entries are W_K[0][c_h] = alpha for one channel c_h of each head,
    the averaged key of head h is alpha e_{c_h}, so z_h = alpha Q[:, c_h] /
    sqrt(d) = X (alpha W_Q[:, c_h] / sqrt(d)): the CAT logits of the pinned
    scores_1d with that W_A column, and the whole forward equals CAT's."""
    rng = np.random.default_rng(60 + H)
    B, N, d = 2, 9, 4
    D = H * d
    X = rng.standard_normal((B, N, D))
    X[:, :, 0] = 1.0
    WQ, WV = rng.standard_normal((D, D)), rng.standard_normal((D, D))
    WK = np.zeros((D, D))
    cs = [h * d + (h + 1) % d for h in range(H)]
    for c in cs:
        WK[0, c] = alpha
    WA = np.stack([alpha * WQ[:, c] / np.sqrt(d) for c in cs], axis=1)
    got = oracle.cat_avgkey_forward_1d(X, WQ, WK, WV, H)
    ref = oracle.cat_forward_1d(X, WA, WV)
    assert np.allclose(got["z"], ref["z"], rtol=1e-12, atol=1e-12)
    assert np.allclose(got["O"], ref["O"], rtol=1e-12, atol=1e-12)


def test_avgkey_matches_reassociated_library_route():
    """z = X (W_Q,h kbar_h) / sqrt(d) with kbar = mean(X) W_K by BLAS (the
    same sums in another association), then scipy's circulant matrix."""
    rng = np.random.default_rng(77)
    B, N, D, H = 2, 11, 12, 3
    d = D // H
    X = rng.standard_normal((B, N, D))
    WQ, WK, WV = (rng.standard_normal((D, D)) for _ in range(3))
    got = oracle.cat_avgkey_forward_1d(X, WQ, WK, WV, H)
    for b in range(B):
        kbar = X[b].mean(axis=0) @ WK
        V = X[b] @ WV
        for h in range(H):
            sl = slice(h * d, (h + 1) * d)
            z = X[b] @ (WQ[:, sl] @ kbar[sl]) / np.sqrt(d)
            assert np.allclose(got["z"][b, h], z, rtol=1e-12, atol=1e-12)
            C = scipy.linalg.circulant(scipy.special.softmax(z))
            assert np.allclose(got["O"][b][:, sl], C @ V[:, sl], rtol=1e-11, atol=1e-12)


def test_avgkey_invariants():
    """Token-constant X gives equal logits, a uniform circulant and O = V;
    rolling X along the tokens leaves the mean key unchanged, so the output
    rolls twice as far, as in CAT."""
    rng = np.random.default_rng(8)
    B, N, D, H = 1, 10, 8, 2
    WQ, WK, WV = (rng.standard_normal((D, D)) for _ in range(3))
    Xc = np.broadcast_to(rng.standard_normal((B, 1, D)), (B, N, D)).copy()
    r = oracle.cat_avgkey_forward_1d(Xc, WQ, WK, WV, H)
    assert np.allclose(r["zstar"], 1.0 / N, atol=1e-15)
    assert np.allclose(r["O"], r["V"], rtol=1e-12, atol=1e-12)
    X = rng.standard_normal((B, N, D))
    O = oracle.cat_avgkey_forward_1d(X, WQ, WK, WV, H)["O"]
    Or = oracle.cat_avgkey_forward_1d(np.roll(X, 3, axis=1), WQ, WK, WV, H)["O"]
    assert np.allclose(Or, np.roll(O, 6, axis=1), atol=1e-12)


def test_planted_avgkey_mistakes_are_caught():
    """A sum instead of a mean, a missing 1/sqrt(d), Q and K swapped, or the
    mean taken over channels instead of tokens each miss the golden digits."""
    g = gold("avgkey_scores_n3_digits.json")
    X, WQ, WK = np.array(g["X"])[None], np.array(g["W_Q"]), np.array(g["W_K"])
    want = np.array(g["z"])
    d = X.shape[2]
    Q, K = X[0] @ WQ, X[0] @ WK
    mutants = {
        "sum": Q @ K.sum(axis=0) / np.sqrt(d),
        "no scale": Q @ K.mean(axis=0),
        "swapped": K @ Q.mean(axis=0) / np.sqrt(d),
        "channel mean": (Q * K.mean(axis=1, keepdims=True)).sum(axis=1) / np.sqrt(d),
    }
    for name, z in mutants.items():
        assert not np.allclose(z, want), name


# ---------------------------------------------------------------- causal CAT
def test_causal_golden_digits():
    g = gold("causal_1d_n3_digits.json")
    O = oracle.causal_1d(np.array(g["z"])[None, None, :], np.array(g["V"])[None])[0]
    np.testing.assert_allclose(O, np.array(g["O"]), rtol=1e-15)
    np.testing.assert_allclose(np.array(g["numerators"]) / np.array(g["denominators"]), np.array(g["O"])[:, 0])


@pytest.mark.parametrize("N,H,d", [(1, 1, 2), (2, 2, 1), (7, 1, 3), (16, 3, 2), (31, 2, 4)])
def test_causal_matches_masked_dense_attention(N, H, d):
    """Against the materialised score matrix S[i][j] = z[(i - j) mod N] (via
    scipy's circulant), the entries j > i set to -inf, scipy's row softmax,
    and a BLAS product."""
    rng = np.random.default_rng(200 + N)
    B, D = 2, H * d
    z = rng.standard_normal((B, H, N)) * 2
    V = rng.standard_normal((B, N, D))
    O = oracle.causal_1d(z, V)
    for b in range(B):
        for h in range(H):
            S = scipy.linalg.circulant(z[b, h]).copy()
            S[np.triu_indices(N, 1)] = -np.inf
            P = scipy.special.softmax(S, axis=1)
            sl = slice(h * d, (h + 1) * d)
            assert np.allclose(O[b][:, sl], P @ V[b][:, sl], rtol=1e-12, atol=1e-12)


def test_causal_special_rows_and_invariants():
    """Row 0 is V[0]; the last row keeps every token and every lag, so it is
    the last row of the (pinned) non-causal circulant; weights sum to one
    (token-constant V is returned); row i depends only on tokens <= i (the
    causal output of a prefix is the prefix of the causal output); a huge
    common shift of the logits changes nothing (max subtraction)."""
    rng = np.random.default_rng(9)
    B, N, H, d = 2, 13, 2, 3
    D = H * d
    z = rng.standard_normal((B, H, N)) * 3
    V = rng.standard_normal((B, N, D))
    O = oracle.causal_1d(z, V)
    assert np.allclose(O[:, 0], V[:, 0], rtol=1e-14, atol=1e-15)
    full = oracle.circulant_1d(oracle.softmax(z), V)
    assert np.allclose(O[:, N - 1], full[:, N - 1], rtol=1e-12, atol=1e-13)
    Vc = np.broadcast_to(rng.standard_normal((B, 1, D)), (B, N, D)).copy()
    assert np.allclose(oracle.causal_1d(z, Vc), Vc, rtol=1e-13, atol=1e-14)
    M = 6
    assert np.allclose(oracle.causal_1d(z[..., :M], V[:, :M]), O[:, :M], rtol=1e-13, atol=1e-14)
    # (adding 4000 rounds each logit by up to 2^-41, about 5e-13)
    assert np.allclose(oracle.causal_1d(z + 4000.0, V), O, rtol=1e-10, atol=1e-11)
    rows = [0, 5, N + 3, 2 * N - 1]
    assert np.allclose(oracle.causal_1d(z, V, rows=rows), O.reshape(B * N, D)[rows], rtol=1e-15, atol=0)


def test_planted_causal_mistakes_are_caught():
    """An anti-causal mask (j >= i), a strict mask (j < i, row 0 undefined,
    so the diagonal is dropped on the others), and masking after a global
    softmax without renormalising each miss the golden digits."""
    g = gold("causal_1d_n3_digits.json")
    z, V, want = np.array(g["z"]), np.array(g["V"])[:, 0], np.array(g["O"])[:, 0]
    N = len(z)
    S = scipy.linalg.circulant(z)

    def masked(keep, renorm=True):
        P = np.where(keep, np.exp(S), 0.0)
        if renorm:
            P = P / np.maximum(P.sum(axis=1, keepdims=True), 1e-300)
        else:
            P = P / np.exp(z).sum()
        return P @ V

    i, j = np.indices((N, N))
    assert not np.allclose(masked(j >= i), want)
    assert not np.allclose(masked((j < i) | (i == 0)), want)
    assert not np.allclose(masked(j <= i, renorm=False), want)
    assert np.allclose(masked(j <= i), want)


@pytest.mark.parametrize("B,N,D,H", [(1, 5, 4, 2), (2, 12, 6, 3)])
def test_cat_causal_forward_composes_pinned_steps(B, N, D, H):
    rng = np.random.default_rng(N)
    X = rng.standard_normal((B, N, D))
    WA, WV = rng.standard_normal((D, H)), rng.standard_normal((D, D))
    r = oracle.cat_causal_forward_1d(X, WA, WV)
    assert np.allclose(r["O"], oracle.causal_1d(np.transpose(X @ WA, (0, 2, 1)), X @ WV), rtol=1e-12, atol=1e-12)
