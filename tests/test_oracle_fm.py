"""Pins of the oracle's GLM factorization machine (ROCS Sec. 3.1.4, Eq. 9-10, two groups): brute
force on tiny inputs, the symmetry and closed forms of the self-interaction blocks, the GLM
invariant (request outputs ignore every candidate; a candidate's outputs depend on its own
embeddings and its request's only), and the index handling shared with the other operators."""
import numpy as np

import oracle
import synth


def tiny(seed, R=3, C=7, n_r=4, n_c=3, d=5, kind="f32"):
    x_r = synth.draw(seed, 1, R * n_r * d, kind).reshape(R, n_r, d)
    x_c = synth.draw(seed, 2, C * n_c * d, kind).reshape(C, n_c, d)
    return x_r, x_c


def test_fm_brute_force():
    x_r, x_c = tiny(1)
    m = np.array([0, 0, 2, 1, 1, 1, 2], dtype=np.int32)
    got = oracle.fm(x_r, x_c, m=m, want_request=True)
    xr, xc = x_r.astype(np.float64), x_c.astype(np.float64)
    for c in range(7):
        r = m[c]
        for i in range(3):
            for n in range(4):
                assert abs(got["y_c"][c, i, n] - sum(xc[c, i, k] * xr[r, n, k] for k in range(5))) < 1e-12
            for n in range(3):
                assert abs(got["y_c"][c, i, 4 + n] - sum(xc[c, i, k] * xc[c, n, k] for k in range(5))) < 1e-12
    for r in range(3):
        for i in range(4):
            for n in range(4):
                assert abs(got["y_r"][r, i, n] - sum(xr[r, i, k] * xr[r, n, k] for k in range(5))) < 1e-12


def test_fm_self_blocks_are_gram_matrices():
    x_r, x_c = tiny(2, n_r=6, n_c=5, d=9)
    m = np.array([1, 0, 2, 2, 0, 1, 1], dtype=np.int32)
    got = oracle.fm(x_r, x_c, m=m, want_request=True)
    cc = got["y_c"][:, :, 6:]
    assert np.array_equal(cc, np.transpose(cc, (0, 2, 1)))          # symmetric
    assert np.all(np.einsum("cii->ci", cc) >= 0)                     # diagonal = squared norms
    assert np.array_equal(got["y_r"], np.transpose(got["y_r"], (0, 2, 1)))
    # orthonormal candidate rows: the self block is the identity
    e = np.zeros((1, 3, 4), dtype=np.float32)
    e[0, 0, 1] = e[0, 1, 3] = e[0, 2, 0] = 1.0
    one = oracle.fm(np.ones((1, 2, 4), dtype=np.float32), e, m=np.zeros(1, dtype=np.int32))
    assert np.array_equal(one["y_c"][0, :, 2:], np.eye(3))
    assert np.array_equal(one["y_c"][0, :, :2], np.ones((3, 2)))


def test_fm_glm_invariant():
    """Request outputs do not depend on any candidate; a candidate's outputs depend only on its own
    embeddings and its request's (Eq. 10's zero block)."""
    x_r, x_c = tiny(3)
    m = np.array([0, 1, 1, 2, 2, 2, 0], dtype=np.int32)
    base = oracle.fm(x_r, x_c, m=m, want_request=True)
    x_c2 = x_c.copy()
    x_c2[4] *= -3.0                                    # change one candidate of request 2
    x_r2 = x_r.copy()
    x_r2[1] += 1.0                                     # change request 1
    after = oracle.fm(x_r2, x_c2, m=m, want_request=True)
    assert np.array_equal(after["y_r"][[0, 2]], base["y_r"][[0, 2]])
    same = [0, 3, 5, 6]                                # not candidate 4, not request 1's candidates
    assert np.array_equal(after["y_c"][same], base["y_c"][same])
    assert not np.array_equal(after["y_c"][4], base["y_c"][4])
    assert not np.array_equal(after["y_c"][[1, 2]], base["y_c"][[1, 2]])


def test_fm_index_paths_and_invalid_rows():
    x_r, x_c = tiny(4, kind="bf16")
    off = np.array([0, 2, 2, 7], dtype=np.int32)       # request 1 has no candidates
    m = np.array([0, 0, 2, 2, 2, 2, 2], dtype=np.int32)
    a = oracle.fm(x_r, x_c, off=off)["y_c"]
    b = oracle.fm(x_r, x_c, m=m)["y_c"]
    assert np.array_equal(a, b)
    bad = m.copy()
    bad[3] = 9                                         # out of range: zeros
    z = oracle.fm(x_r, x_c, m=bad)["y_c"]
    assert np.all(z[3] == 0) and np.array_equal(z[[0, 1, 2, 4, 5, 6]], b[[0, 1, 2, 4, 5, 6]])
    # offsets that cover only part of the candidates: the rest get zeros
    part = oracle.fm(x_r, x_c, off=np.array([0, 2, 2, 5], dtype=np.int32))["y_c"]
    assert np.all(part[5:] == 0) and np.array_equal(part[:5], a[:5])
    # cands selects rows in the order asked
    assert np.array_equal(oracle.fm(x_r, x_c, m=m, cands=[6, 0])["y_c"], b[[6, 0]])
