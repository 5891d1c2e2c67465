"""Pins of the oracle's LCB in its embedding-matrix form (ROCS Sec. 3.1.2 Eq. 5-6, two groups) with
the group-local normalisation of Sec. 3.1.3 Eq. 7: brute force on tiny inputs, the explicit
block-matrix form of Eq. 6 with its zero block, the reduction to the (independently pinned) linear
GLM layer when d = 1, torch's own layer_norm / rms_norm for the norm step, closed forms, the GLM
invariant and the index handling."""
import numpy as np
import pytest
import torch

import oracle
import synth


def case(seed, R=3, C=7, n_r=4, n_c=3, d=5, k_r=2, k_c=6, kind="f32"):
    x_r = synth.draw(seed, 1, R * n_r * d, kind).reshape(R, n_r, d)
    x_c = synth.draw(seed, 2, C * n_c * d, kind).reshape(C, n_c, d)
    w_rr = synth.draw(seed, 3, k_r * n_r, kind).reshape(k_r, n_r)
    w_cr = synth.draw(seed, 4, k_c * n_r, kind).reshape(k_c, n_r)
    w_cc = synth.draw(seed, 5, k_c * n_c, kind).reshape(k_c, n_c)
    return x_r, x_c, w_rr, w_cr, w_cc


MAP = np.array([0, 0, 2, 1, 1, 1, 2], dtype=np.int32)


def test_brute_force_no_norm():
    x_r, x_c, w_rr, w_cr, w_cc = case(1)
    got = oracle.lcb_emb(x_r, x_c, w_rr, w_cr, w_cc, m=MAP, want_request=True)
    xr, xc = x_r.astype(np.float64), x_c.astype(np.float64)
    wrr, wcr, wcc = (w.astype(np.float64) for w in (w_rr, w_cr, w_cc))
    for c in range(7):
        r = MAP[c]
        for o in range(6):
            for j in range(5):
                want = sum(wcr[o, k] * xr[r, k, j] for k in range(4)) + sum(wcc[o, k] * xc[c, k, j] for k in range(3))
                assert abs(got["y_c"][c, o, j] - want) < 1e-12
    for r in range(3):
        for o in range(2):
            for j in range(5):
                assert abs(got["y_r"][r, o, j] - sum(wrr[o, k] * xr[r, k, j] for k in range(4))) < 1e-12


@pytest.mark.parametrize("norm", ["layer", "rms"])
def test_brute_force_norm(norm):
    x_r, x_c, w_rr, w_cr, w_cc = case(2)
    g = synth.draw(2, 6, 5, "f32") + 1.0
    b = synth.draw(2, 7, 5, "f32")
    raw = oracle.lcb_emb(x_r, x_c, w_rr, w_cr, w_cc, m=MAP, want_request=True)
    got = oracle.lcb_emb(x_r, x_c, w_rr, w_cr, w_cc, m=MAP, want_request=True, norm=norm, gamma_c=g,
                         beta_c=b, gamma_r=b, beta_r=g, eps=1e-3)
    for key, gg, bb in (("y_c", g, b), ("y_r", b, g)):
        flat_raw = raw[key].reshape(-1, 5)
        flat_got = got[key].reshape(-1, 5)
        for row, out in zip(flat_raw, flat_got):
            vals = [float(v) for v in row]
            if norm == "layer":
                mean = sum(vals) / 5
                var = sum((v - mean) ** 2 for v in vals) / 5
                want = [(v - mean) / (var + 1e-3) ** 0.5 * float(gg[j]) + float(bb[j]) for j, v in enumerate(vals)]
            else:
                ms = sum(v * v for v in vals) / 5
                want = [v / (ms + 1e-3) ** 0.5 * float(gg[j]) + float(bb[j]) for j, v in enumerate(vals)]
            assert np.max(np.abs(np.array(want) - out)) < 1e-12


def test_block_matrix_form_with_zero_block():
    """Eq. 6: [Y^R; Y^C] = [[W_RR, 0], [W_CR, W_CC]] [X^R; X^C] for each candidate and its request."""
    x_r, x_c, w_rr, w_cr, w_cc = case(3, n_r=5, n_c=4, d=7, k_r=3, k_c=2)
    got = oracle.lcb_emb(x_r, x_c, w_rr, w_cr, w_cc, m=MAP, want_request=True)
    blk = np.zeros((3 + 2, 5 + 4))
    blk[:3, :5] = w_rr
    blk[3:, :5] = w_cr
    blk[3:, 5:] = w_cc
    for c in range(7):
        y = blk @ np.concatenate([x_r[MAP[c]], x_c[c]]).astype(np.float64)
        assert np.allclose(y[:3], got["y_r"][MAP[c]], rtol=0, atol=1e-12)
        assert np.allclose(y[3:], got["y_c"][c], rtol=0, atol=1e-12)


def test_d1_is_the_linear_glm_layer():
    """With d = 1 the row-axis form is the vector form of Eq. 4 (no bias, no activation), which the
    C oracle's glm evaluates through its own block-matrix code."""
    x_r, x_c, w_rr, w_cr, w_cc = case(4, R=4, C=9, n_r=12, n_c=10, d=1, k_r=6, k_c=8, kind="bf16")
    m = np.array([3, 0, 0, 2, 1, 3, 3, 2, 0], dtype=np.int32)
    got = oracle.lcb_emb(x_r, x_c, w_rr, w_cr, w_cc, m=m, want_request=True)
    lin = oracle.glm(x_r[:, :, 0].copy(), x_c[:, :, 0].copy(),
                     [dict(w_rr=w_rr, w_cr=w_cr, w_cc=w_cc, act="none")], m=m, want_request=True)
    assert np.allclose(got["y_c"][:, :, 0], lin["y_c"], rtol=0, atol=1e-12)
    assert np.allclose(got["y_r"][:, :, 0], lin["y_r"], rtol=0, atol=1e-12)


@pytest.mark.parametrize("norm", ["layer", "rms"])
def test_norm_step_is_torchs(norm):
    x_r, x_c, w_rr, w_cr, w_cc = case(5, n_r=8, n_c=8, d=16, k_r=4, k_c=8, kind="bf16")
    g = synth.draw(5, 6, 16, "f32") + 1.0
    b = synth.draw(5, 7, 16, "f32")
    raw = oracle.lcb_emb(x_r, x_c, w_rr, w_cr, w_cc, m=MAP, want_request=True)
    got = oracle.lcb_emb(x_r, x_c, w_rr, w_cr, w_cc, m=MAP, want_request=True, norm=norm, gamma_c=g,
                         beta_c=b, gamma_r=g, beta_r=None, eps=1e-5)
    gt, bt = torch.from_numpy(g.astype(np.float64)), torch.from_numpy(b.astype(np.float64))

    def ref(y, gam, bet):
        y = torch.from_numpy(y)
        if norm == "layer":
            return torch.nn.functional.layer_norm(y, (16,), gam, bet, eps=1e-5).numpy()
        out = torch.nn.functional.rms_norm(y, (16,), gam, eps=1e-5)
        return (out if bet is None else out + bet).numpy()

    assert np.allclose(got["y_c"], ref(raw["y_c"], gt, bt), rtol=0, atol=1e-12)
    assert np.allclose(got["y_r"], ref(raw["y_r"], gt, None), rtol=0, atol=1e-12)


def test_closed_forms():
    # W_CC = I and W_CR = 0 pass the candidate embeddings through; a W_CR row of ones sums the
    # request's embedding rows
    x_r, x_c, _, _, _ = case(6, n_r=4, n_c=3, d=5)
    w_rr = np.eye(4, dtype=np.float32)[:2]
    w_cr = np.zeros((4, 4), dtype=np.float32)
    w_cr[3] = 1.0
    w_cc = np.zeros((4, 3), dtype=np.float32)
    w_cc[:3, :3] = np.eye(3)
    got = oracle.lcb_emb(x_r, x_c, w_rr, w_cr, w_cc, m=MAP, want_request=True)
    assert np.array_equal(got["y_c"][:, :3], x_c.astype(np.float64))
    assert np.allclose(got["y_c"][:, 3], x_r.astype(np.float64)[MAP].sum(axis=1), rtol=0, atol=1e-12)
    assert np.array_equal(got["y_r"], x_r[:, :2].astype(np.float64))
    # LayerNorm of a row with zero variance is beta; RMSNorm of a zero row is beta
    z = oracle.lcb_emb(x_r, x_c, w_rr, np.zeros_like(w_cr), np.zeros_like(w_cc), m=MAP, norm="layer",
                       beta_c=np.arange(5, dtype=np.float32))
    assert np.array_equal(z["y_c"], np.broadcast_to(np.arange(5.0), z["y_c"].shape))


def test_glm_invariant():
    """Request outputs ignore every candidate; a candidate's outputs change only with its own or its
    request's embeddings (Eq. 6's zero block), with the norm applied per group."""
    x_r, x_c, w_rr, w_cr, w_cc = case(7)
    kw = dict(m=MAP, want_request=True, norm="layer")
    base = oracle.lcb_emb(x_r, x_c, w_rr, w_cr, w_cc, **kw)
    x_c2 = x_c.copy()
    x_c2[4] *= -3.0
    x_r2 = x_r.copy()
    x_r2[2] += 1.0
    after = oracle.lcb_emb(x_r2, x_c2, w_rr, w_cr, w_cc, **kw)
    assert np.array_equal(after["y_r"][[0, 1]], base["y_r"][[0, 1]])
    same = [0, 1, 3, 5]                          # not candidate 4, not request 2's candidates (2, 6)
    assert np.array_equal(after["y_c"][same], base["y_c"][same])
    for c in (2, 4, 6):
        assert not np.array_equal(after["y_c"][c], base["y_c"][c])


def test_index_paths_and_invalid_rows():
    x_r, x_c, w_rr, w_cr, w_cc = case(8, kind="bf16")
    off = np.array([0, 2, 2, 7], dtype=np.int32)             # grouped: 2, 0, 5 candidates
    m = synth.cand_to_req_from_counts(np.array([2, 0, 5]))
    a = oracle.lcb_emb(x_r, x_c, w_rr, w_cr, w_cc, off=off, norm="rms")["y_c"]
    b = oracle.lcb_emb(x_r, x_c, w_rr, w_cr, w_cc, m=m, norm="rms")["y_c"]
    assert np.array_equal(a, b)
    bad = m.copy()
    bad[1] = 3
    bad[5] = -1
    z = oracle.lcb_emb(x_r, x_c, w_rr, w_cr, w_cc, m=bad, norm="layer", beta_c=np.ones(5, np.float32))["y_c"]
    assert np.all(z[[1, 5]] == 0)                            # zeros, not beta: no valid request
    sub = oracle.lcb_emb(x_r, x_c, w_rr, w_cr, w_cc, m=m, cands=[6, 0], norm="rms")["y_c"]
    assert np.array_equal(sub, b[[6, 0]])
