"""Pins of the oracle's request-side K/V projection (ROCS Sec. 4.1, the DCA decomposition after
Eq. 14) and request-side attention A^R (Sec. 3.2, Eq. 13): brute force on tiny inputs, exact
closed forms, and the commutation of the projection with the request-to-candidate broadcast
that the pages state."""
import numpy as np

import oracle
import synth


def bf16(a):
    """float values that are exactly bf16 -> bit patterns"""
    f = np.asarray(a, dtype=np.float32)
    bits = f.view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0)
    return (bits >> 16).astype(np.uint16)


def test_decode_bf16_bit_patterns():
    assert list(oracle.decode(np.array([0x3F80, 0xC000, 0x0000, 0x3E80, 0x7F80], dtype=np.uint16))) == \
        [1.0, -2.0, 0.0, 0.25, np.inf]


def test_linear_brute_force_tiny():
    rng = np.random.default_rng(3)
    x = bf16(np.round(rng.normal(size=(3, 8)) * 8) / 8)
    w = bf16(np.round(rng.normal(size=(5, 8)) * 8) / 8)
    y = oracle.linear(x, w)
    xd, wd = oracle.decode(x), oracle.decode(w)
    for i in range(3):
        for n in range(5):
            s = 0.0
            for k in range(8):
                s += xd[i, k] * wd[n, k]
            assert y[i, n] == s        # products and sums of eighths are exact in fp64


def test_linear_identity_and_rows():
    x = synth.draw(7, 1, 6 * 16, "bf16").reshape(6, 16)
    eye = bf16(np.eye(16))
    assert np.array_equal(oracle.linear(x, eye), oracle.decode(x))
    # a permutation weight reorders the columns; selected rows come back in the order asked
    perm = np.eye(16)[::-1]
    assert np.array_equal(oracle.linear(x, bf16(perm), rows=[4, 1]), oracle.decode(x)[[4, 1], ::-1])


def test_projection_commutes_with_the_broadcast():
    """(S_m) W = (S W)_m: projecting the gathered rows equals gathering the projected rows."""
    R, L, d_in, d_out = 4, 3, 32, 24
    s = synth.draw(8, 2, R * L * d_in, "bf16").reshape(R * L, d_in)
    w = synth.draw(8, 3, d_out * d_in, "bf16").reshape(d_out, d_in)
    m = np.array([2, 0, 0, 3, 1, 2], dtype=np.int64)           # candidate -> request
    rows = (m[:, None] * L + np.arange(L)[None, :]).reshape(-1)
    gathered_then_projected = oracle.linear(s, w, rows=rows)
    projected_then_gathered = oracle.linear(s, w)[rows]
    assert np.array_equal(gathered_then_projected, projected_then_gathered)


def test_linear_is_linear_in_w():
    x = synth.draw(9, 4, 5 * 12, "f32").reshape(5, 12)
    w1 = synth.draw(9, 5, 7 * 12, "f32").reshape(7, 12)
    w2 = synth.draw(9, 6, 7 * 12, "f32").reshape(7, 12)
    lhs = oracle.linear(x, (w1.astype(np.float64) + w2.astype(np.float64)).astype(np.float32))
    rhs = oracle.linear(x, w1) + oracle.linear(x, w2)
    assert np.max(np.abs(lhs - rhs)) < 1e-5     # the fp32 rounding of w1 + w2 only


def test_request_attention_is_dca_with_the_identity_map():
    R, L, H, d, Lq = 3, 5, 2, 8, 2
    q = synth.draw(10, 1, R * Lq * H * d, "f32").reshape(R, Lq, H, d)
    k = synth.draw(10, 2, R * L * H * d, "f32").reshape(R, L, H, d)
    v = synth.draw(10, 3, R * L * H * d, "f32").reshape(R, L, H, d)
    got = oracle.request_attention(q, k, v)
    # brute force: softmax over request r's keys only
    qd, kd, vd = (a.astype(np.float64) for a in (q, k, v))
    for r in range(R):
        for t in range(Lq):
            for h in range(H):
                s = kd[r, :, h, :] @ qd[r, t, h, :] / np.sqrt(d)
                p = np.exp(s - s.max())
                want = (p / p.sum()) @ vd[r, :, h, :]
                assert np.max(np.abs(got[r, t, h] - want)) < 1e-12
