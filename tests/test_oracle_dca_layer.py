"""Pins of the oracle's DCA interaction layer (ROCS Sec. 3.2, Eq. 12-13, and the concatenation that
feeds the next layer): pure-Python brute force of a whole layer on tiny shapes (query generator,
the four K/V projections, both attention halves, the [Q | A] order), the GLM invariant of a
two-layer stack (Eq. 11: the request path never sees a candidate), and the index handling."""
import math

import numpy as np

import oracle
import synth


def params(seed, R=2, C=5, k_r=6, k_c=4, L=3, seq_dim=5, q_len=2, heads=2, d=2, kind="f32"):
    W = q_len * heads * d
    x_r = synth.draw(seed, 1, R * k_r, kind).reshape(R, k_r)
    x_c = synth.draw(seed, 2, C * k_c, kind).reshape(C, k_c)
    ly = dict(w_rr=synth.draw(seed, 3, W * k_r, kind, 0.5).reshape(W, k_r),
              w_cr=synth.draw(seed, 4, W * k_r, kind, 0.5).reshape(W, k_r),
              w_cc=synth.draw(seed, 5, W * k_c, kind, 0.5).reshape(W, k_c),
              b_r=synth.draw(seed, 6, W, "f32", 0.1), b_c=synth.draw(seed, 7, W, "f32", 0.1), act="none")
    seq = synth.draw(seed, 8, R * L * seq_dim, kind).reshape(R * L, seq_dim)
    ws = [synth.draw(seed, 9 + i, heads * d * seq_dim, kind, 0.5).reshape(heads * d, seq_dim) for i in range(4)]
    return x_r, x_c, [ly], seq, ws


def attend(q, keys, vals, scale):
    """Softmax attention of one query vector over lists of key and value vectors, by loops."""
    s = [scale * sum(a * b for a, b in zip(q, kk)) for kk in keys]
    mx = max(s)
    e = [math.exp(x - mx) for x in s]
    z = sum(e)
    return [sum(e[j] * vals[j][i] for j in range(len(keys))) / z for i in range(len(q))]


def test_layer_brute_force():
    R, C, k_r, k_c, L, sd, Lq, H, d = 2, 5, 6, 4, 3, 5, 2, 2, 2
    W = Lq * H * d
    x_r, x_c, layers, seq, (wkc, wvc, wkr, wvr) = params(1)
    m = np.array([1, 0, 1, 1, 0], dtype=np.int32)
    got = oracle.dca_layer(x_r, x_c, layers, seq, wkc, wvc, wkr, wvr, q_len=Lq, heads=H, m=m)
    ly = {k: (v.astype(np.float64) if isinstance(v, np.ndarray) else v) for k, v in layers[0].items()}
    xr, xc, S = x_r.astype(np.float64), x_c.astype(np.float64), seq.astype(np.float64)

    def proj(w, row):                       # K or V row: sum_k S[row, k] W[n, k]
        w = w.astype(np.float64)
        return [sum(S[row, k] * w[n, k] for k in range(sd)) for n in range(H * d)]

    scale = 1 / math.sqrt(d)
    for r in range(R):
        q = [sum(ly["w_rr"][n, k] * xr[r, k] for k in range(k_r)) + ly["b_r"][n] for n in range(W)]
        kk = [proj(wkr, r * L + j) for j in range(L)]
        vv = [proj(wvr, r * L + j) for j in range(L)]
        a = []
        for t in range(Lq):
            for h in range(H):
                qv = q[(t * H + h) * d:(t * H + h + 1) * d]
                a += attend(qv, [x[h * d:(h + 1) * d] for x in kk], [x[h * d:(h + 1) * d] for x in vv], scale)
        assert np.max(np.abs(np.array(q + a) - got["y_r"][r])) < 1e-12
    for c in range(C):
        r = m[c]
        q = [sum(ly["w_cr"][n, k] * xr[r, k] for k in range(k_r)) + sum(ly["w_cc"][n, k] * xc[c, k] for k in range(k_c))
             + ly["b_c"][n] for n in range(W)]
        kk = [proj(wkc, r * L + j) for j in range(L)]
        vv = [proj(wvc, r * L + j) for j in range(L)]
        a = []
        for t in range(Lq):
            for h in range(H):
                qv = q[(t * H + h) * d:(t * H + h + 1) * d]
                a += attend(qv, [x[h * d:(h + 1) * d] for x in kk], [x[h * d:(h + 1) * d] for x in vv], scale)
        assert np.max(np.abs(np.array(q + a) - got["y_c"][c])) < 1e-12


def stack(x_r, x_c, layer_params, m):
    """Two layers, the second fed the first's [Q | A] (rounded to fp32, as an fp32 run stores it)."""
    y = None
    for i, (layers, seq, ws) in enumerate(layer_params):
        y = oracle.dca_layer(x_r, x_c, layers, seq, *ws, q_len=2, heads=2, m=m)
        x_r, x_c = y["y_r"].astype(np.float32), y["y_c"].astype(np.float32)
    return y


def test_two_layer_stack_keeps_the_glm_invariant():
    """Eq. 11 over depth: the request outputs after two layers do not depend on any candidate, and a
    candidate's outputs depend only on its own inputs and its request's."""
    x_r, x_c, l1, s1, w1 = params(2)
    W = 8
    _, _, l2, s2, w2 = params(3, k_r=2 * W, k_c=2 * W)
    m = np.array([1, 0, 1, 1, 0], dtype=np.int32)
    base = stack(x_r, x_c, [(l1, s1, w1), (l2, s2, w2)], m)
    x_c2 = x_c.copy()
    x_c2[3] += 1.0                                     # a candidate of request 1
    after = stack(x_r, x_c2, [(l1, s1, w1), (l2, s2, w2)], m)
    assert np.array_equal(after["y_r"], base["y_r"])
    assert np.array_equal(after["y_c"][[0, 1, 2, 4]], base["y_c"][[0, 1, 2, 4]])
    assert not np.array_equal(after["y_c"][3], base["y_c"][3])
    x_r2 = x_r.copy()
    x_r2[0] *= -1.0                                    # request 0: its candidates 1 and 4 change
    after = stack(x_r2, x_c, [(l1, s1, w1), (l2, s2, w2)], m)
    assert np.array_equal(after["y_r"][1], base["y_r"][1])
    assert np.array_equal(after["y_c"][[0, 2, 3]], base["y_c"][[0, 2, 3]])
    assert not np.array_equal(after["y_c"][[1, 4]], base["y_c"][[1, 4]])


def test_layer_index_paths_subsets_and_varlen():
    x_r, x_c, layers, seq, ws = params(4, kind="bf16")
    off = np.array([0, 2, 5], dtype=np.int32)
    m = synth.cand_to_req_from_counts(np.array([2, 3]))
    a = oracle.dca_layer(x_r, x_c, layers, seq, *ws, q_len=2, heads=2, off=off)
    b = oracle.dca_layer(x_r, x_c, layers, seq, *ws, q_len=2, heads=2, m=m)
    assert np.array_equal(a["y_c"], b["y_c"]) and np.array_equal(a["y_r"], b["y_r"])
    sub = oracle.dca_layer(x_r, x_c, layers, seq, *ws, q_len=2, heads=2, m=m, cands=[4, 1])
    assert np.array_equal(sub["y_c"], b["y_c"][[4, 1]])
    bad = m.copy()
    bad[2] = 7
    z = oracle.dca_layer(x_r, x_c, layers, seq, *ws, q_len=2, heads=2, m=bad)["y_c"]
    assert np.all(z[2] == 0)
    # the same rows as two variable-length sequences of 3 give the uniform result
    v = oracle.dca_layer(x_r, x_c, layers, seq, *ws, q_len=2, heads=2, m=m, kv_cu=np.array([0, 3, 6], np.int32))
    assert np.allclose(v["y_c"], b["y_c"], rtol=0, atol=1e-12) and np.allclose(v["y_r"], b["y_r"], rtol=0, atol=1e-12)
