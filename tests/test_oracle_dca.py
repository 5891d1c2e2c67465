"""Pins of the DCA oracle (candidate cross attention, ROCS Sec. 3.2 Eq. 13 A^C; Sec. 4.3.1).

Each pin ties the oracle to something other than itself: a library attention routine, closed
forms, invariances of softmax attention, and index bookkeeping. CPU only."""
import numpy as np
import pytest
import torch

import oracle
import synth


def _f32(seed, tag, shape, scale=1.0):
    return synth.draw(seed, tag, int(np.prod(shape)), "f32", scale).reshape(shape)


def _dyadic(seed, tag, shape, lo=-8, hi=8, denom=8.0):
    """fp32 values on a dyadic grid, so shifts and affine maps stay exact."""
    u = synth.draw(seed, tag, int(np.prod(shape)), "unif")
    return (np.floor(lo + u * (hi - lo + 1)) / denom).astype(np.float32).reshape(shape)


def _torch_attention_per_request(q, k, v, counts, kv_lens, scale, varlen):
    """torch's own scaled_dot_product_attention in fp64, one call per request."""
    C, Lq, H, d = q.shape
    out = np.zeros((C, Lq, H, d))
    c0, k0 = 0, 0
    for r, n in enumerate(counts):
        L = kv_lens[r]
        kr = k[k0:k0 + L] if varlen else k[r]
        vr = v[k0:k0 + L] if varlen else v[r]
        qs = torch.from_numpy(q[c0:c0 + n].astype(np.float64)).reshape(n * Lq, H, d).permute(1, 0, 2)
        ks = torch.from_numpy(kr.astype(np.float64)).permute(1, 0, 2)
        vs = torch.from_numpy(vr.astype(np.float64)).permute(1, 0, 2)
        if n > 0 and L > 0:
            o = torch.nn.functional.scaled_dot_product_attention(qs, ks, vs, scale=scale)
            out[c0:c0 + n] = o.permute(1, 0, 2).reshape(n, Lq, H, d).numpy()
        c0 += n
        k0 += L if varlen else 0
    return out


@pytest.mark.parametrize("Lq,H,d", [(1, 2, 64), (4, 3, 16), (2, 1, 8)])
def test_matches_library_attention_uniform(Lq, H, d):
    counts = np.array([3, 1, 5, 2])
    R, L = len(counts), 13
    C = counts.sum()
    q = _f32(1, 1, (C, Lq, H, d))
    k = _f32(1, 2, (R, L, H, d))
    v = _f32(1, 3, (R, L, H, d))
    m = synth.cand_to_req_from_counts(counts)
    got = oracle.dca(q, k, v, R, m=m)
    want = _torch_attention_per_request(q, k, v, counts, [L] * R, 1.0 / np.sqrt(d), False)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_matches_library_attention_varlen_tiny_workload():
    s = synth.dca_spec("tiny")
    q, k, v = synth.dca_q(s), synth.dca_kv(s, "k"), synth.dca_kv(s, "v")
    k4 = k.reshape(s.R, s.L, s.H, s.d)
    v4 = v.reshape(s.R, s.L, s.H, s.d)
    got = oracle.dca(q, k4, v4, s.R, off=s.offsets)
    want = _torch_attention_per_request(q, k4, v4, s.counts, s.kv_lens, s.scale, False)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    # the same K/V presented as a variable-length store gives the same result
    cu = synth.offsets_from_counts(np.full(s.R, s.L))
    got2 = oracle.dca(q, k, v, s.R, off=s.offsets, kv_cu=cu)
    assert np.array_equal(got, got2)


def test_matches_library_attention_ragged_lengths():
    counts = np.array([2, 0, 4, 1, 3])
    lens = np.array([5, 9, 1, 17, 3])
    R, H, d, Lq = 5, 2, 16, 2
    C = counts.sum()
    q = _f32(2, 1, (C, Lq, H, d))
    k = _f32(2, 2, (lens.sum(), H, d))
    v = _f32(2, 3, (lens.sum(), H, d))
    cu = synth.offsets_from_counts(lens)
    got = oracle.dca(q, k, v, R, m=synth.cand_to_req_from_counts(counts), kv_cu=cu, scale=0.3)
    want = _torch_attention_per_request(q, k, v, counts, lens, 0.3, True)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_bf16_inputs_widen_exactly():
    counts = np.array([2, 3])
    R, L, H, d = 2, 7, 2, 8
    C = counts.sum()
    qb = synth.draw(3, 1, C * H * d, "bf16").reshape(C, 1, H, d)
    kb = synth.draw(3, 2, R * L * H * d, "bf16").reshape(R, L, H, d)
    vb = synth.draw(3, 3, R * L * H * d, "bf16").reshape(R, L, H, d)
    m = synth.cand_to_req_from_counts(counts)
    got = oracle.dca(qb, kb, vb, R, m=m)
    q64, k64, v64 = (synth.bf16_to_f64(x) for x in (qb, kb, vb))
    want = _torch_attention_per_request(q64, k64, v64, counts, [L] * R, 1 / np.sqrt(d), False)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_single_key_returns_v():
    # P2: with L_r = 1 the softmax weight is exactly 1, so O = V[r, 0].
    counts = np.array([3, 2, 4])
    R, H, d = 3, 2, 16
    C = counts.sum()
    q = _f32(4, 1, (C, 2, H, d), 5.0)
    k = _f32(4, 2, (R, 1, H, d))
    v = _f32(4, 3, (R, 1, H, d))
    m = synth.cand_to_req_from_counts(counts)
    got = oracle.dca(q, k, v, R, m=m)
    for c in range(C):
        for t in range(2):
            assert np.array_equal(got[c, t], v[m[c], 0].astype(np.float64))


def test_zero_query_gives_mean_of_values():
    # P7: Q = 0 gives uniform weights, O = mean_j V_j.
    counts = np.array([2, 3])
    R, L, H, d = 2, 11, 2, 8
    q = np.zeros((5, 1, H, d), np.float32)
    k = _f32(5, 2, (R, L, H, d))
    v = _f32(5, 3, (R, L, H, d))
    m = synth.cand_to_req_from_counts(counts)
    got = oracle.dca(q, k, v, R, m=m)
    for c in range(5):
        np.testing.assert_allclose(got[c, 0], v[m[c]].astype(np.float64).mean(axis=0), rtol=0, atol=1e-14)


def test_key_shift_invariance():
    # P5: adding the same vector u to every key of a head adds <q, u> to every score of that
    # query, which the softmax cancels. Dyadic values keep K + u exact in fp32.
    counts = np.array([2, 2, 3])
    R, L, H, d = 3, 9, 2, 8
    q = _dyadic(6, 1, (7, 1, H, d))
    k = _dyadic(6, 2, (R, L, H, d))
    v = _f32(6, 3, (R, L, H, d))
    u = _dyadic(6, 4, (1, 1, H, d))
    m = synth.cand_to_req_from_counts(counts)
    a = oracle.dca(q, k, v, R, m=m)
    b = oracle.dca(q, (k + u).astype(np.float32), v, R, m=m)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_value_affine_equivariance():
    # P6: V' = a V + b gives O' = a O + b (the weights sum to one).
    counts = np.array([4, 1])
    R, L, H, d = 2, 6, 1, 8
    q = _f32(7, 1, (5, 3, H, d))
    k = _f32(7, 2, (R, L, H, d))
    v = _dyadic(7, 3, (R, L, H, d))
    m = synth.cand_to_req_from_counts(counts)
    a = oracle.dca(q, k, v, R, m=m)
    b = oracle.dca(q, k, (2.0 * v + 0.5).astype(np.float32), R, m=m)
    np.testing.assert_allclose(b, 2.0 * a + 0.5, rtol=0, atol=1e-12)


def test_request_tag_and_index_resolution():
    # P8: V[r] == r everywhere makes every output equal to its candidate's request.
    counts = np.array([1, 3, 2, 2])
    R, L, H, d = 4, 5, 2, 4
    C = counts.sum()
    q = _f32(8, 1, (C, 1, H, d))
    k = _f32(8, 2, (R, L, H, d))
    v = np.broadcast_to(np.arange(R, dtype=np.float32)[:, None, None, None], (R, L, H, d)).copy()
    m = synth.cand_to_req_from_counts(counts)
    got = oracle.dca(q, k, v, R, m=m)
    np.testing.assert_allclose(got, np.broadcast_to(m[:, None, None, None], got.shape), atol=1e-13)


def test_permutation_equivariance_and_unsorted_map():
    # P4: permuting candidates together with m permutes the outputs, bit for bit.
    counts = np.array([3, 2, 4])
    R, L, H, d = 3, 7, 2, 8
    C = counts.sum()
    q = _f32(9, 1, (C, 2, H, d))
    k = _f32(9, 2, (R, L, H, d))
    v = _f32(9, 3, (R, L, H, d))
    m = synth.cand_to_req_from_counts(counts)
    perm = np.array([5, 0, 8, 2, 7, 1, 6, 3, 4])
    a = oracle.dca(q, k, v, R, m=m)
    b = oracle.dca(q[perm], k, v, R, m=m[perm])
    assert np.array_equal(a[perm], b)


def test_offsets_and_map_agree():
    # P18: offsets only, map only, and both together give identical outputs.
    s = synth.dca_spec("tiny")
    q, k, v = synth.dca_q(s), synth.dca_kv(s, "k"), synth.dca_kv(s, "v")
    k4, v4 = k.reshape(s.R, s.L, s.H, s.d), v.reshape(s.R, s.L, s.H, s.d)
    a = oracle.dca(q, k4, v4, s.R, m=s.cand_to_req)
    b = oracle.dca(q, k4, v4, s.R, off=s.offsets)
    c = oracle.dca(q, k4, v4, s.R, m=s.cand_to_req, off=s.offsets)
    assert np.array_equal(a, b) and np.array_equal(a, c)
    # A map that disagrees with the offsets: the offsets decide every row (the contiguous grouping
    # the kernels execute on) and the disagreeing entry is counted as one violation.
    bad = s.cand_to_req.copy()
    bad[3] = (bad[3] + 1) % s.R
    got, nv = oracle.dca(q, k4, v4, s.R, m=bad, off=s.offsets, return_violations=True)
    assert nv == 1 and np.array_equal(got, b)
    assert oracle.index_violations(bad, s.offsets, len(bad), s.R) == 1
    # ... and an out-of-range entry inside a valid offset range likewise
    bad[5] = -7
    got, nv = oracle.dca(q, k4, v4, s.R, m=bad, off=s.offsets, return_violations=True)
    assert nv == 2 and np.array_equal(got, b)
    # the map alone for the same entries: row 3 attends another request, row 5 is zero
    alone, nv = oracle.dca(q, k4, v4, s.R, m=bad, return_violations=True)
    assert nv == 1 and np.all(alone[5] == 0) and not np.array_equal(alone[3], b[3])


def test_invalid_request_rows_are_zero_and_counted():
    counts = np.array([2, 2])
    R, L, H, d = 2, 3, 1, 4
    q = _f32(10, 1, (4, 1, H, d))
    k = _f32(10, 2, (R, L, H, d))
    v = _f32(10, 3, (R, L, H, d))
    m = np.array([0, -1, 1, 2], np.int32)
    got, nv = oracle.dca(q, k, v, R, m=m, return_violations=True)
    assert nv == 2
    assert np.all(got[1] == 0) and np.all(got[3] == 0)
    assert np.any(got[0] != 0) and np.any(got[2] != 0)


def test_empty_sequence_and_empty_request():
    # A request with L_r = 0 gives zero rows; a request with no candidates is harmless.
    counts = np.array([2, 0, 1])
    lens = np.array([0, 4, 3])
    H, d = 1, 4
    q = _f32(11, 1, (3, 1, H, d))
    k = _f32(11, 2, (lens.sum(), H, d))
    v = _f32(11, 3, (lens.sum(), H, d))
    got = oracle.dca(q, k, v, 3, m=synth.cand_to_req_from_counts(counts),
                     kv_cu=synth.offsets_from_counts(lens))
    assert np.all(got[:2] == 0) and np.any(got[2] != 0)
    empty = oracle.dca(np.zeros((0, 1, H, d), np.float32), k, v, 3, m=np.zeros(0, np.int32),
                       kv_cu=synth.offsets_from_counts(lens))
    assert empty.shape == (0, 1, H, d)


def test_candidate_subset_matches_full():
    s = synth.dca_spec("tiny")
    q, k, v = synth.dca_q(s), synth.dca_kv(s, "k"), synth.dca_kv(s, "v")
    k4, v4 = k.reshape(s.R, s.L, s.H, s.d), v.reshape(s.R, s.L, s.H, s.d)
    full = oracle.dca(q, k4, v4, s.R, off=s.offsets)
    sub = [0, 7, s.C - 1, 3]
    assert np.array_equal(oracle.dca(q, k4, v4, s.R, off=s.offsets, cands=sub), full[sub])


def test_large_scores_stay_finite():
    # The max subtraction keeps exp() in range for scores far beyond exp's overflow point.
    counts = np.array([1])
    k = np.zeros((1, 3, 1, 4), np.float32)
    k[0, :, 0, 0] = [1000.0, 999.0, -5.0]
    q = np.zeros((1, 1, 1, 4), np.float32)
    q[0, 0, 0, 0] = 2.0
    v = np.zeros((1, 3, 1, 4), np.float32)
    v[0, :, 0, 1] = [1.0, 2.0, 3.0]
    got = oracle.dca(q, k, v, 1, m=np.zeros(1, np.int32), scale=1.0)
    w = np.exp(np.array([0.0, -2.0, -2010.0]))
    w /= w.sum()
    np.testing.assert_allclose(got[0, 0, 0, 1], (w * [1, 2, 3]).sum(), rtol=1e-14)
    assert np.all(np.isfinite(got))
