"""Pins of the GLM / IKBO-LCB / GLM-MLP oracle (ROCS Sec. 3.1, Eq. 1-6, 8, 11, 14). CPU only."""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "normal_cdf_table.txt")


def _f32(seed, tag, shape, scale=1.0):
    return synth.draw(seed, tag, int(np.prod(shape)), "f32", scale).reshape(shape)


def _layer(seed, k_req, k_cand, n_req, n_cand, act="none", base=10, bias=True):
    return {
        "w_rr": _f32(seed, base + 0, (n_req, k_req), 1 / math.sqrt(max(k_req, 1))),
        "w_cr": _f32(seed, base + 1, (n_cand, k_req), 1 / math.sqrt(max(k_req, 1))),
        "w_cc": _f32(seed, base + 2, (n_cand, k_cand), 1 / math.sqrt(max(k_cand, 1))),
        "b_r": _f32(seed, base + 3, (n_req,), 0.1) if bias else None,
        "b_c": _f32(seed, base + 4, (n_cand,), 0.1) if bias else None,
        "act": act,
    }


def _torch_masked_layer(u, ly, k_req):
    """torch F.linear over the concatenated input with the Eq. 6 block weight [[W_RR,0],[W_CR,W_CC]]."""
    w_rr = torch.from_numpy(ly["w_rr"].astype(np.float64))
    w_cr = torch.from_numpy(ly["w_cr"].astype(np.float64))
    w_cc = torch.from_numpy(ly["w_cc"].astype(np.float64))
    top = torch.cat([w_rr, torch.zeros(w_rr.shape[0], w_cc.shape[1], dtype=torch.float64)], dim=1)
    bot = torch.cat([w_cr, w_cc], dim=1)
    W = torch.cat([top, bot], dim=0)
    b = torch.cat([torch.from_numpy(ly["b_r"].astype(np.float64)) if ly["b_r"] is not None else torch.zeros(w_rr.shape[0], dtype=torch.float64),
                   torch.from_numpy(ly["b_c"].astype(np.float64)) if ly["b_c"] is not None else torch.zeros(w_cc.shape[0], dtype=torch.float64)])
    y = torch.nn.functional.linear(u, W, b)
    if ly["act"] == "gelu":
        y = torch.nn.functional.gelu(y, approximate="none")
    return y


def test_gelu_golden_table_and_identities():
    # P15: GELU(x) = x Phi(x) against textbook Phi values; GELU(0) = 0; GELU(x) - GELU(-x) = x.
    rows = [l.split() for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    for xs, ps in rows:
        x, p = float(xs), float(ps)
        assert abs(oracle.gelu(x) - x * p) <= 1e-15 * max(1.0, abs(x))
    assert oracle.gelu(0.0) == 0.0
    for x in np.linspace(-6, 6, 97):
        assert abs(oracle.gelu(x) - oracle.gelu(-x) - x) <= 1e-14
        assert abs(oracle.gelu(x) - 0.5 * x * (1 + math.erf(x / math.sqrt(2)))) <= 1e-15 * max(1, abs(x))


def test_one_by_one_closed_form():
    # P16: K = N = 1: y_c = phi(w_cc x_c + w_cr x_r + b_c), y_r = phi(w_rr x_r + b_r).
    x_r = np.array([[0.75], [-1.5]], np.float32)
    x_c = np.array([[2.0], [-0.25], [0.5]], np.float32)
    m = np.array([1, 0, 1], np.int32)
    ly = {"w_rr": np.array([[0.5]], np.float32), "w_cr": np.array([[-2.0]], np.float32),
          "w_cc": np.array([[1.25]], np.float32), "b_r": np.array([0.125], np.float32),
          "b_c": np.array([-0.375], np.float32), "act": "gelu"}
    out = oracle.glm(x_r, x_c, [ly], m=m, want_request=True)
    g = lambda z: 0.5 * z * (1 + math.erf(z / math.sqrt(2)))
    for c in range(3):
        want = g(1.25 * float(x_c[c, 0]) - 2.0 * float(x_r[m[c], 0]) - 0.375)
        assert out["y_c"][c, 0] == pytest.approx(want, abs=1e-15)
    for r in range(2):
        assert out["y_r"][r, 0] == pytest.approx(g(0.5 * float(x_r[r, 0]) + 0.125), abs=1e-15)


@pytest.mark.parametrize("act", ["none", "gelu"])
def test_decomposition_eq14_and_library_linear(act):
    # P10: the expanded masked form (Eq. 6) equals the decomposition of Eq. 14, computed here
    # with numpy matmuls: Z = W_CR x_r once per request, y_c = phi(W_CC x_c + Z[m] + b_c).
    counts = np.array([3, 1, 4, 2])
    R, C = len(counts), counts.sum()
    Kr, Kc, Nr, Nc = 24, 16, 8, 12
    x_r = _f32(1, 1, (R, Kr))
    x_c = _f32(1, 2, (C, Kc))
    ly = _layer(1, Kr, Kc, Nr, Nc, act)
    m = synth.cand_to_req_from_counts(counts)
    out = oracle.glm(x_r, x_c, [ly], m=m, want_request=True, want_request_per_cand=True)
    phi = (lambda z: 0.5 * z * (1 + np.vectorize(math.erf)(z / math.sqrt(2)))) if act == "gelu" else (lambda z: z)
    Z = x_r.astype(np.float64) @ ly["w_cr"].astype(np.float64).T
    y_c = phi(x_c.astype(np.float64) @ ly["w_cc"].astype(np.float64).T + Z[m] + ly["b_c"].astype(np.float64))
    y_r = phi(x_r.astype(np.float64) @ ly["w_rr"].astype(np.float64).T + ly["b_r"].astype(np.float64))
    np.testing.assert_allclose(out["y_c"], y_c, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out["y_r"], y_r, rtol=1e-12, atol=1e-12)
    # and torch's F.linear on the expanded input with the explicit block weight
    u = torch.cat([torch.from_numpy(x_r[m].astype(np.float64)), torch.from_numpy(x_c.astype(np.float64))], 1)
    t = _torch_masked_layer(u, ly, Kr).numpy()
    np.testing.assert_allclose(out["y_c"], t[:, Nr:], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out["y_r_c"], t[:, :Nr], rtol=1e-12, atol=1e-12)


def test_glm_invariance_and_closure_single_layer():
    # P11/P12: the request-group output ignores candidate inputs (Eq. 1-2), is identical for all
    # candidates of a request, and equals the request-batched evaluation (Eq. 11).
    counts = np.array([4, 2, 3])
    R, C = 3, 9
    x_r = _f32(2, 1, (R, 16))
    x_c = _f32(2, 2, (C, 8))
    ly = _layer(2, 16, 8, 8, 8, "gelu")
    m = synth.cand_to_req_from_counts(counts)
    a = oracle.glm(x_r, x_c, [ly], m=m, want_request=True, want_request_per_cand=True)
    b = oracle.glm(x_r, (x_c * 3.0 - 1.0).astype(np.float32), [ly], m=m, want_request=True,
                   want_request_per_cand=True)
    assert np.array_equal(a["y_r_c"], b["y_r_c"]) and np.array_equal(a["y_r"], b["y_r"])
    assert np.array_equal(a["y_r_c"], a["y_r"][m])
    assert not np.allclose(a["y_c"], b["y_c"])


def test_zero_blocks():
    # P13: W_CC = 0 makes y_c constant within a request; W_CR = 0 makes y_c ignore m.
    counts = np.array([3, 2])
    x_r = _f32(3, 1, (2, 8))
    x_c = _f32(3, 2, (5, 8))
    m = synth.cand_to_req_from_counts(counts)
    ly = _layer(3, 8, 8, 4, 4, "gelu")
    ly0 = dict(ly, w_cc=np.zeros_like(ly["w_cc"]))
    y = oracle.glm(x_r, x_c, [ly0], m=m)["y_c"]
    assert np.array_equal(y[0], y[1]) and np.array_equal(y[0], y[2]) and np.array_equal(y[3], y[4])
    assert not np.array_equal(y[0], y[3])
    ly1 = dict(ly, w_cr=np.zeros_like(ly["w_cr"]))
    y1 = oracle.glm(x_r, x_c, [ly1], m=m)["y_c"]
    y2 = oracle.glm(x_r, x_c, [ly1], m=np.array([1, 1, 0, 0, 1], np.int32))["y_c"]
    assert np.array_equal(y1, y2)


def test_request_tag():
    # P14: x_r[r] = r e0, W_CR = e0 e0^T, W_CC = 0, b = 0, no activation: y_c[c, 0] = m[c].
    R, C, K, N = 5, 9, 4, 3
    x_r = np.zeros((R, K), np.float32)
    x_r[:, 0] = np.arange(R)
    x_c = _f32(4, 2, (C, K))
    w_cr = np.zeros((N, K), np.float32)
    w_cr[0, 0] = 1.0
    ly = {"w_rr": _f32(4, 3, (N, K)), "w_cr": w_cr, "w_cc": np.zeros((N, K), np.float32),
          "b_r": None, "b_c": None, "act": "none"}
    m = np.array([4, 0, 2, 2, 1, 3, 0, 4, 1], np.int32)
    y = oracle.glm(x_r, x_c, [ly], m=m)["y_c"]
    assert np.array_equal(y[:, 0], m.astype(np.float64))
    assert np.all(y[:, 1:] == 0)


def test_two_layer_mlp_matches_library_and_closure():
    # The query MLP of Eq. 12 as a 2-layer GLM stack: torch F.linear layer by layer on the
    # expanded input, and closure (Eq. 11) of the request path under candidate perturbation.
    counts = np.array([2, 3, 1])
    R, C = 3, 6
    x_r = _f32(5, 1, (R, 32))
    x_c = _f32(5, 2, (C, 16))
    l1 = _layer(5, 32, 16, 24, 20, "gelu", base=20)
    l2 = _layer(5, 24, 20, 12, 8, "none", base=30)
    m = synth.cand_to_req_from_counts(counts)
    out = oracle.glm(x_r, x_c, [l1, l2], m=m, want_request=True, want_request_per_cand=True)
    u = torch.cat([torch.from_numpy(x_r[m].astype(np.float64)), torch.from_numpy(x_c.astype(np.float64))], 1)
    h = _torch_masked_layer(u, l1, 32)
    o = _torch_masked_layer(h, l2, 24).numpy()
    np.testing.assert_allclose(out["y_c"], o[:, 12:], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out["y_r_c"], o[:, :12], rtol=1e-12, atol=1e-12)
    assert np.array_equal(out["y_r_c"], out["y_r"][m])
    pert = oracle.glm(x_r, (x_c + 0.5).astype(np.float32), [l1, l2], m=m, want_request=True,
                      want_request_per_cand=True)
    assert np.array_equal(pert["y_r_c"], out["y_r_c"])
    with pytest.raises(oracle.OracleError):
        oracle.glm(x_r, x_c, [l1, _layer(5, 20, 20, 12, 8)], m=m)   # widths do not chain


def test_bf16_and_offsets_paths():
    g = synth.glm_spec("tiny")
    x_r = synth.glm_x(g, "x_r")
    x_c = synth.glm_x(g, "x_c")
    w = synth.glm_weights(g, 0)
    ly = dict(w, act="none")
    a = oracle.glm(x_r, x_c, [ly], m=g.cand_to_req, want_request=True)
    b = oracle.glm(x_r, x_c, [ly], off=g.offsets, want_request=True)
    assert np.array_equal(a["y_c"], b["y_c"]) and np.array_equal(a["y_r"], b["y_r"])
    # bf16 bits widen exactly
    xb_r, xb_c = synth.f32_to_bf16_bits(x_r), synth.f32_to_bf16_bits(x_c)
    lb = {k: (synth.f32_to_bf16_bits(v) if k.startswith("w_") else v) for k, v in ly.items()}
    lf = {k: (synth.bf16_to_f64(v).astype(np.float32) if k.startswith("w_") else v) for k, v in lb.items()}
    c = oracle.glm(xb_r, xb_c, [lb], m=g.cand_to_req)
    d = oracle.glm(synth.bf16_to_f64(xb_r).astype(np.float32), synth.bf16_to_f64(xb_c).astype(np.float32),
                   [lf], m=g.cand_to_req)
    assert np.array_equal(c["y_c"], d["y_c"])


def test_invalid_index_rows_zero():
    x_r = _f32(6, 1, (2, 8))
    x_c = _f32(6, 2, (4, 8))
    ly = _layer(6, 8, 8, 4, 4, "gelu")
    out = oracle.glm(x_r, x_c, [ly], m=np.array([0, 5, 1, -3], np.int32), return_violations=True)
    assert out["violations"] == 2
    assert np.all(out["y_c"][1] == 0) and np.all(out["y_c"][3] == 0)


def test_index_violation_counter():
    m = np.array([0, 0, 1, 1, 2], np.int32)
    off = np.array([0, 2, 4, 5], np.int32)
    assert oracle.index_violations(m, off, 5, 3, True) == 0
    assert oracle.index_violations(np.array([0, 1, 0, 1, 2], np.int32), None, 5, 3, True) == 1
    assert oracle.index_violations(np.array([0, 0, 1, 3, 2], np.int32), None, 5, 3, False) == 1
    assert oracle.index_violations(None, np.array([0, 3, 2, 5], np.int32), 5, 3, False) == 1
    assert oracle.index_violations(m, np.array([0, 1, 4, 5], np.int32), 5, 3, False) == 1
    # the ends of the offsets count once each
    assert oracle.index_violations(None, np.array([1, 2, 4, 5], np.int32), 5, 3, False) == 1
    assert oracle.index_violations(None, np.array([0, 2, 4, 4], np.int32), 5, 3, False) == 1
    assert oracle.index_violations(None, np.array([1, 2, 4, 6], np.int32), 5, 3, False) == 2
    # an unsorted map is a violation only when the caller declares it sorted
    u = np.array([2, 0, 1, 0, 1], np.int32)
    assert oracle.index_violations(u, None, 5, 3, False) == 0
    assert oracle.index_violations(u, None, 5, 3, True) == 2


def test_map_that_disagrees_with_offsets_takes_the_offsets():
    # Both index forms given and disagreeing: each candidate's request comes from the offsets (the
    # contiguous grouping) and every disagreeing entry is one violation.
    x_r = _f32(7, 1, (3, 8))
    x_c = _f32(7, 2, (5, 8))
    ly = _layer(7, 8, 8, 4, 4, "gelu")
    off = np.array([0, 2, 4, 5], np.int32)
    bad = np.array([0, 2, 1, 1, -1], np.int32)
    ref = oracle.glm(x_r, x_c, [ly], off=off)
    out = oracle.glm(x_r, x_c, [ly], m=bad, off=off, return_violations=True)
    assert out["violations"] == 2
    assert np.array_equal(out["y_c"], ref["y_c"])
    assert oracle.request_of(bad, off, 3, 1) == 0 and oracle.request_of(bad, None, 3, 1) == 2
    assert oracle.index_violations(bad, off, 5, 3, False) == 2
