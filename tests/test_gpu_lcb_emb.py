"""GPU parity of the LCB embedding form with the group-local norm (ROCS Sec. 3.1.2 Eq. 5-6, Sec. 3.1.3
Eq. 7, two groups) through the C ABI against the fp64 oracle: every MFMA variant (d, padded
input rows, output blocks) with each norm, the plain-arithmetic paths, both index forms, invalid
and uncovered candidates, the GLM invariant and the full size."""
import math

import numpy as np
import pytest
import torch

import oracle
import request_candidate_broadcast_amd as ikbo
import synth
from gpu_helpers import assert_parity, bf16_bits, down_f64, note, rne_bits_of, up

pytestmark = pytest.mark.gpu

COUNTS = np.array([3, 40, 0, 1, 77, 12, 5])


def make(seed, n_r, n_c, d, k_r, k_c, kind="bf16", counts=COUNTS):
    R, C = len(counts), int(np.sum(counts))
    x_r = synth.draw(seed, 90, R * n_r * d, kind).reshape(R, n_r, d)
    x_c = synth.draw(seed, 91, C * n_c * d, kind).reshape(C, n_c, d)
    w_rr = synth.draw(seed, 92, k_r * n_r, kind, 1 / math.sqrt(n_r)).reshape(k_r, n_r)
    w_cr = synth.draw(seed, 93, k_c * n_r, kind, 1 / math.sqrt(n_r)).reshape(k_c, n_r)
    w_cc = synth.draw(seed, 94, k_c * n_c, kind, 1 / math.sqrt(n_c)).reshape(k_c, n_c)
    g_r = (1.0 + 0.25 * synth.draw(seed, 95, d, "f32")).astype(np.float32)
    b_r = (0.25 * synth.draw(seed, 96, d, "f32")).astype(np.float32)
    g_c = (1.0 + 0.25 * synth.draw(seed, 97, d, "f32")).astype(np.float32)
    b_c = (0.25 * synth.draw(seed, 98, d, "f32")).astype(np.float32)
    return dict(x_r=x_r, x_c=x_c, w_rr=w_rr, w_cr=w_cr, w_cc=w_cc, gamma_r=g_r, beta_r=b_r, gamma_c=g_c,
                beta_c=b_c, m=synth.cand_to_req_from_counts(counts), off=synth.offsets_from_counts(counts))


def run(p, *, norm="layer", use_off=True, m=None, off=None, out_dtype=torch.float32, want_req=True,
        sorted_index=False, affine=True, x_r=None, x_c=None):
    kw = {}
    if m is not None:
        kw["cand_to_req"] = up(m)
    if off is not None:
        kw["req_cand_offsets"] = up(off)
    if not kw:
        kw["req_cand_offsets" if use_off else "cand_to_req"] = up(p["off"] if use_off else p["m"])
    if affine:
        kw.update(gamma_req=up(p["gamma_r"]), beta_req=up(p["beta_r"]), gamma_cand=up(p["gamma_c"]),
                  beta_cand=up(p["beta_c"]))
    y_r, y_c = ikbo.ikbo_lcb_emb_forward(up(p["x_r"] if x_r is None else x_r), up(p["x_c"] if x_c is None else x_c),
                                         up(p["w_rr"]), up(p["w_cr"]), up(p["w_cc"]), norm=norm, out_dtype=out_dtype,
                                         want_request_output=want_req, sorted_index=sorted_index, **kw)
    torch.cuda.synchronize()
    return y_r, y_c


def want(p, *, norm="layer", m=None, off=None, cands=None, affine=True, x_r=None, x_c=None):
    if m is None and off is None:
        off = p["off"]
    aff = dict(gamma_r=p["gamma_r"], beta_r=p["beta_r"], gamma_c=p["gamma_c"], beta_c=p["beta_c"]) if affine else {}
    return oracle.lcb_emb(p["x_r"] if x_r is None else x_r, p["x_c"] if x_c is None else x_c, p["w_rr"], p["w_cr"],
                          p["w_cc"], m=m, off=off, norm=norm, cands=cands, want_request=True, **aff)


# d on the MFMA path; input rows in one 32-row tile, ragged (padded to 16 / 32), and two; output
# rows in one 32-row block, ragged, and two
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("n_c,k_c", [(32, 32), (20, 28), (48, 64), (64, 40), (8, 4)])
def test_lcb_emb_mfma_paths(d, n_c, k_c):
    p = make(100 + d + n_c, 24, n_c, d, 12, k_c)
    for norm in ("none", "layer", "rms"):
        note("lcb_emb d=%d n_c=%d k_c=%d norm=%s" % (d, n_c, k_c, norm))
        y_r, y_c = run(p, norm=norm)
        w = want(p, norm=norm)
        assert_parity(down_f64(y_c), w["y_c"], "bf16", "y_c " + norm)
        assert_parity(down_f64(y_r), w["y_r"], "bf16", "y_r " + norm)
        if norm == "none":
            # products of bf16 are exact in fp32; only the fp32 sums round
            assert np.max(np.abs(down_f64(y_c) - w["y_c"])) < 1e-3
        y16_r, y16_c = run(p, norm=norm, out_dtype=torch.bfloat16)
        assert np.array_equal(bf16_bits(y16_c), rne_bits_of(y_c))
        assert np.array_equal(bf16_bits(y16_r), rne_bits_of(y_r))


def test_lcb_emb_without_affine_parameters():
    p = make(120, 32, 32, 64, 32, 32)
    note("lcb_emb no gamma/beta")
    y_r, y_c = run(p, norm="rms", affine=False)
    w = want(p, norm="rms", affine=False)
    assert_parity(down_f64(y_c), w["y_c"], "bf16", "y_c rms plain")
    assert_parity(down_f64(y_r), w["y_r"], "bf16", "y_r rms plain")


def test_lcb_emb_generic_paths():
    # fp32 inputs (any d), and bf16 with widths the MFMA path does not take
    p = make(121, 6, 12, 20, 5, 8, "f32")
    for norm in ("none", "layer", "rms"):
        note("lcb_emb fp32 norm=%s" % norm)
        y_r, y_c = run(p, norm=norm)
        w = want(p, norm=norm)
        assert_parity(down_f64(y_c), w["y_c"], "f32", "fp32 y_c " + norm)
        assert_parity(down_f64(y_r), w["y_r"], "f32", "fp32 y_r " + norm)
    for n_c, d, k_c in ((12, 48, 8), (80, 64, 16), (16, 64, 72), (8, 200, 3)):
        p = make(122 + n_c, 10, n_c, d, 4, k_c)
        note("lcb_emb bf16 generic n_c=%d d=%d k_c=%d" % (n_c, d, k_c))
        y_r, y_c = run(p, norm="layer", use_off=False)
        w = want(p, norm="layer", m=p["m"])
        assert_parity(down_f64(y_c), w["y_c"], "bf16", "generic y_c")
        assert_parity(down_f64(y_r), w["y_r"], "bf16", "generic y_r")


def test_lcb_emb_index_paths_invalid_and_uncovered():
    p = make(123, 32, 32, 64, 16, 32)
    note("lcb_emb index paths")
    _, a = run(p)
    _, b = run(p, m=p["m"], sorted_index=True)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    bad = p["m"].copy()
    bad[5] = 99
    bad[50] = -1
    _, z = run(p, m=bad)
    zz = down_f64(z)
    assert np.all(zz[[5, 50]] == 0)
    keep = np.setdiff1d(np.arange(len(bad)), [5, 50])
    assert np.array_equal(zz[keep], down_f64(b)[keep])
    part = p["off"].copy()
    part[-1] = p["off"][-1] - 3                  # the last 3 candidates are not covered
    _, q = run(p, off=part)
    assert np.all(down_f64(q)[-3:] == 0)
    assert np.array_equal(down_f64(q)[:-3], down_f64(a)[:-3])
    rng = np.random.default_rng(9)
    mu = rng.integers(0, len(COUNTS), len(bad)).astype(np.int32)
    note("lcb_emb unsorted map")
    _, u = run(p, m=mu)
    assert_parity(down_f64(u), want(p, m=mu)["y_c"], "bf16", "unsorted")


def test_lcb_emb_no_requests():
    """num_req = 0: every candidate lacks a valid request, so every output row is zero."""
    p = make(124, 32, 32, 64, 16, 32, counts=np.array([0]))
    C = 9
    x_c = synth.draw(124, 1, C * 32 * 64, "bf16").reshape(C, 32, 64)
    note("lcb_emb no requests")
    y_r, y_c = ikbo.ikbo_lcb_emb_forward(up(np.zeros((0, 32, 64), np.uint16)), up(x_c), up(p["w_rr"]),
                                         up(p["w_cr"]), up(p["w_cc"]), cand_to_req=up(np.zeros(C, np.int32)),
                                         norm="layer", out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert y_r.shape == (0, 16, 64) and torch.count_nonzero(y_c).item() == 0


def test_lcb_emb_glm_invariant_bitwise():
    """Changing one candidate's embeddings changes only that candidate's outputs; changing one
    request's changes only that request's output and its candidates' (Eq. 6's zero block)."""
    p = make(125, 32, 32, 64, 16, 32)
    note("lcb_emb GLM invariant")
    y_r, y_c = run(p)
    x_c2 = p["x_c"].copy()
    x_c2[10] = synth.draw(126, 1, x_c2[10].size, "bf16").reshape(x_c2[10].shape)
    x_r2 = p["x_r"].copy()
    x_r2[5] = synth.draw(126, 2, x_r2[5].size, "bf16").reshape(x_r2[5].shape)
    y_r2, y_c2 = run(p, x_r=x_r2, x_c=x_c2)
    off = p["off"]
    changed = {10} | set(range(off[5], off[6]))
    same_c = torch.tensor([c for c in range(len(p["m"])) if c not in changed], device=y_c.device)
    assert torch.equal(y_c2[same_c].view(torch.int32), y_c[same_c].view(torch.int32))
    same_r = torch.tensor([r for r in range(len(COUNTS)) if r != 5], device=y_r.device)
    assert torch.equal(y_r2[same_r].view(torch.int32), y_r[same_r].view(torch.int32))


def test_lcb_emb_full_size():
    """128 requests x 2048 candidates, 32 request and 32 candidate embeddings of width 64, 32 output
    rows per group, LayerNorm: sampled candidates (first and last of some requests plus seeded ones)
    and every request output against the oracle."""
    counts = np.full(128, 2048)
    R, C, n, d, k = 128, 128 * 2048, 32, 64, 32
    note("lcb_emb full size")
    x_r = synth.draw(127, 90, R * n * d, "bf16").reshape(R, n, d)
    x_c = synth.draw(127, 91, C * n * d, "bf16").reshape(C, n, d)
    p = make(127, n, n, d, k, k, counts=np.array([1]))
    p.update(x_r=x_r, x_c=x_c, m=synth.cand_to_req_from_counts(counts), off=synth.offsets_from_counts(counts))
    y_r, y_c = run(p, norm="layer")
    assert torch.isfinite(y_c).all()
    rng = np.random.default_rng(127)
    cands = np.unique(np.concatenate([[0, 2047, 2048, 64 * 2048, C - 1], rng.integers(0, C, 24)]))
    w = want(p, norm="layer", m=p["m"], cands=cands)
    assert_parity(down_f64(y_c[torch.from_numpy(cands).to(y_c.device)]), w["y_c"], "bf16", "full y_c sampled")
    assert_parity(down_f64(y_r), w["y_r"], "bf16", "full y_r")
