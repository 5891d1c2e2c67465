"""GPU parity of the GLM factorization machine (ROCS Sec. 3.1.4, Eq. 9-10, two groups) through the
C ABI against the fp64 oracle: every MFMA variant (d, feature-block counts), the plain-arithmetic
path, both index forms, invalid and uncovered candidates, the GLM invariant, and the full size."""
import numpy as np
import pytest
import torch

import oracle
import request_candidate_broadcast_amd as ikbo
import synth
from gpu_helpers import assert_parity, bf16_bits, down_f64, note, rne_bits_of, up

pytestmark = pytest.mark.gpu

COUNTS = np.array([3, 40, 0, 1, 77, 12, 5])


def make(seed, n_r, n_c, d, kind="bf16", counts=COUNTS):
    R, C = len(counts), int(np.sum(counts))
    x_r = synth.draw(seed, 80, R * n_r * d, kind).reshape(R, n_r, d)
    x_c = synth.draw(seed, 81, C * n_c * d, kind).reshape(C, n_c, d)
    return x_r, x_c, synth.cand_to_req_from_counts(counts), synth.offsets_from_counts(counts)


def run(x_r, x_c, *, m=None, off=None, out_dtype=torch.float32, want_req=True, sorted_index=False):
    kw = {}
    if m is not None:
        kw["cand_to_req"] = up(m)
    if off is not None:
        kw["req_cand_offsets"] = up(off)
    y_r, y_c = ikbo.ikbo_fm_forward(up(x_r), up(x_c), out_dtype=out_dtype, want_request_output=want_req,
                                    sorted_index=sorted_index, **kw)
    torch.cuda.synchronize()
    return y_r, y_c


# d on the MFMA path; feature counts in one and two 32-row blocks, ragged within a block
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("n_r,n_c", [(32, 32), (4, 28), (64, 48), (60, 64)])
def test_fm_mfma_paths(d, n_r, n_c):
    x_r, x_c, m, off = make(50 + d, n_r, n_c, d)
    note("fm d=%d n_r=%d n_c=%d" % (d, n_r, n_c))
    y_r, y_c = run(x_r, x_c, off=off)
    want = oracle.fm(x_r, x_c, off=off, want_request=True)
    assert_parity(down_f64(y_c), want["y_c"], "bf16", "y_c")
    assert_parity(down_f64(y_r), want["y_r"], "bf16", "y_r")
    # products of bf16 are exact in fp32; only the fp32 sums round
    assert np.max(np.abs(down_f64(y_c) - want["y_c"])) < 1e-3
    _, y16 = run(x_r, x_c, off=off, out_dtype=torch.bfloat16, want_req=False)
    assert np.array_equal(bf16_bits(y16), rne_bits_of(y_c))


def test_fm_index_paths_invalid_and_uncovered():
    x_r, x_c, m, off = make(60, 32, 32, 64)
    note("fm index paths")
    _, a = run(x_r, x_c, off=off)
    _, b = run(x_r, x_c, m=m, sorted_index=True)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    bad = m.copy()
    bad[5] = 99
    bad[50] = -1
    _, z = run(x_r, x_c, m=bad)
    zz = down_f64(z)
    assert np.all(zz[[5, 50]] == 0)
    keep = np.setdiff1d(np.arange(len(m)), [5, 50])
    assert np.array_equal(zz[keep], down_f64(b)[keep])
    part = off.copy()
    part[-1] = off[-1] - 3                       # the last 3 candidates are not covered
    _, p = run(x_r, x_c, off=part)
    assert np.all(down_f64(p)[-3:] == 0)
    assert np.array_equal(down_f64(p)[:-3], down_f64(a)[:-3])


def test_fm_unsorted_map():
    x_r, x_c, m, _ = make(61, 32, 32, 64)
    rng = np.random.default_rng(7)
    mu = rng.integers(0, len(COUNTS), len(m)).astype(np.int32)
    note("fm unsorted map")
    _, y = run(x_r, x_c, m=mu)
    assert_parity(down_f64(y), oracle.fm(x_r, x_c, m=mu)["y_c"], "bf16", "unsorted")


def test_fm_generic_paths():
    # fp32 inputs (any d), and bf16 with a width the MFMA path does not take
    x_r, x_c, m, off = make(62, 8, 12, 20, "f32")
    note("fm fp32")
    y_r, y_c = run(x_r, x_c, off=off)
    want = oracle.fm(x_r, x_c, off=off, want_request=True)
    assert_parity(down_f64(y_c), want["y_c"], "f32", "fp32 y_c")
    assert_parity(down_f64(y_r), want["y_r"], "f32", "fp32 y_r")
    x_r, x_c, m, off = make(63, 68, 8, 48)
    note("fm bf16 generic")
    y_r, y_c = run(x_r, x_c, m=m)
    want = oracle.fm(x_r, x_c, m=m, want_request=True)
    assert_parity(down_f64(y_c), want["y_c"], "bf16", "generic y_c")
    assert_parity(down_f64(y_r), want["y_r"], "bf16", "generic y_r")


def test_fm_glm_invariant_bitwise():
    """Changing one candidate's embeddings changes only that candidate's outputs; changing one
    request's changes only that request's output and its candidates' (Eq. 10)."""
    x_r, x_c, m, off = make(64, 32, 32, 64)
    note("fm GLM invariant")
    y_r, y_c = run(x_r, x_c, off=off)
    x_c2 = x_c.copy()
    x_c2[10] = synth.draw(65, 1, x_c2[10].size, "bf16").reshape(x_c2[10].shape)
    x_r2 = x_r.copy()
    x_r2[5] = synth.draw(65, 2, x_r2[5].size, "bf16").reshape(x_r2[5].shape)
    y_r2, y_c2 = run(x_r2, x_c2, off=off)
    changed_c = {10} | set(range(off[5], off[6]))
    same_c = torch.tensor([c for c in range(len(m)) if c not in changed_c], device=y_c.device)
    assert torch.equal(y_c2[same_c].view(torch.int32), y_c[same_c].view(torch.int32))
    same_r = torch.tensor([r for r in range(len(COUNTS)) if r != 5], device=y_r.device)
    assert torch.equal(y_r2[same_r].view(torch.int32), y_r[same_r].view(torch.int32))


def test_fm_full_size():
    """128 requests x 2048 candidates, 32 request and 32 candidate features of width 64: sampled
    candidates (first and last of four requests plus seeded ones) and all request outputs."""
    counts = np.full(128, 2048)
    R, C, n_r, n_c, d = 128, 128 * 2048, 32, 32, 64
    note("fm full size")
    x_r = synth.draw(66, 80, R * n_r * d, "bf16").reshape(R, n_r, d)
    x_c = synth.draw(66, 81, C * n_c * d, "bf16").reshape(C, n_c, d)
    off = synth.offsets_from_counts(counts)
    y_r, y_c = ikbo.ikbo_fm_forward(up(x_r), up(x_c), req_cand_offsets=up(off), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.isfinite(y_c).all()
    rng = np.random.default_rng(66)
    cands = np.unique(np.concatenate([[0, 2047, 2048, 64 * 2048, C - 1], rng.integers(0, C, 24)]))
    m = synth.cand_to_req_from_counts(counts)
    want = oracle.fm(x_r, x_c, m=m, cands=cands, want_request=True)
    assert_parity(down_f64(y_c[torch.from_numpy(cands).to(y_c.device)]), want["y_c"], "bf16", "full y_c sampled")
    assert_parity(down_f64(y_r), want["y_r"], "bf16", "full y_r")
