"""The persistent IKBO-LCB launch (request and candidate tiles co-scheduled in one kernel, the
candidate epilogue waiting on per-request-tile ready flags, ROCS Sec. 4.2.3) against the
two-launch form and the fp64 oracle.

The two forms run the same tile code with the same reduction order, so their outputs must agree
bit for bit; the oracle bounds both. IKBO_LCB_FUSED=1 selects the persistent launch."""
import os

import numpy as np
import pytest
import torch

import oracle
import request_candidate_broadcast_amd as ikbo
import synth
from gpu_helpers import assert_parity, bf16_bits, down_f64, note
from test_gpu_lcb import make_layer, make_x, run_lcb

pytestmark = pytest.mark.gpu

COUNTS = np.array([1, 300, 0, 77, 513, 2, 40, 260, 5])


def both_forms(fn):
    """(persistent launch result, two-launch result)"""
    ref = fn()
    os.environ["IKBO_LCB_FUSED"] = "1"
    try:
        return fn(), ref
    finally:
        os.environ.pop("IKBO_LCB_FUSED", None)


def same_bits(a, b):
    if a is None or b is None:
        return a is None and b is None
    if a.dtype == torch.bfloat16:
        return np.array_equal(bf16_bits(a), bf16_bits(b))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


# (k_req, k_cand, n_req, n_cand): request output columns a multiple of the 256-wide tile and not,
# ragged candidate output width, several request row blocks (R > 256 in the second group)
@pytest.mark.parametrize("shape", [(256, 128, 256, 512), (192, 256, 0, 200), (128, 64, 512, 1000), (64, 192, 200, 256)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_fused_equals_two_launch_and_oracle(shape, out):
    k_req, k_cand, n_req, n_cand = shape
    R, C = len(COUNTS), int(COUNTS.sum())
    x_r, x_c = make_x(21, R, C, k_req, k_cand, "bf16")
    ly = make_layer(21, k_req, k_cand, max(n_req, 8), n_cand, "bf16", "gelu")
    if n_req == 0:
        ly["w_rr"] = ly["w_rr"][:0]
        ly["b_r"] = ly["b_r"][:0]
    m = synth.cand_to_req_from_counts(COUNTS)
    od = torch.float32 if out == "f32" else torch.bfloat16
    note("lcb fused shape=%s out=%s" % (shape, out))
    (yr, yc), (yr2, yc2) = both_forms(lambda: run_lcb(x_r, x_c, ly, m=m, out_dtype=od, want_req=n_req > 0))
    assert same_bits(yc, yc2), "candidate output differs between the fused and the two-launch form"
    assert same_bits(yr, yr2), "request output differs between the fused and the two-launch form"
    if out == "f32":
        want = oracle.glm(x_r, x_c, [ly], m=m, want_request=True)
        assert_parity(down_f64(yc), want["y_c"], "bf16", "y_c")
        if n_req > 0:
            assert_parity(down_f64(yr), want["y_r"], "bf16", "y_r")


def test_fused_many_request_blocks_unsorted_map():
    """R = 600 requests (three 256-row request tiles) and a shuffled map: every candidate tile waits
    on all request row blocks of its Z columns."""
    rng = np.random.default_rng(5)
    R, C = 600, 3000
    k_req, k_cand, n_req, n_cand = 128, 128, 256, 384
    x_r, x_c = make_x(22, R, C, k_req, k_cand, "bf16")
    ly = make_layer(22, k_req, k_cand, n_req, n_cand, "bf16", "none")
    m = rng.integers(0, R, C).astype(np.int32)
    note("lcb fused R=600 unsorted")
    (yr, yc), (yr2, yc2) = both_forms(lambda: run_lcb(x_r, x_c, ly, m=m))
    assert same_bits(yc, yc2) and same_bits(yr, yr2)
    cands = np.array(sorted(set(rng.integers(0, C, 64).tolist()) | {0, C - 1}))
    want = oracle.glm(x_r, x_c[cands], [ly], m=m[cands], want_request=True)
    assert_parity(down_f64(yc[torch.from_numpy(cands).to(yc.device)]), want["y_c"], "bf16", "y_c sampled")
    assert_parity(down_f64(yr), want["y_r"], "bf16", "y_r")


def test_fused_repeated_calls_reuse_the_workspace():
    """The ready flags and counters live in the workspace and are cleared by every call: three calls
    in a row on the same workspace give the same bits."""
    R, C = len(COUNTS), int(COUNTS.sum())
    x_r, x_c = make_x(23, R, C, 256, 256, "bf16")
    ly = make_layer(23, 256, 256, 256, 256, "bf16", "gelu")
    m = synth.cand_to_req_from_counts(COUNTS)
    os.environ["IKBO_LCB_FUSED"] = "1"
    try:
        outs = [run_lcb(x_r, x_c, ly, m=m) for _ in range(3)]
    finally:
        os.environ.pop("IKBO_LCB_FUSED", None)
    for yr, yc in outs[1:]:
        assert same_bits(yc, outs[0][1]) and same_bits(yr, outs[0][0])


def fused_with_wait_bound(ns, fn):
    os.environ["IKBO_LCB_FUSED"] = "1"
    os.environ["IKBO_LCB_FUSED_WAIT_NS"] = str(ns)
    try:
        return fn()
    finally:
        os.environ.pop("IKBO_LCB_FUSED", None)
        os.environ.pop("IKBO_LCB_FUSED_WAIT_NS", None)


def test_bounded_waits_give_up_with_nan_tiles():
    """The candidate epilogue's wait on the request tiles' ready flags is bounded in time. Forced
    from the host (IKBO_LCB_FUSED_WAIT_NS < 0: the request tiles withhold their flags, the bound is
    2 us), every wait gives up, the launch still ends, every candidate output is NaN (the documented
    mark), and the request-group output, which needs no flag, is the two-launch result. A normal
    launch on the same workspace afterwards is bit-equal to the two-launch form again."""
    R, C = len(COUNTS), int(COUNTS.sum())
    x_r, x_c = make_x(24, R, C, 256, 128, "bf16")
    ly = make_layer(24, 256, 128, 256, 512, "bf16", "gelu")
    m = synth.cand_to_req_from_counts(COUNTS)
    note("lcb fused: withheld flags, 2 us wait bound")
    ref_r, ref_c = run_lcb(x_r, x_c, ly, m=m)
    yr, yc = fused_with_wait_bound(-2000, lambda: run_lcb(x_r, x_c, ly, m=m))
    assert torch.isnan(yc).all()
    assert same_bits(yr, ref_r)
    note("lcb fused: normal launch after the forced timeouts")
    os.environ["IKBO_LCB_FUSED"] = "1"
    try:
        yr2, yc2 = run_lcb(x_r, x_c, ly, m=m)
    finally:
        os.environ.pop("IKBO_LCB_FUSED", None)
    assert same_bits(yc2, ref_c) and same_bits(yr2, ref_r)


@pytest.mark.parametrize("wait_ns", [0, 4000, 40000])
def test_short_wait_bounds_mark_whole_tiles_only(wait_ns):
    """With a short bound and published flags, a candidate tile whose flags are not set within the
    bound gives up (and, once one has, every later wait stops at once): each 256 x 256 output tile
    is then either bit-equal to the two-launch result or NaN throughout (no partly written tile)."""
    R, C = 700, 2600
    x_r, x_c = make_x(25, R, C, 2048, 64, "bf16")
    ly = make_layer(25, 2048, 64, 256, 512, "bf16", "none")
    m = synth.cand_to_req_from_counts(np.full(R, C // R)) if C % R == 0 else np.sort(
        np.random.default_rng(25).integers(0, R, C)).astype(np.int32)
    note("lcb fused: wait bound %d ns" % wait_ns)
    ref_r, ref_c = run_lcb(x_r, x_c, ly, m=m)
    yr, yc = fused_with_wait_bound(wait_ns, lambda: run_lcb(x_r, x_c, ly, m=m))
    assert same_bits(yr, ref_r)
    got, want = yc.float().cpu().numpy(), ref_c.float().cpu().numpy()
    marked = 0
    for r0 in range(0, C, 256):
        for c0 in range(0, 512, 256):
            g, w = got[r0:r0 + 256, c0:c0 + 256], want[r0:r0 + 256, c0:c0 + 256]
            if np.isnan(g).all():
                marked += 1
            else:
                assert np.array_equal(g.view(np.uint32), w.view(np.uint32)), (r0, c0)
    print("tiles marked NaN: %d of %d" % (marked, ((C + 255) // 256) * 2))
