"""Parity at the full workload sizes, in the launch configuration bench.py times.

The oracle cannot evaluate whole workloads at these sizes, so each test compares sampled
candidates (first and last candidates of requests 0, 1, R/2 and R-1, plus seeded random ones)
one by one against the fp64 oracle, and checks properties that hold at any size over every
output: finiteness, and for attention the convexity bound min_j V <= O <= max_j V per request,
head and channel. The persistent IKBO-LCB launch must equal the two-launch form bit for bit."""
import os

import numpy as np
import pytest
import torch

import oracle
import request_candidate_broadcast_amd as ikbo
import synth
from gpu_helpers import assert_parity, down_f64, note, up

pytestmark = pytest.mark.gpu


def sample_candidates(offsets, R, extra=8, seed=0):
    picks = []
    for r in sorted({0, 1, R // 2, R - 1}):
        if offsets[r + 1] > offsets[r]:
            picks += [int(offsets[r]), int(offsets[r + 1] - 1)]
    rng = np.random.default_rng(seed)
    picks += [int(x) for x in rng.integers(0, int(offsets[-1]), extra)]
    return np.array(sorted(set(picks)), dtype=np.int64)


def convexity_check(out, k_unused, v, s):
    """min_j V[r, j, h, :] <= O[c, t, h, :] <= max_j V[r, j, h, :] for every candidate of request r."""
    off = s.offsets
    for r in range(s.R):
        c0, c1 = int(off[r]), int(off[r + 1])
        if c1 == c0:
            continue
        if s.varlen:
            cu = s.kv_cu
            vr = v[int(cu[r]):int(cu[r + 1])]
        else:
            vr = v[r]
        if vr.shape[0] == 0:
            assert torch.all(out[c0:c1] == 0)
            continue
        vr = vr.float()
        lo = vr.amin(dim=0) - 1e-3      # [H, d]
        hi = vr.amax(dim=0) + 1e-3
        o = out[c0:c1].float()
        assert torch.all(o >= lo) and torch.all(o <= hi), "request %d breaks the convexity bound" % r


@pytest.mark.parametrize("name", ["dca_fixed", "dca_ragged"])
def test_dca_full_size(name):
    s = synth.dca_spec(name)
    note("full-size %s C=%d R=%d" % (name, s.C, s.R))
    q = synth.dca_q(s)
    k, v = synth.dca_kv(s, "k"), synth.dca_kv(s, "v")
    qd, kd, vd = up(q), up(k), up(v)
    kw = {}
    if s.varlen:
        kw["kv_cu_seqlens"] = up(s.kv_cu)
    else:
        kd = kd.view(s.R, s.L, s.H, s.d)
        vd = vd.view(s.R, s.L, s.H, s.d)
    out = ikbo.ikbo_dca_forward(qd, kd, vd, num_req=s.R, req_cand_offsets=up(s.offsets), out_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    convexity_check(out, kd, vd, s)
    cands = sample_candidates(s.offsets, s.R)
    ko = k if s.varlen else k.reshape(s.R, s.L, s.H, s.d)
    vo = v if s.varlen else v.reshape(s.R, s.L, s.H, s.d)
    want = oracle.dca(q, ko, vo, s.R, off=s.offsets, kv_cu=s.kv_cu, cands=cands)
    got = down_f64(out[torch.from_numpy(cands).to(out.device)])
    assert_parity(got, want, "bf16", name)


def test_lcb_full_size():
    g = synth.glm_spec("lcb")
    note("full-size lcb C=%d" % g.C)
    x_r, x_c = synth.glm_x(g, "x_r"), synth.glm_x(g, "x_c")
    w = synth.glm_weights(g, 0)
    wd = {k: up(v) for k, v in w.items()}
    xr_d, xc_d, m_d = up(x_r), up(x_c), up(g.cand_to_req)

    def call():
        return ikbo.ikbo_lcb_forward(xr_d, xc_d, wd["w_rr"], wd["w_cr"], wd["w_cc"], b_r=wd["b_r"], b_c=wd["b_c"],
                                     cand_to_req=m_d, sorted_index=True, activation="gelu", out_dtype=torch.float32)
    y_r, y_c = call()
    torch.cuda.synchronize()
    assert torch.isfinite(y_c).all() and torch.isfinite(y_r).all()
    # the persistent request/candidate launch gives the same bits at full size
    note("full-size lcb, persistent launch")
    os.environ["IKBO_LCB_FUSED"] = "1"
    try:
        y_r2, y_c2 = call()
        torch.cuda.synchronize()
    finally:
        os.environ.pop("IKBO_LCB_FUSED", None)
    assert torch.equal(y_c2.view(torch.int32), y_c.view(torch.int32))
    assert torch.equal(y_r2.view(torch.int32), y_r.view(torch.int32))
    del y_r2, y_c2
    cands = sample_candidates(g.offsets, g.R)
    ly = dict(w, act="gelu")
    # compact oracle inputs: only the sampled candidates' rows
    want = oracle.glm(x_r, x_c[cands], [ly], m=g.cand_to_req[cands], want_request=True)
    assert_parity(down_f64(y_c[torch.from_numpy(cands).to(y_c.device)]), want["y_c"], "bf16", "lcb y_c")
    assert_parity(down_f64(y_r), want["y_r"], "bf16", "lcb y_r (all requests)")


def test_full_block():
    g, s = synth.block_specs()
    note("full-size block C=%d" % g.C)
    x_r, x_c = synth.glm_x(g, "x_r"), synth.glm_x(g, "x_c")
    layers_h = [dict(synth.glm_weights(g, li), act=g.layers[li].act) for li in range(len(g.layers))]
    layers_d = [{k: (up(v) if isinstance(v, np.ndarray) else v) for k, v in ly.items()} for ly in layers_h]
    k, v = synth.dca_kv(s, "k"), synth.dca_kv(s, "v")
    kd = up(k).view(s.R, s.L, s.H, s.d)
    vd = up(v).view(s.R, s.L, s.H, s.d)
    # the launch sequence bench.py times: GLM-MLP to bf16 queries, then DCA
    y_req, y_cand = ikbo.ikbo_glm_mlp_forward(up(x_r), up(x_c), layers_d, cand_to_req=up(g.cand_to_req),
                                              sorted_index=True, out_dtype=torch.bfloat16)
    q = y_cand.view(s.C, s.Lq, s.H, s.d)
    out = ikbo.ikbo_dca_forward(q, kd, vd, req_cand_offsets=up(s.offsets), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(y_cand.float()).all()
    convexity_check(out, kd, vd, s)
    cands = sample_candidates(s.offsets, s.R, extra=4)
    reqs = sorted(set(g.cand_to_req[cands].tolist()))
    # oracle chain in fp64 on compact inputs: the sampled candidates and their requests' K/V
    mlp = oracle.glm(x_r, x_c[cands], layers_h, m=g.cand_to_req[cands], want_request=True)
    kc = np.stack([synth.dca_kv_request(s, "k", r) for r in reqs])
    vc = np.stack([synth.dca_kv_request(s, "v", r) for r in reqs])
    mc = np.array([reqs.index(r) for r in g.cand_to_req[cands]], np.int32)
    want = oracle.dca(mlp["y_c"].reshape(len(cands), s.Lq, s.H, s.d), kc, vc, len(reqs), m=mc)
    got = down_f64(out[torch.from_numpy(cands).to(out.device)])
    assert_parity(got, want, "bf16", "block DCA output")
    # the request-group output is stored in bf16 here (the queries must be bf16 for DCA); it is held
    # to the same bars as the fp32-output runs
    assert_parity(down_f64(y_req), mlp["y_r"], "bf16", "block request-group MLP output")
