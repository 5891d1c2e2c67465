"""Index handling on the GPU, through the C ABI (the map m of ROCS Sec. 4.1 and the contiguous
per-request grouping of Sec. 4.2.1):

* ikbo_check_index counts exactly what the oracle's index_violations counts, case by case;
* an ungrouped map is grouped by a stable sort: each request's candidates in index order;
* with both index arrays given, every entry point takes each candidate's request from the
  offsets (the map is not read), as the oracle does;
* one DCA interaction layer checks every stage's arguments before it launches anything.
Every comparison here is bitwise (integer work, or runs of the same kernels)."""
import math

import numpy as np
import pytest
import torch

import oracle
import request_candidate_broadcast_amd as ikbo
import synth
from gpu_helpers import assert_parity, down_f64, note, up

pytestmark = pytest.mark.gpu


def check_cases():
    """(name, m, off, C, R, sorted_flag) with a known kind of fault each."""
    m = synth.cand_to_req_from_counts(np.array([3, 0, 5, 2]))
    off = synth.offsets_from_counts(np.array([3, 0, 5, 2]))
    C, R = len(m), 4
    rng = np.random.default_rng(3)
    big_counts = rng.integers(0, 40, 300)
    big_m = synth.cand_to_req_from_counts(big_counts)
    big_off = synth.offsets_from_counts(big_counts)
    cases = [("valid grouped, both arrays", m, off, C, R, True),
             ("valid grouped, map only", m, None, C, R, True),
             ("valid grouped, offsets only", None, off, C, R, False),
             ("large valid", big_m, big_off, len(big_m), len(big_counts), True)]
    u = m.copy()
    u[[0, 6]] = u[[6, 0]]
    cases.append(("unsorted map declared sorted", u, None, C, R, True))
    cases.append(("unsorted map not declared sorted", u, None, C, R, False))
    bad = m.copy()
    bad[[1, 4, 9]] = [-1, 4, 1000]
    cases.append(("out-of-range map", bad, None, C, R, False))
    cases.append(("out-of-range map with offsets", bad, off, C, R, True))
    dis = m.copy()
    dis[[2, 7]] = [2, 0]
    cases.append(("map disagrees with offsets", dis, off, C, R, False))
    nm = off.copy()
    nm[2] = 9
    cases.append(("non-monotone offsets", None, nm, C, R, False))
    cases.append(("non-monotone offsets with map", m, nm, C, R, True))
    o0 = off.copy()
    o0[0] = 1
    cases.append(("off[0] != 0", None, o0, C, R, False))
    oR = off.copy()
    oR[R] = C - 1
    cases.append(("off[R] != C", None, oR, C, R, False))
    both = off.copy()
    both[0], both[R] = 2, C + 3
    cases.append(("off[0] != 0 and off[R] != C", None, both, C, R, False))
    bm = big_m.copy()
    bm[rng.integers(0, len(bm), 50)] = rng.integers(-5, len(big_counts) + 5, 50).astype(np.int32)
    cases.append(("large with faults", bm, big_off, len(bm), len(big_counts), True))
    cases.append(("empty", np.zeros(0, np.int32), np.zeros(R + 1, np.int32), 0, R, True))
    return cases


@pytest.mark.parametrize("case", check_cases(), ids=lambda c: c[0])
def test_check_index_counts_match_the_oracle(case):
    name, m, off, C, R, srt = case
    note("check_index %s" % name)
    kw = {}
    if m is not None:
        kw["cand_to_req"] = up(m) if C > 0 else torch.zeros(1, dtype=torch.int32, device="cuda:0")
    if off is not None:
        kw["req_cand_offsets"] = up(off)
    got = ikbo.ikbo_check_index(C, R, sorted_index=srt, **kw)
    want = oracle.index_violations(m, off, C, R, srt)
    assert got == want, (name, got, want)
    if name.startswith("valid") or name in ("large valid", "empty", "unsorted map not declared sorted"):
        assert got == 0
    else:
        assert got > 0


def dca_perm(ws: torch.Tensor, C: int, R: int) -> np.ndarray:
    """The grouping order the DCA computed for a map without offsets, read from its workspace:
    three int32 [R + 1] arrays (each from a 256-byte boundary), then perm [C]."""
    a = (4 * (R + 1) + 255) // 256 * 256
    return ws[3 * a: 3 * a + 4 * C].view(torch.int32).cpu().numpy()


@pytest.mark.parametrize("R,C", [(7, 300), (300, 5000), (70000, 9000)])
def test_ungrouped_map_is_grouped_stably(R, C):
    # one, two and three 8-bit passes (keys 0..R), tiles of several blocks, invalid entries last
    rng = np.random.default_rng(R)
    m = rng.integers(0, R, C).astype(np.int32)
    m[rng.integers(0, C, 9)] = -3
    m[rng.integers(0, C, 9)] = R + 11
    k = up(synth.draw(60, 1, R * 64, "bf16").reshape(R, 1, 1, 64))
    v = up(synth.draw(60, 2, R * 64, "bf16").reshape(R, 1, 1, 64))
    q = up(synth.draw(61, 1, C * 64, "bf16").reshape(C, 1, 1, 64))
    ws = torch.empty(ikbo.ikbo_dca_workspace_size(C, R), dtype=torch.uint8, device="cuda:0")
    note("stable grouping R=%d C=%d" % (R, C))
    out = ikbo.ikbo_dca_forward(q, k, v, num_req=R, cand_to_req=up(m), workspace=ws)
    torch.cuda.synchronize()
    key = np.where((m >= 0) & (m < R), m, R)
    assert np.array_equal(dca_perm(ws, C, R), np.argsort(key, kind="stable"))
    # single key per request: every valid row is its request's V, every invalid row zero
    vv = v.view(R, 64)
    ok = torch.from_numpy((m >= 0) & (m < R)).to(out.device)
    mm = torch.from_numpy(np.clip(m, 0, R - 1)).to(out.device).long()
    assert torch.equal(out.view(C, 64)[ok], vv[mm[ok]])
    assert torch.count_nonzero(out.view(C, 64)[~ok]).item() == 0


def disagreeing(counts):
    m = synth.cand_to_req_from_counts(counts)
    off = synth.offsets_from_counts(counts)
    bad = m.copy()
    bad[[0, len(m) // 2, len(m) - 1]] = [len(counts) - 1, -1, 0]
    assert oracle.index_violations(bad, off, len(m), len(counts)) > 0
    return m, off, bad


def test_both_arrays_the_offsets_decide_dca():
    counts = np.array([40, 0, 170, 9])
    m, off, bad = disagreeing(counts)
    s = synth.custom_dca_spec(62, list(counts), [100] * 4, 2, 128, 2, dtype="bf16")
    q, k, v = synth.dca_q(s), synth.dca_kv(s, "k"), synth.dca_kv(s, "v")
    k4, v4 = up(k).view(4, 100, 2, 128), up(v).view(4, 100, 2, 128)
    note("both arrays: dca")
    a = ikbo.ikbo_dca_forward(up(q), k4, v4, req_cand_offsets=up(off), out_dtype=torch.float32)
    b = ikbo.ikbo_dca_forward(up(q), k4, v4, req_cand_offsets=up(off), cand_to_req=up(bad), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    want = oracle.dca(q, k.reshape(4, 100, 2, 128), v.reshape(4, 100, 2, 128), 4, m=bad, off=off)
    assert_parity(down_f64(b), want, "bf16", "dca both")


def test_both_arrays_the_offsets_decide_lcb_and_mlp():
    counts = np.array([3, 0, 290, 9])
    m, off, bad = disagreeing(counts)
    R, C = 4, int(counts.sum())
    x_r = synth.draw(63, 1, R * 64, "bf16").reshape(R, 64)
    x_c = synth.draw(63, 2, C * 128, "bf16").reshape(C, 128)
    layers = []
    for i, (kr, kc, n, act) in enumerate(((64, 128, 48, "gelu"), (48, 48, 40, "none"))):
        layers.append(dict(w_rr=synth.draw(63, 10 + 8 * i, n * kr, "bf16", 1 / math.sqrt(kr)).reshape(n, kr),
                           w_cr=synth.draw(63, 11 + 8 * i, n * kr, "bf16", 1 / math.sqrt(kr)).reshape(n, kr),
                           w_cc=synth.draw(63, 12 + 8 * i, n * kc, "bf16", 1 / math.sqrt(kc)).reshape(n, kc),
                           b_r=synth.draw(63, 13 + 8 * i, n, "f32", 0.1), b_c=synth.draw(63, 14 + 8 * i, n, "f32", 0.1),
                           act=act))
    dl = [{k: (up(v) if isinstance(v, np.ndarray) else v) for k, v in ly.items()} for ly in layers]
    note("both arrays: lcb")
    l0 = dl[0]
    lcb = lambda **kw: ikbo.ikbo_lcb_forward(up(x_r), up(x_c), l0["w_rr"], l0["w_cr"], l0["w_cc"], b_r=l0["b_r"],
                                             b_c=l0["b_c"], activation="gelu", out_dtype=torch.float32, **kw)[1]
    a, b = lcb(req_cand_offsets=up(off)), lcb(req_cand_offsets=up(off), cand_to_req=up(bad), sorted_index=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert_parity(down_f64(b), oracle.glm(x_r, x_c, layers[:1], m=bad, off=off)["y_c"], "bf16", "lcb both")
    note("both arrays: glm-mlp")
    mlp = lambda **kw: ikbo.ikbo_glm_mlp_forward(up(x_r), up(x_c), dl, out_dtype=torch.float32, **kw)[1]
    a, b = mlp(req_cand_offsets=up(off)), mlp(req_cand_offsets=up(off), cand_to_req=up(bad))
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    # and the map alone really is different (the disagreeing rows move or vanish)
    c = mlp(cand_to_req=up(bad))
    torch.cuda.synchronize()
    assert not torch.equal(a, c)


def test_both_arrays_the_offsets_decide_fm_and_lcb_emb():
    counts = np.array([30, 2, 0, 60])
    m, off, bad = disagreeing(counts)
    R, C, n, d = 4, int(counts.sum()), 32, 64
    x_r = up(synth.draw(64, 1, R * n * d, "bf16").reshape(R, n, d))
    x_c = up(synth.draw(64, 2, C * n * d, "bf16").reshape(C, n, d))
    note("both arrays: fm")
    a = ikbo.ikbo_fm_forward(x_r, x_c, req_cand_offsets=up(off), out_dtype=torch.float32)[1]
    b = ikbo.ikbo_fm_forward(x_r, x_c, req_cand_offsets=up(off), cand_to_req=up(bad), out_dtype=torch.float32)[1]
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    w = [up(synth.draw(64, 3 + i, 32 * 32, "bf16", 1 / math.sqrt(32)).reshape(32, 32)) for i in range(3)]
    note("both arrays: lcb_emb")
    e = lambda **kw: ikbo.ikbo_lcb_emb_forward(x_r, x_c, *w, norm="layer", out_dtype=torch.float32, **kw)[1]
    a, b = e(req_cand_offsets=up(off)), e(req_cand_offsets=up(off), cand_to_req=up(bad))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def layer_params(seed, R, C, d, Lq=2, H=2, L=40, sd=64):
    W = Lq * H * d
    x_r = synth.draw(seed, 1, R * 64, "bf16").reshape(R, 64)
    x_c = synth.draw(seed, 2, C * 48, "bf16").reshape(C, 48)
    layers = []
    for i, (kr, kc, n, act) in enumerate(((64, 48, 32, "gelu"), (32, 32, W, "none"))):
        layers.append(dict(w_rr=synth.draw(seed, 10 + 8 * i, n * kr, "bf16", 1 / math.sqrt(kr)).reshape(n, kr),
                           w_cr=synth.draw(seed, 11 + 8 * i, n * kr, "bf16", 1 / math.sqrt(kr + kc)).reshape(n, kr),
                           w_cc=synth.draw(seed, 12 + 8 * i, n * kc, "bf16", 1 / math.sqrt(kr + kc)).reshape(n, kc),
                           b_r=synth.draw(seed, 13 + 8 * i, n, "f32", 0.1), b_c=synth.draw(seed, 14 + 8 * i, n, "f32", 0.1),
                           act=act))
    dl = [{k: (up(v) if isinstance(v, np.ndarray) else v) for k, v in ly.items()} for ly in layers]
    seq = up(synth.draw(seed, 30, R * L * sd, "bf16").reshape(R * L, sd))
    ws = [up(synth.draw(seed, 31 + i, H * d * sd, "bf16", 1 / math.sqrt(sd)).reshape(H * d, sd)) for i in range(4)]
    return dict(x_r=up(x_r), x_c=up(x_c), layers=dl, seq=seq, ws=ws, Lq=Lq, H=H, d=d, W=W)


def test_both_arrays_the_offsets_decide_dca_layer():
    counts = np.array([5, 0, 9, 1])
    m, off, bad = disagreeing(counts)
    p = layer_params(65, 4, int(counts.sum()), 64)
    note("both arrays: dca layer")
    run = lambda **kw: ikbo.ikbo_dca_layer_forward(p["x_r"], p["x_c"], p["layers"], p["seq"], *p["ws"], q_len=p["Lq"],
                                                   num_heads=p["H"], head_dim=p["d"], **kw)
    a_r, a_c = run(req_cand_offsets=up(off))
    b_r, b_c = run(req_cand_offsets=up(off), cand_to_req=up(bad))
    torch.cuda.synchronize()
    assert torch.equal(a_r.view(torch.int16), b_r.view(torch.int16))
    assert torch.equal(a_c.view(torch.int16), b_c.view(torch.int16))


def test_dca_layer_checks_every_stage_before_launching():
    # bf16 attention is built for head_dim 64 and 128: with 96 the call must fail before the query
    # generator writes anything into the outputs
    counts = np.array([4, 3])
    R, C = 2, 7
    p = layer_params(66, R, C, 96)
    y_r = torch.full((R, 2 * p["W"]), 7.0, dtype=torch.bfloat16, device="cuda:0")
    y_c = torch.full((C, 2 * p["W"]), 7.0, dtype=torch.bfloat16, device="cuda:0")
    note("dca layer: head_dim 96 rejected before any launch")
    with pytest.raises(ikbo.IkboError) as e:
        ikbo.ikbo_dca_layer_forward(p["x_r"], p["x_c"], p["layers"], p["seq"], *p["ws"], q_len=p["Lq"],
                                    num_heads=p["H"], head_dim=96, req_cand_offsets=up(synth.offsets_from_counts(counts)),
                                    y_req=y_r, y_cand=y_c)
    assert e.value.status == ikbo.IKBO_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.all(y_r == 7.0) and torch.all(y_c == 7.0)
