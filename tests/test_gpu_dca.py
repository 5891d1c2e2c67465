"""GPU parity of IKBO-DCA (through the C ABI) against the fp64 oracle, plus exactness checks."""
import numpy as np
import pytest
import torch

import oracle
import request_candidate_broadcast_amd as ikbo
import synth
from gpu_helpers import assert_parity, bf16_bits, down_f64, note, rne_bits_of, up

pytestmark = pytest.mark.gpu


def make_case(seed, counts, kv_lens, H, d, Lq, dtype, varlen=None, scale=1.0):
    s = synth.custom_dca_spec(seed, counts, kv_lens, H, d, Lq, dtype=dtype, varlen=varlen, value_scale=scale)
    q = synth.dca_q(s)
    k = synth.dca_kv(s, "k")
    v = synth.dca_kv(s, "v")
    return s, q, k, v


def run_gpu(s, q, k, v, *, mode="offsets", out_dtype=torch.float32, m=None, perm=None):
    qd = up(q)
    kd, vd = up(k), up(v)
    if not s.varlen:
        kd = kd.view(s.R, s.L, s.H, s.d)
        vd = vd.view(s.R, s.L, s.H, s.d)
    kw = {}
    if s.varlen:
        kw["kv_cu_seqlens"] = up(s.kv_cu)
    if mode == "offsets":
        kw["req_cand_offsets"] = up(s.offsets)
    elif mode == "map":
        kw["cand_to_req"] = up(s.cand_to_req if m is None else m)
        kw["sorted_index"] = m is None
    elif mode == "both":
        kw["req_cand_offsets"] = up(s.offsets)
        kw["cand_to_req"] = up(s.cand_to_req)
        kw["sorted_index"] = True
    out = ikbo.ikbo_dca_forward(qd, kd, vd, num_req=s.R, out_dtype=out_dtype, **kw)
    torch.cuda.synchronize()
    return out


def oracle_out(s, q, k, v, m=None, cands=None):
    kv = dict(kv_cu=s.kv_cu) if s.varlen else {}
    k_ = k if s.varlen else k.reshape(s.R, s.L, s.H, s.d)
    v_ = v if s.varlen else v.reshape(s.R, s.L, s.H, s.d)
    return oracle.dca(q, k_, v_, s.R, m=s.cand_to_req if m is None else m, cands=cands, **kv)


def test_tiny_fp32_workload():
    s = synth.dca_spec("tiny")
    q, k, v = synth.dca_q(s), synth.dca_kv(s, "k"), synth.dca_kv(s, "v")
    note("dca tiny fp32 C=%d" % s.C)
    got = run_gpu(s, q, k, v)
    assert_parity(down_f64(got), oracle_out(s, q, k, v), "f32", "tiny")


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("Lq", [1, 4])
def test_bf16_ragged_tiles(d, Lq):
    # several 256-row tiles, a ragged last tile, an empty request, keys not a multiple of 64
    counts = [1, 37, 300, 0, 64, 129]
    s, q, k, v = make_case(10 + d + Lq, counts, [200] * len(counts), 2, d, Lq, "bf16")
    note("dca bf16 ragged d=%d Lq=%d C=%d" % (d, Lq, s.C))
    got32 = run_gpu(s, q, k, v)
    want = oracle_out(s, q, k, v)
    assert_parity(down_f64(got32), want, "bf16", "d=%d Lq=%d" % (d, Lq))
    got16 = run_gpu(s, q, k, v, out_dtype=torch.bfloat16)
    assert np.array_equal(bf16_bits(got16), rne_bits_of(got32)), "bf16 output must be RNE of the fp32 output"


@pytest.mark.parametrize("d", [128, 64])
def test_bf16_varlen(d):
    counts = [5, 0, 70, 260, 3]
    lens = [1, 65, 300, 0, 64]
    s, q, k, v = make_case(20 + d, counts, lens, 3, d, 2, "bf16", varlen=True)
    note("dca bf16 varlen d=%d" % d)
    got = run_gpu(s, q, k, v)
    want = oracle_out(s, q, k, v)
    assert_parity(down_f64(got), want, "bf16", "varlen")
    # the L_r = 0 request (index 3) gives exact zeros
    off = s.offsets
    assert torch.all(got[off[3]:off[4]] == 0)


def test_fp32_general_head_dims():
    for d in (4, 36, 128):
        s, q, k, v = make_case(30 + d, [3, 17, 1], [9, 40, 70], 2, d, 3, "f32", varlen=True)
        note("dca fp32 d=%d" % d)
        got = run_gpu(s, q, k, v)
        assert_parity(down_f64(got), oracle_out(s, q, k, v), "f32", "fp32 d=%d" % d)


def test_index_paths_agree_bitwise_and_unsorted_map():
    counts = [40, 1, 300, 7, 0, 90]
    s, q, k, v = make_case(40, counts, [130] * 6, 2, 128, 4, "bf16")
    note("dca index paths")
    a = run_gpu(s, q, k, v, mode="offsets")
    b = run_gpu(s, q, k, v, mode="map")
    c = run_gpu(s, q, k, v, mode="both")
    assert torch.equal(a, b) and torch.equal(a, c)
    # unsorted map: permute candidates together with their map entries (P4: bitwise permutation)
    rng = np.random.default_rng(0)
    perm = rng.permutation(s.C)
    qp = q[perm]
    m_p = s.cand_to_req[perm]
    d_ = run_gpu(s, qp, k, v, mode="map", m=m_p)
    assert torch.equal(d_, a[torch.from_numpy(perm).to(a.device)])
    assert_parity(down_f64(a), oracle_out(s, q, k, v), "bf16", "index paths")


def test_invalid_map_rows_are_zero():
    counts = [10, 20]
    s, q, k, v = make_case(41, counts, [64, 64], 1, 64, 1, "bf16")
    m = s.cand_to_req.copy()
    m[[0, 15, 29]] = [-1, 2, 7]
    note("dca invalid map rows")
    got = run_gpu(s, q, k, v, mode="map", m=m)
    want = oracle.dca(q, k.reshape(2, 64, 1, 64), v.reshape(2, 64, 1, 64), 2, m=m)
    for c in (0, 15, 29):
        assert torch.all(got[c] == 0)
    assert_parity(down_f64(got), want, "bf16", "invalid rows")


def test_single_key_is_exact():
    # P2: L_r = 1 -> softmax weight 1 -> O == V[r, 0], bit for bit in both output dtypes. The kernel
    # folds the softmax scale into one FMA, so the weight of the max key is exp2 of that product's
    # rounding residual (|x| < 2^-20); its bf16 rounding, the value the PV product and the row sum
    # both use, is exactly 1, so O = V * 1 / 1.
    counts = [33, 300, 2]
    s, q, k, v = make_case(42, counts, [1, 1, 1], 2, 128, 1, "bf16")
    note("dca single key")
    got = run_gpu(s, q, k, v)
    vv = synth.bf16_to_f64(v.reshape(3, 2, 128))
    want = vv[s.cand_to_req][:, None]
    assert np.array_equal(down_f64(got), want)
    got16 = run_gpu(s, q, k, v, out_dtype=torch.bfloat16)
    assert np.array_equal(bf16_bits(got16), v.reshape(3, 2, 128)[s.cand_to_req][:, None])


def test_request_tag_exact():
    # P8 with one key per request: V[r] == r gives O[c] == m[c] exactly.
    counts = [3, 70, 1, 300]
    R = 4
    s, q, k, v = make_case(43, counts, [1] * R, 2, 64, 2, "bf16")
    vt = synth.f32_to_bf16_bits(np.repeat(np.arange(R, dtype=np.float32), 2 * 64))
    note("dca request tag")
    got = run_gpu(s, q, k, vt)
    want = np.broadcast_to(s.cand_to_req[:, None, None, None].astype(np.float64), tuple(got.shape))
    assert np.array_equal(down_f64(got), want)
    got16 = run_gpu(s, q, k, vt, out_dtype=torch.bfloat16)
    assert np.array_equal(down_f64(got16), want)


def test_zero_query_mean_of_values():
    # P7: Q = 0 gives O = mean_j V_j
    counts = [5, 8]
    s, q, k, v = make_case(44, counts, [300, 300], 2, 128, 1, "bf16")
    q0 = np.zeros_like(q)
    note("dca zero query")
    got = down_f64(run_gpu(s, q0, k, v))
    vv = synth.bf16_to_f64(v).reshape(2, 300, 2, 128).mean(axis=1)
    assert np.abs(got - vv[s.cand_to_req][:, None]).max() < 2e-3


def test_identical_queries_identical_outputs_and_determinism():
    # P9 and run-to-run determinism.
    counts = [300, 200]
    s, q, k, v = make_case(45, counts, [257, 257], 2, 128, 1, "bf16")
    q = q.copy()
    q[7] = q[250]
    q[299] = q[250]
    note("dca identical queries")
    a = run_gpu(s, q, k, v)
    b = run_gpu(s, q, k, v)
    assert torch.equal(a, b)
    assert torch.equal(a[7], a[250]) and torch.equal(a[299], a[250])


def test_empty_inputs():
    s, q, k, v = make_case(46, [0, 0], [8, 8], 1, 64, 1, "bf16")
    note("dca empty")
    got = run_gpu(s, q, k, v)
    assert got.shape == (0, 1, 1, 64)


@pytest.mark.parametrize("d,hot_value", [(64, 8.0), (128, 8.0), (64, 10.0), (128, 10.0), (64, 12.0), (128, 12.0)])
def test_scores_far_above_the_first_tile_take_the_exact_path(d, hot_value):
    # Scores in a later key tile far above the first tile's max overflow the fixed-reference sums;
    # those queries are recomputed against their exact max. Other queries of the same work tile
    # must come out bit for bit as in a run where nothing overflows. The hot key (every element 8)
    # also makes every query's score against it several times its usual size, which magnifies any
    # rounding of the queries or scores (a bf16 rounding of the scaled queries fails here).
    counts = [300]
    L, H = 200, 1
    s, q, k, v = make_case(47, counts, [L], H, d, 1, "bf16")
    big_q = q.copy()
    big_k = k.copy()
    hot = synth.f32_to_bf16_bits(np.full(d, hot_value, np.float32))
    big_q[5, 0, 0] = hot          # candidate 5's query
    big_k[150, 0] = hot           # key 150 (third tile): score hot^2 d / sqrt(d), far past 2^128
    note("dca exact-path fallback d=%d hot=%g" % (d, hot_value))
    got = run_gpu(s, big_q, big_k, v)
    want = oracle.dca(big_q, big_k.reshape(1, L, H, d), v.reshape(1, L, H, d), 1, m=s.cand_to_req)
    assert_parity(down_f64(got), want, "bf16", "fallback")
    ref = run_gpu(s, q, big_k, v)   # same keys, no hot query: nothing overflows
    others = [c for c in range(s.C) if c != 5]
    # queries other than 5 see the hot key too, so compare them with the run that has no hot query
    assert torch.equal(got[others], ref[others])
