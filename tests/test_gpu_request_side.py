"""GPU parity of the request-side DCA path (the rows next to IKBO-DCA): the K/V projection at the
request batch size (ROCS Sec. 4.1, the DCA decomposition after Eq. 14) and the request half A^R of
Eq. 13, through the C ABI, against the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
import request_candidate_broadcast_amd as ikbo
import synth
from gpu_helpers import assert_parity, bf16_bits, down_f64, note, rne_bits_of, up

pytestmark = pytest.mark.gpu


def proj_inputs(seed, rows, d_in, d_out, kind="bf16"):
    s = synth.draw(seed, 70, rows * d_in, kind).reshape(rows, d_in)
    w_k = synth.draw(seed, 71, d_out * d_in, kind, 1 / math.sqrt(d_in)).reshape(d_out, d_in)
    w_v = synth.draw(seed, 72, d_out * d_in, kind, 1 / math.sqrt(d_in)).reshape(d_out, d_in)
    return s, w_k, w_v


# rows across several 256-row tiles with a ragged tail; d_out a multiple of the 256-wide tile and
# not; d_in from one 64-deep k tile to sixteen, and one that is not a multiple of 64
@pytest.mark.parametrize("rows,d_in,d_out", [(1000, 256, 256), (777, 64, 96), (513, 1024, 1024), (300, 200, 520)])
def test_kv_project_bf16(rows, d_in, d_out):
    s, w_k, w_v = proj_inputs(31, rows, d_in, d_out)
    note("kv_project bf16 rows=%d d_in=%d d_out=%d" % (rows, d_in, d_out))
    sd, wkd, wvd = up(s), up(w_k), up(w_v)
    k32, v32 = ikbo.ikbo_kv_project(sd, wkd, wvd, out_dtype=torch.float32)
    k16, v16 = ikbo.ikbo_kv_project(sd, wkd, wvd, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert_parity(down_f64(k32), oracle.linear(s, w_k), "bf16", "K")
    assert_parity(down_f64(v32), oracle.linear(s, w_v), "bf16", "V")
    # a bf16 output is the round-to-nearest-even of the fp32 output
    assert np.array_equal(bf16_bits(k16), rne_bits_of(k32))
    assert np.array_equal(bf16_bits(v16), rne_bits_of(v32))


def test_kv_project_fp32():
    s, w_k, w_v = proj_inputs(32, 300, 64, 48, "f32")
    note("kv_project fp32")
    k, v = ikbo.ikbo_kv_project(up(s), up(w_k), up(w_v))
    torch.cuda.synchronize()
    assert_parity(down_f64(k), oracle.linear(s, w_k), "f32", "K fp32")
    assert_parity(down_f64(v), oracle.linear(s, w_v), "f32", "V fp32")


def test_kv_project_commutes_with_the_broadcast_on_the_gpu():
    """Projecting the rows each candidate would have received equals projecting each request's rows
    once and reading them through the map, bit for bit (the same dot products)."""
    R, L, d_in, d_out = 6, 40, 128, 256
    s, w_k, w_v = proj_inputs(33, R * L, d_in, d_out)
    m = np.array([0, 0, 3, 5, 5, 5, 1], dtype=np.int64)
    rows = (m[:, None] * L + np.arange(L)[None, :]).reshape(-1)
    note("kv_project broadcast commutation")
    k_req, _ = ikbo.ikbo_kv_project(up(s), up(w_k), up(w_v), out_dtype=torch.float32)
    k_cand, _ = ikbo.ikbo_kv_project(up(np.ascontiguousarray(s[rows])), up(w_k), up(w_v), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(k_req[torch.from_numpy(rows).to(k_req.device)], k_cand)


def ra_case(seed, R, L, H, d, Lq, varlen_lens=None):
    kv_lens = varlen_lens if varlen_lens is not None else [L] * R
    s = synth.custom_dca_spec(seed, np.ones(R, dtype=np.int64), kv_lens, H, d, Lq, dtype="bf16",
                              varlen=varlen_lens is not None)
    return s, synth.dca_q(s), synth.dca_kv(s, "k"), synth.dca_kv(s, "v")


def ra_run(s, q, k, v, out_dtype=torch.float32):
    kd, vd = up(k), up(v)
    kw = {}
    if s.varlen:
        kw["kv_cu_seqlens"] = up(s.kv_cu)
    else:
        kd = kd.view(s.R, s.L, s.H, s.d)
        vd = vd.view(s.R, s.L, s.H, s.d)
    out = ikbo.ikbo_request_attention(up(q), kd, vd, out_dtype=out_dtype, **kw)
    torch.cuda.synchronize()
    return out


def ra_oracle(s, q, k, v):
    if s.varlen:
        return oracle.request_attention(q, k, v, kv_cu=s.kv_cu)
    return oracle.request_attention(q, k.reshape(s.R, s.L, s.H, s.d), v.reshape(s.R, s.L, s.H, s.d))


@pytest.mark.parametrize("d", [128, 64])
def test_request_attention_uniform(d):
    # several 64-key tiles and a ragged last one; Lq = 4 rows per request as in the block workload
    s, q, k, v = ra_case(40 + d, 9, 200, 4, d, 4)
    note("request attention uniform d=%d" % d)
    got = ra_run(s, q, k, v)
    assert_parity(down_f64(got), ra_oracle(s, q, k, v), "bf16", "A^R")
    got16 = ra_run(s, q, k, v, torch.bfloat16)
    assert np.array_equal(bf16_bits(got16), rne_bits_of(got))


def test_request_attention_varlen_with_empty_request():
    lens = [130, 0, 64, 1, 300, 65]
    s, q, k, v = ra_case(44, len(lens), 0, 8, 128, 3, varlen_lens=lens)
    note("request attention varlen")
    got = ra_run(s, q, k, v)
    want = ra_oracle(s, q, k, v)
    assert np.all(down_f64(got)[1] == 0.0)           # L_r = 0: zeros
    assert_parity(down_f64(got), want, "bf16", "A^R varlen")


def test_request_attention_equals_dca_on_the_identity_map():
    """The one-wave work tiles (few rows per request) and the eight-wave tiles give the same bits:
    the same queries as candidates of requests that also hold enough other candidates to make the
    eight-wave configuration the one chosen."""
    R, L, H, d, Lq = 5, 150, 2, 128, 4
    s, q, k, v = ra_case(45, R, L, H, d, Lq)
    note("request attention vs dca configurations")
    small = ra_run(s, q, k, v)
    # candidates: request r's own query row first, then 63 filler candidates (avg rows >> 32)
    filler = synth.draw(46, 1, R * 63 * Lq * H * d, "bf16").reshape(R * 63, Lq, H, d)
    qs, offs, own = [], [0], []
    for r in range(R):
        own.append(sum(len(x) for x in qs))
        qs.append(q[r:r + 1])
        qs.append(filler[r * 63:(r + 1) * 63])
        offs.append(offs[-1] + 64)
    qc = np.ascontiguousarray(np.concatenate(qs))
    big = ikbo.ikbo_dca_forward(up(qc), up(k).view(R, L, H, d), up(v).view(R, L, H, d), num_req=R,
                                req_cand_offsets=up(np.array(offs, dtype=np.int32)), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(big[torch.tensor(own, device=big.device)].view(torch.int32), small.view(torch.int32))


def test_request_side_layer_chain():
    """S -> K^R, V^R (projection) -> A^R with q_r, against the oracle on the GPU's own K/V (the
    projection is pinned above): the chain the block's request half runs."""
    R, L, H, d, Lq, d_in = 4, 96, 2, 64, 4, 128
    s, w_k, w_v = proj_inputs(47, R * L, d_in, H * d)
    q = synth.draw(47, 73, R * Lq * H * d, "bf16").reshape(R, Lq, H, d)
    note("request-side chain")
    kd, vd = ikbo.ikbo_kv_project(up(s), up(w_k), up(w_v))            # bf16 K, V
    out = ikbo.ikbo_request_attention(up(q), kd.view(R, L, H, d), vd.view(R, L, H, d), out_dtype=torch.float32)
    torch.cuda.synchronize()
    k_bits = bf16_bits(kd).reshape(R, L, H, d)
    v_bits = bf16_bits(vd).reshape(R, L, H, d)
    assert_parity(down_f64(out), oracle.request_attention(q, k_bits, v_bits), "bf16", "A^R chain")


def test_full_size_request_side():
    """The block workload's request half at full size: 128 requests x 8192 keys, H = 8, d = 128,
    q_len = 4, S rows of width 1024; sampled rows against the oracle, all rows finite."""
    R, L, H, d, Lq, d_in = 128, 8192, 8, 128, 4, 1024
    rows = R * L
    note("full-size request side")
    s = synth.draw(48, 70, rows * d_in, "bf16").reshape(rows, d_in)
    w_k = synth.draw(48, 71, H * d * d_in, "bf16", 1 / math.sqrt(d_in)).reshape(H * d, d_in)
    w_v = synth.draw(48, 72, H * d * d_in, "bf16", 1 / math.sqrt(d_in)).reshape(H * d, d_in)
    q = synth.draw(48, 73, R * Lq * H * d, "bf16").reshape(R, Lq, H, d)
    kd, vd = ikbo.ikbo_kv_project(up(s), up(w_k), up(w_v))
    out = ikbo.ikbo_request_attention(up(q), kd.view(R, L, H, d), vd.view(R, L, H, d), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    pick = np.array([0, 1, 4095, 8192 * 64 + 17, rows - 1], dtype=np.int64)
    k32, _ = ikbo.ikbo_kv_project(up(s), up(w_k), up(w_v), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_parity(down_f64(k32[torch.from_numpy(pick).to(k32.device)]), oracle.linear(s, w_k, rows=pick), "bf16",
                  "K sampled rows")
    del k32
    reqs = [0, 63, 127]
    sel = torch.tensor(reqs, device=kd.device)
    k_bits = bf16_bits(kd.view(R, L, H, d)[sel])
    v_bits = bf16_bits(vd.view(R, L, H, d)[sel])
    want = oracle.request_attention(np.ascontiguousarray(q[reqs]), np.ascontiguousarray(k_bits),
                                    np.ascontiguousarray(v_bits))
    assert_parity(down_f64(out[torch.tensor(reqs, device=out.device)]), want, "bf16", "A^R sampled requests")
