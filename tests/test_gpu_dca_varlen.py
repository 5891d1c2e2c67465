"""IKBO-DCA with per-request K/V lengths (kv_cu_seqlens): a row's result depends only on its own
query and its request's keys, so every output row must carry the same bits as a launch of the same
rows with uniform lengths, or of its request alone. Outputs start as NaN, so a tile that never ran
shows up."""
import numpy as np
import pytest
import torch

import oracle
import request_candidate_broadcast_amd as ikbo
import synth
from gpu_helpers import assert_parity, down_f64, note, up

pytestmark = pytest.mark.gpu


def nan_out(C, Lq, H, d):
    return torch.full((C, Lq, H, d), float("nan"), dtype=torch.float32, device="cuda")


def same_bits(a, b):
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("d,rows", [(64, 20), (64, 100), (128, 100), (64, 1300), (128, 1300)])
def test_varlen_keeps_the_bits_of_the_uniform_launch(d, rows):
    """Equal K/V lengths given as kv_cu_seqlens and as kv_len: bit-equal. Candidate counts vary around `rows` per request (one-, four- and
    eight-wave tiles) and include an empty request."""
    R, L, H, Lq = 40, 333, 2, 1
    counts = synth.uniform_ints(90 + d, 1, R, rows // 2, rows + rows // 2).astype(np.int64)
    counts[7] = 0
    C = int(counts.sum())
    off = synth.offsets_from_counts(counts)
    q = up(synth.draw(90 + d, 2, C * Lq * H * d, "bf16").reshape(C, Lq, H, d))
    k = up(synth.draw(90 + d, 3, R * L * H * d, "bf16").reshape(R * L, H, d))
    v = up(synth.draw(90 + d, 4, R * L * H * d, "bf16").reshape(R * L, H, d))
    cu = up(np.arange(R + 1, dtype=np.int32) * L)
    note("dca varlen d=%d rows=%d: uniform" % (d, rows))
    plain = ikbo.ikbo_dca_forward(q, k.view(R, L, H, d), v.view(R, L, H, d), num_req=R, req_cand_offsets=up(off),
                                  out=nan_out(C, Lq, H, d))
    note("dca varlen d=%d rows=%d: varlen" % (d, rows))
    vl = ikbo.ikbo_dca_forward(q, k, v, num_req=R, req_cand_offsets=up(off), kv_cu_seqlens=cu, kv_len=L,
                                  out=nan_out(C, Lq, H, d))
    torch.cuda.synchronize()
    assert not torch.isnan(vl).any()
    assert same_bits(vl, plain)


@pytest.mark.parametrize("d", [64, 128])
def test_ragged_lengths_match_each_request_alone(d):
    """Ragged lengths (one of them zero, some not a multiple of the 64-key tile) and ragged counts:
    each request's rows equal, bit for bit, a plain launch of that request alone with uniform
    length L_r; the whole output also passes against the oracle."""
    R, H, Lq = 24, 2, 2
    lens = synth.uniform_ints(120 + d, 1, R, 1, 900).astype(np.int64)
    lens[5] = 0
    counts = synth.uniform_ints(120 + d, 2, R, 0, 140).astype(np.int64)
    C = int(counts.sum())
    off = synth.offsets_from_counts(counts)
    cu_np = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    rows = int(cu_np[-1])
    q_np = synth.draw(120 + d, 3, C * Lq * H * d, "bf16").reshape(C, Lq, H, d)
    k_np = synth.draw(120 + d, 4, rows * H * d, "bf16").reshape(rows, H, d)
    v_np = synth.draw(120 + d, 5, rows * H * d, "bf16").reshape(rows, H, d)
    q, k, v = up(q_np), up(k_np), up(v_np)
    note("dca varlen ragged d=%d: all requests" % d)
    out = ikbo.ikbo_dca_forward(q, k, v, num_req=R, req_cand_offsets=up(off), kv_cu_seqlens=up(cu_np),
                                  kv_len=int(lens.max()), out=nan_out(C, Lq, H, d))
    torch.cuda.synchronize()
    assert not torch.isnan(out).any()
    note("dca varlen ragged d=%d: per request" % d)
    for r in range(R):
        c0, c1, l0, l1 = int(off[r]), int(off[r + 1]), int(cu_np[r]), int(cu_np[r + 1])
        if c1 == c0:
            continue
        if l1 == l0:
            # no keys: the documented zero rows
            assert torch.equal(out[c0:c1], torch.zeros_like(out[c0:c1])), r
            continue
        alone = ikbo.ikbo_dca_forward(q[c0:c1], k[l0:l1].reshape(1, l1 - l0, H, d), v[l0:l1].reshape(1, l1 - l0, H, d),
                                      num_req=1, req_cand_offsets=up(np.array([0, c1 - c0], np.int32)),
                                      kv_len=l1 - l0, out=nan_out(c1 - c0, Lq, H, d))
        torch.cuda.synchronize()
        assert same_bits(out[c0:c1], alone), r
    want = oracle.dca(q_np, k_np, v_np, R, off=off, kv_cu=cu_np)
    assert_parity(down_f64(out), want, "bf16", "ragged varlen DCA")


def test_varlen_long_and_short_requests():
    """Several thousand tiles of very different lengths (4096 and 256 keys, interleaved):
    bit-equal to the uniform-length launches of the two halves."""
    R, H, d, Lq = 64, 8, 64, 1
    counts = np.full(R, 300, np.int64)
    lens = np.where(np.arange(R) % 2 == 0, 4096, 256).astype(np.int64)
    C = int(counts.sum())
    off = synth.offsets_from_counts(counts)
    cu_np = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    rows = int(cu_np[-1])
    q = up(synth.draw(131, 1, C * Lq * H * d, "bf16").reshape(C, Lq, H, d))
    k = up(synth.draw(131, 2, rows * H * d, "bf16").reshape(rows, H, d))
    v = up(synth.draw(131, 3, rows * H * d, "bf16").reshape(rows, H, d))
    note("dca varlen long/short: varlen")
    out = ikbo.ikbo_dca_forward(q, k, v, num_req=R, req_cand_offsets=up(off), kv_cu_seqlens=up(cu_np),
                                  kv_len=4096, out=nan_out(C, Lq, H, d))
    torch.cuda.synchronize()
    assert not torch.isnan(out).any()
    note("dca varlen long/short: uniform halves")
    for parity, L in ((0, 4096), (1, 256)):
        reqs = np.arange(parity, R, 2)
        cand = torch.from_numpy(np.concatenate([np.arange(off[r], off[r + 1]) for r in reqs])).to("cuda")
        keys = torch.from_numpy(np.concatenate([np.arange(cu_np[r], cu_np[r + 1]) for r in reqs])).to("cuda")
        sub_off = up(synth.offsets_from_counts(counts[reqs]))
        plain = ikbo.ikbo_dca_forward(q[cand].contiguous(), k[keys].reshape(len(reqs), L, H, d),
                                      v[keys].reshape(len(reqs), L, H, d), num_req=len(reqs), req_cand_offsets=sub_off,
                                      out=nan_out(len(cand), Lq, H, d))
        torch.cuda.synchronize()
        assert same_bits(out[cand], plain), parity
