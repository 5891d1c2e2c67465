"""The three IKBO-DCA work-tile shapes (8 waves x 32 rows, 4 waves, 1 wave) give the same bits for
the same query rows: each row's scores, softmax and sums do not depend on which rows share its
tile. The shape follows the average stacked query rows per request, so the same candidates are
run alone (few rows per request) and among filler candidates (many rows per request)."""
import numpy as np
import pytest
import torch

import oracle
import request_candidate_broadcast_amd as ikbo
import synth
from gpu_helpers import assert_parity, down_f64, note, up

pytestmark = pytest.mark.gpu


def run(q, k, v, counts, R, L, H, d):
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    out = ikbo.ikbo_dca_forward(up(q), up(k).view(R, L, H, d), up(v).view(R, L, H, d), num_req=R,
                                req_cand_offsets=up(off), out_dtype=torch.float32)
    torch.cuda.synchronize()
    return out, off


@pytest.mark.parametrize("d", [64, 128])
def test_tile_shapes_give_the_same_bits(d):
    R, L, H, Lq = 6, 300, 2, 1
    own, fill = 100, 1100                       # 100 rows per request: four waves; 1200: eight waves
    k = synth.draw(80 + d, 2, R * L * H * d, "bf16")
    v = synth.draw(80 + d, 3, R * L * H * d, "bf16")
    q_own = synth.draw(80 + d, 1, R * own * Lq * H * d, "bf16").reshape(R, own, Lq, H, d)
    q_fill = synth.draw(80 + d, 4, R * fill * Lq * H * d, "bf16").reshape(R, fill, Lq, H, d)
    note("dca modes d=%d: four waves" % d)
    a, off_a = run(np.ascontiguousarray(q_own.reshape(-1, Lq, H, d)), k, v, np.full(R, own), R, L, H, d)
    note("dca modes d=%d: eight waves" % d)
    qb = np.ascontiguousarray(np.concatenate([q_own, q_fill], axis=1).reshape(-1, Lq, H, d))
    b, _ = run(qb, k, v, np.full(R, own + fill), R, L, H, d)
    rows_b = np.concatenate([np.arange(r * (own + fill), r * (own + fill) + own) for r in range(R)])
    assert torch.equal(a.view(torch.int32), b[torch.from_numpy(rows_b).to(b.device)].view(torch.int32))
    note("dca modes d=%d: one wave" % d)
    few = 20                                     # 20 rows per request: one wave
    qc = np.ascontiguousarray(q_own[:, :few].reshape(-1, Lq, H, d))
    c, _ = run(qc, k, v, np.full(R, few), R, L, H, d)
    rows_a = np.concatenate([np.arange(r * own, r * own + few) for r in range(R)])
    assert torch.equal(c.view(torch.int32), a[torch.from_numpy(rows_a).to(a.device)].view(torch.int32))
    # and the four-wave run against the oracle
    want = oracle.dca(np.ascontiguousarray(q_own.reshape(-1, Lq, H, d)), k.reshape(R, L, H, d), v.reshape(R, L, H, d),
                      R, off=off_a)
    assert_parity(down_f64(a), want, "bf16", "four-wave tiles")
