"""The entry points inside a captured HIP graph. The library enqueues only kernels (counters and
scratch are cleared by fill kernels, never by memset nodes), so a call captured once replays like
the eager call: every replay is checked bit for bit against an eager call on the same inputs, with
eager work and synchronisations between the replays, and with new input values written into the
captured buffers between replays (the graph reads its inputs at replay time)."""
import numpy as np
import pytest
import torch

import request_candidate_broadcast_amd as ikbo
import synth
from gpu_helpers import note, up

pytestmark = pytest.mark.gpu


def same_bits(a, b):
    return torch.equal(a.view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32),
                       b.view(torch.int16 if b.dtype == torch.bfloat16 else torch.int32))


def eager_noise():
    # unrelated eager work between replays (allocations, a matmul, a reduction), then a sync
    a = torch.randn(512, 512, device="cuda")
    (a @ a).sum().item()
    torch.cuda.synchronize()


def capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                                # warm-up outside the capture (first-call set-up)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("form", ["offsets", "map"])
def test_dca_noalloc_replays_like_eager_calls(form):
    counts, lens, H, d, Lq = [40, 300, 0, 129, 7, 513], [200, 70, 33, 300, 1, 129], 2, 128, 2
    s = synth.custom_dca_spec(140, counts, lens, H, d, Lq, dtype="bf16", varlen=True)
    q = up(synth.dca_q(s))
    k, v = up(synth.dca_kv(s, "k")), up(synth.dca_kv(s, "v"))
    kv_cu = up(s.kv_cu)
    m = up(np.random.default_rng(140).permutation(s.cand_to_req).astype(np.int32))   # ungrouped map
    off = up(s.offsets)
    out = torch.full((s.C, Lq, H, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lib = ikbo.load_library()

    def call():
        st = lib.ikbo_dca_forward_noalloc(q.data_ptr(), s.C, Lq, k.data_ptr(), v.data_ptr(), s.R, kv_cu.data_ptr(), 0,
                                          m.data_ptr() if form == "map" else None,
                                          off.data_ptr() if form == "offsets" else None, 0, H, d, 0.0, ikbo.IKBO_BF16,
                                          ikbo.IKBO_BF16, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert st == ikbo.IKBO_OK, lib.ikbo_last_error_message()

    def eager():
        kw = dict(cand_to_req=m) if form == "map" else dict(req_cand_offsets=off)
        r = ikbo.ikbo_dca_forward(q, k, v, num_req=s.R, kv_cu_seqlens=kv_cu, **kw)
        torch.cuda.synchronize()
        return r

    note("dca graph capture (%s)" % form)
    g = capture(call)
    for rep in range(4):
        if rep == 2:
            # new query values in the captured buffer
            q.copy_(up(synth.draw(141, 1, s.C * Lq * H * d, "bf16").reshape(s.C, Lq, H, d)))
            torch.cuda.synchronize()
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = eager()
        assert same_bits(out, want), rep
        eager_noise()


def test_lcb_replays_like_eager_calls():
    R, C, kr, kc, n = 8, 2000, 512, 256, 256
    counts = synth.uniform_ints(142, 1, R, 100, 400)
    counts[-1] = C - counts[:-1].sum()
    off = up(synth.offsets_from_counts(counts))
    x_r = up(synth.draw(142, 2, R * kr, "bf16").reshape(R, kr))
    x_c = up(synth.draw(142, 3, C * kc, "bf16").reshape(C, kc))
    w_rr = up(synth.draw(142, 4, n * kr, "bf16", 1 / np.sqrt(kr)).reshape(n, kr))
    w_cr = up(synth.draw(142, 5, n * kr, "bf16", 1 / np.sqrt(kr)).reshape(n, kr))
    w_cc = up(synth.draw(142, 6, n * kc, "bf16", 1 / np.sqrt(kc)).reshape(n, kc))
    b_r = up(synth.draw(142, 7, n, "f32", 1 / np.sqrt(kr)))
    b_c = up(synth.draw(142, 8, n, "f32", 1 / np.sqrt(kc)))
    ws = torch.empty(max(1, ikbo.ikbo_lcb_workspace_size(C, R, kr, kc, n, n)), dtype=torch.uint8,
                     device="cuda")
    y_r = torch.empty((R, n), dtype=torch.bfloat16, device="cuda")
    y_c = torch.empty((C, n), dtype=torch.bfloat16, device="cuda")
    args = (x_r, x_c, w_rr, w_cr, w_cc)
    kw = dict(b_r=b_r, b_c=b_c, req_cand_offsets=off, activation="gelu")

    def call():
        ikbo.ikbo_lcb_forward(*args, **kw, y_req=y_r, y_cand=y_c, workspace=ws)

    def eager():
        r = ikbo.ikbo_lcb_forward(*args, **kw)
        torch.cuda.synchronize()
        return r

    note("lcb graph capture")
    g = capture(call)
    for rep in range(4):
        if rep == 2:
            x_c.copy_(up(synth.draw(143, 3, C * kc, "bf16").reshape(C, kc)))
            torch.cuda.synchronize()
        y_r.fill_(float("nan"))
        y_c.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want_r, want_c = eager()
        assert same_bits(y_r, want_r) and same_bits(y_c, want_c), rep
        eager_noise()
