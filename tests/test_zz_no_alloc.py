"""IKBO-DCA without allocation (ikbo_dca_forward_noalloc), called through the C ABI: its outputs
equal ikbo_dca_forward's bit for bit on two calls in a row, the second smaller, so that it runs on
what the first left in the shared scratch array; both with a map that needs the device grouping
(the most scratch) and with offsets; and a call needing more scratch than the fixed array is
refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import request_candidate_broadcast_amd as ikbo
import synth
from gpu_helpers import note, up

pytestmark = pytest.mark.gpu


def ptr(t):
    return None if t is None else t.data_ptr()


def code(t):
    return ikbo.IKBO_BF16 if t.dtype == torch.bfloat16 else ikbo.IKBO_F32


def noalloc(q, k, v, R, out, *, m=None, off=None, kv_cu=None, L=0):
    lib = ikbo.load_library()
    C, Lq, H, d = q.shape
    return lib.ikbo_dca_forward_noalloc(ptr(q), C, Lq, ptr(k), ptr(v), R, ptr(kv_cu), L, ptr(m), ptr(off), 0, H, d, 0.0,
                                        code(q), code(out), ptr(out), torch.cuda.current_stream().cuda_stream)


def inputs(seed, counts, lens, H, d, Lq, varlen):
    s = synth.custom_dca_spec(seed, counts, lens, H, d, Lq, dtype="bf16", varlen=varlen)
    q, k, v = up(synth.dca_q(s)), up(synth.dca_kv(s, "k")), up(synth.dca_kv(s, "v"))
    if not varlen:
        k, v = k.view(s.R, s.L, s.H, s.d), v.view(s.R, s.L, s.H, s.d)
    rng = np.random.default_rng(seed)
    perm = rng.permutation(s.C)
    m = s.cand_to_req[perm].copy()               # an ungrouped map: candidates shuffled
    if s.C > 3:
        m[[1, s.C - 2]] = [-1, s.R + 4]          # and two rows with no valid request
    return s, q[torch.from_numpy(perm).to(q.device)].contiguous(), k, v, m


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_noalloc_equals_the_workspace_entry_point(out_dtype):
    cases = [(80, [40, 300, 0, 129, 7, 513, 2, 64, 90], [200, 70, 33, 300, 1, 129, 64, 500, 8], 2, 128, 4, True),
             (81, [9, 30, 3], [65, 65, 65], 2, 64, 1, False)]           # the second call is smaller
    for seed, counts, lens, H, d, Lq, varlen in cases:
        s, q, k, v, m = inputs(seed, counts, lens, H, d, Lq, varlen)
        kv_cu = up(s.kv_cu) if varlen else None
        L = 0 if varlen else s.L
        for form in ("map", "offsets"):
            note("dca noalloc seed=%d C=%d form=%s out=%s" % (seed, s.C, form, out_dtype))
            idx = dict(m=up(m)) if form == "map" else dict(off=up(s.offsets))
            qq = q if form == "map" else up(synth.dca_q(s))
            got = torch.full((s.C, Lq, H, d), 5.0, dtype=out_dtype, device="cuda:0")
            st = noalloc(qq, k, v, s.R, got, kv_cu=kv_cu, L=L, **idx)
            assert st == ikbo.IKBO_OK, ikbo.load_library().ikbo_last_error_message()
            kw = dict(cand_to_req=idx["m"]) if form == "map" else dict(req_cand_offsets=idx["off"])
            want = ikbo.ikbo_dca_forward(qq, k, v, num_req=s.R, kv_cu_seqlens=kv_cu, kv_len=L, out_dtype=out_dtype, **kw)
            torch.cuda.synchronize()
            assert torch.equal(got.view(torch.int16) if out_dtype == torch.bfloat16 else got,
                               want.view(torch.int16) if out_dtype == torch.bfloat16 else want)


def test_noalloc_refuses_sizes_beyond_its_scratch():
    lib = ikbo.load_library()
    C, R = 2 << 20, 1                                   # about 40 MiB of scratch: above the array
    assert lib.ikbo_dca_workspace_size(C, R) > ikbo.IKBO_DCA_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((C, 1, 1, 64), dtype=torch.bfloat16, device="cuda:0")
    k = torch.zeros((R, 1, 1, 64), dtype=torch.bfloat16, device="cuda:0")
    m = torch.zeros(C, dtype=torch.int32, device="cuda:0")
    out = torch.full((C, 1, 1, 64), 3.0, dtype=torch.bfloat16, device="cuda:0")
    note("dca noalloc size refused")
    st = noalloc(q, k, k, R, out, m=m, L=1)
    assert st == ikbo.IKBO_WORKSPACE_TOO_SMALL
    assert b"fixed" in lib.ikbo_last_error_message()
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
