"""IKBO-DCA at the size limits of the bf16 path.

The K (and V) rows of one request are addressed through a 31-bit buffer range, so a request may
hold up to L_r * H * d * 2 < 2^31 bytes. These tests run the longest request that fits, checked
against a closed form (Q = 0 gives uniform weights, so O is the mean of V over the request's keys),
and one key more, which the library must turn into NaN rows (varlen with no length bound) or
reject (a length bound that exceeds the limit)."""
import pytest
import torch

import request_candidate_broadcast_amd as ikbo
from gpu_helpers import note

pytestmark = pytest.mark.gpu

H, D = 8, 128
L_MAX = (1 << 31) // (H * D * 2) - 1          # 1048575 keys: the last length below the limit


def _kv(L, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    k = torch.randn((L, H, D), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn((L, H, D), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    return k, v


def test_longest_request_that_fits_gives_the_mean_of_v():
    note("dca limit: one request of %d keys" % L_MAX)
    k, v = _kv(L_MAX, 11)
    C = 3
    q = torch.zeros((C, 1, H, D), dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, L_MAX], dtype=torch.int32, device="cuda")
    off = torch.tensor([0, C], dtype=torch.int32, device="cuda")
    out = ikbo.ikbo_dca_forward(q, k, v, kv_cu_seqlens=cu, req_cand_offsets=off, kv_len=L_MAX,
                                out_dtype=torch.float32)
    torch.cuda.synchronize()
    mean = torch.zeros((H, D), dtype=torch.float64, device="cuda")
    for s in range(0, L_MAX, 1 << 18):
        mean += v[s:s + (1 << 18)].double().sum(dim=0)
    mean /= L_MAX
    for c in range(C):
        err = (out[c, 0].double() - mean).abs().max().item()
        assert err < 1e-5, "candidate %d: max |O - mean(V)| = %g" % (c, err)


def test_one_key_past_the_limit():
    L = L_MAX + 1
    note("dca limit: one request of %d keys" % L)
    k, v = _kv(L, 12)
    q = torch.zeros((2, 1, H, D), dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, L], dtype=torch.int32, device="cuda")
    off = torch.tensor([0, 2], dtype=torch.int32, device="cuda")
    # a length bound past the limit is rejected before any launch
    with pytest.raises(RuntimeError, match="2\\^31"):
        ikbo.ikbo_dca_forward(q, k, v, kv_cu_seqlens=cu, req_cand_offsets=off, kv_len=L, out_dtype=torch.float32)
    # with no bound the kernel meets the request and writes NaN rows
    out = ikbo.ikbo_dca_forward(q, k, v, kv_cu_seqlens=cu, req_cand_offsets=off, kv_len=0, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
