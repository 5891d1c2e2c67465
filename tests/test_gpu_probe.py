"""The ceiling probes (include/ikbo_probe.h) on the GPU: each runs, writes what its header says, and
the copy probe moves the bytes it claims to move."""
import pytest
import torch

import request_candidate_broadcast_amd as ikbo
from gpu_helpers import note

pytestmark = pytest.mark.gpu


def test_probes_run_and_write_their_outputs():
    dev = torch.device("cuda:0")
    blocks = 64
    out = torch.full((blocks * 256,), float("nan"), dtype=torch.float32, device=dev)
    note("probe mfma")
    ikbo.ikbo_probe_launch(ikbo.IKBO_PROBE_MFMA_BF16, out, 100, blocks)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and (out > 0).all()
    out.fill_(float("nan"))
    note("probe exp2")
    ikbo.ikbo_probe_launch(ikbo.IKBO_PROBE_EXP2, out, 100, blocks)
    torch.cuda.synchronize()
    # eight chains y <- 2^-y stay in [0.5, 1]: their sum in [4, 8]
    assert torch.isfinite(out).all() and (out >= 4).all() and (out <= 8).all()
    note("probe copy")
    buf = torch.arange(1 << 20, dtype=torch.int32, device=dev)          # 4 MiB: 2 MiB copied
    ikbo.ikbo_probe_launch(ikbo.IKBO_PROBE_COPY, buf, 0, blocks)
    torch.cuda.synchronize()
    half = buf.numel() // 2
    assert torch.equal(buf[half:], torch.arange(half, dtype=torch.int32, device=dev))
    note("probe read")
    src = torch.ones(1 << 20, dtype=torch.int32, device=dev)
    ikbo.ikbo_probe_launch(ikbo.IKBO_PROBE_READ, src, 0, blocks)
    torch.cuda.synchronize()
    # the last blocks * 256 words hold one xor of each thread's reads: ones xor'd in fours -> 0
    assert torch.count_nonzero(src[-blocks * 256:]).item() == 0
    for kind, name in ((ikbo.IKBO_PROBE_LDS_B128, "lds b128"), (ikbo.IKBO_PROBE_LDS_TR16, "lds tr16")):
        note("probe " + name)
        words = torch.full((blocks * 256,), -1, dtype=torch.int32, device=dev)
        ikbo.ikbo_probe_launch(kind, words, 10, blocks)
        torch.cuda.synchronize()
        # every read returns copies of the fill value; an even number of them xor to 0
        assert torch.count_nonzero(words).item() == 0
