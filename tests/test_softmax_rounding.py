"""Why the DCA kernels scale scores in fp32: a CPU emulation of the two ways to reach the exp2
argument, on one query block with a hot key (every element of one key and of one query equal
to `hot`), against the fp64 softmax. Both forms use the kernels' other roundings (bf16 inputs,
fp32 scores, weights rounded to bf16 before the PV product, the row sum over those rounded
weights):
  fma  : s = fp32(q . k), p = bf16(2^(s * scale * log2(e) - m))
  fold : q' = bf16(q * scale * log2(e)), s = fp32(q' . k), p = bf16(2^(s - m))
The fold saves one VALU instruction per score but rounds every score by up to 2^-9 of its size;
a key several times larger than the rest turns that into output errors past the bf16 bar
(max-abs 2e-2), while the fp32 form stays far inside it. Host-only numerics, no GPU."""
import numpy as np
import pytest

BF16_MAX = 2e-2


def bf16(x):
    """Round fp32 values to bf16 (nearest even), returned as fp32."""
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def max_error(d, hot, seed, form, C=300, L=200):
    rng = np.random.default_rng(seed)
    q = bf16(rng.standard_normal((C, d)))
    k = bf16(rng.standard_normal((L, d)))
    v = bf16(rng.standard_normal((L, d)))
    q[5] = hot
    k[150] = hot
    scale = 1.0 / np.sqrt(d)
    s64 = (q.astype(np.float64) @ k.T.astype(np.float64)) * scale
    w = np.exp(s64 - s64.max(1, keepdims=True))
    ref = (w @ v.astype(np.float64)) / w.sum(1, keepdims=True)
    cl2 = np.float32(scale * 1.4426950408889634)
    if form == "fold":
        s = (bf16(q * cl2) @ k.T).astype(np.float32)
    else:
        s = (q @ k.T).astype(np.float32) * cl2
    p = bf16(np.exp2((s - s.max(1, keepdims=True)).astype(np.float32)))
    out = (p @ v) / p.sum(1, keepdims=True)
    return float(np.abs(out - ref).max())


@pytest.mark.parametrize("d", [64, 128])
def test_fp32_scaling_stays_inside_the_bar_and_folding_does_not(d):
    fma = max(max_error(d, hot, seed, "fma") for hot in (6.0, 8.0, 10.0, 12.0) for seed in range(4))
    fold = max(max_error(d, hot, seed, "fold") for hot in (6.0, 8.0, 10.0, 12.0) for seed in range(4))
    assert fma < BF16_MAX / 10, fma
    assert fold > BF16_MAX, fold
