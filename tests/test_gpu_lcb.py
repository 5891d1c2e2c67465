"""GPU parity of IKBO-LCB and the GLM-MLP (through the C ABI) against the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
import request_candidate_broadcast_amd as ikbo
import synth
from gpu_helpers import assert_parity, bf16_bits, down_f64, note, rne_bits_of, up

pytestmark = pytest.mark.gpu


def make_layer(seed, k_req, k_cand, n_req, n_cand, dtype, act, base=50):
    kind = "bf16" if dtype == "bf16" else "f32"
    return {
        "w_rr": synth.draw(seed, base, n_req * k_req, kind, 1 / math.sqrt(k_req)).reshape(n_req, k_req),
        "w_cr": synth.draw(seed, base + 1, n_cand * k_req, kind, 1 / math.sqrt(k_req)).reshape(n_cand, k_req),
        "w_cc": synth.draw(seed, base + 2, n_cand * k_cand, kind, 1 / math.sqrt(k_cand)).reshape(n_cand, k_cand),
        "b_r": synth.draw(seed, base + 3, n_req, "f32", 1 / math.sqrt(k_req)),
        "b_c": synth.draw(seed, base + 4, n_cand, "f32", 1 / math.sqrt(k_cand)),
        "act": act,
    }


def dev_layer(ly):
    return {k: (up(v) if isinstance(v, np.ndarray) else v) for k, v in ly.items()}


def make_x(seed, R, C, k_req, k_cand, dtype):
    kind = "bf16" if dtype == "bf16" else "f32"
    return (synth.draw(seed, 60, R * k_req, kind).reshape(R, k_req),
            synth.draw(seed, 61, C * k_cand, kind).reshape(C, k_cand))


def run_lcb(x_r, x_c, ly, *, m=None, off=None, out_dtype=torch.float32, want_req=True):
    d = dev_layer(ly)
    kw = {}
    if m is not None:
        kw["cand_to_req"] = up(m)
    if off is not None:
        kw["req_cand_offsets"] = up(off)
    y_r, y_c = ikbo.ikbo_lcb_forward(up(x_r), up(x_c), d["w_rr"], d["w_cr"], d["w_cc"], b_r=d["b_r"], b_c=d["b_c"],
                                     activation=ly["act"], out_dtype=out_dtype, want_request_output=want_req, **kw)
    torch.cuda.synchronize()
    return y_r, y_c


def test_tiny_fp32_workload():
    g = synth.glm_spec("tiny")
    x_r, x_c = synth.glm_x(g, "x_r"), synth.glm_x(g, "x_c")
    ly = dict(synth.glm_weights(g, 0), act="none")
    note("lcb tiny fp32")
    y_r, y_c = run_lcb(x_r, x_c, ly, off=g.offsets)
    want = oracle.glm(x_r, x_c, [ly], off=g.offsets, want_request=True)
    assert_parity(down_f64(y_c), want["y_c"], "f32", "y_c")
    assert_parity(down_f64(y_r), want["y_r"], "f32", "y_r")


@pytest.mark.parametrize("act", ["gelu", "none"])
# (k_req, k_cand, n_req, n_cand): k tails, tiny K, long split-K request GEMM, and with K a
# multiple of 64 (direct LDS copies) ragged N over several column tiles; N = 300 has a whole
# column tile with bf16 rows of 600 bytes (direct stores) and fp32 rows of 1200 (staged stores)
@pytest.mark.parametrize("shape", [(136, 264, 72, 200), (64, 8, 40, 203), (4096, 512, 256, 256),
                                   (128, 192, 256, 200), (64, 256, 520, 1000), (64, 128, 40, 300)])
def test_bf16_ragged_shapes(act, shape):
    k_req, k_cand, n_req, n_cand = shape
    counts = np.array([1, 300, 0, 77, 513, 2, 40])
    R, C = len(counts), int(counts.sum())
    x_r, x_c = make_x(7, R, C, k_req, k_cand, "bf16")
    ly = make_layer(7, k_req, k_cand, n_req, n_cand, "bf16", act)
    m = synth.cand_to_req_from_counts(counts)
    note("lcb bf16 shape=%s act=%s" % (shape, act))
    y_r, y_c = run_lcb(x_r, x_c, ly, m=m)
    want = oracle.glm(x_r, x_c, [ly], m=m, want_request=True)
    assert_parity(down_f64(y_c), want["y_c"], "bf16", "y_c")
    assert_parity(down_f64(y_r), want["y_r"], "bf16", "y_r")
    y_r16, y_c16 = run_lcb(x_r, x_c, ly, m=m, out_dtype=torch.bfloat16)
    assert np.array_equal(bf16_bits(y_c16), rne_bits_of(y_c))
    assert np.array_equal(bf16_bits(y_r16), rne_bits_of(y_r))


def test_index_paths_and_invalid_rows():
    counts = np.array([3, 0, 290, 9])
    R, C = 4, int(counts.sum())
    x_r, x_c = make_x(8, R, C, 64, 128, "bf16")
    ly = make_layer(8, 64, 128, 32, 96, "bf16", "gelu")
    m = synth.cand_to_req_from_counts(counts)
    off = synth.offsets_from_counts(counts)
    note("lcb index paths")
    _, a = run_lcb(x_r, x_c, ly, m=m)
    _, b = run_lcb(x_r, x_c, ly, off=off)
    _, c = run_lcb(x_r, x_c, ly, m=m, off=off)
    assert torch.equal(a, b) and torch.equal(a, c)
    # unsorted map: rows depend only on their own request
    rng = np.random.default_rng(1)
    perm = rng.permutation(C)
    _, d = run_lcb(x_r, x_c[perm], ly, m=m[perm])
    assert torch.equal(d, a[torch.from_numpy(perm).to(a.device)])
    bad = m.copy()
    bad[[0, 100, C - 1]] = [-2, 4, 1000]
    _, e = run_lcb(x_r, x_c, ly, m=bad)
    for c_ in (0, 100, C - 1):
        assert torch.all(e[c_] == 0)
    want = oracle.glm(x_r, x_c, [ly], m=bad)
    assert_parity(down_f64(e), want["y_c"], "bf16", "invalid rows")


def test_glm_invariance_and_zero_blocks_bitwise():
    counts = np.array([100, 160, 4])
    R, C = 3, int(counts.sum())
    x_r, x_c = make_x(9, R, C, 128, 64, "bf16")
    ly = make_layer(9, 128, 64, 64, 64, "bf16", "gelu")
    m = synth.cand_to_req_from_counts(counts)
    note("lcb invariance")
    y_r, y_c = run_lcb(x_r, x_c, ly, m=m)
    x_c2 = synth.draw(99, 61, C * 64, "bf16").reshape(C, 64)
    y_r2, y_c2 = run_lcb(x_r, x_c2, ly, m=m)
    assert torch.equal(y_r, y_r2)                      # P11: request outputs ignore candidates
    assert not torch.equal(y_c, y_c2)
    ly0 = dict(ly, w_cc=np.zeros_like(ly["w_cc"]))
    _, y0 = run_lcb(x_r, x_c, ly0, m=m)                 # P13: W_CC = 0 -> rows equal within a request
    off = synth.offsets_from_counts(counts)
    for r in range(R):
        blk = y0[off[r]:off[r + 1]]
        assert torch.equal(blk, blk[:1].expand_as(blk))


def test_request_tag_bitwise():
    # P14: x_r[r] = r e0, W_CR = e0 e0^T, W_CC = 0, b = 0, no activation -> y_c[c, 0] == m[c]
    R, K, N = 6, 64, 32
    counts = np.array([2, 300, 1, 0, 50, 9])
    C = int(counts.sum())
    x_r = np.zeros((R, K), np.float32)
    x_r[:, 0] = np.arange(R)
    x_c = synth.draw(10, 61, C * K, "f32").reshape(C, K)
    w_cr = np.zeros((N, K), np.float32)
    w_cr[0, 0] = 1.0
    ly = {"w_rr": synth.draw(10, 1, N * K, "f32").reshape(N, K), "w_cr": w_cr, "w_cc": np.zeros((N, K), np.float32),
          "b_r": None, "b_c": None, "act": "none"}
    b16 = {k: (synth.f32_to_bf16_bits(v) if isinstance(v, np.ndarray) else v) for k, v in ly.items()}
    m = synth.cand_to_req_from_counts(counts)
    note("lcb request tag")
    _, y_c = run_lcb(synth.f32_to_bf16_bits(x_r), synth.f32_to_bf16_bits(x_c), b16, m=m)
    got = down_f64(y_c)
    assert np.array_equal(got[:, 0], m.astype(np.float64)) and np.all(got[:, 1:] == 0)


def test_no_request_output_and_empty():
    counts = np.array([0, 0])
    x_r, x_c = make_x(11, 2, 0, 64, 64, "bf16")
    ly = make_layer(11, 64, 64, 32, 32, "bf16", "gelu")
    note("lcb empty candidates")
    y_r, y_c = run_lcb(x_r, x_c, ly, m=np.zeros(0, np.int32))
    assert y_c.shape == (0, 32)
    want = oracle.glm(x_r, np.zeros((0, 64), np.uint16), [ly], m=np.zeros(0, np.int32), want_request=True)
    assert_parity(down_f64(y_r), want["y_r"], "bf16", "y_r only")
    counts = np.array([5, 9])
    x_r, x_c = make_x(12, 2, 14, 64, 64, "bf16")
    m = synth.cand_to_req_from_counts(counts)
    yr, yc = run_lcb(x_r, x_c, ly, m=m, want_req=False)
    assert yr is None
    assert_parity(down_f64(yc), oracle.glm(x_r, x_c, [ly], m=m)["y_c"], "bf16", "no y_r")


# ------------------------------------------------------------------------------------------------
def run_mlp(x_r, x_c, layers, *, m=None, off=None, out_dtype=torch.float32):
    kw = {}
    if m is not None:
        kw["cand_to_req"] = up(m)
    if off is not None:
        kw["req_cand_offsets"] = up(off)
    y_r, y_c = ikbo.ikbo_glm_mlp_forward(up(x_r), up(x_c), [dev_layer(l) for l in layers], out_dtype=out_dtype, **kw)
    torch.cuda.synchronize()
    return y_r, y_c


def test_mlp_fp32_exact_path():
    counts = np.array([3, 20, 1])
    R, C = 3, 24
    x_r, x_c = make_x(13, R, C, 32, 16, "f32")
    l1 = make_layer(13, 32, 16, 24, 20, "f32", "gelu", base=20)
    l2 = make_layer(13, 24, 20, 12, 8, "f32", "none", base=30)
    m = synth.cand_to_req_from_counts(counts)
    note("mlp fp32")
    y_r, y_c = run_mlp(x_r, x_c, [l1, l2], m=m)
    want = oracle.glm(x_r, x_c, [l1, l2], m=m, want_request=True)
    assert_parity(down_f64(y_c), want["y_c"], "f32", "mlp y_c")
    assert_parity(down_f64(y_r), want["y_r"], "f32", "mlp y_r")


def test_mlp_bf16_three_layers_and_closure():
    counts = np.array([70, 1, 300])
    R, C = 3, 371
    x_r, x_c = make_x(14, R, C, 256, 128, "bf16")
    layers = [make_layer(14, 256, 128, 128, 136, "bf16", "gelu", base=20),
              make_layer(14, 128, 136, 64, 64, "bf16", "gelu", base=30),
              make_layer(14, 64, 64, 48, 256, "bf16", "none", base=40)]
    m = synth.cand_to_req_from_counts(counts)
    note("mlp bf16 3 layers")
    y_r, y_c = run_mlp(x_r, x_c, layers, m=m)
    want = oracle.glm(x_r, x_c, layers, m=m, want_request=True)
    assert_parity(down_f64(y_c), want["y_c"], "bf16", "mlp y_c")
    assert_parity(down_f64(y_r), want["y_r"], "bf16", "mlp y_r")
    # P17: the request path of the stack ignores candidate inputs, bit for bit
    x_c2 = synth.draw(77, 61, C * 128, "bf16").reshape(C, 128)
    y_r2, _ = run_mlp(x_r, x_c2, layers, m=m)
    assert torch.equal(y_r, y_r2)
    y_r16, y_c16 = run_mlp(x_r, x_c, layers, m=m, out_dtype=torch.bfloat16)
    assert np.array_equal(bf16_bits(y_c16), rne_bits_of(y_c))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("ks", [(100, 262), (262, 1001), (1001, 100), (7, 3)])
def test_misaligned_k_widths(dtype, ks):
    # B5, the alignment rule (Sec. 4.2.4): K widths that break 16-byte rows are zero-padded inside
    # the call (bf16) or read element by element (fp32); the results meet the same bars
    k_req, k_cand = ks
    counts = np.array([2, 130, 0, 41])
    R, C = len(counts), int(counts.sum())
    x_r, x_c = make_x(15, R, C, k_req, k_cand, dtype)
    ly = make_layer(15, k_req, k_cand, 72, 200, dtype, "gelu")
    m = synth.cand_to_req_from_counts(counts)
    note("lcb misaligned k=%s %s" % (ks, dtype))
    y_r, y_c = run_lcb(x_r, x_c, ly, m=m)
    want = oracle.glm(x_r, x_c, [ly], m=m, want_request=True)
    assert_parity(down_f64(y_c), want["y_c"], dtype, "y_c")
    assert_parity(down_f64(y_r), want["y_r"], dtype, "y_r")
    if dtype == "bf16":
        y_r16, y_c16 = run_lcb(x_r, x_c, ly, m=m, out_dtype=torch.bfloat16)
        assert np.array_equal(bf16_bits(y_c16), rne_bits_of(y_c))
        assert np.array_equal(bf16_bits(y_r16), rne_bits_of(y_r))


def test_mlp_misaligned_input_and_hidden_widths():
    # every layer pads its own misaligned inputs, hidden widths included
    counts = np.array([3, 200, 5])
    R, C = 3, 208
    x_r, x_c = make_x(16, R, C, 100, 262, "bf16")
    layers = [make_layer(16, 100, 262, 44, 52, "bf16", "gelu", base=20),
              make_layer(16, 44, 52, 36, 30, "bf16", "none", base=30)]
    m = synth.cand_to_req_from_counts(counts)
    note("mlp bf16 misaligned widths")
    y_r, y_c = run_mlp(x_r, x_c, layers, m=m)
    want = oracle.glm(x_r, x_c, layers, m=m, want_request=True)
    assert_parity(down_f64(y_c), want["y_c"], "bf16", "mlp y_c")
    assert_parity(down_f64(y_r), want["y_r"], "bf16", "mlp y_r")
    y_r16, y_c16 = run_mlp(x_r, x_c, layers, m=m, out_dtype=torch.bfloat16)
    assert np.array_equal(bf16_bits(y_c16), rne_bits_of(y_c))
