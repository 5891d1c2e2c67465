"""The seeded input generator: SplitMix64 stream values, normals, bf16 rounding, workload shapes."""
import numpy as np
import pytest

import synth

MASK = (1 << 64) - 1


def test_splitmix64_published_first_output():
    # SplitMix64 started from state 0 returns 0xE220A8397B1DCDAF first (Steele, Lea, Flood 2014;
    # the value every reference implementation prints for seed 0). Our stream key for a raw state
    # is the state itself, so check the mixer through a stream whose key we solve for: draw i of
    # key k is mix(k + (i+1)*golden); with k = 0, i = 0 this is the published first output.
    lib = synth._get()
    assert lib.synth_raw(0, 0) == 0xE220A8397B1DCDAF


def test_counter_based_slices_agree():
    full = synth.draw(7, 3, 1000, "f64")
    part = synth.draw(7, 3, 100, "f64", start=450)
    assert np.array_equal(full[450:550], part)


def test_normals_moments():
    x = synth.draw(11, 5, 1 << 20, "f64")
    assert abs(x.mean()) < 5e-3
    assert abs(x.std() - 1.0) < 5e-3
    # fraction beyond 2 sigma ~ 2 * (1 - Phi(2)) = 0.0455
    assert abs(np.mean(np.abs(x) > 2.0) - 0.0455) < 2e-3


def test_bf16_rounding_matches_numpy_rne():
    x32 = synth.draw(3, 9, 4096, "f32", scale=3.0)
    b = synth.draw(3, 9, 4096, "bf16", scale=3.0)
    assert np.array_equal(b, synth.f32_to_bf16_bits(x32))
    back = synth.bf16_to_f64(b)
    assert np.all(np.abs(back - x32) <= np.abs(x32) * 2.0 ** -8 + 1e-30)


def test_uniform_ints_in_range():
    v = synth.uniform_ints(0, 1, 10000, 8, 32)
    assert v.min() == 8 and v.max() == 32


@pytest.mark.parametrize("name", ["tiny", "dca_fixed", "dca_ragged", "block"])
def test_dca_specs(name):
    s = synth.dca_spec(name)
    assert s.C == int(s.counts.sum())
    off = s.offsets
    assert off[0] == 0 and off[-1] == s.C
    m = s.cand_to_req
    assert len(m) == s.C and np.all(np.diff(m) >= 0)
    if name == "dca_fixed":
        assert s.flops() == 2.0 ** 38
    if name == "block":
        assert s.flops() == 2.0 ** 45
    if name == "dca_ragged":
        assert s.varlen and s.counts.min() >= 16 and s.counts.max() <= 2048
        assert s.kv_lens.min() >= 256 and s.kv_lens.max() <= 4096


def test_glm_specs():
    g = synth.glm_spec("lcb")
    assert g.C == 524288 and g.R == 512
    assert g.flops() == 2.0 * 524288 * 1024 * 4096 + 2.0 * 512 * 2048 * 8192
