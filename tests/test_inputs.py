"""The seeded input generators (host only): storage rounding and workload recipes."""
import numpy as np
import pytest

from linear_attention_chunked_gdn_amd import inputs


def test_round_to_bf16_is_nearest_even():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: ties go to the even mantissa (1.0);
    # 1 + 3*2^-8 ties between 1 + 2^-7 and 1 + 2^-6 and goes up
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1e-30], np.float32)
    r = inputs.round_to_bf16(x)
    assert r.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, -2.5, r[4]]
    assert np.all(inputs.bf16_bits(r).astype(np.uint32) << 16 == r.view(np.uint32))


def test_round_to_f16_is_exact_in_f16_and_nearest():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(10000).astype(np.float32) * np.float32(30.0)
    r = inputs.round_to_f16(x)
    assert np.array_equal(r.astype(np.float16).astype(np.float32), r)
    # nearest: the error is at most half a unit in the last place (2^-11 relative)
    assert np.all(np.abs(r.astype(np.float64) - x) <= np.abs(x.astype(np.float64)) * 2.0 ** -11 + 2.0 ** -25)
    with pytest.raises(ValueError):
        inputs.round_to_f16(np.array([70000.0], np.float32))


@pytest.mark.parametrize("io", ["f16", "f32"])
def test_workload_io_override_keeps_draws(io):
    a = inputs.make_workload(0)
    b = inputs.make_workload(0, io=io)
    assert b.io == io and a.cu_seqlens.tolist() == b.cu_seqlens.tolist()
    # same draws, only rounded differently; g and beta are fp32 in every case
    assert np.array_equal(a.g, b.g) and np.array_equal(a.beta, b.beta)
    assert np.max(np.abs(a.q - b.q)) <= 2.0 ** -11
    if io == "f16":
        assert "f16" in b.name
        assert np.array_equal(b.v.astype(np.float16).astype(np.float32), b.v)


def test_head_shard_keeps_the_key_head_of_every_value_head():
    # one GPU's share of a GQA batch: key heads [0, Hk / G) and the value heads reading them,
    # renumbered so that value head h' reads key head h' % (Hk / G)
    x = inputs.make_custom(3, [40, 0, 25], 4, 8, io="bf16", init_std=0.1)
    y = inputs.head_shard(x, 2)
    assert (y.Hk, y.Hv, y.N, y.T_tot) == (2, 4, 3, 65)
    picked = [0, 1, 4, 5]   # value heads j + 4 m for j < 2, m < 2
    for hp, h in enumerate(picked):
        assert np.array_equal(y.v[:, hp], x.v[:, h]) and np.array_equal(y.g[:, hp], x.g[:, h])
        assert np.array_equal(y.beta[:, hp], x.beta[:, h])
        assert np.array_equal(y.initial_state[:, hp], x.initial_state[:, h])
        assert np.array_equal(y.k[:, hp % y.Hk], x.k[:, h % x.Hk])
        assert np.array_equal(y.q[:, hp % y.Hk], x.q[:, h % x.Hk])
    assert inputs.head_shard(x, 1) is x
    with pytest.raises(ValueError):
        inputs.head_shard(x, 3)
