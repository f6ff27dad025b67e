"""The seeded generator: determinism, bf16 rounding, length laws."""
import numpy as np
import torch

from variable_length_attention_jfa_amd import inputs as gen


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 3.0e38, -1e-40, 1.00390625, 1.01171875], dtype=np.float32)])
    ours = gen.bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(gen.bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_same_seed_same_bytes():
    wl = gen.small_workload(gen.WORKLOADS[3], B=5, lo=1, hi=300)
    a, b = gen.make_batch(wl), gen.make_batch(wl)
    for name in ("q_bits", "k_bits", "v_bits", "dout_bits", "q_offsets", "kv_offsets"):
        np.testing.assert_array_equal(getattr(a, name), getattr(b, name))
    c = gen.make_batch(wl, seed=wl.seed + 1)
    assert not np.array_equal(a.q_lengths, c.q_lengths) or not np.array_equal(a.q_bits, c.q_bits)


def test_workload_lengths_follow_their_laws():
    rng_lens = {}
    for i, wl in gen.WORKLOADS.items():
        rng = np.random.default_rng(wl.seed)
        lq = wl.q_len.sample(rng, wl.B)
        assert lq.min() >= wl.q_len.lo and lq.max() <= wl.q_len.hi
        rng_lens[i] = lq
    # cfg 2: uniform [1, 1024], mean ~ half the max (sparsity ~0.5)
    assert 350 < rng_lens[2].mean() < 650
    # cfg 3: lognormal(ln 1500, 0.6) clipped to [32, 4096]
    assert 1200 < rng_lens[3].mean() < 2200


def test_offsets_are_prefix_sums():
    lens = np.array([5, 0, 7], dtype=np.int64)
    np.testing.assert_array_equal(gen.offsets_from_lengths(lens), [0, 5, 5, 12])
