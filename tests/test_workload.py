"""The seeded input generator: bf16 rounding and reproducibility (CPU)."""
import numpy as np
import torch

from workload import (WORKLOADS, bf16_bits_to_f32, make_inputs, normal_bf16,
                      round_to_bf16_bits)


def test_round_to_bf16_matches_torch_rne():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0 + 2**-8, 1.0 + 3 * 2**-8, -1.0 - 2**-8, 0.0, -0.0,
                                  3.0e38, 1e-40], dtype=np.float32)])
    ours = round_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_generator_is_deterministic_and_bf16_exact():
    a = normal_bf16((64, 32), 0.02, 77)
    b = normal_bf16((64, 32), 0.02, 77)
    assert np.array_equal(a, b)
    f = bf16_bits_to_f32(a)
    assert abs(float(np.std(f)) - 0.02) < 0.003
    assert np.array_equal(round_to_bf16_bits(f), a)


def test_llama_gate_half_is_scaled_by_8():
    w = WORKLOADS["llama"]
    small = w.__class__(**{**w.__dict__, "M": 4, "D": 64, "I": 32, "Dout": 64})
    x, W1, Wd, dy = make_inputs(small)
    plain = normal_bf16((64, 64), w.w1_std, 1234 + 1)
    assert np.array_equal(W1[:, :32], plain[:, :32])
    assert np.array_equal(bf16_bits_to_f32(W1[:, 32:]), bf16_bits_to_f32(plain[:, 32:]) * 8)


def test_workload_shapes():
    for name, w in WORKLOADS.items():
        assert w.D % 64 == 0 and w.I % 64 == 0 and w.Dout % 64 == 0, name


def test_moe_routing_counts_and_offsets():
    from workload import MOE_WORKLOADS, expert_counts, group_offsets, make_moe_inputs
    w = MOE_WORKLOADS["moe"]
    c = expert_counts(w.tokens, w.top_k, w.experts, w.skew)
    assert c.shape == (w.experts,) and c.sum() == w.M and np.all(c >= 0)
    assert np.array_equal(c, expert_counts(w.tokens, w.top_k, w.experts, w.skew))
    assert c.max() > 2 * c.min()                      # uneven: the grouped GEMM's case
    # each token picks distinct experts: no expert can hold more rows than tokens
    assert c.max() <= w.tokens
    off = group_offsets(c)
    assert off.dtype == np.int32 and off[0] == 0 and off[-1] == w.M and np.all(np.diff(off) == c)
    t = MOE_WORKLOADS["moe_tiny"]
    x, W1, Wd, dy, o = make_moe_inputs(t)
    assert x.shape == (t.M, t.D) and dy.shape == (t.M, t.Dout)
    assert W1.shape == (t.experts, t.D, 2 * t.I) and Wd.shape == (t.experts, t.I, t.Dout)
    assert o[-1] == t.M and len({W1[e].tobytes() for e in range(t.experts)}) == t.experts
    _, W1s, _, _, _ = make_moe_inputs(t, weight_sets=2)
    assert np.array_equal(W1s[0], W1s[2]) and not np.array_equal(W1s[0], W1s[1])
    assert np.array_equal(W1s[1], W1[1])
