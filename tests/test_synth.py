"""The seeded input generators: deterministic bits, one rounding to bf16, and
the planted structure the recipe states (CPU only)."""
import math

import torch

import stem_synth as S


def test_same_seed_same_bits_other_seed_other_bits():
    a = S.make_qkv([256, 384], 4, 2, seed=11)
    b = S.make_qkv([256, 384], 4, 2, seed=11)
    c = S.make_qkv([256, 384], 4, 2, seed=12)
    for x, y, z in zip(a, b, c):
        assert x.dtype == torch.bfloat16 and x.is_contiguous()
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
        assert not torch.equal(x, z)
    t1 = S.make_topic_qkv([512], 4, 2, seed=3)
    t2 = S.make_topic_qkv([512], 4, 2, seed=3)
    assert all(torch.equal(x, y) for x, y in zip(t1, t2))


def test_bf16_is_one_rounding_of_the_fp32_draw():
    f32 = S.make_qkv([512], 4, 2, seed=5, dtype=torch.float32)
    b16 = S.make_qkv([512], 4, 2, seed=5, dtype=torch.bfloat16)
    for x, y in zip(f32, b16):
        assert torch.equal(x.to(torch.bfloat16), y)


def test_sink_keys_and_lognormal_value_rows():
    T, Hkv, d = 4096, 2, 128
    _, k, v = S.make_qkv([T], 4, Hkv, seed=9, dtype=torch.float32)
    kf = k.double()
    for g in range(Hkv):
        # +3 along one unit direction on the first 256 keys; elsewhere mean ~ 0
        assert 2.5 < float(kf[:256, g].mean(0).norm()) < 3.5
        assert float(kf[256:512, g].mean(0).norm()) < 1.5
    # |V_t| = r_t |z_t| with log r ~ N(0, 0.5) and |z_t| ~ sqrt(d)
    logn = torch.log(v.double().norm(dim=-1) / math.sqrt(d))
    assert abs(float(logn.std()) - 0.5) < 0.05 and abs(float(logn.mean())) < 0.05
    _, k0, _ = S.make_qkv([T], 4, Hkv, seed=9, sink=False, dtype=torch.float32)
    assert float(k0.double()[:256, 0].mean(0).norm()) < 1.5


def test_topic_draw_attends_to_its_planted_block():
    """Queries of a block score their planted key block's topic far above the rest."""
    q, k, _ = S.make_topic_qkv([2048], 2, 1, seed=4, topics=8, gain=6.0)
    qb = q[128 * 10:128 * 11, 0].mean(0)
    scores = torch.stack([k[128 * J:128 * (J + 1), 0].mean(0) @ qb for J in range(11)])
    assert float(scores.max() - scores.median()) > 20.0       # ~ gain^2 = 36 for a match


def test_workload_tables_are_consistent():
    for w in list(S.CONFIGS.values()) + [S.fp8_workload(0), S.fp8_workload(35)]:
        assert w.cu_seqlens[-1] == w.total_tokens
        assert len(w.k_start) == len(w.seqlens)
        assert all(L % 128 == 0 for L in w.seqlens)
        assert w.num_q_heads % w.num_kv_heads == 0
    assert list(S.FP8_SEQLENS) == [8192, 16384, 32768, 73728]
    assert sum(S.FP8_SEQLENS) == 131072
