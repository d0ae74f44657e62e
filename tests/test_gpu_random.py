"""GPU parity on seeded random problem shapes: the whole path (scores, lists,
bf16 / fp8 / fp8 with fp16 weights / paged / 64x128 attention, scoring on
e4m3 codes) against the oracle, over random
sequence counts and lengths, head ratios and schedule parameters.  Each
case is deterministic (its seed fixes every draw) and small enough for the
oracle to check every output."""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_stem_amd as stem
import oracle as O
import stem_synth as S
from gpu_common import (BF16_MAX_ABS, BF16_MEAN_REL, FP8_MAX_ABS, check_lse, check_out, check_scores,
                        dequant, dev, f64, lists_equal, make_inputs, note, page_pool, quantize_fp8,
                        random_q64_lists, to_dev)

pytestmark = pytest.mark.gpu


def _case(seed):
    r = np.random.default_rng(1000 + seed)
    n_seq = int(r.integers(1, 5))
    lens = tuple(int(x) * 128 for x in r.integers(1, 25, size=n_seq))
    Hkv = int(r.choice([1, 2, 4]))
    Hq = Hkv * int(r.choice([1, 2, 4]))
    mu = float(r.choice([0.3, 0.5, 0.7, 1.0]))
    alpha = float(r.choice([0.7, 1.0]))
    n_init, n_window = int(r.integers(0, 3)), int(r.integers(0, 3))
    k_start = [int(r.integers(0, L // 128 + 3)) for L in lens]
    beta = float(r.choice([0.0, 0.2, 0.5]))
    return lens, Hq, Hkv, mu, alpha, n_init, n_window, k_start, beta


@pytest.mark.parametrize("seed", range(12))
def test_random_shapes_whole_path(seed):
    lens, Hq, Hkv, mu, alpha, n_init, n_window, k_start, beta = _case(seed)
    note(f"[random {seed}] lens={lens} Hq={Hq} Hkv={Hkv} mu={mu} alpha={alpha} "
         f"init={n_init} window={n_window} k_start={k_start} beta={beta}")
    cu = S.cu_from_lengths(lens)
    p = stem.Problem(cu, Hq, Hkv)
    q, k, v = make_inputs(lens, Hq, Hkv, seed=seed)
    qf, kf, vf = (f64(t) for t in (q, k, v))
    qd, kd, vd = to_dev(q, k, v)
    scale = 1.0 / math.sqrt(128.0)

    # scores, then the lists both ways on the same fp32 scores
    s = stem.stem_score(p, qd, kd, vd, 8, 2048, 1.0, beta)
    ref_s = O.block_scores(qf, kf, O.value_bonus(vf, cu, 128, beta), cu, Hq, Hkv, 128, 8, 2048, 1.0)
    check_scores(s.cpu().numpy(), ref_s, f"random {seed}")
    kcap = stem.stem_max_kept(p, k_start, mu, alpha, n_init, n_window)
    idx, cnt = stem.stem_schedule_topk(p, s, k_start, mu, alpha, n_init, n_window, kcap)
    ri, rc = O.schedule_topk(s.cpu().numpy(), cu, k_start, mu, alpha, n_init, n_window, kcap)
    lists_equal(idx.cpu().numpy(), cnt.cpu().numpy(), ri, rc, f"random {seed}")

    # bf16 attention on those lists
    out, lse = stem.stem_bsa_prefill(p, qd, kd, vd, idx, cnt, scale, want_lse=True)
    ro, rl = O.block_sparse_attention(qf, kf, vf, ri, rc, cu, Hq, Hkv, scale)
    check_out(f64(out), ro, BF16_MAX_ABS, BF16_MEAN_REL, f"random {seed} bf16")
    check_lse(lse.cpu().numpy().astype(np.float64), rl, f"random {seed} bf16")

    # 64 x 128 blocks with their own random lists
    i64, c64 = random_q64_lists(lens, Hq, seed=seed)
    o64 = stem.stem_bsa_prefill_q64(p, qd, kd, vd, torch.from_numpy(i64).to(dev()),
                                    torch.from_numpy(c64).to(dev()), scale)
    r64, _ = O.block_sparse_attention(qf, kf, vf, i64, c64, cu, Hq, Hkv, scale, q_block=64)
    check_out(f64(o64), r64, BF16_MAX_ABS, BF16_MEAN_REL, f"random {seed} 64x128")

    # fp8 on the same lists, contiguous and paged
    (q8, k8, v8), (qs, ks, vs) = quantize_fp8(q, k, v, lens)
    qa, ka, va = to_dev(q8, k8, v8)
    scl = to_dev(qs, ks, vs)
    o8, l8 = stem.stem_bsa_prefill(p, qa, ka, va, idx, cnt, scale, scales=scl, want_lse=True)
    ro8, rl8 = O.block_sparse_attention(dequant(q8, qs), dequant(k8, ks), dequant(v8, vs), ri, rc, cu, Hq, Hkv,
                                        scale)
    check_out(f64(o8), ro8, FP8_MAX_ABS, None, f"random {seed} fp8")
    check_lse(l8.cpu().numpy().astype(np.float64), rl8, f"random {seed} fp8")
    kp, vp, ksp, vsp, table = page_pool(k8, v8, ks, vs, lens, spare=3, seed=seed)
    kpd, vpd, tabd = to_dev(kp, vp, table)
    op, lp = stem.stem_bsa_prefill_paged(p, qa, kpd, vpd, tabd, idx, cnt, scale, scales=to_dev(qs, ksp, vsp),
                                         want_lse=True)
    assert torch.equal(op, o8) and torch.equal(lp, l8), f"random {seed}: paged differs from contiguous"
    o16 = stem.stem_bsa_prefill(p, qa, ka, va, idx, cnt, scale, scales=scl, fp16_weights=True)
    check_out(f64(o16), ro8, BF16_MAX_ABS, BF16_MEAN_REL, f"random {seed} fp8 inputs, fp16 weights")

    # scoring on the e4m3 codes, and the lists selected from those scores
    qq, kq, vq = dequant(q8, qs), dequant(k8, ks), dequant(v8, vs)
    s8 = stem.stem_score(p, qa, ka, va, 8, 2048, 1.0, beta, scales=scl)
    ref8 = O.block_scores(qq, kq, O.value_bonus(vq, cu, 128, beta), cu, Hq, Hkv, 128, 8, 2048, 1.0)
    check_scores(s8.cpu().numpy(), ref8, f"random {seed} e4m3 scoring")
    i8, c8 = stem.stem_schedule_topk(p, s8, k_start, mu, alpha, n_init, n_window, kcap)
    ri8, rc8 = O.schedule_topk(s8.cpu().numpy(), cu, k_start, mu, alpha, n_init, n_window, kcap)
    lists_equal(i8.cpu().numpy(), c8.cpu().numpy(), ri8, rc8, f"random {seed} e4m3 scoring")
