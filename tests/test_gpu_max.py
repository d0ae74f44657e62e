"""GPU parity at the largest sequence the scoring and selection stages accept:
262 144 tokens, i.e. 2048 key blocks of 128 (the row-length limit of the
top-k stage), alone and packed behind a short sequence.

Heads are cut to 8 query heads over 2 KV heads so the oracle's fp64 copies
stay small; every per-head quantity (scores, lists, attention) has the same
size as in a 32-head layer.  Checked:
  * scores on sampled rows, the last row included (2048 key blocks);
  * every list of every head and row, bit-exact against the oracle's
    selection on the GPU's fp32 scores;
  * bf16 block-sparse, 64 x 128 and dense attention on sampled rows;
  * fp8 attention (e4m3 and fp16 weights) and its paged form on the packed
    batch;
  * with every block kept the lists are 0..I (2048 entries on the last row)
    and the block-sparse call equals the dense call bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_stem_amd as stem
import oracle as O
import stem_synth as S
from gpu_common import (BF16_MAX_ABS, BF16_MEAN_REL, FP8_MAX_ABS, check_lse, check_out, check_scores, dev,
                        lists_equal, note, page_pool, quantize_fp8, to_dev)

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(128.0)
LMAX = 2048 * 128
HQ, HKV = 8, 2
MU, ALPHA, N_INIT, N_WINDOW = 0.5, 0.7, 1, 2


def _sample_rows(seqlens):
    """First, second, middle, second-to-last and last block rows of every sequence."""
    rows, r0 = [], 0
    for L in seqlens:
        nb = L // 128
        rows += sorted({r0, r0 + 1, r0 + nb // 2, r0 + nb - 2, r0 + nb - 1})
        r0 += nb
    return rows


def _rows_of(x, rows):
    """[T][Hq][d] -> float64 [Hq * len(rows)][128][d], head-major."""
    return np.stack([x[r * 128:(r + 1) * 128, h, :].to(torch.float64).cpu().numpy()
                     for h in range(HQ) for r in rows])


def _lse_of(lse, rows):
    return np.stack([lse[h, r * 128:(r + 1) * 128].to(torch.float64).cpu().numpy()
                     for h in range(HQ) for r in rows])


def _ref_rows(o, lse, rows):
    return (np.stack([o[r * 128:(r + 1) * 128, h, :] for h in range(HQ) for r in rows]),
            np.stack([lse[h, r * 128:(r + 1) * 128] for h in range(HQ) for r in rows]))


def _stages(p, qd, kd, vd, k_start):
    kcap = stem.stem_max_kept(p, k_start, MU, ALPHA, N_INIT, N_WINDOW)
    scores = stem.stem_score(p, qd, kd, vd)
    idx, cnt = stem.stem_schedule_topk(p, scores, k_start, MU, ALPHA, N_INIT, N_WINDOW, kcap)
    return kcap, scores, idx, cnt


@pytest.fixture(scope="module")
def single():
    """One 256K-token sequence, bf16, about a quarter of the block pairs kept."""
    lens, k_start = (LMAX,), [552]
    note(f"[max bf16] T={LMAX} Hq={HQ} Hkv={HKV} k_start={k_start}")
    q, k, v = S.make_qkv(lens, HQ, HKV, 128, seed=7, sink=True)
    p = stem.Problem(S.cu_from_lengths(lens), HQ, HKV)
    qd, kd, vd = to_dev(q, k, v)
    kcap, scores, idx, cnt = _stages(p, qd, kd, vd, k_start)
    rows = _sample_rows(lens)
    out, lse = stem.stem_bsa_prefill(p, qd, kd, vd, idx, cnt, SCALE, want_lse=True)
    o64, l64 = stem.stem_bsa_prefill_q64(p, qd, kd, vd, idx.repeat_interleave(2, dim=1).contiguous(),
                                         cnt.repeat_interleave(2, dim=1).contiguous(), SCALE, want_lse=True)
    dout = stem.stem_dense_prefill(p, qd, kd, vd, SCALE)
    torch.cuda.synchronize()
    res = dict(lens=lens, k_start=k_start, kcap=kcap, rows=rows,
               scores=scores.cpu().numpy(), idx=idx.cpu().numpy(), cnt=cnt.cpu().numpy(),
               out=_rows_of(out, rows), lse=_lse_of(lse, rows), o64=_rows_of(o64, rows),
               l64=_lse_of(l64, rows), dout=_rows_of(dout, rows[-1:]))
    del qd, kd, vd, scores, idx, cnt, out, lse, o64, l64, dout
    torch.cuda.empty_cache()
    res["ref_inputs"] = tuple(t.to(torch.float64).numpy() for t in (q, k, v))
    return res


def test_max_scores_on_sampled_rows(single):
    qf, kf, vf = single["ref_inputs"]
    cu = S.cu_from_lengths(single["lens"])
    bonus = O.value_bonus(vf, cu, 128, S.BETA)
    ref = O.block_scores(qf, kf, bonus, cu, HQ, HKV, 128, 8, 128, 1.0, rows=single["rows"])
    rows = single["rows"]
    check_scores(single["scores"][:, rows], ref[:, rows], f"256K {HQ} heads x {len(rows)} rows")


def test_max_every_list_bit_exact(single):
    ri, rc = O.schedule_topk(single["scores"], S.cu_from_lengths(single["lens"]), single["k_start"], MU,
                             ALPHA, N_INIT, N_WINDOW, single["kcap"])
    note(f"  lists 256K: {rc.size} rows, {int(rc.sum())} kept blocks, k_cap {single['kcap']}")
    lists_equal(single["idx"], single["cnt"], ri, rc, "256K")


def test_max_attention_on_sampled_rows(single):
    qf, kf, vf = single["ref_inputs"]
    cu = S.cu_from_lengths(single["lens"])
    rows = single["rows"]
    pairs = [(h, r) for h in range(HQ) for r in rows]
    ro, rl = O.block_sparse_attention(qf, kf, vf, single["idx"], single["cnt"], cu, HQ, HKV, SCALE, rows=pairs)
    ref_o, ref_l = _ref_rows(ro, rl, rows)
    check_out(single["out"], ref_o, BF16_MAX_ABS, BF16_MEAN_REL, f"256K bsa {len(pairs)} rows")
    check_lse(single["lse"], ref_l, "256K bsa")
    # the 64 x 128 variant with each half given its row's list: same result
    check_out(single["o64"], ref_o, BF16_MAX_ABS, BF16_MEAN_REL, f"256K q64 {len(pairs)} rows")
    check_lse(single["l64"], ref_l, "256K q64")


def test_max_dense_last_row(single):
    """Every query of the last block row against all 262 144 keys."""
    qf, kf, vf = single["ref_inputs"]
    cu = S.cu_from_lengths(single["lens"])
    t0 = LMAX - 128
    ro, _ = O.dense_causal_attention(qf, kf, vf, cu, HQ, HKV, SCALE, q_range=(t0, LMAX))
    ref = np.stack([ro[t0:LMAX, h, :] for h in range(HQ)])
    check_out(single["dout"], ref, BF16_MAX_ABS, BF16_MEAN_REL, "256K dense last row, all heads")


def test_max_all_blocks_kept_lists_and_dense_identity():
    """k_start far above the row length keeps every causal block: the lists are
    0..I (2048 entries on the last row), and attention over them is the dense
    call bit for bit."""
    lens = (LMAX,)
    q, k, v = S.make_qkv(lens, 2, 1, 128, seed=8, sink=True)
    p = stem.Problem(S.cu_from_lengths(lens), 2, 1)
    qd, kd, vd = to_dev(q, k, v)
    kcap = stem.stem_max_kept(p, [1e6], MU, 1.0, N_INIT, N_WINDOW)
    assert kcap == 2048
    scores = stem.stem_score(p, qd, kd, vd)
    idx, cnt = stem.stem_schedule_topk(p, scores, [1e6], MU, 1.0, N_INIT, N_WINDOW, kcap)
    fi, fc = O.full_lists(S.cu_from_lengths(lens), 2)
    lists_equal(idx.cpu().numpy(), cnt.cpu().numpy(), fi, fc, "256K every block kept")
    out = stem.stem_bsa_prefill(p, qd, kd, vd, idx, cnt, SCALE)
    dout = stem.stem_dense_prefill(p, qd, kd, vd, SCALE)
    torch.cuda.synchronize()
    assert torch.equal(out, dout), "every block listed must equal the dense call"


def test_max_fp8_packed_behind_a_short_sequence():
    """fp8 varlen batch [384, 262144]: e4m3 weights, fp16 weights and the paged
    form on the scheduled lists, checked on sampled rows of both sequences."""
    lens, k_start = (384, LMAX), [2, 552]
    note(f"[max fp8] lens={lens} Hq={HQ} Hkv={HKV}")
    cu = S.cu_from_lengths(lens)
    q, k, v = S.make_qkv(lens, HQ, HKV, 128, seed=9, sink=True)
    p = stem.Problem(cu, HQ, HKV)
    kcap, scores, idx, cnt = _stages(p, *to_dev(q, k, v), k_start)
    (q8, k8, v8), (qs, ks, vs) = quantize_fp8(q, k, v, lens)
    qa, ka, va = to_dev(q8, k8, v8)
    sc = to_dev(qs, ks, vs)
    out, lse = stem.stem_bsa_prefill(p, qa, ka, va, idx, cnt, SCALE, scales=sc, want_lse=True)
    o16, l16 = stem.stem_bsa_prefill(p, qa, ka, va, idx, cnt, SCALE, scales=sc, want_lse=True, fp16_weights=True)
    kp, vp, ksp, vsp, table = page_pool(k8, v8, ks, vs, lens, spare=4, seed=9)
    kpd, vpd, tabd = to_dev(kp, vp, table)
    po, pl = stem.stem_bsa_prefill_paged(p, qa, kpd, vpd, tabd, idx, cnt, SCALE, scales=to_dev(qs, ksp, vsp),
                                         want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(po, out) and torch.equal(pl, lse), "paged differs from contiguous"
    rows = _sample_rows(lens)
    g_out, g_lse, g_o16, g_l16 = _rows_of(out, rows), _lse_of(lse, rows), _rows_of(o16, rows), _lse_of(l16, rows)
    ri, rc = O.schedule_topk(scores.cpu().numpy(), cu, k_start, MU, ALPHA, N_INIT, N_WINDOW, kcap)
    lists_equal(idx.cpu().numpy(), cnt.cpu().numpy(), ri, rc, "fp8 varlen [384, 256K]")
    del qa, ka, va, kpd, vpd, tabd, out, lse, o16, l16, po, pl, scores, idx, cnt
    torch.cuda.empty_cache()
    qf, kf, vf = (O.dequantize_blocks(c.numpy(), s.numpy(), 128) for c, s in ((q8, qs), (k8, ks), (v8, vs)))
    pairs = [(h, r) for h in range(HQ) for r in rows]
    ro, rl = O.block_sparse_attention(qf, kf, vf, ri, rc, cu, HQ, HKV, SCALE, rows=pairs)
    ref_o, ref_l = _ref_rows(ro, rl, rows)
    check_out(g_out, ref_o, FP8_MAX_ABS, None, f"fp8 [384, 256K] {len(pairs)} rows")
    check_lse(g_lse, ref_l, "fp8 [384, 256K]")
    check_out(g_o16, ref_o, BF16_MAX_ABS, BF16_MEAN_REL, f"fp8/fp16 weights [384, 256K] {len(pairs)} rows")
    check_lse(g_l16, ref_l, "fp8/fp16 weights [384, 256K]")
