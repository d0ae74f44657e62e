"""GPU parity: every entry point through the C ABI against the CPU oracle.

Small cases are compared element by element; they span several tiles, a
ragged last score tile and several packed sequences.  Lists are compared
bit-exactly both ways on identical fp32 scores; attention is compared on the
same lists on both sides so its error is isolated from selection.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_stem_amd as stem
import oracle as O
import stem_synth as S
from gpu_common import (BF16_MAX_ABS, BF16_MEAN_REL, FP8_MAX_ABS, check_lse, check_out,
                        check_scores, dequant, dev, f64, lists_equal, make_inputs, note,
                        page_pool, quantize_fp8, random_q64_lists, to_dev)

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(128.0)


def _oracle_scores(qf, kf, vf, w_cu, Hq, Hkv, beta=0.2, chunk=2048):
    bonus = O.value_bonus(vf, w_cu, 128, beta)
    return O.block_scores(qf, kf, bonus, w_cu, Hq, Hkv, 128, 8, chunk, 1.0)


# --------------------------------------------------------------- config 1 ----

@pytest.fixture(scope="module")
def n2k():
    w = S.CONFIGS["n2k_2q1kv"]
    q, k, v = S.make_workload_qkv(w)
    note(f"[n2k] T={w.total_tokens} Hq={w.num_q_heads} Hkv={w.num_kv_heads}")
    return w, (q, k, v), [f64(t) for t in (q, k, v)]


def test_n2k_scores(n2k):
    w, (q, k, v), (qf, kf, vf) = n2k
    p = stem.Problem(w.cu_seqlens, w.num_q_heads, w.num_kv_heads)
    qd, kd, vd = to_dev(q, k, v)
    s = stem.stem_score(p, qd, kd, vd, w.stride, w.chunk_size, w.norm, w.beta)
    torch.cuda.synchronize()
    ref = _oracle_scores(qf, kf, vf, w.cu_seqlens, w.num_q_heads, w.num_kv_heads, w.beta)
    check_scores(s.cpu().numpy(), ref, "n2k")


def test_n2k_topk_both_ways(n2k):
    w, (q, k, v), (qf, kf, vf) = n2k
    p = stem.Problem(w.cu_seqlens, w.num_q_heads, w.num_kv_heads)
    qd, kd, vd = to_dev(q, k, v)
    s_gpu = stem.stem_score(p, qd, kd, vd, w.stride, w.chunk_size, w.norm, w.beta)
    s_ref = _oracle_scores(qf, kf, vf, w.cu_seqlens, w.num_q_heads, w.num_kv_heads, w.beta)
    kcap = stem.stem_max_kept(p, w.k_start, w.mu, w.alpha, w.n_init, w.n_window)
    # GPU selection on the oracle's fp32 scores
    idx, cnt = stem.stem_schedule_topk(p, torch.from_numpy(s_ref).to(dev()), w.k_start, w.mu,
                                       w.alpha, w.n_init, w.n_window, kcap)
    ri, rc = O.schedule_topk(s_ref, w.cu_seqlens, w.k_start, w.mu, w.alpha, w.n_init, w.n_window, kcap)
    lists_equal(idx.cpu().numpy(), cnt.cpu().numpy(), ri, rc, "gpu-select on oracle scores")
    # oracle selection on the GPU's scores
    sg = s_gpu.cpu().numpy()
    idx2, cnt2 = stem.stem_schedule_topk(p, s_gpu, w.k_start, w.mu, w.alpha, w.n_init, w.n_window, kcap)
    ri2, rc2 = O.schedule_topk(sg, w.cu_seqlens, w.k_start, w.mu, w.alpha, w.n_init, w.n_window, kcap)
    lists_equal(idx2.cpu().numpy(), cnt2.cpu().numpy(), ri2, rc2, "oracle-select on gpu scores")
    assert int(rc.sum()) == 2 * 71


def test_n2k_bsa_and_dense_bf16(n2k):
    w, (q, k, v), (qf, kf, vf) = n2k
    p = stem.Problem(w.cu_seqlens, w.num_q_heads, w.num_kv_heads)
    qd, kd, vd = to_dev(q, k, v)
    s_ref = _oracle_scores(qf, kf, vf, w.cu_seqlens, w.num_q_heads, w.num_kv_heads, w.beta)
    kcap = stem.stem_max_kept(p, w.k_start, w.mu, w.alpha, w.n_init, w.n_window)
    ri, rc = O.schedule_topk(s_ref, w.cu_seqlens, w.k_start, w.mu, w.alpha, w.n_init, w.n_window, kcap)
    out, lse = stem.stem_bsa_prefill(p, qd, kd, vd, torch.from_numpy(ri).to(dev()),
                                     torch.from_numpy(rc).to(dev()), SCALE, want_lse=True)
    ro, rl = O.block_sparse_attention(qf, kf, vf, ri, rc, w.cu_seqlens, 2, 1, SCALE)
    check_out(f64(out), ro, BF16_MAX_ABS, BF16_MEAN_REL, "n2k bsa")
    check_lse(lse.cpu().numpy().astype(np.float64), rl, "n2k bsa")
    dout, dlse = stem.stem_dense_prefill(p, qd, kd, vd, SCALE, want_lse=True)
    do, dl = O.dense_causal_attention(qf, kf, vf, w.cu_seqlens, 2, 1, SCALE)
    check_out(f64(dout), do, BF16_MAX_ABS, BF16_MEAN_REL, "n2k dense")
    check_lse(dlse.cpu().numpy().astype(np.float64), dl, "n2k dense")


def test_full_lists_equal_dense_kernel(n2k):
    """Listing every causal block through the sparse kernel reproduces the
    dense kernel bit for bit (same tile loop, same order)."""
    w, (q, k, v), _ = n2k
    p = stem.Problem(w.cu_seqlens, 2, 1)
    qd, kd, vd = to_dev(q, k, v)
    fi, fc = O.full_lists(w.cu_seqlens, 2)
    a = stem.stem_bsa_prefill(p, qd, kd, vd, torch.from_numpy(fi).to(dev()), torch.from_numpy(fc).to(dev()), SCALE)
    b = stem.stem_dense_prefill(p, qd, kd, vd, SCALE)
    assert torch.equal(a, b)


# --------------------------------------------------------------- varlen ------

@pytest.fixture(scope="module")
def varlen():
    lens = (384, 1152, 128, 1664)      # ragged score tiles (nb = 3, 9, 1, 13)
    q, k, v = make_inputs(lens, 4, 2, seed=7)
    note(f"[varlen] lens={lens} Hq=4 Hkv=2")
    return lens, (q, k, v), [f64(t) for t in (q, k, v)]


def test_varlen_scores_and_lists(varlen):
    lens, (q, k, v), (qf, kf, vf) = varlen
    cu = S.cu_from_lengths(lens)
    p = stem.Problem(cu, 4, 2)
    qd, kd, vd = to_dev(q, k, v)
    s = stem.stem_score(p, qd, kd, vd, 8, 1024, 1.0, 0.2)
    ref = _oracle_scores(qf, kf, vf, cu, 4, 2, 0.2)
    check_scores(s.cpu().numpy(), ref, "varlen")
    ks = [3, 5, 1, 6]
    for (mu, alpha, ni, nw) in [(0.5, 0.7, 1, 2), (0.7, 1.0, 0, 1), (1.0, 1.0, 2, 0), (0.3, 1.0, 4, 4)]:
        kcap = stem.stem_max_kept(p, ks, mu, alpha, ni, nw)
        idx, cnt = stem.stem_schedule_topk(p, torch.from_numpy(ref).to(dev()), ks, mu, alpha, ni, nw, kcap + 3)
        ri, rc = O.schedule_topk(ref, cu, ks, mu, alpha, ni, nw, kcap + 3)
        lists_equal(idx.cpu().numpy(), cnt.cpu().numpy(), ri, rc, f"varlen mu={mu} a={alpha} {ni}/{nw}")


def test_varlen_bsa_dense_bf16(varlen):
    lens, (q, k, v), (qf, kf, vf) = varlen
    cu = S.cu_from_lengths(lens)
    p = stem.Problem(cu, 4, 2)
    qd, kd, vd = to_dev(q, k, v)
    ref = _oracle_scores(qf, kf, vf, cu, 4, 2, 0.2)
    ks = [2, 4, 1, 5]
    kcap = stem.stem_max_kept(p, ks, 0.5, 1.0, 1, 1)
    ri, rc = O.schedule_topk(ref, cu, ks, 0.5, 1.0, 1, 1, kcap)
    out, lse = stem.stem_bsa_prefill(p, qd, kd, vd, torch.from_numpy(ri).to(dev()),
                                     torch.from_numpy(rc).to(dev()), SCALE, want_lse=True)
    ro, rl = O.block_sparse_attention(qf, kf, vf, ri, rc, cu, 4, 2, SCALE)
    check_out(f64(out), ro, BF16_MAX_ABS, BF16_MEAN_REL, "varlen bsa")
    check_lse(lse.cpu().numpy().astype(np.float64), rl, "varlen bsa")
    dout = stem.stem_dense_prefill(p, qd, kd, vd, SCALE)
    do, _ = O.dense_causal_attention(qf, kf, vf, cu, 4, 2, SCALE)
    check_out(f64(dout), do, BF16_MAX_ABS, BF16_MEAN_REL, "varlen dense")


def test_empty_lists_give_zero_and_minus_inf(varlen):
    lens, (q, k, v), _ = varlen
    cu = S.cu_from_lengths(lens)
    p = stem.Problem(cu, 4, 2)
    qd, kd, vd = to_dev(q, k, v)
    s = stem.stem_score(p, qd, kd, vd)
    idx, cnt = stem.stem_schedule_topk(p, s, 0, 0.5, 1.0, 0, 0)   # k_start 0, nothing forced
    assert int(cnt.sum()) == 0 and bool((idx == -1).all())
    out, lse = stem.stem_bsa_prefill(p, qd, kd, vd, idx, cnt, SCALE, want_lse=True)
    assert bool((out == 0).all()) and bool(torch.isneginf(lse).all())


def _empty_some_rows(idx, cnt, seed):
    """The same lists with a seeded third of the (head, row) lists emptied."""
    g = torch.Generator().manual_seed(seed)
    drop = torch.rand(cnt.shape, generator=g) < 1.0 / 3.0
    ci, ii = cnt.cpu().clone(), idx.cpu().clone()
    ci[drop] = 0
    ii[drop] = -1
    return ii, ci


def test_empty_rows_between_full_ones(varlen, fp8_small):
    """A third of the rows with empty lists, spread among full ones, so the
    persistent workgroups pass from empty rows to full ones and back: bf16,
    e4m3 weights and fp16 weights against the oracle on the same lists
    (an empty row gives 0 and lse -inf)."""
    lens, (q, k, v), (qf, kf, vf) = varlen
    cu = S.cu_from_lengths(lens)
    p = stem.Problem(cu, 4, 2)
    qd, kd, vd = to_dev(q, k, v)
    s = stem.stem_score(p, qd, kd, vd)
    idx, cnt = stem.stem_schedule_topk(p, s, [3, 5, 1, 6], 0.5, 1.0, 1, 1)
    ii, ci = _empty_some_rows(idx, cnt, 31)
    assert 0 < int((ci == 0).sum()) < ci.numel()
    out, lse = stem.stem_bsa_prefill(p, qd, kd, vd, ii.to(dev()), ci.to(dev()), SCALE, want_lse=True)
    ro, rl = O.block_sparse_attention(qf, kf, vf, ii.numpy(), ci.numpy(), cu, 4, 2, SCALE)
    check_out(f64(out), ro, BF16_MAX_ABS, BF16_MEAN_REL, "bf16 with empty rows")
    check_lse(lse.cpu().numpy().astype(np.float64), rl, "bf16 with empty rows")

    lens8, _, (q8, k8, v8), (qs, ks, vs), (qf8, kf8, vf8) = fp8_small
    cu8 = S.cu_from_lengths(lens8)
    p8 = stem.Problem(cu8, 4, 2)
    s8 = stem.stem_score(p8, *to_dev(*fp8_small[1]))
    idx8, cnt8 = stem.stem_schedule_topk(p8, s8, [1, 3, 4], 0.5, 1.0, 1, 1)
    ii8, ci8 = _empty_some_rows(idx8, cnt8, 32)
    assert 0 < int((ci8 == 0).sum()) < ci8.numel()
    ro8, _ = O.block_sparse_attention(qf8, kf8, vf8, ii8.numpy(), ci8.numpy(), cu8, 4, 2, SCALE)
    sc = to_dev(qs, ks, vs)
    for fp16_weights in (False, True):
        o8 = stem.stem_bsa_prefill(p8, *to_dev(q8, k8, v8), ii8.to(dev()), ci8.to(dev()), SCALE, scales=sc,
                                   fp16_weights=fp16_weights)
        check_out(f64(o8), ro8, FP8_MAX_ABS, None, f"fp8 with empty rows, fp16_weights={fp16_weights}")


@pytest.mark.parametrize("gain", [1.0, 4.0])
def test_diagonal_block_only_lists(gain):
    """Every row lists only its own (diagonal) block, so the causal mask inside
    one block decides every weight and the first queries of each block see one
    to a few keys (on the e4m3 path both 64-key halves of that block take the
    residual pass, and the queries of the first half see no key of the
    second).  bf16, e4m3 weights and fp16 weights against the oracle; gain
    scales Q (peaked logits at 4)."""
    lens = (256, 640)
    q, k, v = make_inputs(lens, 4, 2, seed=11)
    q = (q.float() * gain).to(q.dtype)
    cu = S.cu_from_lengths(lens)
    p = stem.Problem(cu, 4, 2)
    ri = np.full((4, p.R, 1), -1, dtype=np.int32)
    rc = np.ones((4, p.R), dtype=np.int32)
    for z in range(len(lens)):
        r0, r1 = cu[z] // 128, cu[z + 1] // 128
        ri[:, r0:r1, 0] = np.arange(r1 - r0, dtype=np.int32)
    idx, cnt = to_dev(torch.from_numpy(ri), torch.from_numpy(rc))
    qf, kf, vf = (f64(t) for t in (q, k, v))
    out, lse = stem.stem_bsa_prefill(p, *to_dev(q, k, v), idx, cnt, SCALE, want_lse=True)
    ro, rl = O.block_sparse_attention(qf, kf, vf, ri, rc, cu, 4, 2, SCALE)
    check_out(f64(out), ro, BF16_MAX_ABS, BF16_MEAN_REL, f"bf16 diagonal-only lists, gain {gain}")
    check_lse(lse.cpu().numpy().astype(np.float64), rl, f"bf16 diagonal-only lists, gain {gain}")

    (q8, k8, v8), (qs, ks, vs) = quantize_fp8(q, k, v, lens)
    qd8, kd8, vd8 = dequant(q8, qs), dequant(k8, ks), dequant(v8, vs)
    ro8, rl8 = O.block_sparse_attention(qd8, kd8, vd8, ri, rc, cu, 4, 2, SCALE)
    sc = to_dev(qs, ks, vs)
    o8, l8 = stem.stem_bsa_prefill(p, *to_dev(q8, k8, v8), idx, cnt, SCALE, scales=sc, want_lse=True)
    check_out(f64(o8), ro8, FP8_MAX_ABS, None, f"fp8 diagonal-only lists, gain {gain}")
    if gain == 1.0:
        check_lse(l8.cpu().numpy().astype(np.float64), rl8, f"fp8 diagonal-only lists, gain {gain}")
    o16 = stem.stem_bsa_prefill(p, *to_dev(q8, k8, v8), idx, cnt, SCALE, scales=sc, fp16_weights=True)
    check_out(f64(o16), ro8, BF16_MAX_ABS, BF16_MEAN_REL, f"fp8 inputs, fp16 weights, diagonal-only lists, gain {gain}")


def test_chunk_size_changes_no_score(varlen):
    lens, (q, k, v), _ = varlen
    p = stem.Problem(S.cu_from_lengths(lens), 4, 2)
    qd, kd, vd = to_dev(q, k, v)
    outs = [stem.stem_score(p, qd, kd, vd, 8, c).cpu() for c in (128, 1024, 2048, 4096)]
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
    # and on the e4m3 codes
    (q8, k8, v8), scl = quantize_fp8(q, k, v, lens)
    qa, ka, va = to_dev(q8, k8, v8)
    sc = to_dev(*scl)
    outs8 = [stem.stem_score(p, qa, ka, va, 8, c, scales=sc).cpu() for c in (128, 1024, 2048, 4096)]
    for o in outs8[1:]:
        assert torch.equal(o, outs8[0])


def test_many_sequences_span_several_launches():
    lens = tuple([128, 256, 384] * 24)          # 72 sequences > 64 per launch
    q, k, v = make_inputs(lens, 2, 1, seed=11)
    qf, kf, vf = (f64(t) for t in (q, k, v))
    cu = S.cu_from_lengths(lens)
    p = stem.Problem(cu, 2, 1)
    qd, kd, vd = to_dev(q, k, v)
    s = stem.stem_score(p, qd, kd, vd)
    ref = _oracle_scores(qf, kf, vf, cu, 2, 1)
    check_scores(s.cpu().numpy(), ref, "72 seqs")
    idx, cnt = stem.stem_schedule_topk(p, torch.from_numpy(ref).to(dev()), 2, 0.5, 1.0, 1, 1)
    ri, rc = O.schedule_topk(ref, cu, [2] * len(lens), 0.5, 1.0, 1, 1, idx.shape[2])
    lists_equal(idx.cpu().numpy(), cnt.cpu().numpy(), ri, rc, "72 seqs")
    out, lse = stem.stem_bsa_prefill(p, qd, kd, vd, idx, cnt, SCALE, want_lse=True)
    ro, rl = O.block_sparse_attention(qf, kf, vf, ri, rc, cu, 2, 1, SCALE)
    check_out(f64(out), ro, BF16_MAX_ABS, BF16_MEAN_REL, "72 seqs")
    check_lse(lse.cpu().numpy().astype(np.float64), rl, "72 seqs")
    dout = stem.stem_dense_prefill(p, qd, kd, vd, SCALE)
    do, _ = O.dense_causal_attention(qf, kf, vf, cu, 2, 1, SCALE)
    check_out(f64(dout), do, BF16_MAX_ABS, BF16_MEAN_REL, "72 seqs dense")
    i64, c64 = random_q64_lists(lens, 2, seed=11)
    o64 = stem.stem_bsa_prefill_q64(p, qd, kd, vd, torch.from_numpy(i64).to(dev()), torch.from_numpy(c64).to(dev()),
                                    SCALE)
    r64, _ = O.block_sparse_attention(qf, kf, vf, i64, c64, cu, 2, 1, SCALE, q_block=64)
    check_out(f64(o64), r64, BF16_MAX_ABS, BF16_MEAN_REL, "72 seqs 64x128")
    # fp8, contiguous and paged: the block table is indexed across launches
    (q8, k8, v8), (qs, ks, vs) = quantize_fp8(q, k, v, lens)
    qa, ka, va = to_dev(q8, k8, v8)
    o8, l8 = stem.stem_bsa_prefill(p, qa, ka, va, idx, cnt, SCALE, scales=to_dev(qs, ks, vs), want_lse=True)
    ro8, rl8 = O.block_sparse_attention(dequant(q8, qs), dequant(k8, ks), dequant(v8, vs), ri, rc, cu, 2, 1, SCALE)
    check_out(f64(o8), ro8, FP8_MAX_ABS, None, "72 seqs fp8")
    check_lse(l8.cpu().numpy().astype(np.float64), rl8, "72 seqs fp8")
    kp, vp, ksp, vsp, table = page_pool(k8, v8, ks, vs, lens, spare=6, seed=11)
    kpd, vpd, tabd = to_dev(kp, vp, table)
    op, lp = stem.stem_bsa_prefill_paged(p, qa, kpd, vpd, tabd, idx, cnt, SCALE, scales=to_dev(qs, ksp, vsp),
                                         want_lse=True)
    assert torch.equal(op, o8) and torch.equal(lp, l8), "72 seqs: paged differs from contiguous"


def test_topk_tie_stress():
    """Scores from a tiny integer set: ties everywhere; lower index must win."""
    lens = (2048, 1280)
    cu = S.cu_from_lengths(lens)
    p = stem.Problem(cu, 4, 2)
    for seed, ties in ((0, 2), (1, 3), (2, 5)):
        sc = S.random_scores_like(4, lens, ties=ties, seed=seed)
        sc[0, 3, 1] = float("nan")               # NaN ranks as -inf
        ks = [5, 4]
        idx, cnt = stem.stem_schedule_topk(p, sc.to(dev()), ks, 0.6, 1.0, 1, 1)
        ri, rc = O.schedule_topk(sc.numpy(), cu, ks, 0.6, 1.0, 1, 1, idx.shape[2])
        lists_equal(idx.cpu().numpy(), cnt.cpu().numpy(), ri, rc, f"ties={ties}")
    # -0.0 and +0.0 are equal scores: half the zeros of a two-value draw get a minus sign
    sc = S.random_scores_like(4, lens, ties=2, seed=7)
    flip = torch.rand(sc.shape, generator=torch.Generator().manual_seed(8)) < 0.5
    sc = torch.where((sc == 0) & flip, torch.full_like(sc, -0.0), sc)
    assert bool(torch.signbit(sc[sc == 0]).any()) and bool((~torch.signbit(sc[sc == 0])).any())
    idx, cnt = stem.stem_schedule_topk(p, sc.to(dev()), [5, 4], 0.6, 1.0, 1, 1)
    ri, rc = O.schedule_topk(sc.numpy(), cu, [5, 4], 0.6, 1.0, 1, 1, idx.shape[2])
    lists_equal(idx.cpu().numpy(), cnt.cpu().numpy(), ri, rc, "signed zeros")


# ---------------------------------------------------------------- fp8 --------

@pytest.fixture(scope="module")
def fp8_small():
    lens = (256, 768, 1280)
    q, k, v = make_inputs(lens, 4, 2, seed=3)
    (q8, k8, v8), (qs, ks, vs) = quantize_fp8(q, k, v, lens)
    note(f"[fp8] lens={lens}")
    deq = [dequant(q8, qs), dequant(k8, ks), dequant(v8, vs)]
    return lens, (q, k, v), (q8, k8, v8), (qs, ks, vs), deq


def test_fp8_bsa_and_dense(fp8_small):
    lens, (q, k, v), (q8, k8, v8), (qs, ks, vs), (qf, kf, vf) = fp8_small
    cu = S.cu_from_lengths(lens)
    p = stem.Problem(cu, 4, 2)
    qd, kd, vd = to_dev(q, k, v)
    s = stem.stem_score(p, qd, kd, vd)
    idx, cnt = stem.stem_schedule_topk(p, s, [1, 3, 4], 0.5, 1.0, 1, 1)
    ri, rc = idx.cpu().numpy(), cnt.cpu().numpy()
    sc = to_dev(qs, ks, vs)
    out = stem.stem_bsa_prefill(p, *to_dev(q8, k8, v8), idx, cnt, SCALE, scales=sc)
    ro, _ = O.block_sparse_attention(qf, kf, vf, ri, rc, cu, 4, 2, SCALE)
    check_out(f64(out), ro, FP8_MAX_ABS, None, "fp8 bsa")
    dout = stem.stem_dense_prefill(p, *to_dev(q8, k8, v8), SCALE, scales=sc)
    do, _ = O.dense_causal_attention(qf, kf, vf, cu, 4, 2, SCALE)
    check_out(f64(dout), do, FP8_MAX_ABS, None, "fp8 dense")


def test_fp8_scores_and_lists(fp8_small):
    """stem_score_fp8 on the e4m3 codes: the oracle's scores of the dequantised
    values (value bonus included) to the score bar, and the lists selected
    from them bit-exact; also with beta = 0 and norm = 2."""
    lens, _, (q8, k8, v8), (qs, ks, vs), (qf, kf, vf) = fp8_small
    cu = S.cu_from_lengths(lens)
    p = stem.Problem(cu, 4, 2)
    qa, ka, va = to_dev(q8, k8, v8)
    sc = to_dev(qs, ks, vs)
    for beta, norm in ((0.2, 1.0), (0.0, 2.0)):
        s = stem.stem_score(p, qa, ka, va, 8, 2048, norm, beta, scales=sc)
        ref = O.block_scores(qf, kf, O.value_bonus(vf, cu, 128, beta), cu, 4, 2, 128, 8, 2048, norm)
        check_scores(s.cpu().numpy(), ref, f"fp8 scores beta {beta} norm {norm}")
    idx, cnt = stem.stem_schedule_topk(p, s, [1, 3, 4], 0.5, 1.0, 1, 1)
    ri, rc = O.schedule_topk(s.cpu().numpy(), cu, [1, 3, 4], 0.5, 1.0, 1, 1, idx.shape[2])
    lists_equal(idx.cpu().numpy(), cnt.cpu().numpy(), ri, rc, "fp8 scores")
    # the whole fp8 layer through stem_prefill with fp8 scoring equals the three calls
    s1 = stem.stem_score(p, qa, ka, va, scales=sc)
    i1, c1 = stem.stem_schedule_topk(p, s1, [1, 3, 4], 0.5, 1.0, 2, 2)
    o1 = stem.stem_bsa_prefill(p, qa, ka, va, i1, c1, scales=sc)
    o2 = stem.stem_prefill(p, None, None, None, [1, 3, 4], 0.5, 1.0, n_init=2, n_window=2,
                           fp8_inputs=(qa, ka, va, sc), fp8_scoring=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_fp8_full_lists_equal_dense(fp8_small):
    lens, _, (q8, k8, v8), (qs, ks, vs), _ = fp8_small
    cu = S.cu_from_lengths(lens)
    p = stem.Problem(cu, 4, 2)
    fi, fc = O.full_lists(cu, 4)
    sc = to_dev(qs, ks, vs)
    a = stem.stem_bsa_prefill(p, *to_dev(q8, k8, v8), torch.from_numpy(fi).to(dev()),
                              torch.from_numpy(fc).to(dev()), SCALE, scales=sc)
    b = stem.stem_dense_prefill(p, *to_dev(q8, k8, v8), SCALE, scales=sc)
    assert torch.equal(a, b)


# ------------------------------------------------------- head-group shapes ----

@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 1), (10, 2), (9, 3)])
def test_head_group_ratios(Hq, Hkv):
    """Multi-head (1 query head per KV head), 8 query heads on one KV head, and
    odd group sizes (5 and 3 query heads per KV head, an odd KV head count):
    scores, lists and attention through the whole path, bf16 and fp8."""
    lens = (640, 1408)
    cu = S.cu_from_lengths(lens)
    q, k, v = make_inputs(lens, Hq, Hkv, seed=11)
    qf, kf, vf = f64(q), f64(k), f64(v)
    note(f"[heads] Hq={Hq} Hkv={Hkv} lens={lens}")
    p = stem.Problem(cu, Hq, Hkv)
    qd, kd, vd = to_dev(q, k, v)
    s = stem.stem_score(p, qd, kd, vd)
    ref = _oracle_scores(qf, kf, vf, cu, Hq, Hkv)
    check_scores(s.cpu().numpy(), ref, f"Hq={Hq} Hkv={Hkv}")
    ks = [2, 4]
    idx, cnt = stem.stem_schedule_topk(p, s, ks, 0.5, 0.7, 1, 2)
    ri, rc = O.schedule_topk(s.cpu().numpy(), cu, ks, 0.5, 0.7, 1, 2, idx.shape[2])
    lists_equal(idx.cpu().numpy(), cnt.cpu().numpy(), ri, rc, f"Hq={Hq} Hkv={Hkv}")
    out, lse = stem.stem_bsa_prefill(p, qd, kd, vd, idx, cnt, SCALE, want_lse=True)
    ro, rl = O.block_sparse_attention(qf, kf, vf, ri, rc, cu, Hq, Hkv, SCALE)
    check_out(f64(out), ro, BF16_MAX_ABS, BF16_MEAN_REL, f"bsa Hq={Hq} Hkv={Hkv}")
    check_lse(lse.cpu().numpy().astype(np.float64), rl, f"bsa Hq={Hq} Hkv={Hkv}")
    dout = stem.stem_dense_prefill(p, qd, kd, vd, SCALE)
    do, _ = O.dense_causal_attention(qf, kf, vf, cu, Hq, Hkv, SCALE)
    check_out(f64(dout), do, BF16_MAX_ABS, BF16_MEAN_REL, f"dense Hq={Hq} Hkv={Hkv}")
    (q8, k8, v8), (qs, kss, vs) = quantize_fp8(q, k, v, lens)
    o8, l8 = stem.stem_bsa_prefill(p, *to_dev(q8, k8, v8), idx, cnt, SCALE, scales=to_dev(qs, kss, vs),
                                   want_lse=True)
    ro8, rl8 = O.block_sparse_attention(dequant(q8, qs), dequant(k8, kss), dequant(v8, vs), ri, rc, cu, Hq, Hkv,
                                        SCALE)
    check_out(f64(o8), ro8, FP8_MAX_ABS, None, f"fp8 bsa Hq={Hq} Hkv={Hkv}")
    check_lse(l8.cpu().numpy().astype(np.float64), rl8, f"fp8 bsa Hq={Hq} Hkv={Hkv}")
    # scoring on the e4m3 codes and its lists, same head layout
    qq, kq, vq = dequant(q8, qs), dequant(k8, kss), dequant(v8, vs)
    s8 = stem.stem_score(p, *to_dev(q8, k8, v8), scales=to_dev(qs, kss, vs))
    check_scores(s8.cpu().numpy(), _oracle_scores(qq, kq, vq, cu, Hq, Hkv), f"e4m3 scoring Hq={Hq} Hkv={Hkv}")
    i8, c8 = stem.stem_schedule_topk(p, s8, ks, 0.5, 0.7, 1, 2)
    ri8, rc8 = O.schedule_topk(s8.cpu().numpy(), cu, ks, 0.5, 0.7, 1, 2, i8.shape[2])
    lists_equal(i8.cpu().numpy(), c8.cpu().numpy(), ri8, rc8, f"e4m3 scoring Hq={Hq} Hkv={Hkv}")


def test_score_parameters_beta_zero_and_norm():
    """beta = 0 (no value bonus: the plain strided routing score) and an extra
    normaliser n = 2 reach the scores exactly as the oracle defines them."""
    lens = (1024, 896)
    cu = S.cu_from_lengths(lens)
    q, k, v = make_inputs(lens, 4, 2, seed=12)
    qf, kf, vf = f64(q), f64(k), f64(v)
    p = stem.Problem(cu, 4, 2)
    qd, kd, vd = to_dev(q, k, v)
    for beta, norm in [(0.0, 1.0), (0.2, 2.0), (0.5, 0.5)]:
        s = stem.stem_score(p, qd, kd, vd, 8, 2048, norm, beta)
        bonus = O.value_bonus(vf, cu, 128, beta)
        ref = O.block_scores(qf, kf, bonus, cu, 4, 2, 128, 8, 2048, norm)
        check_scores(s.cpu().numpy(), ref, f"beta={beta} norm={norm}")


def test_lists_with_spare_capacity_are_padded():
    """A list row stride far above the largest kept count: every entry past
    the count is -1 and attention reads only the counted prefix."""
    lens = (1536,)
    cu = S.cu_from_lengths(lens)
    q, k, v = make_inputs(lens, 2, 1, seed=13)
    qf, kf, vf = f64(q), f64(k), f64(v)
    p = stem.Problem(cu, 2, 1)
    qd, kd, vd = to_dev(q, k, v)
    s = stem.stem_score(p, qd, kd, vd)
    kcap = 12                                     # max_nb: every row could hold all its blocks
    idx, cnt = stem.stem_schedule_topk(p, s, [3], 0.5, 1.0, 1, 1, kcap)
    ri, rc = O.schedule_topk(s.cpu().numpy(), cu, [3], 0.5, 1.0, 1, 1, kcap)
    lists_equal(idx.cpu().numpy(), cnt.cpu().numpy(), ri, rc, "spare capacity")
    ig, cg = idx.cpu().numpy(), cnt.cpu().numpy()
    for h in range(2):
        for r in range(12):
            assert np.all(ig[h, r, cg[h, r]:] == -1)
    out = stem.stem_bsa_prefill(p, qd, kd, vd, idx, cnt, SCALE)
    ro, _ = O.block_sparse_attention(qf, kf, vf, ri, rc, cu, 2, 1, SCALE)
    check_out(f64(out), ro, BF16_MAX_ABS, BF16_MEAN_REL, "spare capacity")


# ------------------------------------------------------------ paged fp8 ----

def test_fp8_paged_matches_oracle_and_contiguous(fp8_small):
    """K/V scattered over a shuffled page pool (spare pages hold NaN codes):
    the paged kernel matches the oracle on the dequantised contiguous tensors
    and reproduces the contiguous fp8 path bit for bit."""
    lens, (q, k, v), (q8, k8, v8), (qs, ks, vs), (qf, kf, vf) = fp8_small
    cu = S.cu_from_lengths(lens)
    p = stem.Problem(cu, 4, 2)
    qd, kd, vd = to_dev(q, k, v)
    s = stem.stem_score(p, qd, kd, vd)
    idx, cnt = stem.stem_schedule_topk(p, s, [1, 3, 4], 0.5, 1.0, 1, 1)
    ri, rc = idx.cpu().numpy(), cnt.cpu().numpy()
    kp, vp, ksp, vsp, table = page_pool(k8, v8, ks, vs, lens, spare=7, seed=21)
    note(f"  pool of {kp.shape[0]} pages, table stride {table.shape[1]}")
    sc_paged = to_dev(qs, ksp, vsp)
    q8d, kpd, vpd, tabd = to_dev(q8, kp, vp, table)
    out, lse = stem.stem_bsa_prefill_paged(p, q8d, kpd, vpd, tabd, idx, cnt, SCALE, scales=sc_paged,
                                           want_lse=True)
    ro, rl = O.block_sparse_attention(qf, kf, vf, ri, rc, cu, 4, 2, SCALE)
    check_out(f64(out), ro, FP8_MAX_ABS, None, "fp8 paged bsa")
    check_lse(lse.cpu().numpy().astype(np.float64), rl, "fp8 paged bsa")
    ref_out, ref_lse = stem.stem_bsa_prefill(p, *to_dev(q8, k8, v8), idx, cnt, SCALE,
                                             scales=to_dev(qs, ks, vs), want_lse=True)
    assert torch.equal(out, ref_out), "paged and contiguous fp8 outputs differ"
    assert torch.equal(lse, ref_lse)
    # every block listed: the paged path equals dense attention
    fi, fc = O.full_lists(cu, 4)
    fout = stem.stem_bsa_prefill_paged(p, q8d, kpd, vpd, tabd, *to_dev(torch.from_numpy(fi), torch.from_numpy(fc)),
                                       SCALE, scales=sc_paged)
    do, _ = O.dense_causal_attention(qf, kf, vf, cu, 4, 2, SCALE)
    check_out(f64(fout), do, FP8_MAX_ABS, None, "fp8 paged all blocks")


# ------------------------------------------------ 64-query rows (64 x 128) ---

def test_q64_random_lists_match_oracle(varlen):
    """Rows of 64 queries against 128-key blocks, each row with its own random
    list (empty rows, rows without the diagonal block), vs the oracle."""
    lens, (q, k, v), (qf, kf, vf) = varlen
    cu = S.cu_from_lengths(lens)
    p = stem.Problem(cu, 4, 2)
    qd, kd, vd = to_dev(q, k, v)
    ri, rc = random_q64_lists(lens, 4, seed=31)
    assert (rc == 0).any() and ri.shape[1] == 2 * p.R
    out, lse = stem.stem_bsa_prefill_q64(p, qd, kd, vd, torch.from_numpy(ri).to(dev()),
                                         torch.from_numpy(rc).to(dev()), SCALE, want_lse=True)
    ro, rl = O.block_sparse_attention(qf, kf, vf, ri, rc, cu, 4, 2, SCALE, q_block=64)
    check_out(f64(out), ro, BF16_MAX_ABS, BF16_MEAN_REL, "q64 random lists")
    check_lse(lse.cpu().numpy().astype(np.float64), rl, "q64 random lists")


def test_q64_parent_lists_match_square_rows(varlen):
    """Both 64-query halves given the Stem list of their 128-query row: the
    oracle's square-row result, and the square-row kernel's within the bar."""
    lens, (q, k, v), (qf, kf, vf) = varlen
    cu = S.cu_from_lengths(lens)
    p = stem.Problem(cu, 4, 2)
    qd, kd, vd = to_dev(q, k, v)
    ref = _oracle_scores(qf, kf, vf, cu, 4, 2, 0.2)
    ks = [2, 4, 1, 5]
    kcap = stem.stem_max_kept(p, ks, 0.5, 1.0, 1, 1)
    ri, rc = O.schedule_topk(ref, cu, ks, 0.5, 1.0, 1, 1, kcap)
    idx64 = torch.from_numpy(np.repeat(ri, 2, axis=1)).to(dev())
    cnt64 = torch.from_numpy(np.repeat(rc, 2, axis=1)).to(dev())
    out, lse = stem.stem_bsa_prefill_q64(p, qd, kd, vd, idx64, cnt64, SCALE, want_lse=True)
    ro, rl = O.block_sparse_attention(qf, kf, vf, ri, rc, cu, 4, 2, SCALE)
    check_out(f64(out), ro, BF16_MAX_ABS, BF16_MEAN_REL, "q64 parent lists")
    check_lse(lse.cpu().numpy().astype(np.float64), rl, "q64 parent lists")
    sq = stem.stem_bsa_prefill(p, qd, kd, vd, torch.from_numpy(ri).to(dev()), torch.from_numpy(rc).to(dev()),
                               SCALE)
    check_out(f64(out), f64(sq), BF16_MAX_ABS, None, "q64 vs square-row kernel")


def test_q64_every_block_listed_equals_dense(n2k):
    w, (q, k, v), (qf, kf, vf) = n2k
    cu = w.cu_seqlens
    p = stem.Problem(cu, w.num_q_heads, w.num_kv_heads)
    qd, kd, vd = to_dev(q, k, v)
    fi, fc = O.full_lists(cu, w.num_q_heads, 128, q_block=64)
    out = stem.stem_bsa_prefill_q64(p, qd, kd, vd, torch.from_numpy(fi).to(dev()),
                                    torch.from_numpy(fc).to(dev()), SCALE)
    do, _ = O.dense_causal_attention(qf, kf, vf, cu, w.num_q_heads, w.num_kv_heads, SCALE)
    check_out(f64(out), do, BF16_MAX_ABS, BF16_MEAN_REL, "q64 all blocks vs dense")


# ------------------------------------------------------ one-call wrapper ----

def test_stem_prefill_equals_the_three_calls(fp8_small):
    """stem_prefill (score -> schedule -> attention in one call) gives exactly
    what the three entry points give, for bf16 and for e4m3 inputs (with e4m3
    and with fp16 weights for P.V)."""
    lens, (q, k, v), (q8, k8, v8), (qs, ks, vs), _ = fp8_small
    cu = S.cu_from_lengths(lens)
    p = stem.Problem(cu, 4, 2)
    qd, kd, vd = to_dev(q, k, v)
    kstart, mu, alpha = [1, 3, 4], 0.5, 0.7
    s = stem.stem_score(p, qd, kd, vd)
    idx, cnt = stem.stem_schedule_topk(p, s, kstart, mu, alpha, 1, 2)
    a = stem.stem_prefill(p, qd, kd, vd, kstart, mu, alpha, n_init=1, n_window=2, softmax_scale=SCALE)
    assert torch.equal(a, stem.stem_bsa_prefill(p, qd, kd, vd, idx, cnt, SCALE))
    f8 = to_dev(q8, k8, v8)
    sc = to_dev(qs, ks, vs)
    for w16 in (False, True):
        b = stem.stem_prefill(p, qd, kd, vd, kstart, mu, alpha, n_init=1, n_window=2, softmax_scale=SCALE,
                              fp8_inputs=(*f8, sc), fp16_weights=w16)
        assert torch.equal(b, stem.stem_bsa_prefill(p, *f8, idx, cnt, SCALE, scales=sc, fp16_weights=w16))
