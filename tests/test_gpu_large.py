"""GPU parity at the full workload sizes: 32K and 128K bf16 layers and the
128K fp8 varlen layer at both alpha values of its layer schedule (1.0 and 0.7).

The GPU runs every stage on the whole workload through the C ABI, with the
entry points, arguments and preallocated workspaces the benchmark times.
The oracle then checks, at sizes it can afford:
  * block scores on sampled (head, row) pairs, every key block of each row;
  * every list of every head and row, selected by the oracle from the GPU's
    own fp32 scores (bit-exact);
  * attention output and LSE on sampled (head, row) pairs, on the GPU's lists;
  * dense attention on sampled heads and query ranges.
The oracle is fed head subsets (whole GQA groups) so its fp64 copies stay a
few GB; a subset keeps each query head with its own KV head.
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_stem_amd as stem
import oracle as O
import stem_synth as S
from gpu_common import (BF16_MAX_ABS, BF16_MEAN_REL, FP8_MAX_ABS, check_lse, check_out,
                        check_scores, dev, lists_equal, note, page_pool, to_dev)

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(128.0)
HS = [0, 1, 2, 3, 12, 13, 14, 15, 28, 29, 30, 31]    # query heads of KV groups 0, 3, 7
KS = [0, 3, 7]


def _subset64(q, k, v):
    return (q[:, HS].to(torch.float64).numpy(), k[:, KS].to(torch.float64).numpy(),
            v[:, KS].to(torch.float64).numpy())


def _sample_rows(w):
    """First, second, middle and last q-block rows of every sequence."""
    rows, r0 = [], 0
    for L in w.seqlens:
        nb = L // 128
        rows += sorted({r0, r0 + 1, r0 + nb // 2, r0 + nb - 1})
        r0 += nb
    return rows


def _gather_rows(x, rows):
    """x [T][Hq][d] on the GPU -> {(h_sub, r): [128][d] float64} for h in HS."""
    out = {}
    for hi, h in enumerate(HS):
        for r in rows:
            out[(hi, r)] = x[r * 128:(r + 1) * 128, h, :].to(torch.float64).cpu().numpy()
    return out


def _random_half_lists(w, idx, cnt, seed=64):
    """Lists for the second 64-query half of every row: for the sampled heads
    a seeded random ascending subset of [0, I] with the row's own count (so
    the two halves of a row list mostly different blocks); for the other
    heads the row's list."""
    rng = np.random.default_rng(seed)
    out = idx.copy()
    local = np.concatenate([np.arange(L // 128) for L in w.seqlens])
    for h in HS:
        for r, I in enumerate(local):
            n = int(cnt[h, r])
            out[h, r, :n] = np.sort(rng.choice(int(I) + 1, size=n, replace=False))
            out[h, r, n:] = -1
    return out


def _run(w, fp8):
    note(f"[{w.name}] generating T={w.total_tokens} Hq={w.num_q_heads} Hkv={w.num_kv_heads}")
    q, k, v = S.make_workload_qkv(w)
    p = stem.Problem(w.cu_seqlens, w.num_q_heads, w.num_kv_heads)
    qd, kd, vd = to_dev(q, k, v)
    ws = torch.empty(stem.stem_score_workspace_bytes(p), dtype=torch.uint8, device=dev())
    scores = torch.empty((p.Hq, p.R, p.max_nb), dtype=torch.float32, device=dev())
    kcap = stem.stem_max_kept(p, w.k_start, w.mu, w.alpha, w.n_init, w.n_window)
    idx = torch.empty((p.Hq, p.R, kcap), dtype=torch.int32, device=dev())
    cnt = torch.empty((p.Hq, p.R), dtype=torch.int32, device=dev())
    note(f"[{w.name}] score + schedule (k_cap {kcap})")
    stem.stem_score(p, qd, kd, vd, w.stride, w.chunk_size, w.norm, w.beta, scores, ws)
    stem.stem_schedule_topk(p, scores, w.k_start, w.mu, w.alpha, w.n_init, w.n_window, kcap, idx, cnt)
    dt = stem.STEM_DTYPE_FP8_E4M3 if fp8 else stem.STEM_DTYPE_BF16
    aws = torch.empty(stem.stem_attn_workspace_bytes(p, dt), dtype=torch.uint8, device=dev())
    out = torch.empty((p.T, p.Hq, p.d), dtype=torch.bfloat16, device=dev())
    dout = torch.empty_like(out)
    lse = torch.empty((p.Hq, p.T), dtype=torch.float32, device=dev())
    scales = None
    if fp8:
        # the harness quantiser: per (128-token block, head) scale amax / 448
        (q8, qs), (k8, ks), (v8, vs) = (S.quantize_e4m3_per_block(t, w.seqlens) for t in (q, k, v))
        qa, ka, va = to_dev(q8, k8, v8)
        scales = to_dev(qs, ks, vs)
        # the oracle sees the dequantised values of the same codes
        hq, hk, hv = (O.dequantize_blocks(c.numpy(), s.numpy(), 128) for c, s in
                      ((q8[:, HS], qs[:, HS]), (k8[:, KS], ks[:, KS]), (v8[:, KS], vs[:, KS])))
        ref_inputs = (hq, hk, hv)
    else:
        qa, ka, va = qd, kd, vd
        ref_inputs = None
    note(f"[{w.name}] {'fp8' if fp8 else 'bf16'} block-sparse and dense attention")
    stem.stem_bsa_prefill(p, qa, ka, va, idx, cnt, SCALE, scales=scales, out=out, lse=lse, workspace=aws)
    paged_equal = None
    if fp8:
        # the same layer from a shuffled page pool must give the same bits
        kp, vp, ksp, vsp, table = page_pool(k8, v8, ks, vs, w.seqlens, spare=5, seed=w.seed)
        kpd, vpd, tabd = to_dev(kp, vp, table)
        pout = torch.empty_like(out)
        plse = torch.empty_like(lse)
        stem.stem_bsa_prefill_paged(p, qa, kpd, vpd, tabd, idx, cnt, SCALE, scales=to_dev(qs, ksp, vsp),
                                    out=pout, lse=plse, workspace=aws)
        torch.cuda.synchronize()
        paged_equal = bool(torch.equal(pout, out)) and bool(torch.equal(plse, lse))
        note(f"[{w.name}] paged ({kp.shape[0]} pages) equals contiguous: {paged_equal}")
        del kpd, vpd, tabd, pout, plse
        # scoring on the e4m3 codes (stem_score_fp8), with its own lists
        scores8 = torch.empty_like(scores)
        stem.stem_score(p, qa, ka, va, w.stride, w.chunk_size, w.norm, w.beta, scores8, ws, scales=scales)
        fp8_scores = scores8.cpu().numpy()
        del scores8
        # the same lists with fp16 weights for P.V
        out16, lse16 = torch.empty_like(out), torch.empty_like(lse)
        stem.stem_bsa_prefill(p, qa, ka, va, idx, cnt, SCALE, scales=scales, out=out16, lse=lse16, workspace=aws,
                              fp16_weights=True)
    out64 = lse64 = None
    if not fp8:
        # 64-query rows, each half given its 128-query row's list
        out64, lse64 = torch.empty_like(out), torch.empty_like(lse)
        stem.stem_bsa_prefill_q64(p, qa, ka, va, idx.repeat_interleave(2, dim=1).contiguous(),
                                  cnt.repeat_interleave(2, dim=1).contiguous(), SCALE, out=out64, lse=lse64,
                                  workspace=aws)
        # and with independent half lists (half 1 random, same counts): the
        # kernel then skips, per half, the blocks that half does not list
        idx_np, cnt_np = idx.cpu().numpy(), cnt.cpu().numpy()
        idx_b = _random_half_lists(w, idx_np, cnt_np)
        idx64d = np.stack((idx_np, idx_b), axis=2).reshape(p.Hq, 2 * p.R, kcap)
        cnt64d = np.stack((cnt_np, cnt_np), axis=2).reshape(p.Hq, 2 * p.R)
        out64d, lse64d = torch.empty_like(out), torch.empty_like(lse)
        stem.stem_bsa_prefill_q64(p, qa, ka, va, torch.from_numpy(np.ascontiguousarray(idx64d)).to(dev()),
                                  torch.from_numpy(np.ascontiguousarray(cnt64d)).to(dev()), SCALE, out=out64d,
                                  lse=lse64d, workspace=aws)
    stem.stem_dense_prefill(p, qa, ka, va, SCALE, scales=scales, out=dout, workspace=aws)
    torch.cuda.synchronize()
    rows = _sample_rows(w)
    res = dict(w=w, p=p, kcap=kcap, rows=rows, paged_equal=paged_equal,
               scores=scores.cpu().numpy(), idx=idx.cpu().numpy(), cnt=cnt.cpu().numpy(),
               out=_gather_rows(out, rows), dout=_gather_rows(dout, rows),
               lse={(hi, r): lse[h, r * 128:(r + 1) * 128].to(torch.float64).cpu().numpy()
                    for hi, h in enumerate(HS) for r in rows})
    if fp8:
        res["fp8_scores"] = fp8_scores
        res["out16"] = _gather_rows(out16, rows)
        res["lse16"] = {(hi, r): lse16[h, r * 128:(r + 1) * 128].to(torch.float64).cpu().numpy()
                        for hi, h in enumerate(HS) for r in rows}
        del out16, lse16
    if out64 is not None:
        res["out64"] = _gather_rows(out64, rows)
        res["lse64"] = {(hi, r): lse64[h, r * 128:(r + 1) * 128].to(torch.float64).cpu().numpy()
                        for hi, h in enumerate(HS) for r in rows}
        del out64, lse64
        res["out64d"] = _gather_rows(out64d, rows)
        res["lse64d"] = {(hi, r): lse64d[h, r * 128:(r + 1) * 128].to(torch.float64).cpu().numpy()
                         for hi, h in enumerate(HS) for r in rows}
        res["idx64d"], res["cnt64d"] = idx64d[HS], cnt64d[HS]
        del out64d, lse64d
    del qd, kd, vd, out, dout, lse, scores, idx, cnt, aws, ws
    torch.cuda.empty_cache()
    bf = _subset64(q, k, v)
    res["bf16_ref_inputs"] = bf
    res["attn_ref_inputs"] = ref_inputs if fp8 else bf
    return res


@pytest.fixture(scope="module", params=["n32k_32q8kv", "n128k_32q8kv", "fp8_layer0", "fp8_layer5"])
def big(request):
    # fp8 layers 0-4 of the 36-layer schedule use alpha 1.0, layers 5-35 alpha 0.7
    if request.param.startswith("fp8_layer"):
        return _run(S.fp8_workload(int(request.param[len("fp8_layer"):])), fp8=True)
    return _run(S.CONFIGS[request.param], fp8=False)


def test_scores_on_sampled_rows(big):
    w, rows = big["w"], big["rows"]
    qs, ks, vs = big["bf16_ref_inputs"]
    bonus = O.value_bonus(vs, w.cu_seqlens, 128, w.beta)
    # chunk width 128 changes no value (pinned on the CPU) and keeps each row cheap
    ref = O.block_scores(qs, ks, bonus, w.cu_seqlens, len(HS), len(KS), 128, w.stride, 128, w.norm,
                         rows=rows)
    gpu = big["scores"][HS][:, rows]
    check_scores(gpu, ref[:, rows], f"{w.name} {len(HS)} heads x {len(rows)} rows")


def test_fp8_scores_on_sampled_rows_and_their_lists(big):
    """Scoring on the e4m3 codes: the oracle's scores of the dequantised values
    on sampled rows, and every list selected from those scores bit-exact."""
    if "fp8_scores" not in big:
        pytest.skip("bf16 layer: e4m3 scoring applies to the fp8 layer")
    w, rows = big["w"], big["rows"]
    qs, ks, vs = big["attn_ref_inputs"]
    bonus = O.value_bonus(vs, w.cu_seqlens, 128, w.beta)
    ref = O.block_scores(qs, ks, bonus, w.cu_seqlens, len(HS), len(KS), 128, w.stride, 128, w.norm, rows=rows)
    check_scores(big["fp8_scores"][HS][:, rows], ref[:, rows], f"{w.name} e4m3 scoring {len(HS)} heads x {len(rows)} rows")
    ri, rc = O.schedule_topk(big["fp8_scores"], w.cu_seqlens, w.k_start, w.mu, w.alpha, w.n_init, w.n_window,
                             big["kcap"])
    idx, cnt = stem.stem_schedule_topk(stem.Problem(w.cu_seqlens, w.num_q_heads, w.num_kv_heads),
                                       torch.from_numpy(big["fp8_scores"]).to(dev()), w.k_start, w.mu, w.alpha,
                                       w.n_init, w.n_window, big["kcap"])
    lists_equal(idx.cpu().numpy(), cnt.cpu().numpy(), ri, rc, f"{w.name} e4m3 scoring")


def test_every_list_bit_exact(big):
    w = big["w"]
    ri, rc = O.schedule_topk(big["scores"], w.cu_seqlens, w.k_start, w.mu, w.alpha, w.n_init,
                             w.n_window, big["kcap"])
    note(f"  lists {w.name}: {rc.size} rows, {int(rc.sum())} kept blocks")
    lists_equal(big["idx"], big["cnt"], ri, rc, w.name)


def _compare_rows(big, ref_o, ref_lse, gpu_rows, gpu_lse, bar, where):
    rows = big["rows"]
    g = np.stack([gpu_rows[(hi, r)] for hi in range(len(HS)) for r in rows])
    rr = np.stack([ref_o[r * 128:(r + 1) * 128, hi, :] for hi in range(len(HS)) for r in rows])
    check_out(g, rr, bar[0], bar[1], where)
    if gpu_lse is not None:
        gl = np.stack([gpu_lse[(hi, r)] for hi in range(len(HS)) for r in rows])
        rl = np.stack([ref_lse[hi, r * 128:(r + 1) * 128] for hi in range(len(HS)) for r in rows])
        check_lse(gl, rl, where)


def test_block_sparse_attention_on_sampled_rows(big):
    w = big["w"]
    fp8 = w.fp8
    qs, ks, vs = big["attn_ref_inputs"]
    idx_sub, cnt_sub = big["idx"][HS], big["cnt"][HS]
    pairs = [(hi, r) for hi in range(len(HS)) for r in big["rows"]]
    ro, rl = O.block_sparse_attention(qs, ks, vs, idx_sub, cnt_sub, w.cu_seqlens, len(HS), len(KS),
                                      SCALE, rows=pairs)
    bar = (FP8_MAX_ABS, None) if fp8 else (BF16_MAX_ABS, BF16_MEAN_REL)
    _compare_rows(big, ro, rl, big["out"], big["lse"], bar, f"{w.name} bsa {len(pairs)} rows")


def test_q64_rows_on_sampled_rows(big):
    """The 64 x 128 variant with each half given its row's list: the same
    oracle result as the square rows (a pinned identity of the oracle)."""
    if "out64" not in big:
        pytest.skip("fp8 layer: the 64-query variant is bf16 only")
    w = big["w"]
    qs, ks, vs = big["attn_ref_inputs"]
    pairs = [(hi, r) for hi in range(len(HS)) for r in big["rows"]]
    ro, rl = O.block_sparse_attention(qs, ks, vs, big["idx"][HS], big["cnt"][HS], w.cu_seqlens, len(HS),
                                      len(KS), SCALE, rows=pairs)
    _compare_rows(big, ro, rl, big["out64"], big["lse64"], (BF16_MAX_ABS, BF16_MEAN_REL),
                  f"{w.name} q64 {len(pairs)} rows")


def test_q64_independent_half_lists_on_sampled_rows(big):
    """The 64 x 128 variant with half 1 given a random list of the same count
    (the halves then share few blocks): every sampled 64-query row against
    the oracle with 64-query rows on the same lists."""
    if "out64d" not in big:
        pytest.skip("fp8 layer: the 64-query variant is bf16 only")
    w = big["w"]
    qs, ks, vs = big["attn_ref_inputs"]
    pairs = [(hi, 2 * r + s) for hi in range(len(HS)) for r in big["rows"] for s in (0, 1)]
    ro, rl = O.block_sparse_attention(qs, ks, vs, big["idx64d"], big["cnt64d"], w.cu_seqlens, len(HS), len(KS),
                                      SCALE, rows=pairs, q_block=64)
    _compare_rows(big, ro, rl, big["out64d"], big["lse64d"], (BF16_MAX_ABS, BF16_MEAN_REL),
                  f"{w.name} q64 independent halves {len(pairs)} half rows")


def test_fp8_fp16_weights_on_sampled_rows(big):
    """The fp8 layer with fp16 weights for P.V: the bf16 output bar on the
    oracle's attention over the dequantised codes."""
    if "out16" not in big:
        pytest.skip("bf16 layer: fp16 weights are an fp8 mode")
    w = big["w"]
    qs, ks, vs = big["attn_ref_inputs"]
    pairs = [(hi, r) for hi in range(len(HS)) for r in big["rows"]]
    ro, rl = O.block_sparse_attention(qs, ks, vs, big["idx"][HS], big["cnt"][HS], w.cu_seqlens, len(HS),
                                      len(KS), SCALE, rows=pairs)
    _compare_rows(big, ro, rl, big["out16"], big["lse16"], (BF16_MAX_ABS, BF16_MEAN_REL),
                  f"{w.name} fp16 weights {len(pairs)} rows")


def test_dense_attention_on_sampled_rows(big):
    w = big["w"]
    fp8 = w.fp8
    qs, ks, vs = big["attn_ref_inputs"]
    rows = big["rows"]
    # one head per sampled KV group: a middle row (the last row of the first
    # sequence when packed) and the last row overall
    checks = [(0, rows[2] if len(w.seqlens) == 1 else rows[3]), (6, rows[-1]), (11, rows[-1])]
    seq_start = {}
    r0 = 0
    for z, L in enumerate(w.seqlens):
        for I in range(L // 128):
            seq_start[r0 + I] = (w.cu_seqlens[z], I)
        r0 += L // 128
    bar = (FP8_MAX_ABS, None) if fp8 else (BF16_MAX_ABS, BF16_MEAN_REL)
    for hi, r in checks:
        a, I = seq_start[r]
        t0 = I * 128
        ro, _ = O.dense_causal_attention(qs, ks, vs, w.cu_seqlens, len(HS), len(KS), SCALE,
                                         heads=[hi], q_range=(t0, t0 + 128))
        check_out(big["dout"][(hi, r)], ro[a + t0:a + t0 + 128, hi, :], bar[0], bar[1],
                  f"{w.name} dense head {HS[hi]} row {r}")


def test_fp8_paged_equals_contiguous_at_full_size(big):
    """Paged K/V (shuffled pool, NaN-filled spare pages) reproduce the
    contiguous fp8 output and LSE bit for bit over the whole layer."""
    if big["paged_equal"] is None:
        pytest.skip("bf16 layer: the paged path is fp8 only")
    assert big["paged_equal"]
