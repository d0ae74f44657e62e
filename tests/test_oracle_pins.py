"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

None of these re-types an oracle formula and compares it with itself: each
check is a brute-force evaluation, a closed form, a special case that reduces
to a textbook quantity, an invariant, a library routine, or a hand example.
"""
import itertools
import json
import math
from fractions import Fraction
import os

import numpy as np
import pytest
import torch

import oracle as O
import stem_synth as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- P1 / P2 -----

def test_strided_scores_equal_bruteforce_antidiagonal_sums():
    """P1: the reshaped-GEMM form equals explicit anti-diagonal tile sums of the
    token-level Q K^T (pairs (t, s-1-t) inside every s x s tile)."""
    r = _rng(1)
    L, d, s = 96, 8, 4
    q, k = r.standard_normal((L, d)), r.standard_normal((L, d))
    scale = 0.37
    A = O.strided_scores(q, k, s, scale)
    n = L // s
    for i in range(n):
        for j in range(n):
            if j > i:
                assert A[i, j] == -np.inf
                continue
            acc = 0.0
            for t in range(s):
                acc += float(np.dot(q[i * s + t], k[j * s + (s - 1 - t)]))
            assert abs(A[i, j] - scale * acc) < 1e-12 * max(1.0, abs(acc))


def test_stride_one_reduces_to_blockmax_of_causal_logits():
    """P2: with s = 1 the block score is the max of q.k / (sqrt(d) n) over the
    causal token pairs of the block, plus the value bonus (bonus zeroed here)."""
    r = _rng(2)
    L, H, d, bs = 64, 2, 16, 16
    q = r.standard_normal((L, H, d))
    k = r.standard_normal((L, 1, d))
    bonus = np.zeros((1, L // bs))
    norm = 1.5
    Sc = O.block_scores(q, k, bonus, [0, L], H, 1, block_size=bs, stride=1, chunk_size=32, norm=norm)
    for h in range(H):
        logits = (q[:, h, :] @ k[:, 0, :].T) / (math.sqrt(d) * norm)
        for I in range(L // bs):
            for J in range(L // bs):
                if J > I:
                    assert Sc[h, I, J] == -np.inf
                    continue
                best = -np.inf
                for a in range(I * bs, I * bs + bs):
                    for b in range(J * bs, J * bs + bs):
                        if b <= a:
                            best = max(best, logits[a, b])
                assert abs(Sc[h, I, J] - np.float32(best)) <= 1e-6 * max(1, abs(best))


def test_chunk_width_changes_no_value():
    """P8: chunk widths 256 / 512 / 1024 give identical block scores."""
    q, k, v = S.make_qkv((1024,), 2, 1, 128, seed=3, sink=True)
    qf, kf, vf = (t.to(torch.float64).numpy() for t in (q, k, v))
    bonus = O.value_bonus(vf, [0, 1024], 128, 0.2)
    outs = [O.block_scores(qf, kf, bonus, [0, 1024], 2, 1, 128, 8, c, 1.0) for c in (256, 512, 1024)]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_row_and_head_restriction_and_fp32_views_change_no_value():
    """P8: restricting block_scores to some rows and heads, and passing the
    bf16 values as fp32 arrays instead of fp64, leaves those rows' scores
    bit-identical (every product is formed in fp64 either way); the other
    rows and heads stay -inf."""
    lens = (384, 640)
    cu = S.cu_from_lengths(lens)
    q, k, v = S.make_qkv(lens, 4, 2, 128, seed=5, sink=True)
    qf, kf, vf = (t.to(torch.float64).numpy() for t in (q, k, v))
    q32, k32 = (t.to(torch.float32).numpy() for t in (q, k))
    bonus = O.value_bonus(vf, cu, 128, 0.2)
    full = O.block_scores(qf, kf, bonus, cu, 4, 2, 128, 8, 256, 1.0)
    rows, heads = [0, 2, 4, 7], [1, 2]
    part = O.block_scores(q32, k32, bonus, cu, 4, 2, 128, 8, 128, 1.0, heads=heads, rows=rows)
    for h in range(4):
        for r in range(full.shape[1]):
            if h in heads and r in rows:
                assert np.array_equal(part[h, r], full[h, r])
            else:
                assert np.all(np.isneginf(part[h, r]))


# ---------------------------------------------------------------- P3 (OAM) -----

def test_value_bonus_hand_example():
    """P3: two key blocks with l = (0, 2): mean 1, population std 1, so
    z = (-1, +1)/(1 + 1e-6) and bonus = (0, beta/(1 + 1e-6))."""
    bs, d = 4, 3
    v = np.zeros((2 * bs, 1, d))
    v[:bs, 0, 0] = 1.0                       # ||V||^2 = 1   -> ln 1 = 0
    v[bs:, 0, 0] = math.exp(1.0)             # ||V||^2 = e^2 -> ln = 2
    v[1, 0, 0] = 0.5                         # smaller rows do not change the block max
    b = O.value_bonus(v, [0, 2 * bs], bs, beta=0.2)
    assert b[0, 0] == 0.0
    assert abs(b[0, 1] - 0.2 / (1 + 1e-6)) < 1e-15


def test_value_bonus_scale_invariant_and_single_block_zero():
    """P3: scaling V by c shifts every l_J by 2 ln c and leaves the z-score
    (hence the bonus) unchanged; a one-block sequence has zero spread -> 0."""
    r = _rng(4)
    v = r.standard_normal((512, 2, 16)) * np.exp(0.5 * r.standard_normal((512, 2, 1)))
    b1 = O.value_bonus(v, [0, 256, 512], 64, 0.2)
    b2 = O.value_bonus(7.5 * v, [0, 256, 512], 64, 0.2)
    assert np.allclose(b1, b2, atol=1e-12)
    one = O.value_bonus(v[:64], [0, 64], 64, 0.2)
    assert np.all(one == 0.0)


def test_zero_queries_give_pure_bonus_and_beta_zero_gives_route_score():
    """P3: with Q = 0 every causal block score equals the bonus exactly; with
    beta = 0 the score is the pure routing score (independent brute force)."""
    q, k, v = S.make_qkv((512,), 2, 1, 32, seed=5, sink=False)
    qf, kf, vf = (t.to(torch.float64).numpy() for t in (q, k, v))
    bonus = O.value_bonus(vf, [0, 512], 128, 0.2)
    S0 = O.block_scores(np.zeros_like(qf), kf, bonus, [0, 512], 2, 1, 128, 8, 256, 1.0)
    for I in range(4):
        assert np.array_equal(S0[:, I, :I + 1], np.broadcast_to(bonus[0, :I + 1].astype(np.float32), (2, I + 1)))
    Sb = O.block_scores(qf, kf, np.zeros_like(bonus), [0, 512], 2, 1, 128, 8, 256, 1.0)
    scale = 1 / (math.sqrt(32) * 8)
    for h in range(2):
        tok = qf[:, h, :] @ kf[:, 0, :].T
        for I in range(4):
            for J in range(I + 1):
                best = -np.inf
                for i in range(16 * I, 16 * I + 16):
                    for j in range(16 * J, min(16 * J + 16, i + 1)):
                        acc = sum(tok[i * 8 + t, j * 8 + 7 - t] for t in range(8))
                        best = max(best, acc * scale)
                assert abs(Sb[h, I, J] - best) < 1e-5


def test_log_transform_keeps_the_ranking():
    """P3 / [HPC] §二.2.2: selecting on route + beta*ReLU(z) picks the same
    blocks as selecting on the product exp(route) * exp(beta*ReLU(z))."""
    r = _rng(6)
    route = r.standard_normal(40)
    bon = 0.2 * np.maximum(0, r.standard_normal(40))
    additive = route + bon
    product = np.exp(route) * np.exp(bon)
    for kept in (3, 10, 25):
        f = O.forced_blocks(39, 1, 2)
        assert O.select_row(additive, 39, kept, f) == O.select_row(product, 39, kept, f)


# ---------------------------------------------------------------- P4 (TPD) -----

@pytest.mark.parametrize("k_start,mu,alpha,nb", [(8, 0.5, 1.0, 16), (70, 0.5, 0.7, 256),
                                                 (276, 0.5, 0.7, 1024), (13, 0.7, 1.0, 37),
                                                 (100, 0.3, 0.7, 500)])
def test_tpd_budget_closed_form_properties(k_start, mu, alpha, nb):
    """P4 ([ZH] §2.1): k(0) = floor(k_start'); the budget is non-increasing and
    linear, reaching k_end = mu * k_start' one block past the end; midpoint is
    the mean of the two ends (k_start' = alpha * k_start)."""
    from fractions import Fraction as F
    ke = F(repr(float(alpha))) * k_start
    mu_f = F(repr(float(mu)))
    ks = [O.tpd_budget(I, nb, k_start, mu, alpha) for I in range(nb + 1)]
    assert ks[0] == math.floor(ke)
    assert all(a >= b for a, b in zip(ks, ks[1:]))
    assert ks[nb] == math.floor(mu_f * ke)
    if nb % 2 == 0:
        assert ks[nb // 2] == math.floor((1 + mu_f) * ke / 2)
    # every step drops by at most ceil of the per-block slope
    slope = ke * (1 - mu_f) / nb
    assert all(a - b <= math.ceil(slope) for a, b in zip(ks, ks[1:]))


def test_tpd_mu_one_is_uniform_topk():
    """P4: mu = 1 is the uniform per-row budget the pages compare against."""
    assert {O.tpd_budget(I, 100, 30, 1.0, 0.7) for I in range(100)} == {21}


def test_kept_count_respects_forced_and_causal_limits():
    for I in range(40):
        f = O.forced_blocks(I, 2, 3)
        assert len(f) == len(set(f)) and all(0 <= j <= I for j in f)
        kc = O.kept_count(I, 40, 5, 0.5, 1.0, 2, 3)
        assert len(f) <= kc <= I + 1


# ---------------------------------------------------------------- P5 (top-k) ----

@pytest.mark.parametrize("seed", range(12))
def test_topk_matches_exhaustive_subset_search(seed):
    """P5: for tiny rows, enumerate every subset of the free candidates and
    require the oracle's choice to be the unique one whose every member
    precedes every non-member under (score desc, index asc); ties are common
    because scores come from a small integer set."""
    r = _rng(100 + seed)
    I = int(r.integers(0, 10))
    n_init, n_window = int(r.integers(0, 3)), int(r.integers(0, 3))
    row = r.integers(0, 3, size=I + 1).astype(np.float32)
    if seed % 3 == 0:
        row[r.integers(0, I + 1)] = np.nan
    forced = O.forced_blocks(I, n_init, n_window)
    kept = int(r.integers(len(forced), I + 2))
    got = O.select_row(row, I, kept, forced)
    free = [J for J in range(I + 1) if J not in forced]
    need = kept - len(forced)

    def val(J):
        x = float(row[J])
        return -np.inf if math.isnan(x) else x

    def precedes(a, b):
        return val(a) > val(b) or (val(a) == val(b) and a < b)

    winners = []
    for sub in itertools.combinations(free, need):
        rest = [J for J in free if J not in sub]
        if all(precedes(a, b) for a in sub for b in rest):
            winners.append(sorted(list(sub) + forced))
    assert len(winners) == 1
    assert got == winners[0]
    assert got == sorted(got) and len(got) == kept


# ---------------------------------------------------------------- P6 / P7 (BSA) -

def _tiny_qkv(seed, L=(96, 64), Hq=4, Hkv=2, d=16):
    r = _rng(seed)
    T = sum(L)
    return (r.standard_normal((T, Hq, d)), r.standard_normal((T, Hkv, d)),
            r.standard_normal((T, Hkv, d)), [0] + list(np.cumsum(L)))


def test_dense_equals_python_loop_softmax():
    """P6: dense causal attention equals an explicit per-query loop."""
    q, k, v, cu = _tiny_qkv(7, L=(48, 32), Hq=2, Hkv=1, d=8)
    sc = 0.3
    Od, lse = O.dense_causal_attention(q, k, v, cu, 2, 1, sc)
    for (a, b) in zip(cu[:-1], cu[1:]):
        for h in range(2):
            for t in range(a, b):
                logits = [sc * float(np.dot(q[t, h], k[u, 0])) for u in range(a, t + 1)]
                m = max(logits)
                w = [math.exp(x - m) for x in logits]
                den = sum(w)
                o = sum(wi * v[a + i, 0] for i, wi in enumerate(w)) / den
                assert np.allclose(Od[t, h], o, atol=1e-12)
                assert abs(lse[h, t] - (m + math.log(den))) < 1e-12


def test_dense_equals_torch_sdpa_fp64():
    """P6 library cross-check: torch's causal SDPA in fp64 on the CPU."""
    q, k, v, cu = _tiny_qkv(8, L=(128,), Hq=4, Hkv=2, d=16)
    sc = 1 / 4.0
    Od, _ = O.dense_causal_attention(q, k, v, cu, 4, 2, sc)
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(np.repeat(k, 2, axis=1)).permute(1, 0, 2)[None]
    vt = torch.from_numpy(np.repeat(v, 2, axis=1)).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=sc)
    assert np.allclose(Od, ref[0].permute(1, 0, 2).numpy(), atol=1e-12)


def test_all_blocks_kept_equals_dense():
    """P6: listing every causal block reproduces dense causal attention."""
    q, k, v, cu = _tiny_qkv(9)
    idx, cnt = O.full_lists(cu, 4, block_size=16)
    Ob, lb = O.block_sparse_attention(q, k, v, idx, cnt, cu, 4, 2, 0.25, block_size=16)
    Od, ld = O.dense_causal_attention(q, k, v, cu, 4, 2, 0.25)
    assert np.allclose(Ob, Od, atol=1e-12) and np.allclose(lb, ld, atol=1e-12)


def test_skipped_blocks_equal_minus_inf_masking():
    """P7 ([HPC] §三.3.1): attending only to the listed blocks equals dense
    attention with every non-listed key's logit set to -inf (the pages'
    pseudo-sparse fallback: expand the mask, then dense attention)."""
    q, k, v, cu = _tiny_qkv(10)
    bs, Hq, Hkv, sc = 16, 4, 2, 0.25
    r = _rng(11)
    nbs = [(b - a) // bs for a, b in zip(cu[:-1], cu[1:])]
    R = sum(nbs)
    idx = np.full((Hq, R, max(nbs)), -1, np.int32)
    cnt = np.zeros((Hq, R), np.int32)
    row = 0
    for nb in nbs:
        for I in range(nb):
            for h in range(Hq):
                sel = sorted(set(r.choice(I + 1, size=int(r.integers(1, I + 2)), replace=False).tolist()) | {I})
                idx[h, row, :len(sel)] = sel
                cnt[h, row] = len(sel)
            row += 1
    Ob, _ = O.block_sparse_attention(q, k, v, idx, cnt, cu, Hq, Hkv, sc, block_size=bs)
    row0 = 0
    for (a, b), nb in zip(zip(cu[:-1], cu[1:]), nbs):
        L = b - a
        for h in range(Hq):
            g = h // 2
            x = sc * (q[a:b, h] @ k[a:b, g].T)
            mask = np.full((L, L), -np.inf)
            for I in range(nb):
                for J in idx[h, row0 + I, :cnt[h, row0 + I]]:
                    mask[I * bs:(I + 1) * bs, J * bs:(J + 1) * bs] = 0.0
            mask[np.triu_indices(L, 1)] = -np.inf
            x = x + mask
            p = np.exp(x - x.max(axis=1, keepdims=True))
            ref = (p / p.sum(axis=1, keepdims=True)) @ v[a:b, g]
            assert np.allclose(Ob[a:b, h], ref, atol=1e-12)
        row0 += nb


def test_half_height_rows_listing_every_block_equal_dense():
    """P6 for rectangular blocks ([HPC] §三.3.1: 64x128 next to 128x128), here
    8-query rows against 16-key blocks: listing every block that holds a key
    <= the row's last query reproduces dense causal attention."""
    q, k, v, cu = _tiny_qkv(13)
    idx, cnt = O.full_lists(cu, 4, block_size=16, q_block=8)
    assert idx.shape[1] == (96 + 64) // 8
    assert [int(c) for c in cnt[0, :4]] == [1, 1, 2, 2]     # rows 0,1 -> block 0; rows 2,3 -> blocks 0,1
    Ob, lb = O.block_sparse_attention(q, k, v, idx, cnt, cu, 4, 2, 0.25, block_size=16, q_block=8)
    Od, ld = O.dense_causal_attention(q, k, v, cu, 4, 2, 0.25)
    assert np.allclose(Ob, Od, atol=1e-12) and np.allclose(lb, ld, atol=1e-12)


def test_half_height_rows_with_the_parent_lists_equal_square_rows():
    """Both halves of a square row, given the square row's list, see exactly
    the keys the square row sees: same output and LSE."""
    q, k, v, cu = _tiny_qkv(14)
    bs, Hq, Hkv, sc = 16, 4, 2, 0.25
    r = _rng(15)
    nbs = [(b - a) // bs for a, b in zip(cu[:-1], cu[1:])]
    R = sum(nbs)
    idx = np.full((Hq, R, max(nbs)), -1, np.int32)
    cnt = np.zeros((Hq, R), np.int32)
    row = 0
    for nb in nbs:
        for I in range(nb):
            for h in range(Hq):
                sel = sorted(set(r.choice(I + 1, size=int(r.integers(1, I + 2)), replace=False).tolist()) | {I})
                idx[h, row, :len(sel)] = sel
                cnt[h, row] = len(sel)
            row += 1
    Os, ls = O.block_sparse_attention(q, k, v, idx, cnt, cu, Hq, Hkv, sc, block_size=bs)
    Oh, lh = O.block_sparse_attention(q, k, v, np.repeat(idx, 2, axis=1), np.repeat(cnt, 2, axis=1), cu,
                                      Hq, Hkv, sc, block_size=bs, q_block=bs // 2)
    assert np.allclose(Oh, Os, atol=1e-12) and np.allclose(lh, ls, atol=1e-12)


def test_half_height_rows_equal_token_level_masking():
    """Rectangular rows with their own random lists (some without the
    diagonal block, some empty) equal dense attention whose logits are -inf
    outside the listed (row, block) rectangles; an empty row gives 0."""
    q, k, v, cu = _tiny_qkv(16)
    bs, qb, Hq, Hkv, sc = 16, 8, 4, 2, 0.25
    r = _rng(17)
    nrows = [(b - a) // qb for a, b in zip(cu[:-1], cu[1:])]
    R = sum(nrows)
    idx = np.full((Hq, R, 8), -1, np.int32)
    cnt = np.zeros((Hq, R), np.int32)
    row = 0
    for n in nrows:
        for I in range(n):
            top = (I * qb + qb - 1) // bs                # the row's diagonal key block
            for h in range(Hq):
                if r.random() < 0.1:
                    continue                             # empty row
                sel = sorted(r.choice(top + 1, size=int(r.integers(1, top + 2)), replace=False).tolist())
                idx[h, row, :len(sel)] = sel
                cnt[h, row] = len(sel)
            row += 1
    assert (cnt == 0).any() and any(cnt[h, i] > 0 and idx[h, i, cnt[h, i] - 1] < (i % 12) * qb // bs
                                    for h in range(Hq) for i in range(12))
    Ob, _ = O.block_sparse_attention(q, k, v, idx, cnt, cu, Hq, Hkv, sc, block_size=bs, q_block=qb)
    row0 = 0
    for (a, b), n in zip(zip(cu[:-1], cu[1:]), nrows):
        L = b - a
        for h in range(Hq):
            g = h // 2
            x = sc * (q[a:b, h] @ k[a:b, g].T)
            mask = np.full((L, L), -np.inf)
            for I in range(n):
                for J in idx[h, row0 + I, :cnt[h, row0 + I]]:
                    mask[I * qb:(I + 1) * qb, J * bs:(J + 1) * bs] = 0.0
            mask[np.triu_indices(L, 1)] = -np.inf
            x = x + mask
            for t in range(L):
                if np.all(x[t] == -np.inf):
                    assert np.all(Ob[a + t, h] == 0.0)
                    continue
                p = np.exp(x[t] - x[t].max())
                assert np.allclose(Ob[a + t, h], (p / p.sum()) @ v[a:b, g], atol=1e-12)
        row0 += n


def test_empty_row_gives_zero_and_minus_inf_lse():
    q, k, v, cu = _tiny_qkv(12, L=(32,), Hq=2, Hkv=1, d=8)
    idx = np.full((2, 2, 2), -1, np.int32)
    cnt = np.zeros((2, 2), np.int32)
    Ob, lb = O.block_sparse_attention(q, k, v, idx, cnt, cu, 2, 1, 0.5, block_size=16)
    assert np.all(Ob == 0) and np.all(lb == -np.inf)


# ---------------------------------------------------------------- P9 (fp8) ------

def test_e4m3fn_decoder_matches_torch_on_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.decode_e4m3fn(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])


def test_e4m3fn_decoder_spec_values():
    """OCP 8-bit FP spec: 0x38 = 1, 0x7E = 448 (max), 0x08 = 2^-6 (min normal),
    0x01 = 2^-9 (min subnormal), 0x7F / 0xFF = NaN, 0x80 = -0."""
    spec = json.load(open(os.path.join(GOLDEN, "e4m3fn_spec_values.json")))
    for code, val in spec["values"].items():
        got = O.decode_e4m3fn(np.array([int(code, 16)], np.uint8))[0]
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val))


def test_dequantized_blocks_round_trip_within_half_ulp():
    x = torch.randn(256, 2, 32, generator=torch.Generator().manual_seed(0)).to(torch.bfloat16)
    codes, scales = S.quantize_e4m3_per_block(x, (128, 128), 128)
    deq = O.dequantize_blocks(codes.numpy(), scales.numpy(), 128)
    xf = x.to(torch.float64).numpy()
    sc = np.repeat(scales.numpy().astype(np.float64), 128, axis=0)[:, :, None]
    # relative error of a 3-bit mantissa is at most 2^-4 for normals; subnormals
    # have absolute spacing 2^-9 in code units
    err = np.abs(deq - xf)
    assert np.all(err <= np.maximum(np.abs(xf) * 2.0 ** -4, sc * 2.0 ** -10) + 1e-12)


# ---------------------------------------------------------------- golden --------

def test_kstart_table_matches_derivation_script():
    """The k_start values in stem_synth were written by the committed script
    tests/golden/derive_kstart.py, which calls the oracle only."""
    g = json.load(open(os.path.join(GOLDEN, "kstart.json")))
    assert tuple(g["n32k_32q8kv"]) == S.CONFIGS["n32k_32q8kv"].k_start
    assert tuple(g["n128k_32q8kv"]) == S.CONFIGS["n128k_32q8kv"].k_start
    assert {float(k): v for k, v in g["n64k_sweep"].items()} == S.SWEEP_N64K
    assert tuple(g["fp8_varlen_128k"]) == S.FP8_KSTART


def test_n2k_budget_sequence():
    """Config 1 (k_start 8 of 16 blocks, mu 0.5, alpha 1): the decay from 8 to
    mu*8 = 4 over 16 blocks, and the forced sink + window counted inside."""
    ks = [O.tpd_budget(I, 16, 8, 0.5, 1.0) for I in range(16)]
    assert ks == [8, 7, 7, 7, 7, 6, 6, 6, 6, 5, 5, 5, 5, 4, 4, 4]
    kept = [O.kept_count(I, 16, 8, 0.5, 1.0, 1, 1) for I in range(16)]
    assert kept[:9] == [1, 2, 3, 4, 5, 6, 6, 6, 6]
    assert sum(kept) == 71


def test_varlen_packing_equals_separate_sequences():
    """Packing sequences with cu_seqlens changes no score or bonus: each packed
    sequence is scored exactly as if it were alone (no cross-sequence terms)."""
    lens = (256, 512, 384)
    q, k, v = S.make_qkv(lens, 2, 1, 32, seed=13, sink=True)
    qf, kf, vf = (t.to(torch.float64).numpy() for t in (q, k, v))
    cu = S.cu_from_lengths(lens)
    bon = O.value_bonus(vf, cu, 128, 0.2)
    Sp = O.block_scores(qf, kf, bon, cu, 2, 1, 128, 8, 256, 1.0)
    r0 = 0
    for z, L in enumerate(lens):
        a, b = cu[z], cu[z + 1]
        bz = O.value_bonus(vf[a:b], [0, L], 128, 0.2)
        assert np.array_equal(bz, bon[:, a // 128:b // 128])
        Sz = O.block_scores(qf[a:b], kf[a:b], bz, [0, L], 2, 1, 128, 8, 256, 1.0)
        nb = L // 128
        assert np.array_equal(Sp[:, r0:r0 + nb, :nb], Sz[:, :, :nb])
        assert np.all(Sp[:, r0:r0 + nb, nb:] == -np.inf)
        r0 += nb


def _kept_closed_form(I, nb, k_start, mu, alpha, n_init, n_window):
    """gist.science Stem summary §2.1 budget, written out with exact rationals:
    floor(ke - ke (1 - mu) I / nb), ke = alpha k_start, then at least the
    forced blocks and at most the I + 1 causal ones."""
    ke = Fraction(str(alpha)) * Fraction(str(k_start))
    k = math.floor(ke - ke * (1 - Fraction(str(mu))) * Fraction(I, nb))
    forced = len(set(range(min(n_init, I + 1))) | set(range(max(0, I - n_window + 1), I + 1)))
    return min(I + 1, max(k, forced))


@pytest.mark.parametrize("seed", range(3))
def test_schedule_topk_packed_batch_equals_separate_sequences(seed):
    """A packed batch is scheduled row by row exactly as each sequence alone:
    sequence z uses its own k_start[z] and block count, and its rows sit at
    global rows r0(z) .. r0(z) + nb_z - 1.  Every row's count is the closed
    form above, every list is ascending, causal and holds the forced blocks."""
    lens = (384, 1024, 128, 768)
    k_start = [2, 5, 1, 4]
    mu, alpha, n_init, n_window = 0.6, 0.7, 1, 2
    cu = S.cu_from_lengths(lens)
    sc = S.random_scores_like(3, lens, ties=3 if seed == 1 else None, seed=seed).numpy()
    k_cap = max(L // 128 for L in lens) + 2
    idx, cnt = O.schedule_topk(sc, cu, k_start, mu, alpha, n_init, n_window, k_cap)
    r0 = 0
    for z, L in enumerate(lens):
        nb = L // 128
        iz, cz = O.schedule_topk(sc[:, r0:r0 + nb, :nb].copy(), [0, L], [k_start[z]], mu, alpha,
                                 n_init, n_window, k_cap)
        assert np.array_equal(idx[:, r0:r0 + nb], iz) and np.array_equal(cnt[:, r0:r0 + nb], cz)
        for I in range(nb):
            want = _kept_closed_form(I, nb, k_start[z], mu, alpha, n_init, n_window)
            forced = set(range(min(n_init, I + 1))) | set(range(max(0, I - n_window + 1), I + 1))
            for h in range(3):
                row = idx[h, r0 + I, :cnt[h, r0 + I]].tolist()
                assert cnt[h, r0 + I] == want
                assert row == sorted(set(row)) and all(0 <= J <= I for J in row)
                assert forced <= set(row)
                assert np.all(idx[h, r0 + I, cnt[h, r0 + I]:] == -1)
        r0 += nb


def test_signed_zero_scores_tie():
    """-0.0 and +0.0 are equal scores: the lower block index wins either way."""
    row = np.array([1.0, -0.0, 0.0, -0.0, 0.0, -1.0], dtype=np.float32)
    for kept, want in ((2, [0, 1]), (3, [0, 1, 2]), (4, [0, 1, 2, 3])):
        assert O.select_row(row, 5, kept, []) == want
    row2 = np.array([0.0, -0.0, 0.0, 2.0], dtype=np.float32)
    assert O.select_row(row2, 3, 2, []) == [0, 3]
