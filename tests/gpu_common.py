"""Helpers shared by the GPU parity tests (inputs, oracle calls, tolerances)."""
import math
import sys

import numpy as np
import torch

import block_sparse_attention_stem_amd as stem
import oracle as O
import stem_synth as S

# Tolerances of the acceptance bar for this path.
SCORE_REL = 1e-3            # |d| <= 1e-3 * max(|ref|, 1) on finite entries
BF16_MAX_ABS = 1e-2
BF16_MEAN_REL = 2e-3
FP8_MAX_ABS = 6e-2


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda:0")


def f64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def make_inputs(seqlens, Hq, Hkv, seed=0, sink=True):
    q, k, v = S.make_qkv(seqlens, Hq, Hkv, 128, seed, sink)
    return q, k, v


def to_dev(*ts):
    return [t.to(dev()) for t in ts]


def check_scores(gpu, ref, where=""):
    gpu = gpu.astype(np.float64)
    ref = ref.astype(np.float64)
    ninf_g, ninf_r = np.isneginf(gpu), np.isneginf(ref)
    assert np.array_equal(ninf_g, ninf_r), f"-inf pattern differs {where}"
    fin = ~ninf_r
    err = np.abs(gpu[fin] - ref[fin]) / np.maximum(np.abs(ref[fin]), 1.0)
    worst = float(err.max()) if err.size else 0.0
    note(f"  scores {where}: {fin.sum()} finite entries, max scaled err {worst:.3e}")
    assert worst <= SCORE_REL, f"score error {worst} {where}"


def bf16_half_ulp(x):
    """Half the spacing of bf16 numbers at |x| (8 significant bits)."""
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - 8), 0.0)


def check_out(gpu, ref, max_abs, mean_rel=None, where=""):
    """Output bar: |gpu - ref| <= max_abs + half a bf16 ulp of ref, element-wise.

    The output is stored in bf16; storing a value rounds it by up to half an
    ulp, which alone exceeds 1e-2 once |O| >= 4.  The max-abs bar therefore
    bounds the arithmetic error on top of that unavoidable storage rounding.
    The mean-rel bar (mean |d| / mean |ref|) is applied as is.
    """
    g = gpu.astype(np.float64)
    r = ref.astype(np.float64)
    ok = ~np.isnan(r)
    d = np.abs(g[ok] - r[ok])
    excess = d - bf16_half_ulp(r[ok])
    ma = float(d.max())
    me = float(excess.max())
    mr = float(d.mean() / max(np.abs(r[ok]).mean(), 1e-30))
    note(f"  out {where}: max-abs {ma:.3e} (beyond bf16 storage rounding {me:.3e})  "
         f"mean-rel {mr:.3e}  ({ok.sum()} values)")
    assert me <= max_abs, f"max-abs beyond storage rounding {me} > {max_abs} {where}"
    if mean_rel is not None:
        assert mr <= mean_rel, f"mean-rel {mr} > {mean_rel} {where}"


def check_lse(gpu, ref, where=""):
    ok = ~np.isnan(ref)
    fin = ok & np.isfinite(ref)
    assert np.array_equal(np.isneginf(gpu[ok]), np.isneginf(ref[ok])), where
    d = float(np.abs(gpu[fin] - ref[fin]).max()) if fin.any() else 0.0
    note(f"  lse {where}: max-abs {d:.3e}")
    assert d <= 1e-3, f"lse error {d} {where}"


def lists_equal(idx_g, cnt_g, idx_r, cnt_r, where=""):
    assert np.array_equal(cnt_g, cnt_r), f"counts differ {where}"
    assert np.array_equal(idx_g, idx_r), f"lists differ {where}"


def quantize_fp8(q, k, v, seqlens):
    q8, qs = S.quantize_e4m3_per_block(q, seqlens)
    k8, ks = S.quantize_e4m3_per_block(k, seqlens)
    v8, vs = S.quantize_e4m3_per_block(v, seqlens)
    return (q8, k8, v8), (qs, ks, vs)


def dequant(codes, scales):
    return O.dequantize_blocks(codes.numpy(), scales.numpy(), 128)


def page_pool(k8, v8, ks, vs, seqlens, spare=7, seed=0):
    """Scatter the per-block e4m3 K/V codes and scales of packed sequences
    into a shuffled page pool with `spare` unused pages filled with NaN codes
    (0x7F) and NaN scales, so that any read of a wrong page shows up.
    Returns (k_pages, v_pages, k_scale_pages, v_scale_pages, table), CPU."""
    T, Hkv, d = k8.shape
    R = T // 128
    n_pages = R + spare
    perm = torch.randperm(n_pages, generator=torch.Generator().manual_seed(seed))
    kp = torch.full((n_pages, 128, Hkv, d), 0x7F, dtype=torch.uint8)
    vp = torch.full((n_pages, 128, Hkv, d), 0x7F, dtype=torch.uint8)
    ksp = torch.full((n_pages, Hkv), float("nan"), dtype=torch.float32)
    vsp = torch.full((n_pages, Hkv), float("nan"), dtype=torch.float32)
    kp[perm[:R]] = k8.reshape(R, 128, Hkv, d)
    vp[perm[:R]] = v8.reshape(R, 128, Hkv, d)
    ksp[perm[:R]] = ks
    vsp[perm[:R]] = vs
    nbs = [int(n) // 128 for n in seqlens]
    stride = max(nbs) + 3
    table = torch.full((len(nbs), stride), -5, dtype=torch.int32)   # unused columns hold garbage
    r = 0
    for z, nb in enumerate(nbs):
        table[z, :nb] = perm[r:r + nb].to(torch.int32)
        r += nb
    return kp, vp, ksp, vsp, table


def random_q64_lists(seqlens, Hq, seed=0, p_empty=0.1, spare=2):
    """Random lists for 64-query rows (row 2r + s of a sequence lists
    128-token key blocks in [0, r]): ascending, random sizes, about p_empty
    of the rows empty and many without the diagonal block; -1 padded to the
    longest list plus `spare`.  Returns (idx [Hq][R64][k_cap], cnt [Hq][R64]) int32."""
    rng = np.random.default_rng(seed)
    rows = []                                   # diagonal block of every 64-query row
    for L in seqlens:
        rows += [r64 // 2 for r64 in range(int(L) // 64)]
    k_cap = max(rows) + 1 + spare
    idx = np.full((Hq, len(rows), k_cap), -1, np.int32)
    cnt = np.zeros((Hq, len(rows)), np.int32)
    for h in range(Hq):
        for i, top in enumerate(rows):
            if rng.random() < p_empty:
                continue
            sel = np.sort(rng.choice(top + 1, size=int(rng.integers(1, top + 2)), replace=False))
            idx[h, i, :sel.size] = sel
            cnt[h, i] = sel.size
    return idx, cnt
