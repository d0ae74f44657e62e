"""CPU oracle for Stem's sparse-prefill attention path.

TEST INFRASTRUCTURE ONLY.  This module is a plain, slow, obviously-correct
numpy implementation (fp64 arithmetic, fp32 stored scores) used to check the
HIP path.  Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import it; the product library never calls into it, and it shares no
code, header, table or helper with the HIP kernels.

Sources (the pages as published; cited by title and section):
  [DOC]   AngelSlim documentation, "Stem: Rethinking Causal Information Flow in
          Sparse Attention" (features/sparse_attention/stem.md): §2.1 Block-Level
          Scoring (score formula), §2.2 Top-k Schedule, §2.3 Block-Sparse
          Attention, §6 parameter table.
  [ZH]    gist.science Chinese summary of the Stem paper: §2.1 TPD (budget
          formula), §2.2 OAM, §2.3 overall flow.
  [DE]    gist.science German summary of the Stem paper: §2A TPD, §2B OAM, §2C.
  [FORUM] zhichai.net summary of the AngelSlim Stem page: §三 (TPD, sinks and
          windows), §四 Steps 1-3.
  [HPC]   youleyou.com article on Stem and the HPC-BSA operators: §二.2.2 (log
          turns the product into a sum), §三.3.1 (skipped block == -inf).

Readings taken where the pages are silent or disagree (each is listed with its
reason in the design notes of the repository):
  * score = Q.K^T / (sqrt(d) * s * n) + beta * ReLU(vbar_J)   ([DOC] §2.1), with
    vbar the z-scored log of the block max of ||V_t||^2, z-scored per
    (sequence, KV head) over that sequence's key blocks, population std, eps 1e-6.
  * The strided score pairs the anti-diagonal of every stride x stride token
    tile ([ZH] §2.3, [DE] §2C): query token i*s+t meets key token j*s+(s-1-t).
  * Strided causal mask j <= i; pooled 128x128 block score = max over the
    16x16 strided cells of the block (no softmax, [ZH] §2.2 "avoid exponentials").
  * TPD budget k(I) = floor(ke - ke*(1-mu)*I/nb) with ke = alpha*k_start, I the
    0-based query block index and nb the sequence's block count ([ZH] §2.1).
  * Forced blocks: sinks [0, n_init) and the window [I-n_window+1, I]; kept(I)
    = min(I+1, max(k(I), |F(I)|)); the rest are the top-scoring causal blocks,
    ties to the lower block index, NaN treated as -inf.  Lists are ascending.
  * softmax scale 1/sqrt(d).

Parity unpinned: the absolute score values at real shapes and the choice
among the readings above (standardisation scope, pooling granularity, how
alpha composes with mu) have no printed value on the pages to pin against;
the checks in tests/test_oracle_pins.py pin everything else.
"""
from __future__ import annotations

import math
from fractions import Fraction
from typing import List, Sequence, Tuple

import numpy as np

NEG_INF = float("-inf")


# --------------------------------------------------------------------------
# O1: inputs.  The oracle takes float64 arrays that are exact upcasts of the
# bf16 inputs; fp8 inputs come as raw e4m3fn codes plus per-block scales and
# are decoded here from the OCP 8-bit floating point definition.
# --------------------------------------------------------------------------

def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """Decode OCP e4m3fn codes (uint8) to float64.

    Layout S.EEEE.MMM, exponent bias 7, no infinities, S.1111.111 is NaN,
    exponent field 0 encodes subnormals m * 2^-9 (OCP 8-bit FP spec).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = (1.0 + m / 8.0) * np.power(2.0, e - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    val = np.where(e == 0, sub, normal) * sign
    val = np.where((e == 0xF) & (m == 0x7), np.nan, val)
    return val


def dequantize_blocks(codes: np.ndarray, scales: np.ndarray, block_size: int = 128) -> np.ndarray:
    """codes [T][H][d] uint8, scales [T/block][H] -> float64 [T][H][d]."""
    x = decode_e4m3fn(codes)
    T, H, d = x.shape
    s = np.asarray(scales, dtype=np.float64)
    return (x.reshape(T // block_size, block_size, H, d) * s[:, None, :, None]).reshape(T, H, d)


def _seq_bounds(cu_seqlens: Sequence[int]) -> List[Tuple[int, int]]:
    return [(int(cu_seqlens[z]), int(cu_seqlens[z + 1])) for z in range(len(cu_seqlens) - 1)]


# --------------------------------------------------------------------------
# O2: the output-aware value bonus ([DOC] §2.1: lambda * ReLU(vbar_j), vbar the
# standardised log value norm; [ZH] §2.2: block-wise max pooling of the value
# magnitude, no exponentials).
# --------------------------------------------------------------------------

def block_log_value_norm(v_seq: np.ndarray, block_size: int) -> np.ndarray:
    """l_J = ln(max_{t in block J} ||V_t||^2) for one sequence, one KV head."""
    e = np.sum(v_seq.astype(np.float64) ** 2, axis=-1)            # [L]
    emax = e.reshape(-1, block_size).max(axis=1)                  # [nb]
    return np.log(np.maximum(emax, 1e-30))


def value_bonus(v: np.ndarray, cu_seqlens: Sequence[int], block_size: int = 128,
                beta: float = 0.2) -> np.ndarray:
    """bonus[g][global key block] = beta * max(0, zscore(l_J)) per (sequence, KV head)."""
    T, Hkv, _ = v.shape
    out = np.zeros((Hkv, T // block_size), dtype=np.float64)
    for (a, b) in _seq_bounds(cu_seqlens):
        for g in range(Hkv):
            ell = block_log_value_norm(v[a:b, g, :], block_size)
            mu = ell.mean()
            sd = math.sqrt(float(np.mean((ell - mu) ** 2)))       # population std
            z = (ell - mu) / (sd + 1e-6)
            out[g, a // block_size:b // block_size] = beta * np.maximum(0.0, z)
    return out


# --------------------------------------------------------------------------
# O3/O4: strided anti-diagonal scores, max-pooled to block scores
# ([DOC] §2.1 strided group GEMM with stride s and chunk width; [FORUM] §四
# Step 1; [ZH] §2.3 anti-diagonal down-sampling).
# --------------------------------------------------------------------------

def strided_scores(q_seq: np.ndarray, k_seq: np.ndarray, stride: int, scale: float,
                   row0: int = 0, row1: int = -1) -> np.ndarray:
    """A[i, j] for strided query rows [row0, row1) against strided key rows [0, row1).

    A[i, j] = scale * sum_t q[i*s + t] . k[j*s + s-1-t]; entries with j > i are -inf.
    Written as one GEMM on the reshaped rows: query rows take their s tokens in
    order, key rows take theirs reversed, so each product pairs an
    anti-diagonal of the s x s token tile.
    """
    L, d = q_seq.shape
    n = L // stride
    if row1 < 0:
        row1 = n
    qr = q_seq[row0 * stride:row1 * stride].astype(np.float64).reshape(row1 - row0, stride * d)
    kr = k_seq[:row1 * stride].astype(np.float64).reshape(row1, stride, d)[:, ::-1, :].reshape(row1, stride * d)
    A = (qr @ kr.T) * scale
    i = np.arange(row0, row1)[:, None]
    j = np.arange(row1)[None, :]
    A[j > i] = NEG_INF
    return A


def block_scores(q: np.ndarray, k: np.ndarray, bonus: np.ndarray, cu_seqlens: Sequence[int],
                 num_q_heads: int, num_kv_heads: int, block_size: int = 128, stride: int = 8,
                 chunk_size: int = 2048, norm: float = 1.0,
                 heads: Sequence[int] = None, rows: Sequence[int] = None) -> np.ndarray:
    """S[h][global q block][J] (fp32) = max-pooled strided score + bonus[kv(h)][J].

    Entries with J > I or J >= nb of the sequence are -inf.  The query axis is
    processed `chunk_size` tokens at a time, as the scoring stage does; the
    chunk width changes the memory footprint only, never a value.
    `heads` restricts the computation to a subset of query heads and `rows` to
    a subset of global query-block rows (everything else stays -inf).
    """
    T, _, d = q.shape
    m = block_size // stride
    seqs = _seq_bounds(cu_seqlens)
    nbs = [(b - a) // block_size for a, b in seqs]
    R, maxnb = sum(nbs), max(nbs)
    S = np.full((num_q_heads, R, maxnb), NEG_INF, dtype=np.float32)
    scale = 1.0 / (math.sqrt(d) * stride * norm)
    group = num_q_heads // num_kv_heads
    hs = range(num_q_heads) if heads is None else heads
    want = None if rows is None else set(int(r) for r in rows)
    r0 = 0
    for (a, b), nb in zip(seqs, nbs):
        for h in hs:
            g = h // group
            qs, ks = q[a:b, h, :], k[a:b, g, :]
            for c0 in range(0, b - a, chunk_size):
                c1 = min(c0 + chunk_size, b - a)
                I0, I1 = c0 // block_size, c1 // block_size
                if want is not None and not any(r0 + I in want for I in range(I0, I1)):
                    continue
                A = strided_scores(qs, ks, stride, scale, c0 // stride, c1 // stride)
                ncol = A.shape[1]
                pooled = A.reshape(I1 - I0, m, ncol // m, m).max(axis=(1, 3))   # [I][J]
                for I in range(I0, I1):
                    if want is not None and r0 + I not in want:
                        continue
                    row = pooled[I - I0, :I + 1] + bonus[g, a // block_size:a // block_size + I + 1]
                    S[h, r0 + I, :I + 1] = row.astype(np.float32)
        r0 += nb
    return S


# --------------------------------------------------------------------------
# O5: Token-Position-Decay budget ([ZH] §2.1: k(i) = floor(k_start -
# k_start (1 - mu) i / N), decaying linearly to k_end = mu k_start; [DOC] §2.2
# per-layer alpha; [FORUM] §三 sinks and window always kept).
# --------------------------------------------------------------------------

def _exact(x) -> Fraction:
    # Decimal reading of a parameter as the user wrote it (0.7 means 7/10).
    return Fraction(repr(x)) if isinstance(x, float) else Fraction(x)


ALPHA_SCALES_KSTART = True   # reading R10: ke = alpha * k_start (alternative: alpha is mu)


def tpd_budget(I: int, nb: int, k_start, mu, alpha) -> int:
    """k(I) for local query block I of a sequence with nb blocks, exact rationals."""
    if ALPHA_SCALES_KSTART:
        ke = _exact(alpha) * _exact(k_start)
        mu_f = _exact(mu)
    else:  # pragma: no cover - the rival reading, kept as a one-line switch
        ke = _exact(k_start)
        mu_f = _exact(alpha)
    val = ke - ke * (1 - mu_f) * Fraction(I, nb)
    return math.floor(val)


def forced_blocks(I: int, n_init: int, n_window: int) -> List[int]:
    """Sink blocks [0, n_init) and window blocks [I - n_window + 1, I], clipped to [0, I]."""
    f = set(range(0, min(n_init, I + 1)))
    f.update(range(max(0, I - n_window + 1), I + 1))
    return sorted(f)


def kept_count(I: int, nb: int, k_start, mu, alpha, n_init: int, n_window: int) -> int:
    k = tpd_budget(I, nb, k_start, mu, alpha)
    return min(I + 1, max(k, len(forced_blocks(I, n_init, n_window))))


# --------------------------------------------------------------------------
# O6: per-query-block top-k into compact ascending lists ([FORUM] §四 Step 2-3;
# [DOC] §2.3 top-k mask).
# --------------------------------------------------------------------------

def select_row(scores_row: np.ndarray, I: int, kept: int, forced: Sequence[int]) -> List[int]:
    """Forced blocks plus the best (kept - |F|) other causal blocks, ascending.

    Order: score descending, then block index ascending; NaN counts as -inf.
    """
    fset = set(forced)
    cand = [J for J in range(I + 1) if J not in fset]
    def key(J):
        s = float(scores_row[J])
        if math.isnan(s):
            s = NEG_INF
        return (-s, J)
    cand.sort(key=key)
    need = max(0, kept - len(fset))
    return sorted(list(fset) + cand[:need])


def schedule_topk(S: np.ndarray, cu_seqlens: Sequence[int], k_start: Sequence, mu, alpha,
                  n_init: int, n_window: int, k_cap: int, block_size: int = 128,
                  heads: Sequence[int] = None):
    """idx int32 [H][R][k_cap] (ascending, -1 padded) and cnt int32 [H][R]."""
    H, R, _ = S.shape
    idx = np.full((H, R, k_cap), -1, dtype=np.int32)
    cnt = np.zeros((H, R), dtype=np.int32)
    hs = range(H) if heads is None else heads
    r = 0
    for z, (a, b) in enumerate(_seq_bounds(cu_seqlens)):
        nb = (b - a) // block_size
        for I in range(nb):
            kept = kept_count(I, nb, k_start[z], mu, alpha, n_init, n_window)
            forced = forced_blocks(I, n_init, n_window)
            for h in hs:
                sel = select_row(S[h, r], I, kept, forced)
                assert len(sel) <= k_cap
                idx[h, r, :len(sel)] = sel
                cnt[h, r] = len(sel)
            r += 1
    return idx, cnt


# --------------------------------------------------------------------------
# O7: causal block-sparse attention on the listed blocks ([DOC] §2.3; [FORUM]
# §四 Step 3: exact softmax and aggregation on the selected blocks only).
# --------------------------------------------------------------------------

def block_sparse_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, idx: np.ndarray,
                           cnt: np.ndarray, cu_seqlens: Sequence[int], num_q_heads: int,
                           num_kv_heads: int, softmax_scale: float, block_size: int = 128,
                           rows: Sequence[Tuple[int, int]] = None, q_block: int = None):
    """O float64 [T][Hq][d] and lse float64 [Hq][T] (natural log).

    For each (head h, query block I) gather the key/value tokens of the listed
    blocks, mask keys later than the query, softmax in fp64 and aggregate.  An
    empty list gives O = 0 and lse = -inf.  `rows` restricts the work to the
    listed (h, global q block) pairs (other outputs stay NaN).

    Query blocks have `q_block` tokens (default: `block_size`) and key blocks
    `block_size` tokens: the rectangular block shapes of the HPC-BSA operators
    ([HPC] §三.3.1 names 64x128 next to 128x128).  Row I of a sequence covers
    queries [I q_block, (I+1) q_block); its list holds key-block ids.
    """
    T, _, d = q.shape
    qb_len = block_size if q_block is None else int(q_block)
    group = num_q_heads // num_kv_heads
    O = np.full((T, num_q_heads, d), np.nan)
    lse = np.full((num_q_heads, T), np.nan)
    seqs = _seq_bounds(cu_seqlens)
    row_seq = []
    for z, (a, b) in enumerate(seqs):
        for I in range((b - a) // qb_len):
            row_seq.append((z, I))
    work = rows if rows is not None else [(h, r) for h in range(num_q_heads) for r in range(len(row_seq))]
    for (h, r) in work:
        z, I = row_seq[r]
        a = seqs[z][0]
        g = h // group
        q0 = a + I * qb_len
        qb = q[q0:q0 + qb_len, h, :].astype(np.float64)
        blocks = [int(J) for J in idx[h, r, :int(cnt[h, r])]]
        if not blocks:
            O[q0:q0 + qb_len, h, :] = 0.0
            lse[h, q0:q0 + qb_len] = NEG_INF
            continue
        kpos = np.concatenate([np.arange(J * block_size, (J + 1) * block_size) for J in blocks])
        ks = k[a + kpos, g, :].astype(np.float64)
        vs = v[a + kpos, g, :].astype(np.float64)
        x = softmax_scale * (qb @ ks.T)                              # [q_block][n]
        qpos = np.arange(I * qb_len, (I + 1) * qb_len)[:, None]
        x[kpos[None, :] > qpos] = NEG_INF
        mx = x.max(axis=1, keepdims=True)
        p = np.exp(x - mx)
        den = p.sum(axis=1, keepdims=True)
        O[q0:q0 + qb_len, h, :] = (p @ vs) / den
        lse[h, q0:q0 + qb_len] = (mx + np.log(den))[:, 0]
    return O, lse


# --------------------------------------------------------------------------
# O8: dense causal attention, the baseline every speedup is measured against.
# Written as the plain full-matrix definition, not through the block lists.
# --------------------------------------------------------------------------

def dense_causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_seqlens: Sequence[int],
                           num_q_heads: int, num_kv_heads: int, softmax_scale: float,
                           heads: Sequence[int] = None, q_range: Tuple[int, int] = None):
    """softmax(scale * q k^T + causal mask) v per sequence and head, fp64.

    `heads` / `q_range` (local token range applied to every sequence) restrict
    the work; outputs outside it stay NaN.
    """
    T, _, d = q.shape
    group = num_q_heads // num_kv_heads
    O = np.full((T, num_q_heads, d), np.nan)
    lse = np.full((num_q_heads, T), np.nan)
    hs = range(num_q_heads) if heads is None else heads
    for (a, b) in _seq_bounds(cu_seqlens):
        t0, t1 = (0, b - a) if q_range is None else (q_range[0], min(q_range[1], b - a))
        for h in hs:
            g = h // group
            qs = q[a + t0:a + t1, h, :].astype(np.float64)
            ks = k[a:a + t1, g, :].astype(np.float64)
            vs = v[a:a + t1, g, :].astype(np.float64)
            x = softmax_scale * (qs @ ks.T)
            qp = np.arange(t0, t1)[:, None]
            kp = np.arange(t1)[None, :]
            x[kp > qp] = NEG_INF
            mx = x.max(axis=1, keepdims=True)
            p = np.exp(x - mx)
            den = p.sum(axis=1, keepdims=True)
            O[a + t0:a + t1, h, :] = (p @ vs) / den
            lse[h, a + t0:a + t1] = (mx + np.log(den))[:, 0]
    return O, lse


def full_lists(cu_seqlens: Sequence[int], num_q_heads: int, block_size: int = 128,
               q_block: int = None):
    """Every causal block listed (idx, cnt), for the all-kept special case.

    With `q_block`, rows are query blocks of that many tokens; row I lists
    every key block holding a key <= its last query.
    """
    qb_len = block_size if q_block is None else int(q_block)
    seqs = _seq_bounds(cu_seqlens)
    nrows = [(b - a) // qb_len for a, b in seqs]
    R = sum(nrows)
    last = [((n * qb_len - 1) // block_size) + 1 for n in nrows]
    idx = np.full((num_q_heads, R, max(last)), -1, dtype=np.int32)
    cnt = np.zeros((num_q_heads, R), dtype=np.int32)
    r = 0
    for n in nrows:
        for I in range(n):
            c = ((I + 1) * qb_len - 1) // block_size + 1
            idx[:, r, :c] = np.arange(c)
            cnt[:, r] = c
            r += 1
    return idx, cnt
