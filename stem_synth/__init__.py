"""Seeded synthetic inputs for the Stem sparse-prefill path.

This module is shared by the tests, the benchmark and the CPU oracle's
checks.  It holds no part of the method's arithmetic (no scoring, no budget,
no selection, no attention): it only draws tensors and packs them, so both
the HIP path and the oracle can be fed the very same bits.

Workload shapes follow the models the Stem paper evaluates (Llama-3.1-8B and
Qwen3-8B: 32 query heads sharing 8 KV heads, head_dim 128; paper summary,
"Results" section) at the context lengths it reports (up to 128K tokens).
The pages publish no tensors, so every input is drawn from a counter-free,
seeded CPU generator and is therefore identical on every machine.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import torch

BLOCK = 128          # attention block size (AngelSlim Stem doc, "Parameters" table)
STRIDE = 8           # scoring down-sampling stride (same table)
CHUNK = 2048         # scoring chunk width (same table)
NORM = 1.0           # extra scoring normaliser n (same table)
BETA = 0.2           # OAM balance coefficient (Stem paper summary, Sec. 2.2 / ablations)
E4M3_MAX = 448.0     # largest finite OCP e4m3fn magnitude


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic attention layer (batch of packed sequences)."""
    name: str
    seqlens: tuple
    num_q_heads: int
    num_kv_heads: int
    head_dim: int = 128
    seed: int = 0
    sink: bool = True            # +3 sigma shared key direction on the first 256 keys
    k_start: tuple = ()          # per sequence, in blocks, before alpha
    mu: float = 0.5
    alpha: float = 1.0
    beta: float = BETA
    n_init: int = 1
    n_window: int = 1
    block_size: int = BLOCK
    stride: int = STRIDE
    chunk_size: int = CHUNK
    norm: float = NORM
    fp8: bool = False

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seqlens))

    @property
    def cu_seqlens(self) -> List[int]:
        cu = [0]
        for n in self.seqlens:
            cu.append(cu[-1] + int(n))
        return cu


def cu_from_lengths(lengths: Sequence[int]) -> List[int]:
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    return cu


# k_start values below were chosen by tests/golden/derive_kstart.py, which
# evaluates the oracle's budget rule and picks the integer whose kept
# block-pair fraction is closest to the target density.
CONFIGS = {
    # 2 query heads share 1 KV head, N = 2048; 8 of 16 key blocks at the start.
    "n2k_2q1kv": Workload("n2k_2q1kv", (2048,), 2, 1, seed=0, sink=False,
                          k_start=(8,), mu=0.5, alpha=1.0, n_init=1, n_window=1),
    # Qwen3-8B-shaped layer at 32K, keep ~25 %.
    "n32k_32q8kv": Workload("n32k_32q8kv", (32768,), 32, 8, seed=0, k_start=(70,),
                            mu=0.5, alpha=0.7, n_init=1, n_window=2),
    # The 128K headline shape, keep ~25 %.
    "n128k_32q8kv": Workload("n128k_32q8kv", (131072,), 32, 8, seed=0, k_start=(276,),
                             mu=0.5, alpha=0.7, n_init=1, n_window=2),
}

# Density sweep at N = 65536: target keep ratio -> k_start (same derivation).
SWEEP_N64K = {1.00: 1461, 0.50: 322, 0.25: 139, 0.20: 108, 0.10: 52}


def sweep_workload(keep: float) -> Workload:
    return Workload(f"n64k_keep{int(round(keep * 100))}", (65536,), 32, 8, seed=0,
                    k_start=(SWEEP_N64K[keep],), mu=0.5, alpha=0.7, n_init=1, n_window=2)


# fp8 varlen batch: four packed sequences, 131072 tokens, 36-layer alpha list
# ([1.0] x 5 + [0.7] x 31, the per-layer example of the AngelSlim Stem doc's
# Python API section).
FP8_SEQLENS = (8192, 16384, 32768, 73728)
FP8_KSTART = (18, 35, 70, 156)
FP8_ALPHAS = tuple([1.0] * 5 + [0.7] * 31)


def fp8_workload(layer: int) -> Workload:
    return Workload(f"fp8_varlen_128k_layer{layer}", FP8_SEQLENS, 32, 8, seed=layer,
                    k_start=FP8_KSTART, mu=0.5, alpha=FP8_ALPHAS[layer],
                    n_init=1, n_window=2, fp8=True)


def make_qkv(seqlens: Sequence[int], num_q_heads: int, num_kv_heads: int,
             head_dim: int = 128, seed: int = 0, sink: bool = True,
             dtype: torch.dtype = torch.bfloat16, device: str = "cpu"):
    """Draw Q, K, V token-major ([T][H][d]).

    Recipe: Q, K, V ~ N(0, 1); each V row is rescaled by a lognormal(0, 0.5)
    norm factor; with `sink`, the first 256 keys of every sequence get a
    shared unit direction times 3 added (attention-sink structure).  Drawn in
    fp32 and rounded once to `dtype` (round-to-nearest-even).

    The draw runs on `device` with a generator seeded there: the default CPU
    draw gives the same bits on every machine (every parity test uses it); a
    GPU draw has the same distribution but other bits, and serves timing runs
    that need many large fresh layers quickly.
    """
    T = int(sum(seqlens))
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    q = torch.randn(T, num_q_heads, head_dim, generator=g, dtype=torch.float32, device=device)
    k = torch.randn(T, num_kv_heads, head_dim, generator=g, dtype=torch.float32, device=device)
    v = torch.randn(T, num_kv_heads, head_dim, generator=g, dtype=torch.float32, device=device)
    r = torch.exp(0.5 * torch.randn(T, num_kv_heads, generator=g, dtype=torch.float32, device=device))
    v.mul_(r.unsqueeze(-1))
    if sink:
        u = torch.randn(num_kv_heads, head_dim, generator=g, dtype=torch.float32, device=device)
        u = u / u.norm(dim=-1, keepdim=True)
        start = 0
        for n in seqlens:
            m = min(256, int(n))
            k[start:start + m] += 3.0 * u
            start += int(n)
    return q.to(dtype), k.to(dtype), v.to(dtype)


def make_workload_qkv(w: Workload, dtype: torch.dtype = torch.bfloat16, device: str = "cpu"):
    return make_qkv(w.seqlens, w.num_q_heads, w.num_kv_heads, w.head_dim, w.seed, w.sink, dtype, device)


def make_topic_qkv(seqlens: Sequence[int], num_q_heads: int, num_kv_heads: int,
                   head_dim: int = 128, seed: int = 0, topics: int = 8, gain: float = 6.0,
                   value_sigma: float = 0.5, block_size: int = BLOCK,
                   dtype: torch.dtype = torch.float64):
    """Q, K, V ([T][H][d]) with planted block-level attention structure.

    Recipe, per sequence and KV head: `topics` random unit directions; every
    key block takes one of them at random and adds `gain` times it to each of
    its keys; every value block is scaled by exp(value_sigma * N(0, 1)).  Per
    query head, every query block adds `gain` times the direction of one
    uniformly drawn causal key block (itself included).  With gain 6 and
    d = 128 a same-topic key scores about gain^2 / sqrt(d) = 3.2 nats above the
    rest, so attention concentrates on the matching blocks, unlike the plain
    Gaussian draw of `make_qkv`, where it is nearly flat.  Base draws are
    N(0, 1) as in `make_qkv`.
    """
    T = int(sum(seqlens))
    grp = num_q_heads // num_kv_heads
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    q = torch.randn(T, num_q_heads, head_dim, generator=g, dtype=torch.float64)
    k = torch.randn(T, num_kv_heads, head_dim, generator=g, dtype=torch.float64)
    v = torch.randn(T, num_kv_heads, head_dim, generator=g, dtype=torch.float64)
    start = 0
    for n in seqlens:
        n = int(n)
        assert n % block_size == 0
        nb = n // block_size
        c = torch.randn(num_kv_heads, topics, head_dim, generator=g, dtype=torch.float64)
        c = c / c.norm(dim=-1, keepdim=True)
        topic = torch.randint(0, topics, (num_kv_heads, nb), generator=g)
        vz = torch.randn(nb, num_kv_heads, generator=g, dtype=torch.float64)
        pick = torch.rand(num_q_heads, nb, generator=g, dtype=torch.float64)
        kb = k[start:start + n].view(nb, block_size, num_kv_heads, head_dim)
        vb = v[start:start + n].view(nb, block_size, num_kv_heads, head_dim)
        qb = q[start:start + n].view(nb, block_size, num_q_heads, head_dim)
        heads = torch.arange(num_kv_heads)
        kb += gain * c[heads[None, :], topic.T][:, None]               # [nb][1][Hkv][d]
        vb *= torch.exp(value_sigma * vz)[:, None, :, None]
        src = (pick * (torch.arange(nb, dtype=torch.float64) + 1)).long()   # [Hq][nb], <= I
        hk = torch.arange(num_q_heads) // grp
        qtopic = topic[hk[:, None], src]                                # [Hq][nb]
        qb += gain * c[hk[:, None], qtopic].permute(1, 0, 2)[:, None]   # [nb][1][Hq][d]
        start += n
    return q.to(dtype), k.to(dtype), v.to(dtype)


def quantize_e4m3_per_block(x: torch.Tensor, seqlens: Sequence[int], block_size: int = BLOCK):
    """Per-(128-token block, head) symmetric e4m3fn quantisation of a [T][H][d] tensor.

    scale = amax / 448 (1 where amax == 0); codes = RNE(x / scale) via torch's
    float8_e4m3fn cast.  Returns (codes uint8 [T][H][d], scales fp32 [nblocks][H]).
    Blocks are counted per sequence (every length must be a multiple of the
    block size), so scale row b belongs to packed tokens [128 b, 128 b + 128).
    """
    T, H, d = x.shape
    assert T % block_size == 0
    for n in seqlens:
        assert int(n) % block_size == 0
    xf = x.to(torch.float32).reshape(T // block_size, block_size, H, d)
    amax = xf.abs().amax(dim=(1, 3))                      # [nb][H]
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    y = xf / scale[:, None, :, None]
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).reshape(T, H, d)
    return codes.contiguous(), scale.contiguous()


def random_scores_like(num_heads: int, seqlens: Sequence[int], block_size: int = BLOCK,
                       seed: int = 0, ties: Optional[int] = None):
    """Random fp32 block-score rows [H][total_qblocks][max_nb] for selection tests.

    Entries J > I (non-causal) and J >= nb of the row's sequence are -inf, as
    the scoring stage writes them.  With `ties`, values are drawn from a small
    integer set {0..ties-1} so that equal scores are common.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    nbs = [int(n) // block_size for n in seqlens]
    R, maxnb = sum(nbs), max(nbs)
    if ties:
        s = torch.randint(0, ties, (num_heads, R, maxnb), generator=g).to(torch.float32)
    else:
        s = torch.randn(num_heads, R, maxnb, generator=g, dtype=torch.float32)
    r = 0
    for nb in nbs:
        for I in range(nb):
            s[:, r, I + 1:] = float("-inf")
            r += 1
    return s
