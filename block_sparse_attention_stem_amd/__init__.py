"""Python binding of libstem.so: the MI355X Stem sparse-prefill path.

Argument marshalling only.  Every step of the path runs in the library's
HIP kernels; torch is used for device memory and the current stream.  The
functions carry the C names (include/stem.h):

    stem_score(problem, q, k, v, ...)           -> block scores
    stem_schedule_topk(problem, scores, ...)    -> (block_idx, block_cnt)
    stem_bsa_prefill(problem, q, k, v, idx, cnt, ...) -> out (and lse)
    stem_dense_prefill(problem, q, k, v, ...)   -> out (and lse)

Importing this module never falls back to anything: if libstem.so is missing
or fails to load, calls raise.

Streams: work goes on `stream` (a torch.cuda.Stream), else on torch's current
stream.  Tensors a call allocates itself (outputs, workspaces) come from
torch's caching allocator on the current stream; with another stream, make it
wait on the current one first (stream.wait_stream) or pass preallocated
tensors.  Temporaries a call drops before returning (its own workspaces, the
intermediate scores and lists of stem_prefill) are recorded on `stream`, so
their memory is not handed out again before the work queued there is done.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libstem.so")

STEM_OK = 0
STEM_DTYPE_BF16 = 0
STEM_DTYPE_FP8_E4M3 = 1
STEM_DTYPE_FP8_E4M3_PV16 = 2     # e4m3 inputs, P.V with fp16 weights
STATUS = {0: "STEM_OK", 1: "STEM_ERR_INVALID_ARG", 2: "STEM_ERR_UNSUPPORTED",
          3: "STEM_ERR_CAPACITY", 4: "STEM_ERR_WORKSPACE", 5: "STEM_ERR_HIP"}

# Defaults of the AngelSlim Stem parameter table (doc §6); beta from the
# paper's OAM setting.
DEFAULTS = dict(block_size=128, stride=8, chunk_size=2048, norm=1.0,
                initial_blocks=4, window_size=4, stem_alpha=1.0, beta=0.2)

EXPORTED = ("stem_status_string", "stem_score_workspace_bytes", "stem_score", "stem_score_fp8",
            "stem_score_noalloc",
            "stem_schedule_topk", "stem_tpd_budget", "stem_kept_count", "stem_max_kept",
            "stem_attn_workspace_bytes", "stem_bsa_prefill", "stem_dense_prefill",
            "stem_bsa_prefill_paged", "stem_bsa_prefill_q64")


class StemError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {STATUS.get(status, status)}")
        self.status = status


class stem_problem_t(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32),
                ("cu_seqlens_host", ctypes.POINTER(ctypes.c_int32)),
                ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libstem.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m block_sparse_attention_stem_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(stem_problem_t)
    vp, i32, f32, f64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_double, ctypes.c_size_t
    lib.stem_status_string.argtypes = [ctypes.c_int]
    lib.stem_status_string.restype = ctypes.c_char_p
    lib.stem_score_workspace_bytes.argtypes = [P]
    lib.stem_score_workspace_bytes.restype = sz
    lib.stem_score.argtypes = [P, vp, vp, vp, i32, i32, f32, f32, vp, vp, sz, vp]
    lib.stem_score.restype = ctypes.c_int
    lib.stem_score_noalloc.argtypes = [P, vp, vp, vp, i32, i32, f32, f32, vp, vp]
    lib.stem_score_noalloc.restype = ctypes.c_int
    lib.stem_score_fp8.argtypes = [P, vp, vp, vp, vp, vp, vp, i32, i32, f32, f32, vp, vp, sz, vp]
    lib.stem_score_fp8.restype = ctypes.c_int
    lib.stem_schedule_topk.argtypes = [P, vp, ctypes.POINTER(f64), f64, f64, i32, i32, i32, vp, vp, vp]
    lib.stem_schedule_topk.restype = ctypes.c_int
    lib.stem_tpd_budget.argtypes = [i32, i32, f64, f64, f64]
    lib.stem_tpd_budget.restype = i32
    lib.stem_kept_count.argtypes = [i32, i32, f64, f64, f64, i32, i32]
    lib.stem_kept_count.restype = i32
    lib.stem_max_kept.argtypes = [P, ctypes.POINTER(f64), f64, f64, i32, i32]
    lib.stem_max_kept.restype = i32
    lib.stem_attn_workspace_bytes.argtypes = [P, i32]
    lib.stem_attn_workspace_bytes.restype = sz
    lib.stem_bsa_prefill.argtypes = [P, i32, vp, vp, vp, vp, vp, vp, vp, vp, i32, f32, vp, vp, vp, sz, vp]
    lib.stem_bsa_prefill.restype = ctypes.c_int
    lib.stem_dense_prefill.argtypes = [P, i32, vp, vp, vp, vp, vp, vp, f32, vp, vp, vp, sz, vp]
    lib.stem_dense_prefill.restype = ctypes.c_int
    lib.stem_bsa_prefill_paged.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, i32, f32, vp, vp,
                                           vp, sz, vp]
    lib.stem_bsa_prefill_paged.restype = ctypes.c_int
    lib.stem_bsa_prefill_q64.argtypes = [P, vp, vp, vp, vp, vp, i32, f32, vp, vp, vp, sz, vp]
    lib.stem_bsa_prefill_q64.restype = ctypes.c_int
    _lib = lib
    return lib


class Problem:
    """Shape of one packed batch: cu_seqlens (token offsets) and head counts."""

    def __init__(self, cu_seqlens: Sequence[int], num_q_heads: int, num_kv_heads: int,
                 head_dim: int = 128, block_size: int = 128):
        self.cu = [int(x) for x in cu_seqlens]
        self._cu_arr = (ctypes.c_int32 * len(self.cu))(*self.cu)
        self.c = stem_problem_t(len(self.cu) - 1, self._cu_arr, num_q_heads, num_kv_heads,
                                head_dim, block_size)
        self.Hq, self.Hkv, self.d, self.bs = num_q_heads, num_kv_heads, head_dim, block_size
        self.T = self.cu[-1]
        self.nbs = [(b - a) // block_size for a, b in zip(self.cu[:-1], self.cu[1:])]
        self.R = sum(self.nbs)
        self.max_nb = max(self.nbs)

    @property
    def ref(self):
        return ctypes.byref(self.c)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on_stream(t: Optional[torch.Tensor], stream):
    """Record a temporary on `stream` (see the module docstring)."""
    if stream is not None and t is not None:
        t.record_stream(stream)


def _check(fn: str, st: int):
    if st != STEM_OK:
        raise StemError(fn, st)


def _need(t: torch.Tensor, name: str, dtype, shape):
    if not t.is_cuda or t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name}: expected contiguous cuda {dtype} {tuple(shape)}, got "
                         f"{t.device} {t.dtype} {tuple(t.shape)}")


def stem_score_workspace_bytes(p: Problem) -> int:
    return int(load_library().stem_score_workspace_bytes(p.ref))


def stem_score(p: Problem, q, k, v, stride: int = 8, chunk_size: int = 2048, norm: float = 1.0,
               beta: float = 0.2, scores: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None, stream=None, scales=None) -> torch.Tensor:
    """Block scores fp32 [Hq][R][max_nb] (-inf for J > I and J >= nb).

    bf16 q, k, v; or e4m3 codes with scales = (q_scale, k_scale, v_scale) as in
    stem_bsa_prefill (stem_score_fp8: the scores of the dequantised values)."""
    lib = load_library()
    fp8 = q.dtype != torch.bfloat16
    if fp8:
        q, k, v = (t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t for t in (q, k, v))
        if scales is None or len(scales) != 3:
            raise ValueError("e4m3 scoring needs (q_scale, k_scale, v_scale)")
        _need(scales[0], "q_scale", torch.float32, (p.R, p.Hq))
        _need(scales[1], "k_scale", torch.float32, (p.R, p.Hkv))
        _need(scales[2], "v_scale", torch.float32, (p.R, p.Hkv))
    elif scales is not None:
        raise ValueError("bf16 scoring takes no scales")
    dt = torch.uint8 if fp8 else torch.bfloat16
    _need(q, "q", dt, (p.T, p.Hq, p.d))
    _need(k, "k", dt, (p.T, p.Hkv, p.d))
    _need(v, "v", dt, (p.T, p.Hkv, p.d))
    if scores is None:
        scores = torch.empty((p.Hq, p.R, p.max_nb), dtype=torch.float32, device=q.device)
    _need(scores, "scores", torch.float32, (p.Hq, p.R, p.max_nb))
    nbytes = stem_score_workspace_bytes(p)
    own_ws = workspace is None
    if own_ws:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    wsb = workspace.numel() * workspace.element_size()
    if fp8:
        st = lib.stem_score_fp8(p.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(scales[0]), _ptr(scales[1]), _ptr(scales[2]),
                                stride, chunk_size, float(norm), float(beta), _ptr(scores), _ptr(workspace), wsb,
                                _stream(stream))
        _check("stem_score_fp8", st)
    else:
        st = lib.stem_score(p.ref, _ptr(q), _ptr(k), _ptr(v), stride, chunk_size, float(norm),
                            float(beta), _ptr(scores), _ptr(workspace), wsb, _stream(stream))
        _check("stem_score", st)
    if own_ws:
        _on_stream(workspace, stream)
    return scores


STEM_SCORE_SCRATCH_BYTES = (1 << 20) + 4096   # the library's own scratch per GPU (stem_score_noalloc)


def stem_score_noalloc(p: Problem, q, k, v, scores: torch.Tensor, stride: int = 8, chunk_size: int = 2048,
                       norm: float = 1.0, beta: float = 0.2, stream=None) -> torch.Tensor:
    """stem_score without a workspace: the library's own device scratch array
    stands in for it, and nothing is allocated here either (`scores` must be
    preallocated fp32 [Hq][R][max_nb]).  Calls that overlap on one GPU race."""
    lib = load_library()
    for name, t, h in (("q", q, p.Hq), ("k", k, p.Hkv), ("v", v, p.Hkv)):
        _need(t, name, torch.bfloat16, (p.T, h, p.d))
    _need(scores, "scores", torch.float32, (p.Hq, p.R, p.max_nb))
    st = lib.stem_score_noalloc(p.ref, _ptr(q), _ptr(k), _ptr(v), stride, chunk_size, float(norm), float(beta),
                                _ptr(scores), _stream(stream))
    _check("stem_score_noalloc", st)
    return scores


def _kstart_arr(p: Problem, k_start):
    """One k_start per sequence (a scalar applies to every sequence)."""
    n = len(p.cu) - 1
    ks = [float(k_start)] * n if isinstance(k_start, (int, float)) else [float(x) for x in k_start]
    if len(ks) != n:
        raise ValueError(f"k_start: expected {n} values (one per sequence), got {len(ks)}")
    return (ctypes.c_double * n)(*ks)


def stem_max_kept(p: Problem, k_start, mu: float, alpha: float, n_init: int, n_window: int) -> int:
    return int(load_library().stem_max_kept(p.ref, _kstart_arr(p, k_start), mu, alpha, n_init, n_window))


def stem_tpd_budget(I: int, nb: int, k_start: float, mu: float, alpha: float) -> int:
    return int(load_library().stem_tpd_budget(I, nb, k_start, mu, alpha))


def stem_kept_count(I: int, nb: int, k_start: float, mu: float, alpha: float,
                    n_init: int, n_window: int) -> int:
    return int(load_library().stem_kept_count(I, nb, k_start, mu, alpha, n_init, n_window))


def stem_schedule_topk(p: Problem, scores: torch.Tensor, k_start, mu: float, alpha: float,
                       n_init: int, n_window: int, k_cap: Optional[int] = None,
                       block_idx: Optional[torch.Tensor] = None,
                       block_cnt: Optional[torch.Tensor] = None, stream=None):
    """Compact ascending block lists: (idx int32 [Hq][R][k_cap], cnt int32 [Hq][R])."""
    lib = load_library()
    _need(scores, "scores", torch.float32, (p.Hq, p.R, p.max_nb))
    ks = _kstart_arr(p, k_start)
    if k_cap is None:
        k_cap = max(1, int(lib.stem_max_kept(p.ref, ks, mu, alpha, n_init, n_window)))
    if block_idx is None:
        block_idx = torch.empty((p.Hq, p.R, k_cap), dtype=torch.int32, device=scores.device)
    if block_cnt is None:
        block_cnt = torch.empty((p.Hq, p.R), dtype=torch.int32, device=scores.device)
    _need(block_idx, "block_idx", torch.int32, (p.Hq, p.R, k_cap))
    _need(block_cnt, "block_cnt", torch.int32, (p.Hq, p.R))
    st = lib.stem_schedule_topk(p.ref, _ptr(scores), ks, float(mu), float(alpha), int(n_init),
                                int(n_window), int(k_cap), _ptr(block_idx), _ptr(block_cnt),
                                _stream(stream))
    _check("stem_schedule_topk", st)
    return block_idx, block_cnt


def _attn_inputs(p: Problem, q, k, v, scales, fp16_weights: bool = False):
    if q.dtype == torch.bfloat16:
        dt = STEM_DTYPE_BF16
        for name, t, h in (("q", q, p.Hq), ("k", k, p.Hkv), ("v", v, p.Hkv)):
            _need(t, name, torch.bfloat16, (p.T, h, p.d))
        if scales is not None:
            raise ValueError("bf16 attention takes no scales")
        if fp16_weights:
            raise ValueError("fp16_weights applies to e4m3 inputs only")
        return dt, (None, None, None)
    dt = STEM_DTYPE_FP8_E4M3_PV16 if fp16_weights else STEM_DTYPE_FP8_E4M3
    for name, t, h in (("q", q, p.Hq), ("k", k, p.Hkv), ("v", v, p.Hkv)):
        if t.dtype == torch.float8_e4m3fn:
            t = t.view(torch.uint8)
        _need(t, name, torch.uint8, (p.T, h, p.d))
    if scales is None or len(scales) != 3:
        raise ValueError("fp8 attention needs (q_scale, k_scale, v_scale)")
    qs, kss, vs = scales
    _need(qs, "q_scale", torch.float32, (p.R, p.Hq))
    _need(kss, "k_scale", torch.float32, (p.R, p.Hkv))
    _need(vs, "v_scale", torch.float32, (p.R, p.Hkv))
    return dt, (qs, kss, vs)


def stem_attn_workspace_bytes(p: Problem, dtype: int = STEM_DTYPE_BF16) -> int:
    return int(load_library().stem_attn_workspace_bytes(p.ref, dtype))


def _attn_workspace(p: Problem, dt: int, workspace, device, stream):
    n = stem_attn_workspace_bytes(p, dt)
    if workspace is None:
        workspace = torch.empty(n, dtype=torch.uint8, device=device)
        _on_stream(workspace, stream)     # dropped on return, read by work queued on `stream`
    if workspace.numel() * workspace.element_size() < n:
        raise ValueError(f"workspace: need {n} bytes")
    return workspace


def stem_bsa_prefill(p: Problem, q, k, v, block_idx, block_cnt, softmax_scale: Optional[float] = None,
                     scales=None, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                     want_lse: bool = False, workspace: Optional[torch.Tensor] = None, stream=None,
                     fp16_weights: bool = False):
    """Causal block-sparse attention over the lists: out bf16 [T][Hq][d] (+ lse fp32 [Hq][T]).

    fp16_weights (e4m3 inputs only): P.V with fp16 instead of e4m3 weights."""
    lib = load_library()
    dt, (qs, kss, vs) = _attn_inputs(p, q, k, v, scales, fp16_weights)
    _need(block_cnt, "block_cnt", torch.int32, (p.Hq, p.R))
    if block_idx.dtype != torch.int32 or block_idx.dim() != 3 or tuple(block_idx.shape[:2]) != (p.Hq, p.R) \
            or not block_idx.is_contiguous():
        raise ValueError("block_idx: expected contiguous int32 [Hq][R][k_cap]")
    scale = 1.0 / math.sqrt(p.d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty((p.T, p.Hq, p.d), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, (p.T, p.Hq, p.d))
    if want_lse and lse is None:
        lse = torch.empty((p.Hq, p.T), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, (p.Hq, p.T))
    ws = _attn_workspace(p, dt, workspace, q.device, stream)
    st = lib.stem_bsa_prefill(p.ref, dt, _ptr(q), _ptr(k), _ptr(v), _ptr(qs), _ptr(kss), _ptr(vs),
                              _ptr(block_idx), _ptr(block_cnt), int(block_idx.shape[2]), scale,
                              _ptr(out), _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(),
                              _stream(stream))
    _check("stem_bsa_prefill", st)
    return (out, lse) if lse is not None else out


def stem_bsa_prefill_q64(p: Problem, q, k, v, block_idx, block_cnt, softmax_scale: Optional[float] = None,
                         out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                         want_lse: bool = False, workspace: Optional[torch.Tensor] = None, stream=None):
    """bf16 block-sparse attention over 64-query rows: block_idx int32 [Hq][2R][k_cap],
    block_cnt int32 [Hq][2R]; list row 2r + s covers queries [64 s, 64 s + 64) of block row r."""
    lib = load_library()
    if q.dtype != torch.bfloat16:
        raise ValueError("stem_bsa_prefill_q64: bf16 inputs only")
    dt, _ = _attn_inputs(p, q, k, v, None)
    _need(block_cnt, "block_cnt", torch.int32, (p.Hq, 2 * p.R))
    if block_idx.dtype != torch.int32 or block_idx.dim() != 3 or tuple(block_idx.shape[:2]) != (p.Hq, 2 * p.R) \
            or not block_idx.is_contiguous():
        raise ValueError("block_idx: expected contiguous int32 [Hq][2R][k_cap]")
    scale = 1.0 / math.sqrt(p.d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty((p.T, p.Hq, p.d), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, (p.T, p.Hq, p.d))
    if want_lse and lse is None:
        lse = torch.empty((p.Hq, p.T), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, (p.Hq, p.T))
    ws = _attn_workspace(p, dt, workspace, q.device, stream)
    st = lib.stem_bsa_prefill_q64(p.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(block_idx), _ptr(block_cnt),
                                  int(block_idx.shape[2]), scale, _ptr(out), _ptr(lse), _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream))
    _check("stem_bsa_prefill_q64", st)
    return (out, lse) if lse is not None else out


def stem_bsa_prefill_paged(p: Problem, q, k_pages, v_pages, block_table, block_idx, block_cnt,
                           softmax_scale: Optional[float] = None, scales=None,
                           out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                           want_lse: bool = False, workspace: Optional[torch.Tensor] = None, stream=None):
    """Block-sparse fp8 attention with K/V in a page pool.

    q: e4m3 [T][Hq][d]; k_pages, v_pages: e4m3 [num_pages][128][Hkv][d];
    block_table: int32 [num_seqs][table_stride] (page of key block J of sequence z);
    scales = (q_scale [R][Hq], k_scale [num_pages][Hkv], v_scale [num_pages][Hkv]).
    """
    lib = load_library()
    q8 = q.view(torch.uint8) if q.dtype == torch.float8_e4m3fn else q
    kp = k_pages.view(torch.uint8) if k_pages.dtype == torch.float8_e4m3fn else k_pages
    vpg = v_pages.view(torch.uint8) if v_pages.dtype == torch.float8_e4m3fn else v_pages
    _need(q8, "q", torch.uint8, (p.T, p.Hq, p.d))
    n_pages = int(kp.shape[0])
    _need(kp, "k_pages", torch.uint8, (n_pages, 128, p.Hkv, p.d))
    _need(vpg, "v_pages", torch.uint8, (n_pages, 128, p.Hkv, p.d))
    if scales is None or len(scales) != 3:
        raise ValueError("paged fp8 attention needs (q_scale, k_scale, v_scale)")
    qs, kss, vs = scales
    _need(qs, "q_scale", torch.float32, (p.R, p.Hq))
    _need(kss, "k_scale", torch.float32, (n_pages, p.Hkv))
    _need(vs, "v_scale", torch.float32, (n_pages, p.Hkv))
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != len(p.nbs) \
            or not block_table.is_contiguous():
        raise ValueError("block_table: expected contiguous int32 [num_seqs][table_stride]")
    _need(block_cnt, "block_cnt", torch.int32, (p.Hq, p.R))
    if block_idx.dtype != torch.int32 or block_idx.dim() != 3 or tuple(block_idx.shape[:2]) != (p.Hq, p.R) \
            or not block_idx.is_contiguous():
        raise ValueError("block_idx: expected contiguous int32 [Hq][R][k_cap]")
    scale = 1.0 / math.sqrt(p.d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty((p.T, p.Hq, p.d), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, (p.T, p.Hq, p.d))
    if want_lse and lse is None:
        lse = torch.empty((p.Hq, p.T), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, (p.Hq, p.T))
    ws = _attn_workspace(p, STEM_DTYPE_FP8_E4M3, workspace, q.device, stream)
    st = lib.stem_bsa_prefill_paged(p.ref, _ptr(q8), _ptr(kp), _ptr(vpg), _ptr(qs), _ptr(kss), _ptr(vs),
                                    _ptr(block_table), int(block_table.shape[1]), n_pages, _ptr(block_idx),
                                    _ptr(block_cnt), int(block_idx.shape[2]), scale, _ptr(out), _ptr(lse),
                                    _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check("stem_bsa_prefill_paged", st)
    return (out, lse) if lse is not None else out


def stem_dense_prefill(p: Problem, q, k, v, softmax_scale: Optional[float] = None, scales=None,
                       out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                       want_lse: bool = False, workspace: Optional[torch.Tensor] = None, stream=None,
                       fp16_weights: bool = False):
    """Dense causal attention with the same tile kernel (fp16_weights as in stem_bsa_prefill)."""
    lib = load_library()
    dt, (qs, kss, vs) = _attn_inputs(p, q, k, v, scales, fp16_weights)
    scale = 1.0 / math.sqrt(p.d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty((p.T, p.Hq, p.d), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, (p.T, p.Hq, p.d))
    if want_lse and lse is None:
        lse = torch.empty((p.Hq, p.T), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, (p.Hq, p.T))
    ws = _attn_workspace(p, dt, workspace, q.device, stream)
    st = lib.stem_dense_prefill(p.ref, dt, _ptr(q), _ptr(k), _ptr(v), _ptr(qs), _ptr(kss), _ptr(vs),
                                scale, _ptr(out), _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(),
                                _stream(stream))
    _check("stem_dense_prefill", st)
    return (out, lse) if lse is not None else out


def stem_prefill(p: Problem, q, k, v, k_start, mu: float = 0.5, alpha: float = 1.0,
                 n_init: int = DEFAULTS["initial_blocks"], n_window: int = DEFAULTS["window_size"],
                 stride: int = DEFAULTS["stride"], chunk_size: int = DEFAULTS["chunk_size"],
                 norm: float = DEFAULTS["norm"], beta: float = DEFAULTS["beta"],
                 fp8_inputs=None, softmax_scale: Optional[float] = None, stream=None,
                 fp16_weights: bool = False, fp8_scoring: bool = False):
    """The whole path for one layer: score -> schedule/top-k -> block-sparse attention.

    Scoring runs on the bf16 q, k, v.  With `fp8_inputs = (q8, k8, v8, (qs, ks, vs))`
    the attention stage runs on those e4m3 tensors instead (with fp16_weights,
    P.V keeps fp16 weights; see stem_bsa_prefill), and with fp8_scoring the
    scoring stage too (stem_score_fp8; q, k, v may then be None).
    """
    if fp8_scoring:
        if fp8_inputs is None:
            raise ValueError("fp8_scoring needs fp8_inputs")
        q8, k8, v8, sc = fp8_inputs
        s = stem_score(p, q8, k8, v8, stride, chunk_size, norm, beta, stream=stream, scales=sc)
    else:
        s = stem_score(p, q, k, v, stride, chunk_size, norm, beta, stream=stream)
    idx, cnt = stem_schedule_topk(p, s, k_start, mu, alpha, n_init, n_window, stream=stream)
    for t in (s, idx, cnt):
        _on_stream(t, stream)             # intermediates, dropped on return
    if fp8_inputs is None:
        if fp16_weights:
            raise ValueError("fp16_weights applies to fp8_inputs only")
        return stem_bsa_prefill(p, q, k, v, idx, cnt, softmax_scale, stream=stream)
    q8, k8, v8, sc = fp8_inputs
    return stem_bsa_prefill(p, q8, k8, v8, idx, cnt, softmax_scale, scales=sc, stream=stream,
                            fp16_weights=fp16_weights)
