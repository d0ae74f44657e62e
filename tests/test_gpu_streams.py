"""The library enqueues its work on the caller's stream and nowhere else:
the whole path run on a side stream equals the default-stream run bit for
bit, and the path captured into a HIP graph (every buffer allocated before
the capture; the path issues kernel launches only, no memsets or copies)
replays correctly on new inputs, each replay checked against an eager run
with eager work and synchronisation in between."""
import math

import torch
import pytest

import block_sparse_attention_stem_amd as stem
import stem_synth as S
from gpu_common import dev, note, to_dev

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(128.0)
LENS = (512, 1280, 768)
HQ, HKV = 8, 2
KSTART, MU, ALPHA = [2, 5, 3], 0.5, 0.7


class Buffers:
    """Every output and workspace of one pass, allocated up front."""

    def __init__(self, p):
        d = dev()
        self.kcap = stem.stem_max_kept(p, KSTART, MU, ALPHA, 1, 2)
        self.scores = torch.empty((p.Hq, p.R, p.max_nb), dtype=torch.float32, device=d)
        self.sws = torch.empty(stem.stem_score_workspace_bytes(p), dtype=torch.uint8, device=d)
        self.idx = torch.empty((p.Hq, p.R, self.kcap), dtype=torch.int32, device=d)
        self.cnt = torch.empty((p.Hq, p.R), dtype=torch.int32, device=d)
        self.aws = torch.empty(stem.stem_attn_workspace_bytes(p), dtype=torch.uint8, device=d)
        self.out = torch.empty((p.T, p.Hq, 128), dtype=torch.bfloat16, device=d)
        self.lse = torch.empty((p.Hq, p.T), dtype=torch.float32, device=d)


def _pass(p, q, k, v, b, stream=None):
    stem.stem_score(p, q, k, v, scores=b.scores, workspace=b.sws, stream=stream)
    stem.stem_schedule_topk(p, b.scores, KSTART, MU, ALPHA, 1, 2, b.kcap, b.idx, b.cnt, stream=stream)
    stem.stem_bsa_prefill(p, q, k, v, b.idx, b.cnt, SCALE, out=b.out, lse=b.lse, workspace=b.aws, stream=stream)


def _same(a, b):
    return all(torch.equal(x, y) for x, y in ((a.scores, b.scores), (a.idx, b.idx), (a.cnt, b.cnt),
                                              (a.out, b.out), (a.lse, b.lse)))


def test_side_stream_equals_default_stream():
    p = stem.Problem(S.cu_from_lengths(LENS), HQ, HKV)
    q, k, v = to_dev(*S.make_qkv(LENS, HQ, HKV, 128, 21, True))
    ref, side_b = Buffers(p), Buffers(p)
    _pass(p, q, k, v, ref)
    side = torch.cuda.Stream()                     # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _pass(p, q, k, v, side_b)                  # the wrapper passes torch's current stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert _same(ref, side_b)
    # and an explicit stream argument from the default stream's context
    exp_b = Buffers(p)
    side.wait_stream(torch.cuda.current_stream())
    _pass(p, q, k, v, exp_b, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert _same(ref, exp_b)


def test_graph_capture_replays_match_eager():
    p = stem.Problem(S.cu_from_lengths(LENS), HQ, HKV)
    q, k, v = to_dev(*S.make_qkv(LENS, HQ, HKV, 128, 31, True))
    gb = Buffers(p)
    # warm up on a side stream, as graph capture expects
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _pass(p, q, k, v, gb)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _pass(p, q, k, v, gb)
    eb = Buffers(p)
    for rep, seed in enumerate((41, 42, 43)):
        nq, nk, nv = to_dev(*S.make_qkv(LENS, HQ, HKV, 128, seed, True))
        q.copy_(nq)
        k.copy_(nk)
        v.copy_(nv)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _pass(p, q, k, v, eb)                      # eager, same inputs
        torch.cuda.synchronize()
        note(f"  graph replay {rep} (inputs seed {seed})")
        assert _same(gb, eb), f"replay {rep} differs from the eager pass"


def test_side_stream_with_the_calls_own_temporaries():
    """stem_prefill on a side stream allocates its workspaces, scores and lists
    itself and drops them on return; while its kernels may still run, the
    current stream allocates and fills fresh memory.  The temporaries are
    recorded on the side stream, so that memory is not handed out again early
    and the result equals the default-stream call."""
    p = stem.Problem(S.cu_from_lengths(LENS), HQ, HKV)
    q, k, v = to_dev(*S.make_qkv(LENS, HQ, HKV, 128, 51, True))
    ref = stem.stem_prefill(p, q, k, v, KSTART, MU, ALPHA, 1, 2)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    for rep in range(3):
        side.wait_stream(torch.cuda.current_stream())
        out = stem.stem_prefill(p, q, k, v, KSTART, MU, ALPHA, 1, 2, stream=side)
        junk = [torch.full((1 << 18,), float(rep), device=dev()) for _ in range(16)]
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        note(f"  side-stream stem_prefill {rep}: {len(junk)} buffers filled meanwhile")
        assert torch.equal(out, ref), f"side-stream call {rep} differs"
        del junk


def test_graph_capture_of_the_fp8_layer_with_e4m3_scoring():
    """Scoring on e4m3 codes, selection and fp8 attention captured into one HIP
    graph; three replays on new codes and scales equal eager runs."""
    from gpu_common import quantize_fp8
    p = stem.Problem(S.cu_from_lengths(LENS), HQ, HKV)

    def codes(seed):
        q, k, v = S.make_qkv(LENS, HQ, HKV, 128, seed, True)
        (q8, k8, v8), (qs, ks, vs) = quantize_fp8(q, k, v, LENS)
        return to_dev(q8, k8, v8, qs, ks, vs)

    x = codes(61)
    kcap = stem.stem_max_kept(p, KSTART, MU, ALPHA, 1, 2)
    d = dev()

    def bufs():
        return dict(s=torch.empty((p.Hq, p.R, p.max_nb), dtype=torch.float32, device=d),
                    sws=torch.empty(stem.stem_score_workspace_bytes(p), dtype=torch.uint8, device=d),
                    idx=torch.empty((p.Hq, p.R, kcap), dtype=torch.int32, device=d),
                    cnt=torch.empty((p.Hq, p.R), dtype=torch.int32, device=d),
                    aws=torch.empty(stem.stem_attn_workspace_bytes(p, stem.STEM_DTYPE_FP8_E4M3), dtype=torch.uint8,
                                    device=d),
                    out=torch.empty((p.T, p.Hq, 128), dtype=torch.bfloat16, device=d))

    def run(b):
        q8, k8, v8, qs, ks, vs = x
        stem.stem_score(p, q8, k8, v8, scores=b["s"], workspace=b["sws"], scales=(qs, ks, vs))
        stem.stem_schedule_topk(p, b["s"], KSTART, MU, ALPHA, 1, 2, kcap, b["idx"], b["cnt"])
        stem.stem_bsa_prefill(p, q8, k8, v8, b["idx"], b["cnt"], SCALE, scales=(qs, ks, vs), out=b["out"],
                              workspace=b["aws"])

    gb, eb = bufs(), bufs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(gb)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(gb)
    for rep, seed in enumerate((62, 63, 64)):
        for dst, src in zip(x, codes(seed)):
            dst.copy_(src)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        run(eb)
        torch.cuda.synchronize()
        note(f"  fp8 graph replay {rep} (codes seed {seed})")
        for key in ("s", "idx", "cnt", "out"):
            assert torch.equal(gb[key], eb[key]), f"replay {rep}: {key} differs from the eager pass"
