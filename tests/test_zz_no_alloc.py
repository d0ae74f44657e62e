"""stem_score_noalloc (the score stage with the library's own device scratch
array in place of a workspace) against stem_score (caller's workspace),
through the C ABI: two calls in a row, the second on a smaller problem, each
equal to the workspace call bit for bit (same kernels, same inputs) and
within the score bar of the oracle."""
import numpy as np
import pytest
import torch

import block_sparse_attention_stem_amd as stem
import oracle as O
import stem_synth as S
from gpu_common import check_scores, dev, f64, note, to_dev

pytestmark = pytest.mark.gpu


def _one(lens, Hq, Hkv, seed, beta):
    note(f"[noalloc] lens={lens} Hq={Hq} Hkv={Hkv} seed={seed} beta={beta}")
    cu = S.cu_from_lengths(lens)
    p = stem.Problem(cu, Hq, Hkv)
    q, k, v = S.make_qkv(lens, Hq, Hkv, 128, seed, True)
    qd, kd, vd = to_dev(q, k, v)
    ref = stem.stem_score(p, qd, kd, vd, 8, 2048, 1.0, beta)
    out = torch.full_like(ref, float("nan"))
    stem.stem_score_noalloc(p, qd, kd, vd, out, 8, 2048, 1.0, beta)
    torch.cuda.synchronize()
    assert torch.equal(out, ref), "no-alloc scores differ from the workspace call"
    want = O.block_scores(f64(q), f64(k), O.value_bonus(f64(v), cu, 128, beta), cu, Hq, Hkv, 128, 8, 2048, 1.0)
    check_scores(out.cpu().numpy(), want, f"no-alloc lens={lens}")


def test_noalloc_scores_equal_workspace_scores_on_two_calls():
    # the second call is smaller: every entry it reads must have been rewritten by it
    _one((1280, 640, 384), 8, 2, seed=21, beta=0.2)
    _one((512,), 4, 1, seed=22, beta=0.5)


def test_noalloc_scores_on_more_sequences_than_one_launch_takes():
    # 72 sequences: two launches of the score kernel, each with its own work-queue
    # counters in the scratch array, then a one-launch call again
    _one((128,) * 40 + (256,) * 30 + (384, 128), 4, 2, seed=23, beta=0.2)
    _one((640, 128), 4, 2, seed=24, beta=0.2)
