"""Synthetic reconstruction-error probe, run on the oracle alone.

The Stem paper's ablations compare, on trained models, the token-position
decay budget (TPD) with a uniform budget, and the output-aware metric (OAM:
block score plus the value-magnitude bonus) with the score-only metric (SAM).
The second comparison is reported as a lower reconstruction error of the
attention output (Stem paper summary, ablation paragraph of the results).
Without a model this probe measures that metric,

    err(head) = ||O_sparse - O_dense||_F / ||O_dense||_F    (mean over heads),

on synthetic layers, for selections of equal computed density:

    stem          TPD (mu 0.5) + OAM (beta 0.2)
    sam           TPD (mu 0.5), beta 0
    uniform       mu 1 (a constant budget) + OAM, the constant matched to stem's density
    uniform_sam   the same constant, beta 0
    random        stem's per-row counts and forced blocks, the rest drawn at random
    mass          stem's per-row counts, the rest chosen by each block's exact
                  share of the dense softmax (an ideal the score estimates)

on two input families: the plain Gaussian draw of the benchmark layers, whose
attention is nearly flat, and a planted block-topic draw whose attention
concentrates on a few blocks per query block.

Pinned: SAM and OAM lists have equal sizes; the matched uniform budget is
within 3% of stem's density; at full density every policy is exact; on the
planted draw every informed selection has under half the error of the random
one.  The OAM-vs-SAM and TPD-vs-uniform differences are printed, not
asserted: one synthetic layer settles neither (TPD's case on the pages is
downstream accuracy, which a single layer cannot show).
"""
import math

import numpy as np
import pytest

import oracle as O
import stem_synth as S

T, HQ, HKV, BS = 8192, 4, 1, 128
NB = T // BS
CU = [0, T]
SCALE = 1.0 / math.sqrt(128.0)
K_START, N_INIT, N_WINDOW = 16, 1, 2


def _pairs(cnt_rows):
    """Computed token pairs of lists whose row I holds cnt blocks, diagonal included."""
    return sum((c - 1) * BS * BS + BS * (BS + 1) // 2 for c in cnt_rows)


def _counts(k_start, mu):
    return [O.kept_count(I, NB, k_start, mu, 1.0, N_INIT, N_WINDOW) for I in range(NB)]


def _rel_err(Os, Od):
    return float(np.mean([np.linalg.norm(Os[:, h] - Od[:, h]) / np.linalg.norm(Od[:, h])
                          for h in range(HQ)]))


def _block_mass(q, k):
    """[HQ][NB][NB] share of each key block in the dense causal softmax, summed over the q block."""
    tri = np.triu_indices(T, 1)
    mass = np.zeros((HQ, NB, NB))
    for h in range(HQ):
        x = SCALE * (q[:, h] @ k[:, h // (HQ // HKV)].T)
        x[tri] = -np.inf
        p = np.exp(x - x.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        mass[h] = p.reshape(NB, BS, NB, BS).sum(axis=(1, 3))
    return mass


def _probe(q, k, v, k_start, mu=0.5):
    Od, _ = O.dense_causal_attention(q, k, v, CU, HQ, HKV, SCALE)
    causal = np.tril(np.ones((NB, NB), bool))[None]

    def scores(beta):
        return O.block_scores(q, k, O.value_bonus(v, CU, BS, beta), CU, HQ, HKV, BS, 8, 2048, 1.0)

    def run(S_, ks, mu):
        idx, cnt = O.schedule_topk(S_, CU, [ks], mu, 1.0, N_INIT, N_WINDOW, NB)
        Os, _ = O.block_sparse_attention(q, k, v, idx, cnt, CU, HQ, HKV, SCALE)
        return dict(err=_rel_err(Os, Od), cnt=cnt, density=_pairs(cnt.ravel()) / (HQ * T * (T + 1) / 2))

    target = _pairs(_counts(k_start, mu))
    ku = min(range(1, NB + 1), key=lambda c: abs(_pairs(_counts(c, 1.0)) - target))
    s_oam, s_sam = scores(0.2), scores(0.0)
    rnd = np.where(causal, np.random.default_rng(1).random((HQ, NB, NB)), -np.inf).astype(np.float32)
    mass = np.where(causal, _block_mass(q, k), -np.inf).astype(np.float32)
    return {"stem": run(s_oam, k_start, mu), "sam": run(s_sam, k_start, mu),
            "uniform": run(s_oam, ku, 1.0), "uniform_sam": run(s_sam, ku, 1.0),
            "random": run(rnd, k_start, mu), "mass": run(mass, k_start, mu), "_ku": ku}


@pytest.fixture(scope="module")
def probe():
    gauss = tuple(x.double().numpy() for x in S.make_qkv([T], HQ, HKV, seed=0))
    planted = tuple(x.numpy() for x in S.make_topic_qkv([T], HQ, HKV, seed=0))
    return {"gaussian": (gauss, _probe(*gauss, K_START)),
            "planted": (planted, _probe(*planted, K_START))}


def test_report(probe):
    for fam, (_, res) in probe.items():
        print(f"\n[{fam}] T={T} Hq={HQ} Hkv={HKV}, k_start {K_START}, uniform budget {res['_ku']}")
        for name, r in res.items():
            if not name.startswith("_"):
                print(f"  {name:12s} density {r['density']:.4f}  relative error {r['err']:.4f}")


def test_equal_density(probe):
    for fam, (_, res) in probe.items():
        assert np.array_equal(res["stem"]["cnt"], res["sam"]["cnt"]), fam
        assert np.array_equal(res["stem"]["cnt"], res["random"]["cnt"]), fam
        assert np.array_equal(res["stem"]["cnt"], res["mass"]["cnt"]), fam
        assert np.array_equal(res["uniform"]["cnt"], res["uniform_sam"]["cnt"]), fam
        assert abs(res["uniform"]["density"] / res["stem"]["density"] - 1) < 0.03, fam


def test_full_density_is_exact(probe):
    q, k, v = probe["planted"][0]
    full = _probe(q, k, v, NB, mu=1.0)       # a constant budget of every block
    for name, r in full.items():
        if not name.startswith("_"):
            assert r["density"] == 1.0 and r["err"] < 1e-12, (name, r["err"])


def test_informed_selection_beats_random_on_planted_structure(probe):
    res = probe["planted"][1]
    for name in ("stem", "sam", "uniform", "uniform_sam", "mass"):
        assert res[name]["err"] < 0.5 * res["random"]["err"], (name, res[name]["err"], res["random"]["err"])
