"""CPU-only checks of the C ABI: the library loads, exports every symbol that
include/stem.h declares, its host-side budget rule equals the oracle's exact
rational TPD on every row of every workload, and invalid calls are rejected
before anything touches a device (no compute calls here)."""
import ctypes
import os
import re

import pytest
import torch

import block_sparse_attention_stem_amd as stem
import oracle as O
import stem_synth as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    src = open(os.path.join(ROOT, "include", "stem.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(stem_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = stem.load_library()
    names = _declared_symbols()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(stem.EXPORTED)


def test_status_strings():
    lib = stem.load_library()
    for code, name in stem.STATUS.items():
        assert lib.stem_status_string(code).decode() == name
    assert lib.stem_status_string(99).decode() == "STEM_ERR_UNKNOWN"


def _all_workloads():
    ws = list(S.CONFIGS.values()) + [S.sweep_workload(k) for k in S.SWEEP_N64K] + \
        [S.fp8_workload(0), S.fp8_workload(5)]
    return ws


@pytest.mark.parametrize("w", _all_workloads(), ids=lambda w: w.name)
def test_host_budget_matches_oracle_exact_rationals_on_every_row(w):
    for z, L in enumerate(w.seqlens):
        nb = L // 128
        for I in range(nb):
            assert stem.stem_tpd_budget(I, nb, w.k_start[z], w.mu, w.alpha) == \
                O.tpd_budget(I, nb, w.k_start[z], w.mu, w.alpha)
            assert stem.stem_kept_count(I, nb, w.k_start[z], w.mu, w.alpha, w.n_init, w.n_window) == \
                O.kept_count(I, nb, w.k_start[z], w.mu, w.alpha, w.n_init, w.n_window)


@pytest.mark.parametrize("params", [(13, 0.7, 1.0, 1, 1), (100, 0.3, 0.7, 4, 4), (5, 1.0, 0.7, 0, 0),
                                    (37, 0.55, 0.9, 2, 3), (0, 0.5, 1.0, 2, 0)])
def test_host_budget_matches_oracle_other_parameters(params):
    ks, mu, alpha, ni, nw = params
    for nb in (1, 7, 64, 333):
        for I in range(nb):
            assert stem.stem_kept_count(I, nb, ks, mu, alpha, ni, nw) == \
                O.kept_count(I, nb, ks, mu, alpha, ni, nw)


def test_max_kept_is_the_row_maximum():
    w = S.fp8_workload(6)
    p = stem.Problem(w.cu_seqlens, 32, 8)
    got = stem.stem_max_kept(p, w.k_start, w.mu, w.alpha, w.n_init, w.n_window)
    ref = max(O.kept_count(I, L // 128, w.k_start[z], w.mu, w.alpha, w.n_init, w.n_window)
              for z, L in enumerate(w.seqlens) for I in range(L // 128))
    assert got == ref


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation


def _score(p, stride=8, chunk=2048, norm=1.0, beta=0.2, ws=FAKE, wsb=1 << 20, q=FAKE):
    return stem.load_library().stem_score(p.ref, q, FAKE, FAKE, stride, chunk, norm, beta, FAKE,
                                          ws, wsb, None)


def test_score_argument_errors():
    p = stem.Problem([0, 1024], 4, 2)
    assert _score(p, q=None) == 1
    assert _score(p, stride=3) == 1
    assert _score(p, stride=4) == 2                      # valid, not implemented
    assert _score(p, chunk=100) == 1
    assert _score(p, norm=0.0) == 1
    assert _score(p, beta=-1.0) == 1
    assert _score(p, ws=None) == 4
    assert _score(p, wsb=8) == 4
    assert _score(p, ws=ctypes.c_void_p(0x1004)) == 4    # misaligned
    assert _score(stem.Problem([0, 1000], 4, 2)) == 2    # ragged tail block
    assert _score(stem.Problem([0, 1024], 4, 3)) == 1    # Hq % Hkv != 0
    assert _score(stem.Problem([0, 1024], 4, 2, head_dim=64)) == 2
    assert _score(stem.Problem([0, 1024], 4, 2, block_size=64)) == 2
    assert _score(stem.Problem([0, 1024, 1024], 4, 2)) == 1   # empty sequence
    assert _score(stem.Problem([0, 128 * 65537], 4, 2), wsb=1 << 30) == 2   # longer than 65536 blocks
    # 2 x 8 fp32 block values, then 8 queue counters, each part padded to 256 bytes
    assert stem.stem_score_workspace_bytes(stem.Problem([0, 1024], 4, 2)) == 512
    assert stem.stem_score_workspace_bytes(stem.Problem([0] + [128 * (i + 1) for i in range(65)], 4, 2)) == 1024   # 520 -> 768, two launches of counters -> 256
    # e4m3 scoring: every scale pointer is required; the rest as stem_score
    lib = stem.load_library()
    p = stem.Problem([0, 1024], 4, 2)

    def s8(qs=FAKE, ks=FAKE, vs=FAKE, stride=8, ws=FAKE):
        return lib.stem_score_fp8(p.ref, FAKE, FAKE, FAKE, qs, ks, vs, stride, 2048, 1.0, 0.2, FAKE, ws, 1 << 20, None)
    assert s8(qs=None) == 1
    assert s8(ks=None) == 1
    assert s8(vs=None) == 1
    assert s8(stride=4) == 2
    assert s8(ws=None) == 4


def test_schedule_argument_errors():
    lib = stem.load_library()
    p = stem.Problem([0, 4096], 4, 2)
    ks = (ctypes.c_double * 1)(10.0)

    def call(mu=0.5, alpha=1.0, ni=1, nw=1, cap=32, kss=ks, idx=FAKE):
        return lib.stem_schedule_topk(p.ref, FAKE, kss, mu, alpha, ni, nw, cap, idx, FAKE, None)
    assert call(mu=0.0) == 1
    assert call(mu=1.5) == 1
    assert call(alpha=0.0) == 1
    assert call(ni=-1) == 1
    assert call(idx=None) == 1
    assert call(kss=(ctypes.c_double * 1)(-1.0)) == 1
    assert stem.stem_max_kept(p, 10.0, 0.5, 1.0, 1, 1) == 8   # rows 7..9 keep 8 blocks
    assert call(cap=7) == 3
    big = stem.Problem([0, 128 * 4096], 4, 2)
    assert lib.stem_schedule_topk(big.ref, FAKE, ks, 0.5, 1.0, 1, 1, 4096, FAKE, FAKE, None) == 2


def test_attention_argument_errors():
    lib = stem.load_library()
    p = stem.Problem([0, 1024], 4, 2)
    f = FAKE
    W = 1 << 30
    assert lib.stem_bsa_prefill(p.ref, 0, f, f, f, None, None, None, None, f, 8, 0.1, f, None, f, W, None) == 1
    assert lib.stem_bsa_prefill(p.ref, 0, f, f, f, f, None, None, f, f, 8, 0.1, f, None, f, W, None) == 1
    assert lib.stem_bsa_prefill(p.ref, 1, f, f, f, None, None, None, f, f, 8, 0.1, f, None, f, W, None) == 1
    assert lib.stem_bsa_prefill(p.ref, 7, f, f, f, None, None, None, f, f, 8, 0.1, f, None, f, W, None) == 2
    assert lib.stem_bsa_prefill(p.ref, 0, f, f, f, None, None, None, f, f, 0, 0.1, f, None, f, W, None) == 1
    assert lib.stem_bsa_prefill(p.ref, 0, f, f, f, None, None, None, f, f, 8, 0.1, f, None, None, W, None) == 4
    assert lib.stem_bsa_prefill(p.ref, 0, f, f, f, None, None, None, f, f, 8, 0.1, f, None, f, 100, None) == 4
    assert lib.stem_dense_prefill(p.ref, 0, f, f, f, None, None, None, -1.0, f, None, f, W, None) == 1
    assert lib.stem_dense_prefill(p.ref, 0, None, f, f, None, None, None, 0.1, f, None, f, W, None) == 1
    assert lib.stem_dense_prefill(p.ref, 0, f, f, f, None, None, None, 0.1, f, None, ctypes.c_void_p(0x1010),
                                  W, None) == 4
    # dtype 2 (e4m3 inputs, fp16 weights for P.V) needs the fp8 scales and workspace too
    assert lib.stem_bsa_prefill(p.ref, 2, f, f, f, None, None, None, f, f, 8, 0.1, f, None, f, W, None) == 1
    assert lib.stem_dense_prefill(p.ref, 2, f, f, f, f, f, f, 0.1, f, None, f, 100, None) == 4
    assert lib.stem_dense_prefill(p.ref, 3, f, f, f, f, f, f, 0.1, f, None, f, W, None) == 2
    # the V^T images (and fp8 row scales), then 256 bytes of work-queue counters
    # (8 per launch of up to 64 sequences)
    assert stem.stem_attn_workspace_bytes(p, 0) == 1024 * 2 * 272 + 256
    assert stem.stem_attn_workspace_bytes(p, 1) == (1024 * 2 * 416 + (1024 // 128) * 2 * 8 + 255) // 256 * 256 + 256
    p70 = stem.Problem([128 * i for i in range(71)], 4, 2)            # 70 sequences: two launches
    assert stem.stem_attn_workspace_bytes(p70, 0) == 70 * 128 * 2 * 272 + 256
    assert stem.stem_attn_workspace_bytes(p, 2) == stem.stem_attn_workspace_bytes(p, 1)
    assert stem.stem_attn_workspace_bytes(p, 5) == 0
    with pytest.raises(ValueError):
        stem.stem_dense_prefill(p, torch.zeros(1024, 4, 128, dtype=torch.bfloat16),
                                torch.zeros(1024, 2, 128, dtype=torch.bfloat16),
                                torch.zeros(1024, 2, 128, dtype=torch.bfloat16), fp16_weights=True)


def test_paged_attention_argument_errors():
    """Every call below carries one invalid argument, so nothing is launched."""
    lib = stem.load_library()
    p = stem.Problem([0, 1024], 4, 2)                 # 8 key blocks
    f = FAKE
    W = 1 << 30
    call = lib.stem_bsa_prefill_paged
    # null table, empty pool, table rows shorter than the longest sequence
    assert call(p.ref, f, f, f, f, f, f, None, 8, 16, f, f, 8, 0.1, f, None, f, W, None) == 1
    assert call(p.ref, f, f, f, f, f, f, f, 8, 0, f, f, 8, 0.1, f, None, f, W, None) == 1
    assert call(p.ref, f, f, f, f, f, f, f, 7, 16, f, f, 8, 0.1, f, None, f, W, None) == 1
    # fp8 scales are required; lists are required; workspace size
    assert call(p.ref, f, f, f, None, f, f, f, 8, 16, f, f, 8, 0.1, f, None, f, W, None) == 1
    assert call(p.ref, f, f, f, f, f, f, f, 8, 16, None, f, 8, 0.1, f, None, f, W, None) == 1
    assert call(p.ref, f, f, f, f, f, f, f, 8, 16, f, f, 8, 0.1, f, None, f, 100, None) == 4
    # a ragged sequence length is reported before anything else
    bad = stem.Problem([0, 1000], 4, 2)
    assert call(bad.ref, f, f, f, f, f, f, f, 8, 16, f, f, 8, 0.1, f, None, f, W, None) == 2


def test_q64_attention_argument_errors():
    """Every call below carries one invalid argument, so nothing is launched."""
    lib = stem.load_library()
    p = stem.Problem([0, 1024], 4, 2)
    f = FAKE
    W = 1 << 30
    call = lib.stem_bsa_prefill_q64
    assert call(p.ref, None, f, f, f, f, 8, 0.1, f, None, f, W, None) == 1        # null q
    assert call(p.ref, f, f, f, None, f, 8, 0.1, f, None, f, W, None) == 1        # null lists
    assert call(p.ref, f, f, f, f, f, 0, 0.1, f, None, f, W, None) == 1           # k_cap 0
    assert call(p.ref, f, f, f, f, f, 8, -1.0, f, None, f, W, None) == 1          # scale
    assert call(p.ref, f, f, f, f, f, 8, 0.1, f, None, f, 100, None) == 4         # workspace size
    assert call(stem.Problem([0, 1000], 4, 2).ref, f, f, f, f, f, 8, 0.1, f, None, f, W, None) == 2
    assert call(stem.Problem([0, 128 * 4097], 4, 2).ref, f, f, f, f, f, 8, 0.1, f, None, f, W, None) == 2


def test_binding_rejects_mismatched_scoring_arguments():
    """The binding's e4m3-scoring checks fire before any device call."""
    p = stem.Problem([0, 1024], 4, 2)
    codes = [torch.zeros(1024, h, 128, dtype=torch.uint8) for h in (4, 2, 2)]
    with pytest.raises(ValueError, match="e4m3 scoring needs"):
        stem.stem_score(p, *codes)
    bf = [torch.zeros(1024, h, 128, dtype=torch.bfloat16) for h in (4, 2, 2)]
    with pytest.raises(ValueError, match="takes no scales"):
        stem.stem_score(p, *bf, scales=(torch.ones(8, 4), torch.ones(8, 2), torch.ones(8, 2)))
    with pytest.raises(ValueError, match="fp8_scoring needs fp8_inputs"):
        stem.stem_prefill(p, *bf, [4], fp8_scoring=True)


def test_package_defaults_match_the_doc_table():
    import json
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "stem_doc_defaults.json")))
    for k, v in g["defaults"].items():
        assert stem.DEFAULTS[k] == v, k
    assert stem.DEFAULTS["beta"] == g["beta"]["value"]
    a = g["alpha_list_example"]
    assert list(S.FP8_ALPHAS) == [a["warmup_alpha"]] * a["warmup_layers"] + [a["later_alpha"]] * a["later_layers"]


def test_header_is_plain_c_and_links_from_c(tmp_path):
    """include/stem.h compiles as C99 (-pedantic), and a C program linked
    against libstem.so calls the host-only entry points (status strings, the
    budget rule, argument validation) without a GPU."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "abi.c"
    src.write_text(r'''
#include <stdio.h>
#include <string.h>
#include "stem.h"
int main(void) {
  int32_t cu[2] = {0, 4096};
  stem_problem_t p = {1, cu, 4, 2, 128, 128};
  double ks = 10.0;
  if (strcmp(stem_status_string(STEM_ERR_CAPACITY), "STEM_ERR_CAPACITY") != 0) return 1;
  if (stem_tpd_budget(0, 8, 10.0, 0.5, 1.0) != 10) return 2;
  if (stem_max_kept(&p, &ks, 0.5, 1.0, 1, 1) != 8) return 3;
  if (stem_score_workspace_bytes(&p) != 512) return 4;
  /* a null q is rejected before anything touches a device */
  if (stem_score(&p, NULL, NULL, NULL, 8, 2048, 1.0f, 0.2f, NULL, NULL, 0, NULL) != STEM_ERR_INVALID_ARG) return 5;
  printf("ok\n");
  return 0;
}
''')
    lib_dir = os.path.dirname(stem.LIB_PATH)
    exe = tmp_path / "abi"
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe), "-L", lib_dir, "-lstem", "-Wl,-rpath," + lib_dir], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout, r.stderr)


def test_noalloc_score_rejects_problems_beyond_its_scratch():
    """stem_score_noalloc checks the problem against its fixed scratch array
    before touching the device: the score workspace (Hkv * R floats, then the
    work-queue counters) must fit in STEM_SCORE_SCRATCH_BYTES, else
    STEM_ERR_WORKSPACE (no launch, no GPU)."""
    lib = stem.load_library()
    assert stem.STEM_SCORE_SCRATCH_BYTES == (1 << 20) + 4096
    # the documented guarantee: Hkv * R <= 262144 with at most 8192 sequences fits
    assert stem.stem_score_workspace_bytes(stem.Problem([0, 128 * 32768], 8, 8)) <= stem.STEM_SCORE_SCRATCH_BYTES
    many = stem.Problem([128 * i for i in range(8193)], 32, 32)      # 8192 one-block sequences, R * Hkv = 262144
    assert stem.stem_score_workspace_bytes(many) <= stem.STEM_SCORE_SCRATCH_BYTES
    dummy = ctypes.c_void_p(256)
    for Hkv, nblk in ((64, 4113), (8, 32897)):
        p = stem.Problem([0, 128 * nblk], Hkv, Hkv)
        assert stem.stem_score_workspace_bytes(p) > stem.STEM_SCORE_SCRATCH_BYTES
        st = lib.stem_score_noalloc(p.ref, dummy, dummy, dummy, 8, 2048, 1.0, 0.2, dummy, None)
        assert st == 4, stem.STATUS.get(st, st)                  # STEM_ERR_WORKSPACE
    # invalid problems are rejected as in stem_score
    p = stem.Problem([0, 100], 2, 1)
    assert lib.stem_score_noalloc(p.ref, dummy, dummy, dummy, 8, 2048, 1.0, 0.2, dummy, None) == 2
