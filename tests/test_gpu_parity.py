"""HIP path vs the CPU oracle, call by call and composed, on seeded inputs.

Tolerances (written here, derived in the design notes):
  * attention output: max-abs 2e-2 for bf16 output, 1e-5 for fp32;
  * confidence: |dc| <= 1e-3 absolute, and relative 1e-4 (fp32 accumulation
    over H terms of exact inputs perturbs a logit by ~1e-5 at most);
  * argmax: equal except where the oracle's top-2 logit gap is <= 1e-4;
  * key-norm importance and score: relative 1e-5;
  * kept indices, pruned K/V and unmask sets: bit-exact on identical inputs.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from sparse_prefix_kv_amd import sprint, synth
from sparse_prefix_kv_amd.block import SprintBlock, _to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def _f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def _u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def _np(t):
    return t.detach().float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


# ============================================================ LM-head confidence

def _check_lmhead(X, W, conf, amax, lse, rows=None):
    Xo = X if rows is None else X[rows]
    c_o, a_o, l_o = oracle.lmhead_confidence(Xo, W)
    gap = oracle.lmhead_top2_gap(Xo, W)
    c_g = conf if rows is None else conf[rows]
    a_g = amax if rows is None else amax[rows]
    assert np.max(np.abs(c_g - c_o)) <= 1e-3
    assert np.max(np.abs(c_g - c_o) / c_o) <= 1e-4
    if lse is not None:
        l_g = lse if rows is None else lse[rows]
        assert np.max(np.abs(l_g - l_o)) <= 1e-4 * max(1.0, np.max(np.abs(l_o)))
    diff = a_g != a_o
    assert np.all(gap[diff] <= 1e-4), (np.nonzero(diff)[0], gap[diff])
    return int(diff.sum())


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M,H,V", [(1, 64, 100), (5, 128, 4096 + 77), (32, 256, 4096),
                                   (33, 256, 1000), (200, 128, 3000), (300, 2048, 513),
                                   (1, 512, 100), (17, 512, 4096 + 77), (40, 1024, 1000),
                                   (64, 512, 257), (48, 256, 65536 + 11),
                                   (1000, 256, 20000)])
def test_lmhead_small(dtype, M, H, V):
    """(1000, 256, 20000) in bf16 gives 316 GEMM tiles, so some blocks of the
    one-block-per-CU grid take two tiles, with ragged last token and
    vocabulary tiles."""
    X = synth.normal_array((M, H), 11 + M, 1.0, dtype)
    W = synth.normal_array((V, H), 12 + V, 0.02, dtype)
    conf, amax, lse = sprint.lmhead_confidence(_to_dev(X, dtype, DEV), _to_dev(W, dtype, DEV),
                                               want_lse=True)
    _check_lmhead(X, W, _np(conf), _np(amax), _np(lse))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_lmhead_planted_confident_rows(dtype):
    M, H, V = 40, 256, 4096
    X = synth.normal_array((M, H), 21, 1.0, dtype)
    W = synth.normal_array((V, H), 22, 0.02, dtype)
    pairs = [(0, 7), (3, 4095), (17, 0), (39, 2048), (20, 2049)]
    W = synth.plant_rows(W, X, pairs, 0.1, dtype)        # z ~ 0.1*|x|^2 ~ 25 -> c ~ 1
    conf, amax, lse = sprint.lmhead_confidence(_to_dev(X, dtype, DEV), _to_dev(W, dtype, DEV),
                                               want_lse=True)
    c = _np(conf)
    a = _np(amax)
    for r, v in pairs:
        assert a[r] == v and c[r] > 0.99
    _check_lmhead(X, W, c, a, _np(lse))


def test_lmhead_zero_weights_tie_to_lowest():
    X = synth.normal_array((7, 128), 1, 1.0, "bf16")
    W = np.zeros((1000, 128), np.float32)
    conf, amax = sprint.lmhead_confidence(_to_dev(X, "bf16", DEV), _to_dev(W, "bf16", DEV))
    assert np.all(_np(amax) == 0)
    np.testing.assert_allclose(_np(conf), 1e-3, rtol=1e-6)


@pytest.mark.parametrize("M,V", [(32, 32768), (4096, 32768), (256, 65536), (32, 163840)])
def test_lmhead_full_size_sampled(M, V):
    H = 2048
    X = synth.normal_array((M, H), 31, 1.0, "bf16")
    W = synth.normal_array((V, H), 32, 0.02, "bf16")
    conf, amax, lse = sprint.lmhead_confidence(_to_dev(X, "bf16", DEV), _to_dev(W, "bf16", DEV),
                                               want_lse=True)
    rng = np.random.default_rng(M + V)
    rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, size=min(M, 48))]))
    _check_lmhead(X, W, _np(conf), _np(amax), _np(lse), rows)


def test_lmhead_generic_tile_path_bf16():
    """bf16 with more than 64 rows and a hidden size that is not a multiple
    of 128: the generic tile kernel, against the oracle."""
    M, H, V = 100, 192, 3000
    X = synth.normal_array((M, H), 4301, 1.0, "bf16")
    W = synth.normal_array((V, H), 4302, 0.02, "bf16")
    conf, amax, lse = sprint.lmhead_confidence(_to_dev(X, "bf16", DEV), _to_dev(W, "bf16", DEV),
                                               want_lse=True)
    _check_lmhead(X, W, _np(conf), _np(amax), _np(lse))


def test_lmhead_generic_small_m_over_2gib():
    """A few rows against a vocabulary matrix just over 2 GiB whose hidden
    size (65 x 64) fits neither the ring nor the buffer-load paths: the
    generic small-M kernel with 64-bit addressing.  W is zero but for two
    planted rows, so the planted closed form gives the result (LLaDA2.0-Uni,
    Sparse Prefix Retention: c = max_v softmax): logit g on one word and 0 on
    the other V - 1 give c = 1 / (1 + (V - 1) e^-g) and lse = log(e^g + V - 1);
    a zero row gives c = 1/V, argmax 0 (lowest index) and lse = log V."""
    H, V = 4160, 258200
    assert V * H * 2 >= 1 << 31
    va, vb = V - 1, 129001
    W = torch.zeros((V, H), dtype=torch.bfloat16, device=DEV)
    W[va, 0] = 12.0
    W[vb, 1] = 5.0
    X = torch.zeros((3, H), dtype=torch.bfloat16, device=DEV)
    X[0, 0] = 1.0
    X[1, 1] = 2.0                       # logit 10 on word vb
    conf, amax, lse = sprint.lmhead_confidence(X, W, want_lse=True)
    torch.cuda.synchronize()
    del W
    want_c = [1.0 / (1.0 + (V - 1) * math.exp(-12.0)), 1.0 / (1.0 + (V - 1) * math.exp(-10.0)),
              1.0 / V]
    want_l = [math.log(math.exp(12.0) + V - 1), math.log(math.exp(10.0) + V - 1), math.log(V)]
    np.testing.assert_allclose(_np(conf), want_c, rtol=1e-4)
    np.testing.assert_allclose(_np(lse), want_l, rtol=1e-5)
    assert _np(amax).tolist() == [va, vb, 0]


@pytest.mark.parametrize("case", range(16))
def test_lmhead_random_shapes(case):
    """Random token counts (one row to several token tiles), hidden sizes
    (multiples of 64) and vocabulary sizes, in both dtypes: the per-step ring
    (M <= 64), the persistent XCD-grouped GEMM with tile counts that leave
    remainders across the eight XCDs, and the fallbacks for other hidden
    sizes, against the oracle."""
    rng = np.random.default_rng(4000 + case)
    dtype = ["bf16", "f32"][case % 2]
    M = int(rng.choice([1, 7, 32, 33, 64, 65, 200, 513, 1500]))
    H = 64 * int(rng.integers(1, 33))
    if dtype == "bf16" and M > 64:
        H = 256 * max(1, H // 256)                 # the tiled GEMM's hidden sizes
    V = int(rng.integers(100, max(101, min(40000, 20_000_000 // M))))
    X = synth.normal_array((M, H), 5000 + case, 1.0, dtype)
    W = synth.normal_array((V, H), 6000 + case, 0.02, dtype)
    conf, amax, lse = sprint.lmhead_confidence(_to_dev(X, dtype, DEV), _to_dev(W, dtype, DEV),
                                               want_lse=True)
    _check_lmhead(X, W, _np(conf), _np(amax), _np(lse))


@pytest.mark.parametrize("M,V", [(32768, 163840), (76375, 65536)])
def test_lmhead_prefix_large_sampled(M, V):
    """The prefix-wide LM head at the long-prefix shapes: 32768 prefix rows
    over a 163840-word vocabulary (128 x 640 tiles of the XCD-grouped GEMM),
    and the 8-sequence ragged prefix of 76375 rows (a ragged last token tile)
    over 65536 words.  Both tails, both sides of tile edges and random rows,
    72 in all, against the oracle: confidence, argmax and log-sum-exp."""
    H = 2048
    X = synth.normal_array((M, H), 33, 1.0, "bf16")
    W = synth.normal_array((V, H), 34, 0.02, "bf16")
    conf, amax, lse = sprint.lmhead_confidence(_to_dev(X, "bf16", DEV), _to_dev(W, "bf16", DEV),
                                               want_lse=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(M ^ V)
    edges = [0, 1, 2, 3, 255, 256, 257, 2047, 2048, M // 2, M - 257, M - 256, M - 5, M - 4,
             M - 3, M - 2, M - 1]
    rows = np.unique(np.concatenate([edges, rng.integers(0, M, size=72 - len(edges))]))
    while len(rows) < 72:
        rows = np.unique(np.concatenate([rows, rng.integers(0, M, size=72 - len(rows))]))
    assert len(rows) >= 64
    _check_lmhead(X, W, _np(conf), _np(amax), _np(lse), rows)


# ============================================================ score

def _check_score(K, conf, cu, dtype, Hkv, D, alpha=0.5):
    ib, sc = sprint.sprint_score(_to_dev(K, dtype, DEV), _f32(conf), _i32(cu), alpha)
    ib_o = oracle.key_norm_importance(K, cu)
    sc_o = oracle.composite_score(ib_o, conf, alpha)
    ib_g, sc_g = _np(ib), _np(sc)
    np.testing.assert_allclose(ib_g, ib_o, rtol=1e-5, atol=1e-7)
    np.testing.assert_allclose(sc_g, sc_o, rtol=1e-5, atol=1e-7)
    for s in range(len(cu) - 1):
        L = cu[s + 1] - cu[s]
        if L:
            assert abs(ib_g[cu[s]:cu[s + 1]].sum() - L) <= 1e-4 * L


@pytest.mark.parametrize("dtype,Hkv,D", [("f32", 2, 64), ("bf16", 4, 128), ("bf16", 3, 64),
                                         ("f32", 1, 128)])
def test_score_small_ragged(dtype, Hkv, D):
    lens = [0, 100, 1000, 257, 1]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    K = synth.lognormal_rows(synth.normal_array((cu[-1], Hkv, D), 41, 1.0, "f32"), 42)
    if dtype == "bf16":
        K = synth.bf16_round(K)
    conf = synth.random_scores(cu[-1], 43) / 2
    _check_score(K, conf, cu, dtype, Hkv, D)
    _check_score(K, conf, cu, dtype, Hkv, D, alpha=0.25)


@pytest.mark.parametrize("case", range(12))
def test_score_random_shapes(case):
    """Random sequence counts and lengths (empty ones included), KV heads,
    head sizes, dtypes and blend weights against the oracle."""
    rng = np.random.default_rng(8000 + case)
    dtype = ["bf16", "f32"][case % 2]
    Hkv, D = int(rng.choice([1, 2, 3, 4, 8])), int(rng.choice([64, 128]))
    lens = [int(v) for v in rng.integers(0, 5000, int(rng.integers(1, 6)))]
    lens[int(rng.integers(0, len(lens)))] += 1                 # at least one position
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    K = synth.lognormal_rows(synth.normal_array((cu[-1], Hkv, D), 8100 + case, 1.0, "f32"),
                             8200 + case)
    if dtype == "bf16":
        K = synth.bf16_round(K)
    conf = synth.random_scores(cu[-1], 8300 + case) / 2
    _check_score(K, conf, cu, dtype, Hkv, D, alpha=float(rng.choice([0.5, 0.25, 0.9])))


def test_score_zero_keys():
    cu = np.array([0, 10, 30], np.int32)
    K = np.zeros((30, 4, 128), np.float32)
    K[10:] = synth.normal_array((20, 4, 128), 1, 1.0, "bf16")
    ib, sc = sprint.sprint_score(_to_dev(K, "bf16", DEV), _f32(np.full(30, 0.5)), _i32(cu))
    assert np.all(_np(ib)[:10] == 1.0)


def test_score_long_sequences():
    """Sequences of more than 512 chunks of 64 positions: each lane of the
    score kernel reads several rounds of eight chunk sums and then a ragged
    remainder (70001 positions = 1094 chunks, 33000 = 516)."""
    lens = [70001, 17, 33000]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    K = synth.bf16_round(synth.lognormal_rows(
        synth.normal_array((cu[-1], 4, 128), 47, 1.0, "f32"), 48))
    conf = synth.random_scores(cu[-1], 49) / 2
    _check_score(K, conf, cu, "bf16", 4, 128)


@pytest.mark.parametrize("name", ["interleaved32k", "ragged8"])
def test_score_full_size(name):
    x = synth.make_inputs(synth.WORKLOADS[name], 0, with_lmhead=False)
    conf = synth.random_scores(x.layout.total_L, 44) / 2
    _check_score(x.K, conf, x.layout.cu_len, "bf16", 4, 128)


# ============================================================ prune

def _run_prune(score, lay, keep, K, V, dtype):
    nseq = lay.nseq
    keep = np.asarray(keep, np.int64).reshape(nseq, 2)
    eff = np.stack([np.minimum(keep[:, 0], lay.n_text), np.minimum(keep[:, 1], lay.n_img)], 1)
    cu_kept = np.concatenate([[0], np.cumsum(eff.sum(1))]).astype(np.int32)
    total = int(cu_kept[-1])
    Ko, Vo, idx = sprint.sprint_prune_kv(_f32(score), _u8(lay.modality), _i32(lay.cu_len),
                                         _i32(keep.reshape(-1)), _i32(cu_kept), total,
                                         _to_dev(K, dtype, DEV), _to_dev(V, dtype, DEV))
    want = oracle.select_kept(score, lay.modality, lay.cu_len, keep)
    got = _np(idx).astype(np.int64)
    np.testing.assert_array_equal(got, want)
    Kp, Vp = oracle.compact(K, V, want)
    assert np.array_equal(_np(Ko).view(np.uint32), Kp.astype(np.float32).view(np.uint32))
    assert np.array_equal(_np(Vo).view(np.uint32), Vp.astype(np.float32).view(np.uint32))
    return got


PRUNE_LAYOUTS = [
    [((0, 192), (1, 64))],
    [((1, 5), (0, 2), (1, 5))],
    [((0, 1),), ((1, 1),), ((0, 3), (1, 4)), ((1, 2000), (0, 70), (1, 1000))],
    [((0, 100),)],
    [((1, 3333),)],
    [((0, 10), (1, 5)), (), ((1, 20),), ()],          # empty sequences
]


@pytest.mark.parametrize("li", range(len(PRUNE_LAYOUTS)))
@pytest.mark.parametrize("levels", [0, 3])
@pytest.mark.parametrize("dtype,Hkv,D", [("bf16", 4, 128), ("f32", 2, 64)])
def test_prune_small(li, levels, dtype, Hkv, D):
    lay = synth.layout_from_runs(PRUNE_LAYOUTS[li])
    n = lay.total_L
    score = synth.random_scores(n, 50 + li, levels)
    K = synth.normal_array((n, Hkv, D), 51, 1.0, dtype)
    V = synth.normal_array((n, Hkv, D), 52, 1.0, dtype)
    for rt, ri in [(1.0, 0.8), (1.0, 1.0), (0.5, 0.3), (0.0, 0.0), (0.0, 1.0)]:
        keep = [[oracle.keep_count(rt, lay.n_text[s]), oracle.keep_count(ri, lay.n_img[s])]
                for s in range(lay.nseq)]
        _run_prune(score, lay, keep, K, V, dtype)


@pytest.mark.parametrize("nbin", [1, 2, 63, 64, 65])
@pytest.mark.parametrize("dup", [False, True])
def test_prune_few_keys_left_under_the_prefix(nbin, dup):
    """Scores in [1, 2): the keys first differ at the mantissa's top bit, so
    the first radix window bins mantissa bits 22..15.  `nbin` scores share
    bin 0x80 ([1.5, 1.5 + 2^-9), up to 2^11 steps of 2^-20, or 8 steps for
    many duplicates), 300 lie above it and 500 below.  The k-th largest
    falls inside the bin (or at its edges), where 64 keys or fewer are
    ranked directly instead of by more windows."""
    rng = np.random.default_rng(100 + 2 * nbin + dup)
    above = rng.uniform(1.6, 1.99, 300)
    below = rng.uniform(1.0, 1.45, 500)
    inbin = 1.5 + rng.integers(0, 8 if dup else 1 << 11, nbin) * 2.0 ** -20
    score = np.concatenate([above, inbin, below]).astype(np.float32)
    score = score[rng.permutation(len(score))]
    n = len(score)
    lay = synth.layout_from_runs([((1, n),)])
    K = synth.normal_array((n, 1, 64), 61, 1.0, "f32")
    V = synth.normal_array((n, 1, 64), 62, 1.0, "f32")
    for k in sorted({299, 300, 301, 300 + (nbin + 1) // 2, 300 + nbin, 301 + nbin}):
        _run_prune(score, lay, [[0, k]], K, V, "f32")


def _random_scores(rng, n, kind):
    if kind == "uniform":
        return rng.uniform(0.0, 2.0, n)
    if kind == "signed_wide":
        return rng.standard_normal(n) * 10.0 ** rng.uniform(-3, 3, n)
    if kind == "levels":
        return rng.integers(0, int(rng.integers(2, 40)), n) * 0.25
    # clustered: one value plus noise a few ulps wide, so the radix windows
    # run deep and the last bins hold a few keys with near ties
    base = rng.uniform(0.5, 4.0)
    return base + rng.integers(-200, 200, n) * np.spacing(np.float32(base))


@pytest.mark.parametrize("case", range(24))
def test_prune_random_distributions(case):
    """Random layouts (1-4 sequences, runs of both modalities, empty ones
    included), score distributions and keep ratios; the kept set bit for bit
    against the oracle."""
    rng = np.random.default_rng(1000 + case)
    nseq = int(rng.integers(1, 5))
    runs = []
    for _ in range(nseq):
        seq = tuple((int(rng.integers(0, 2)), int(rng.integers(0, 3000)))
                    for _ in range(int(rng.integers(0, 4))))
        runs.append(seq)
    if sum(length for seq in runs for _, length in seq) == 0:
        runs[0] = ((1, 500),)          # at least one position; empty sequences stay
    lay = synth.layout_from_runs(runs)
    n = lay.total_L
    kind = ["uniform", "signed_wide", "levels", "clustered"][case % 4]
    score = _random_scores(rng, n, kind).astype(np.float32)
    K = synth.normal_array((n, 1, 64), 63, 1.0, "f32")
    V = synth.normal_array((n, 1, 64), 64, 1.0, "f32")
    rt, ri = rng.uniform(0, 1, 2)
    keep = [[oracle.keep_count(rt, lay.n_text[s]), oracle.keep_count(ri, lay.n_img[s])]
            for s in range(lay.nseq)]
    _run_prune(score, lay, keep, K, V, "f32")


def test_prune_all_equal_scores_keep_lowest():
    lay = synth.layout_from_runs([((0, 50), (1, 3000))])
    got = _run_prune(np.ones(3050, np.float32), lay, [[10, 2000]],
                     synth.normal_array((3050, 4, 128), 1, 1.0, "bf16"),
                     synth.normal_array((3050, 4, 128), 2, 1.0, "bf16"), "bf16")
    np.testing.assert_array_equal(got, np.concatenate([np.arange(10), 50 + np.arange(2000)]))


# Sequences on both sides of 32768 positions counted from the start rounded
# down to 16 (the selection holds up to that many keys per thread block and
# reads longer ones again per radix window), a start that is not a multiple
# of 16, and an end of the arrays inside a 16-position chunk.
BOUNDARY_RUNS = [
    ((0, 5),),
    ((1, 20000), (0, 12763)),           # positions 5..32767: 32768 from 0
    ((0, 40000), (1, 1)),               # 40001 positions
    ((1, 32767),),                      # 72769..105535: 32768 from 72768
    ((0, 1), (1, 32768)),               # 32769 positions from a multiple of 16
    ((1, 17), (0, 15)),                 # ends the arrays at 138337 (not / 16)
]


def _signed_wide_scores(n, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(n) * 10.0 ** rng.uniform(-3, 3, n)).astype(np.float32)


@pytest.mark.parametrize("offset", [0, 1])
@pytest.mark.parametrize("kind", ["uniform", "ties", "signed_wide"])
def test_prune_long_short_and_unaligned_sequences(offset, kind):
    """Kept sets at the 32768-key boundary, over sign and exponent spread.
    offset 1 hands the scores and modality over at addresses that are not
    16-byte aligned."""
    lay = synth.layout_from_runs(BOUNDARY_RUNS)
    n = lay.total_L
    score = {"uniform": lambda: synth.random_scores(n, 70),
             "ties": lambda: synth.random_scores(n, 71, 8),
             "signed_wide": lambda: _signed_wide_scores(n, 72)}[kind]()
    K = synth.normal_array((n, 1, 64), 73, 1.0, "f32")
    V = synth.normal_array((n, 1, 64), 74, 1.0, "f32")
    sbuf = torch.zeros(n + offset, dtype=torch.float32, device=DEV)
    sbuf[offset:] = _f32(score)
    mbuf = torch.zeros(n + 3 * offset, dtype=torch.uint8, device=DEV)
    mbuf[3 * offset:] = _u8(lay.modality)
    for rt, ri in [(0.5, 0.3), (1.0, 0.8), (0.01, 0.99)]:
        keep = np.array([[oracle.keep_count(rt, lay.n_text[s]),
                          oracle.keep_count(ri, lay.n_img[s])] for s in range(lay.nseq)])
        eff = np.stack([np.minimum(keep[:, 0], lay.n_text), np.minimum(keep[:, 1], lay.n_img)], 1)
        cu_kept = np.concatenate([[0], np.cumsum(eff.sum(1))]).astype(np.int32)
        Ko, Vo, idx = sprint.sprint_prune_kv(sbuf[offset:], mbuf[3 * offset:], _i32(lay.cu_len),
                                             _i32(keep.reshape(-1)), _i32(cu_kept),
                                             int(cu_kept[-1]), _to_dev(K, "f32", DEV),
                                             _to_dev(V, "f32", DEV))
        want = oracle.select_kept(score, lay.modality, lay.cu_len, keep)
        np.testing.assert_array_equal(_np(idx).astype(np.int64), want)
        Kp, Vp = oracle.compact(K, V, want)
        assert np.array_equal(_np(Ko), Kp.astype(np.float32))
        assert np.array_equal(_np(Vo), Vp.astype(np.float32))


@pytest.mark.parametrize("name", ["interleaved32k", "ragged8", "single4k"])
def test_prune_full_size(name):
    wl = synth.WORKLOADS[name]
    x = synth.make_inputs(wl, 0, with_lmhead=False)
    lay = x.layout
    for levels in (0, 64):
        score = synth.random_scores(lay.total_L, 60, levels)
        keep = [[oracle.keep_count(wl.r_text, lay.n_text[s]),
                 oracle.keep_count(wl.r_img, lay.n_img[s])] for s in range(lay.nseq)]
        got = _run_prune(score, lay, keep, x.K, x.V, "bf16")
        if name == "interleaved32k":
            assert len(got) == 27852        # pooled image keep floor(0.8 * 24576)


# ============================================================ attention

def _attend_case(dtype, Hq, Hkv, D, Lq, kv_lens, block, seed):
    nseq = len(kv_lens)
    cu = np.concatenate([[0], np.cumsum(kv_lens)]).astype(np.int32)
    Q = synth.normal_array((nseq, Lq, Hq, D), seed, 1.0, dtype)
    Kp = synth.lognormal_rows(synth.normal_array((cu[-1], Hkv, D), seed + 1, 1.0, "f32"), seed + 2)
    Kp = synth.bf16_round(Kp) if dtype == "bf16" else Kp
    Vp = synth.normal_array((cu[-1], Hkv, D), seed + 3, 1.0, dtype)
    Kb = synth.normal_array((nseq, Lq, Hkv, D), seed + 4, 1.0, dtype) if block else None
    Vb = synth.normal_array((nseq, Lq, Hkv, D), seed + 5, 1.0, dtype) if block else None
    O = sprint.block_attend(_to_dev(Q, dtype, DEV), _to_dev(Kp, dtype, DEV), _to_dev(Vp, dtype, DEV),
                            _i32(cu), max(kv_lens),
                            None if Kb is None else _to_dev(Kb, dtype, DEV),
                            None if Vb is None else _to_dev(Vb, dtype, DEV))
    O_o = oracle.attention(Q, Kp, Vp, cu, Kb, Vb)
    err = np.max(np.abs(_np(O) - O_o))
    tol = 2e-2 if dtype == "bf16" else 1e-5
    assert err <= tol, err
    return err


@pytest.mark.parametrize("dtype,Hq,Hkv,D", [("f32", 4, 2, 64), ("bf16", 16, 4, 128),
                                            ("bf16", 8, 8, 64), ("f32", 16, 4, 128),
                                            ("bf16", 2, 1, 128)])
@pytest.mark.parametrize("kv_lens,block,Lq", [([256], True, 32), ([0, 37, 300], True, 32),
                                              ([1000, 5], False, 32), ([33], True, 5),
                                              ([4100, 1, 64], True, 16)])
def test_attend_small(dtype, Hq, Hkv, D, kv_lens, block, Lq):
    if (Hq // Hkv) * Lq > 256:
        pytest.skip("more query rows per KV head than one block holds")
    _attend_case(dtype, Hq, Hkv, D, Lq, kv_lens, block, 70 + len(kv_lens))


@pytest.mark.parametrize("kv_lens", [[3481], [4096], [13209], [27852],
                                     [2048, 16384, 9000, 5000, 3001, 12000, 7777, 2500]])
def test_attend_full_size(kv_lens):
    _attend_case("bf16", 16, 4, 128, 32, kv_lens, True, 80)


@pytest.mark.parametrize("dtype,Hq,D,kv_len", [("f32", 2, 64, 20000), ("bf16", 4, 64, 12000),
                                                ("f32", 4, 128, 6000), ("bf16", 2, 128, 20000)])
def test_attend_many_key_ranges(dtype, Hq, D, kv_len):
    """One KV head, so the plan cuts the cache into 48-157 key ranges of 128
    keys: the combine folds them in batches of 16 per lane, one to three
    batches deep."""
    _attend_case(dtype, Hq, 1, D, 32, [kv_len], True, 85)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_attend_max_kv_below_a_sequence(dtype):
    """max_kv only sizes the split of each cache: with three sequences, two of
    them longer than the max_kv given, every key is still attended (the last
    key range of a sequence runs to its end)."""
    kv_lens = [5000, 300, 9000]
    nseq, Lq, Hq, Hkv, D = 3, 32, 16, 4, 128
    cu = np.concatenate([[0], np.cumsum(kv_lens)]).astype(np.int32)
    Q = synth.normal_array((nseq, Lq, Hq, D), 90, 1.0, dtype)
    Kp = synth.normal_array((cu[-1], Hkv, D), 91, 1.0, dtype)
    Vp = synth.normal_array((cu[-1], Hkv, D), 92, 1.0, dtype)
    Kb = synth.normal_array((nseq, Lq, Hkv, D), 93, 1.0, dtype)
    Vb = synth.normal_array((nseq, Lq, Hkv, D), 94, 1.0, dtype)
    O_o = oracle.attention(Q, Kp, Vp, cu, Kb, Vb)
    tol = 2e-2 if dtype == "bf16" else 1e-5
    for max_kv in (1000, 200, 9000):
        O = sprint.block_attend(_to_dev(Q, dtype, DEV), _to_dev(Kp, dtype, DEV),
                                _to_dev(Vp, dtype, DEV), _i32(cu), max_kv,
                                _to_dev(Kb, dtype, DEV), _to_dev(Vb, dtype, DEV))
        err = np.max(np.abs(_np(O) - O_o))
        assert err <= tol, (max_kv, err)


@pytest.mark.parametrize("kv_lens", [[27852], [3000, 700]])
def test_attend_value_scale_is_exact_across_splits(kv_lens):
    """bf16 V of any magnitude: scaling V by a power of two scales O by it
    bit for bit, through the key-range partials and their combine, from
    values far past fp16's range (2^17 * N(0,1)) down to 2^-60.  The unscaled
    call matches the oracle."""
    nseq, Lq, Hq, Hkv, D = len(kv_lens), 32, 16, 4, 128
    cu = np.concatenate([[0], np.cumsum(kv_lens)]).astype(np.int32)
    Q = synth.normal_array((nseq, Lq, Hq, D), 95, 1.0, "bf16")
    Kp = synth.normal_array((cu[-1], Hkv, D), 96, 1.0, "bf16")
    Vp = synth.normal_array((cu[-1], Hkv, D), 97, 1.0, "bf16")
    Kb = synth.normal_array((nseq, Lq, Hkv, D), 98, 1.0, "bf16")
    Vb = synth.normal_array((nseq, Lq, Hkv, D), 99, 1.0, "bf16")
    args = [_to_dev(a, "bf16", DEV) for a in (Q, Kp, Vp)]
    Kb_d, Vb_d = _to_dev(Kb, "bf16", DEV), _to_dev(Vb, "bf16", DEV)
    O1 = sprint.block_attend(args[0], args[1], args[2], _i32(cu), max(kv_lens), Kb_d, Vb_d)
    O_o = oracle.attention(Q, Kp, Vp, cu, Kb, Vb)
    assert np.max(np.abs(_np(O1) - O_o)) <= 2e-2
    for e in (17, 30, -60):
        f = 2.0 ** e
        Ob = sprint.block_attend(args[0], args[1], args[2] * f, _i32(cu), max(kv_lens), Kb_d,
                                 Vb_d * f)
        assert torch.isfinite(Ob.float()).all()
        assert torch.equal(Ob, (O1.float() * f).to(torch.bfloat16)), e


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
def test_attend_eight_row_waves(dtype, D):
    """256 query rows per KV head (G 8 x 32 block tokens): the blocks of
    eight row-waves, over ragged caches with and without one long enough
    for many key ranges."""
    _attend_case(dtype, 16, 2, D, 32, [3000, 17, 0, 900], True, 4100 + D)
    _attend_case(dtype, 8, 1, D, 32, [9000], False, 4200 + D)


@pytest.mark.parametrize("case", range(24))
def test_attend_random_shapes(case):
    """Random GQA ratios, block lengths, head sizes, sequence counts and
    cache lengths (up to 6000 keys, empty caches included when the block's
    own keys are attended), in both dtypes, against the oracle."""
    rng = np.random.default_rng(2000 + case)
    dtype = ["bf16", "f32"][case % 2]
    D = [64, 128][(case // 2) % 2]
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4, 8]))
    Lq = int(rng.choice([1, 5, 16, 32, 64]))
    while G * Lq > 256:
        Lq //= 2
    block = bool(rng.integers(0, 2))
    kv_lens = [int(v) for v in rng.integers(0, 6001, int(rng.integers(1, 5)))]
    if not block:
        kv_lens = [max(v, 1) for v in kv_lens]
    _attend_case(dtype, G * Hkv, Hkv, D, Lq, kv_lens, block, 3000 + case)


def test_attend_full_retention_equals_unpruned():
    x = synth.make_inputs(synth.WORKLOADS["single4k"], 0, with_lmhead=False)
    lay = x.layout
    Q, K, V = (_to_dev(a, "bf16", DEV) for a in (x.Q, x.K, x.V))
    Kb, Vb = _to_dev(x.Kb, "bf16", DEV), _to_dev(x.Vb, "bf16", DEV)
    cu = _i32(lay.cu_len)
    O1 = sprint.block_attend(Q, K, V, cu, lay.total_L, Kb, Vb)
    keep = [[int(lay.n_text[0]), int(lay.n_img[0])]]
    Kp, Vp, _ = sprint.sprint_prune_kv(_f32(synth.random_scores(lay.total_L, 1)), _u8(lay.modality),
                                       cu, _i32(np.array(keep).reshape(-1)),
                                       _i32([0, lay.total_L]), lay.total_L, K, V)
    O2 = sprint.block_attend(Q, Kp, Vp, _i32([0, lay.total_L]), lay.total_L, Kb, Vb)
    assert torch.equal(O1, O2)


# ============================================================ unmask

@pytest.mark.parametrize("Lq", [1, 7, 32, 64])
@pytest.mark.parametrize("ties", [0, 4])
@pytest.mark.parametrize("steps_left", [-1, 0, 1, 3, 8, 1 << 30])
def test_unmask_parity(Lq, ties, steps_left):
    nseq = 5
    tau = np.float32(0.95)
    conf, amax, masked, tokens = synth.random_unmask_state(nseq, Lq, 1000, 90 + Lq + ties, tau,
                                                           tie_levels=ties)
    conf[0, :] = tau                                   # exactly tau is not accepted by '>'
    masked[1, :] = 0                                   # nothing masked
    m_d, t_d = _u8(masked), _i32(tokens)
    n = sprint.unmask_select(_f32(conf), _i32(amax), m_d, t_d, float(tau), steps_left)
    m_o, t_o, n_o = oracle.unmask_select(conf, amax, masked, tokens, tau, steps_left)
    np.testing.assert_array_equal(_np(m_d), m_o)
    np.testing.assert_array_equal(_np(t_d), t_o)
    np.testing.assert_array_equal(_np(n), n_o)


@pytest.mark.parametrize("case", range(24))
def test_unmask_random(case):
    """Random batches (1-16 sequences, 1-64 positions), confidence laws with
    and without ties and values above tau, mask densities, thresholds and
    steps left, against the oracle bit for bit."""
    rng = np.random.default_rng(7000 + case)
    nseq, Lq = int(rng.integers(1, 17)), int(rng.integers(1, 65))
    tau = np.float32(rng.choice([0.5, 0.9, 0.95, 1.5]))
    if case % 3 == 0:
        conf = rng.integers(0, 6, (nseq, Lq)).astype(np.float32) / 5.0     # many ties
    else:
        conf = rng.uniform(0, 1, (nseq, Lq)).astype(np.float32)
    amax = rng.integers(0, 50000, (nseq, Lq)).astype(np.int32)
    masked = (rng.uniform(0, 1, (nseq, Lq)) < rng.uniform(0, 1)).astype(np.uint8)
    tokens = np.where(masked == 1, -1, rng.integers(0, 50000, (nseq, Lq))).astype(np.int32)
    steps_left = int(rng.choice([-2, 0, 1, 2, 5, 9, 1 << 30]))
    m_d, t_d = _u8(masked), _i32(tokens)
    n = sprint.unmask_select(_f32(conf), _i32(amax), m_d, t_d, float(tau), steps_left)
    m_o, t_o, n_o = oracle.unmask_select(conf, amax, masked, tokens, tau, steps_left)
    np.testing.assert_array_equal(_np(m_d), m_o)
    np.testing.assert_array_equal(_np(t_d), t_o)
    np.testing.assert_array_equal(_np(n), n_o)


def test_unmask_schedule_terminates():
    conf = np.linspace(0.1, 0.2, 32, dtype=np.float32)[None]
    masked = _u8(np.ones((1, 32)))
    tokens = _i32(np.full((1, 32), -1))
    got = []
    for t in range(9):
        n = sprint.unmask_select(_f32(conf), _i32(np.arange(32)[None]), masked, tokens, 2.0, 9 - t)
        got.append(int(_np(n)[0]))
    assert got == [4, 4, 4, 4, 4, 3, 3, 3, 3]
    assert int(masked.sum()) == 0


# ============================================================ composed block

def _unique_order(c, masked, rel=1e-5):
    """True when no two masked confidences are within `rel` of each other."""
    v = np.sort(c[masked == 1])
    return len(v) < 2 or np.all(np.diff(v) > rel * v[1:])


def _compare_block(blk, res, n_steps, att_tol):
    torch.cuda.synchronize()
    lay = blk.layout
    # scores and the kept set
    np.testing.assert_allclose(_np(blk.conf_prefix), res.conf_prefix, rtol=1e-4, atol=1e-7)
    np.testing.assert_allclose(_np(blk.score), res.score, rtol=1e-4, atol=1e-6)
    kept = _np(blk.kept_idx).astype(np.int64)
    assert len(kept) == len(res.kept_idx)
    if not np.array_equal(kept, res.kept_idx):
        # only a near-tie in the oracle's scores may separate the two sets
        for s in range(lay.nseq):
            a, b = lay.cu_len[s], lay.cu_len[s + 1]
            for m in (0, 1):
                pool = np.arange(a, b)[lay.modality[a:b] == m]
                ks = np.intersect1d(kept, pool)
                ev = np.setdiff1d(pool, ks)
                if len(ks) and len(ev):
                    assert res.score[ks].min() >= res.score[ev].max() - 1e-5
    return kept


def test_block_tiny_composition():
    wl = synth.WORKLOADS["tiny"]
    x = synth.make_inputs(wl, 0)
    lay = x.layout
    n_steps = 31
    blk = SprintBlock(x, DEV)
    blk.reset()
    blk.pruning_pass()
    torch.cuda.synchronize()
    res = oracle.run_block(x.Q, x.K, x.V, x.Kb, x.Vb, x.hidden, x.W, lay.cu_len, lay.modality,
                           wl.r_text, wl.r_img, np.float32(wl.tau), wl.T, n_steps)
    kept = _compare_block(blk, res, n_steps, 1e-5)
    assert len(kept) == 243
    O0 = _np(blk.O)
    assert np.max(np.abs(O0 - res.outputs[0])) <= 1e-5
    c0 = _np(blk.conf_blk).reshape(1, -1)
    np.testing.assert_allclose(c0, res.confs[0], rtol=1e-4)
    masks = [_np(blk.masked).copy()]
    for t in range(1, n_steps + 1):
        blk.pruned_step(t)
        torch.cuda.synchronize()
        masks.append(_np(blk.masked).copy())
        if t == 1 and np.array_equal(kept, res.kept_idx):
            assert np.max(np.abs(_np(blk.O) - res.outputs[1])) <= 1e-5
            np.testing.assert_allclose(_np(blk.conf_blk).reshape(1, -1), res.confs[1], rtol=1e-4)
    # one acceptance per step ("at least one per step", no confidence above tau);
    # the sets must agree until a near-tie in the oracle's confidences allows
    # either choice, after which only the count is comparable
    diverged = False
    for t in range(n_steps + 1):
        prev = np.ones((1, 32)) if t == 0 else masks[t - 1]
        assert int(prev.sum() - masks[t].sum()) == 1
        if not diverged and _unique_order(res.confs[min(t, 1)][0], prev[0]):
            np.testing.assert_array_equal(masks[t], res.masks[t])
        else:
            diverged = True
    assert masks[-1].sum() == 0


def test_block_single4k_composition():
    wl = synth.WORKLOADS["single4k"]
    x = synth.make_inputs(wl, 0)
    lay = x.layout
    blk = SprintBlock(x, DEV)
    blk.run_block(8)
    torch.cuda.synchronize()
    res = oracle.run_block(x.Q, x.K, x.V, x.Kb, x.Vb, x.hidden, x.W, lay.cu_len, lay.modality,
                           wl.r_text, wl.r_img, np.float32(wl.tau), wl.T, 1)
    kept = _compare_block(blk, res, 1, 2e-2)
    assert len(kept) == 3481
    # the kept set from the GPU's own scores is the oracle's, bit for bit
    keep = np.array([[oracle.keep_count(wl.r_text, lay.n_text[0]),
                      oracle.keep_count(wl.r_img, lay.n_img[0])]])
    want = oracle.select_kept(_np(blk.score), lay.modality, lay.cu_len, keep)
    np.testing.assert_array_equal(kept, want)
    # the last pruned step's attention over the GPU's kept rows (every pruned
    # step attends to the same cache with the same queries)
    Kp, Vp = oracle.compact(x.K, x.V, kept)
    O_o = oracle.attention(x.Q, Kp, Vp, [0, len(kept)], x.Kb, x.Vb)
    assert np.max(np.abs(_np(blk.O) - O_o)) <= 2e-2
    assert int(blk.masked.sum()) == 0          # the 9-step budget finishes the block
