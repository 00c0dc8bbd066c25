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
                                   (64, 512, 257), (48, 256, 65536 + 11)])
def test_lmhead_small(dtype, M, H, V):
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


def test_score_zero_keys():
    cu = np.array([0, 10, 30], np.int32)
    K = np.zeros((30, 4, 128), np.float32)
    K[10:] = synth.normal_array((20, 4, 128), 1, 1.0, "bf16")
    ib, sc = sprint.sprint_score(_to_dev(K, "bf16", DEV), _f32(np.full(30, 0.5)), _i32(cu))
    assert np.all(_np(ib)[:10] == 1.0)


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


def test_prune_all_equal_scores_keep_lowest():
    lay = synth.layout_from_runs([((0, 50), (1, 3000))])
    got = _run_prune(np.ones(3050, np.float32), lay, [[10, 2000]],
                     synth.normal_array((3050, 4, 128), 1, 1.0, "bf16"),
                     synth.normal_array((3050, 4, 128), 2, 1.0, "bf16"), "bf16")
    np.testing.assert_array_equal(got, np.concatenate([np.arange(10), 50 + np.arange(2000)]))


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
    if np.array_equal(kept, res.kept_idx):
        assert np.max(np.abs(_np(blk.O) - res.outputs[1])) <= 2e-2
    assert int(blk.masked.sum()) == 0          # the 9-step budget finishes the block
