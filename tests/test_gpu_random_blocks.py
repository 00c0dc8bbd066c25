"""Whole SPRINT blocks on seeded random layouts, every stage checked against
the oracle fed the GPU's own inputs for that stage.

Each case draws: fp32 or bf16; head shape; 1-4 sequences of 0-3 runs of
random modality and length (empty runs and empty sequences included); block
length 16 or 32; vocabulary 1000 or 4173; keep ratios (0 included); step
budget T (None = at least one per step); threshold tau; and a power-of-two
scale of the LM head (x1, x32, x128) so that some confidences exceed tau.

Checks, per stage (tolerances as in test_gpu_parity, except that the
relative confidence bound grows with the logits' magnitude, see _check_conf):
  * prefix confidence vs the oracle on the same hidden states and LM head;
  * score vs the oracle's composite of its key-norm importance and the GPU's
    prefix confidences;
  * kept indices: bit-exact against the oracle's selection on the GPU's
    scores; pruned K/V bit-exact against the oracle's compaction;
  * attention (the pass over the full prefix, each step over the GPU's kept
    rows) vs the oracle's softmax attention;
  * block confidence and argmax vs the oracle's LM head on the GPU's stored
    attention output (argmax equal except at near-ties);
  * every unmask step bit-exact against the oracle's rule on the GPU's
    confidences, argmax and the state before the step.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from sparse_prefix_kv_amd import synth
from sparse_prefix_kv_amd.block import SprintBlock

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _np(t):
    return t.detach().float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def _case(seed):
    rng = np.random.default_rng(7000 + seed)
    dtype = "f32" if seed % 2 == 0 else "bf16"
    Hq, Hkv, D = [(4, 2, 64), (8, 2, 128), (16, 4, 128), (6, 3, 64)][int(rng.integers(4))]
    Lq = int(rng.choice([16, 32]))
    nseq = int(rng.integers(1, 5))
    runs = []
    for _ in range(nseq):
        runs.append(tuple((int(rng.integers(0, 2)), int(rng.integers(0, 300)))
                          for _ in range(int(rng.integers(0, 4)))))
    if sum(n for r in runs for _, n in r) == 0:
        runs[0] = ((synth.IMAGE, 37),)
    wl = synth.Workload(
        f"random{seed}", dtype, Hq=Hq, Hkv=Hkv, D=D, Lq=Lq,
        vocab=int(rng.choice([1000, 4173])), segments=tuple(runs),
        r_text=float(rng.choice([0.0, 0.5, 1.0])), r_img=float(rng.choice([0.3, 0.8, 1.0])),
        tau=float(rng.choice([0.5, 0.95, 2.0])), T=[None, 4, 9][int(rng.integers(3))])
    w_scale = float(rng.choice([1.0, 32.0, 128.0]))
    return wl, w_scale


def _check_conf(X, W, conf, amax):
    c_o, a_o, _ = oracle.lmhead_confidence(X, W)
    assert np.max(np.abs(conf - c_o)) <= 1e-3
    # The relative bound of 1e-4 holds for logits of magnitude up to ~4 (the
    # N(0, 0.02) head gives at most 4.2 here).  fp32 accumulation error grows
    # in proportion to the logits, so for the scaled heads the row's bound is
    # 1e-4 * max(1, max|z| / 4).
    zmax = np.max(np.abs(np.asarray(X, np.float64) @ np.asarray(W, np.float64).T), axis=1)
    rel_tol = 1e-4 * np.maximum(1.0, zmax / 4.0)
    assert np.all(np.abs(conf - c_o) / c_o <= rel_tol)
    diff = amax != a_o
    if diff.any():
        gap = oracle.lmhead_top2_gap(X, W)
        assert np.all(gap[diff] <= 1e-4), (np.nonzero(diff)[0], gap[diff])


def _check_unmask(blk, wl, t, prev_mask, prev_tok):
    conf = _np(blk.conf_blk).reshape(prev_mask.shape)
    amax = _np(blk.argmax_blk).reshape(prev_mask.shape).astype(np.int64)
    m_o, t_o, n_o = oracle.unmask_select(conf, amax, prev_mask.copy(), prev_tok.copy(),
                                         np.float32(wl.tau), blk.steps_left(t))
    np.testing.assert_array_equal(_np(blk.masked), m_o)
    np.testing.assert_array_equal(_np(blk.tokens).astype(np.int64), t_o)
    np.testing.assert_array_equal(_np(blk.n_acc).astype(np.int64), np.asarray(n_o))


@pytest.mark.parametrize("seed", range(32))
def test_random_block(seed):
    wl, w_scale = _case(seed)
    x = synth.make_inputs(wl, seed)
    if w_scale != 1.0:
        # a power of two keeps bf16 values exact
        x = dataclasses.replace(x, W=(x.W * np.float32(w_scale)).astype(np.float32))
    lay = x.layout
    nseq, Lq, H = lay.nseq, wl.Lq, wl.H
    att_tol = 1e-5 if wl.dtype == "f32" else 2e-2
    print(f"case {seed}: {wl.dtype} Hq/Hkv/D {wl.Hq}/{wl.Hkv}/{wl.D} Lq {Lq} runs {lay.runs} "
          f"V {wl.vocab} r {wl.r_text}/{wl.r_img} tau {wl.tau} T {wl.T} W x{w_scale}", flush=True)

    blk = SprintBlock(x, DEV)
    blk.reset()
    mask0, tok0 = _np(blk.masked).copy(), _np(blk.tokens).astype(np.int64)
    blk.pruning_pass()
    torch.cuda.synchronize()

    # prefix confidence, score, kept set and compaction
    _check_conf(x.hidden, x.W, _np(blk.conf_prefix), _np(blk.argmax_prefix))
    ibar = oracle.key_norm_importance(x.K, lay.cu_len)
    score_o = oracle.composite_score(ibar, _np(blk.conf_prefix).astype(np.float64), wl.alpha)
    score_g = _np(blk.score)
    np.testing.assert_allclose(score_g, score_o, rtol=1e-5, atol=1e-7)
    keep = np.array([[oracle.keep_count(wl.r_text, int(lay.n_text[s])),
                      oracle.keep_count(wl.r_img, int(lay.n_img[s]))] for s in range(nseq)])
    kept_o = oracle.select_kept(score_g, lay.modality, lay.cu_len, keep)
    kept_g = _np(blk.kept_idx).astype(np.int64)
    np.testing.assert_array_equal(kept_g, kept_o)
    Kp_o, Vp_o = oracle.compact(x.K, x.V, kept_o)
    np.testing.assert_array_equal(_np(blk.K_pr), Kp_o)
    np.testing.assert_array_equal(_np(blk.V_pr), Vp_o)
    cu_kept = np.zeros(nseq + 1, dtype=np.int64)
    cu_kept[1:] = np.cumsum(keep.sum(axis=1))

    # the pass: attention over the full prefix, block confidence, unmasking
    O = _np(blk.O)
    O_o = oracle.attention(x.Q, x.K, x.V, lay.cu_len, x.Kb, x.Vb)
    assert np.max(np.abs(O - O_o)) <= att_tol
    _check_conf(O.reshape(nseq * Lq, H), x.W, _np(blk.conf_blk), _np(blk.argmax_blk))
    _check_unmask(blk, wl, 0, mask0, tok0)

    # pruned steps: attention over the kept rows
    n_steps = (wl.T - 1) if wl.T is not None else 4
    O_p = oracle.attention(x.Q, Kp_o, Vp_o, cu_kept, x.Kb, x.Vb)
    for t in range(1, n_steps + 1):
        prev_mask, prev_tok = _np(blk.masked).copy(), _np(blk.tokens).astype(np.int64)
        blk.pruned_step(t)
        torch.cuda.synchronize()
        O = _np(blk.O)
        assert np.max(np.abs(O - O_p)) <= att_tol
        _check_conf(O.reshape(nseq * Lq, H), x.W, _np(blk.conf_blk), _np(blk.argmax_blk))
        _check_unmask(blk, wl, t, prev_mask, prev_tok)
    if wl.T is not None:
        assert int(blk.masked.sum()) == 0     # the step budget finishes every block
