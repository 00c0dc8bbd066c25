"""Multi-block generation on seeded random layouts: every block's prefix and
pass checked against the oracle fed the GPU's own state.

Each case draws fp32 or bf16, a head shape, 1-3 sequences of 0-3 runs of
random modality and length, block length 16 or 32, keep ratios, the step
budget, the generated blocks' modality, whether prefix confidences are
carried from finished blocks or recomputed from their stored outputs, and a
power-of-two scale of the LM head.  Three blocks are generated.

For block b (checked after its steps, before its rows join the prefix):
  * its prefix (K, V, modality, offsets) equals the oracle's append of block
    b-1's own K/V rows to block b-1's prefix, bit for bit;
  * carried confidences equal the oracle's append of block b-1's prefix
    confidences and its last step's block confidences, bit for bit;
    recomputed ones match the oracle's LM head on the prefix hidden states,
    which hold block b-1's stored outputs after the original rows;
  * the score matches the oracle on the GPU's confidences; the kept set and
    the compaction are bit-exact from the GPU's scores;
  * the last step's attention over the kept rows and its block confidences
    match the oracle (tolerances as in test_gpu_parity; the relative
    confidence bound grows with the logits, as in test_gpu_random_blocks);
  * the step budget leaves no position masked.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from sparse_prefix_kv_amd import synth
from sparse_prefix_kv_amd.gen import SprintGeneration

pytestmark = pytest.mark.gpu
DEV = "cuda"
B = 3


def _np(t):
    return t.detach().float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def _case(seed):
    rng = np.random.default_rng(9000 + seed)
    dtype = "f32" if seed % 2 == 0 else "bf16"
    Hq, Hkv, D = [(4, 2, 64), (8, 2, 128), (16, 4, 128)][int(rng.integers(3))]
    Lq = int(rng.choice([16, 32]))
    nseq = int(rng.integers(1, 4))
    runs = []
    for _ in range(nseq):
        runs.append(tuple((int(rng.integers(0, 2)), int(rng.integers(0, 200)))
                          for _ in range(int(rng.integers(0, 4)))))
    if sum(n for r in runs for _, n in r) == 0:
        runs[0] = ((synth.TEXT, 29),)
    wl = synth.Workload(
        f"randgen{seed}", dtype, Hq=Hq, Hkv=Hkv, D=D, Lq=Lq, vocab=1000, segments=tuple(runs),
        r_text=float(rng.choice([0.0, 0.5, 1.0])), r_img=float(rng.choice([0.3, 0.8, 1.0])),
        tau=float(rng.choice([0.5, 0.95])), T=int(rng.choice([4, 9])),
        gen_modality=int(rng.integers(0, 2)))
    carry = bool(rng.integers(0, 2))
    w_scale = float(rng.choice([1.0, 32.0]))
    return wl, carry, w_scale


def _check_conf(X, W, conf, amax):
    c_o, a_o, _ = oracle.lmhead_confidence(X, W)
    assert np.max(np.abs(conf - c_o)) <= 1e-3
    zmax = np.max(np.abs(np.asarray(X, np.float64) @ np.asarray(W, np.float64).T), axis=1)
    assert np.all(np.abs(conf - c_o) / c_o <= 1e-4 * np.maximum(1.0, zmax / 4.0))
    diff = amax != a_o
    if diff.any():
        gap = oracle.lmhead_top2_gap(X, W)
        assert np.all(gap[diff] <= 1e-4), (np.nonzero(diff)[0], gap[diff])


@pytest.mark.parametrize("seed", range(16))
def test_random_generation(seed):
    wl, carry, w_scale = _case(seed)
    x = synth.make_inputs(wl, seed)
    if w_scale != 1.0:
        x = dataclasses.replace(x, W=(x.W * np.float32(w_scale)).astype(np.float32))
    lay = x.layout
    nseq, Lq, H = lay.nseq, wl.Lq, wl.H
    att_tol = 1e-5 if wl.dtype == "f32" else 2e-2
    print(f"case {seed}: {wl.dtype} Hq/Hkv/D {wl.Hq}/{wl.Hkv}/{wl.D} Lq {Lq} runs {lay.runs} "
          f"r {wl.r_text}/{wl.r_img} tau {wl.tau} T {wl.T} gen_modality {wl.gen_modality} "
          f"carry {carry} W x{w_scale}", flush=True)

    gen = SprintGeneration(x, B, DEV, seed=seed, carry_conf=carry)
    seen = []

    def grab(b):
        torch.cuda.synchronize()
        k = gen.blk
        seen.append(dict(
            K=_np(k.K), V=_np(k.V), mod=_np(k.modality), cu=_np(k.cu_len).astype(np.int64),
            hidden=None if k.hidden is None else _np(k.hidden), conf=_np(k.conf_prefix),
            amax_prefix=_np(k.argmax_prefix), score=_np(k.score),
            kept=_np(k.kept_idx).astype(np.int64), K_pr=_np(k.K_pr), V_pr=_np(k.V_pr),
            O=_np(k.O), conf_blk=_np(k.conf_blk), amax_blk=_np(k.argmax_blk),
            masked=_np(k.masked), tokens=_np(k.tokens)))
    gen.run(wl.T - 1, on_block=grab)
    torch.cuda.synchronize()

    inputs = [(x.Q, x.Kb, x.Vb)] + [synth.make_block_inputs(wl, nseq, b, seed)
                                    for b in range(1, B)]
    K_e, V_e, mod_e, cu_e, hid_e = x.K, x.V, lay.modality, lay.cu_len.astype(np.int64), x.hidden
    for b in range(B):
        g = seen[b]
        Q_b, Kb_b, Vb_b = inputs[b]
        if b > 0:
            p = seen[b - 1]
            _, Kb_p, Vb_p = inputs[b - 1]
            cu_p = cu_e
            K_e, cu_e = oracle.append_block(K_e, cu_p, Kb_p)
            V_e, _ = oracle.append_block(V_e, cu_p, Vb_p)
            mod_e, _ = oracle.append_block(mod_e, cu_p,
                                           np.full((nseq, Lq), wl.gen_modality, np.uint8))
            if carry:
                conf_e, _ = oracle.append_block(p["conf"], cu_p, p["conf_blk"].reshape(nseq, Lq))
            else:
                hid_e, _ = oracle.append_block(hid_e, cu_p, p["O"].reshape(nseq, Lq, H))
        # the grown prefix
        assert g["cu"].tolist() == cu_e.tolist()
        np.testing.assert_array_equal(g["K"], K_e)
        np.testing.assert_array_equal(g["V"], V_e)
        np.testing.assert_array_equal(g["mod"], mod_e)
        if b > 0 and carry:
            np.testing.assert_array_equal(g["conf"], conf_e)
        else:
            np.testing.assert_array_equal(g["hidden"], hid_e)
            _check_conf(hid_e, x.W, g["conf"], g["amax_prefix"])
        # score, kept set, compaction
        ibar = oracle.key_norm_importance(K_e, cu_e)
        score_o = oracle.composite_score(ibar, g["conf"].astype(np.float64), wl.alpha)
        np.testing.assert_allclose(g["score"], score_o, rtol=1e-5, atol=1e-7)
        keep = np.array([[oracle.keep_count(wl.r_text, int(np.sum(mod_e[cu_e[s]:cu_e[s + 1]] == 0))),
                          oracle.keep_count(wl.r_img, int(np.sum(mod_e[cu_e[s]:cu_e[s + 1]] == 1)))]
                         for s in range(nseq)])
        kept_o = oracle.select_kept(g["score"], mod_e, cu_e, keep)
        np.testing.assert_array_equal(g["kept"], kept_o)
        Kp_o, Vp_o = oracle.compact(K_e, V_e, kept_o)
        np.testing.assert_array_equal(g["K_pr"], Kp_o)
        np.testing.assert_array_equal(g["V_pr"], Vp_o)
        cu_kept = np.zeros(nseq + 1, dtype=np.int64)
        cu_kept[1:] = np.cumsum(keep.sum(axis=1))
        # the last pruned step
        O_o = oracle.attention(Q_b, Kp_o, Vp_o, cu_kept, Kb_b, Vb_b)
        assert np.max(np.abs(g["O"] - O_o)) <= att_tol
        _check_conf(g["O"].reshape(nseq * Lq, H), x.W, g["conf_blk"], g["amax_blk"])
        assert g["masked"].sum() == 0
        assert np.all((g["tokens"] >= 0) & (g["tokens"] < wl.vocab))
