"""lmhead_confidence_unmask (the end of a denoising step in one call) against
lmhead_confidence followed by unmask_select, bit for bit, and against the
oracle's unmasking rule.

The fused form (bf16, nseq * Lq <= 64, H a multiple of 256) merges each row
in its own block and lets the block that finishes a sequence's last row run
that sequence's unmasking step; the other shapes run the two calls' kernels
in turn.  Each case walks a whole block of steps from an all-masked state,
with some positions planted confident so that the threshold accepts them,
and repeats the walk so that differently ordered row arrivals are seen."""
import numpy as np
import pytest
import torch

import oracle
from sparse_prefix_kv_amd import sprint, synth
from sparse_prefix_kv_amd.block import SprintBlock

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(rng, nseq, Lq, H, V, dtype, n_planted, gamma=24.0):
    """Hidden rows and an LM head with `n_planted` rows per sequence aligned
    to a vocabulary row (confidence close to 1), the rest random."""
    W = rng.standard_normal((V, H)).astype(np.float32) * 0.02
    X = rng.standard_normal((nseq * Lq, H)).astype(np.float32)
    for s in range(nseq):
        for i in rng.choice(Lq, n_planted, replace=False):
            v = int(rng.integers(0, V))
            # logit gamma for row v, about gamma * W[u].W[v] / |W[v]|^2 (small) elsewhere
            X[s * Lq + i] = gamma * W[v] / float(W[v] @ W[v])
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    if dtype == "bf16":
        X, W = synth.bf16_round(X), synth.bf16_round(W)
    return (torch.from_numpy(X).to(tdt).to(DEV), torch.from_numpy(W).to(tdt).to(DEV), X, W)


def _walk(fused, X, W, nseq, Lq, tau, T):
    """All the steps of one block from the all-masked state; the state after
    every step."""
    masked = torch.ones((nseq, Lq), dtype=torch.uint8, device=DEV)
    tokens = torch.full((nseq, Lq), -1, dtype=torch.int32, device=DEV)
    M = nseq * Lq
    conf = torch.empty(M, dtype=torch.float32, device=DEV)
    amax = torch.empty(M, dtype=torch.int32, device=DEV)
    nacc = torch.empty(nseq, dtype=torch.int32, device=DEV)
    dt = sprint.BF16 if X.dtype == torch.bfloat16 else sprint.F32
    H, V = X.shape[1], W.shape[0]
    if fused:
        # start from a workspace full of junk: the call must set what it needs
        ws = torch.full((sprint.lmhead_confidence_unmask_ws(nseq, Lq, H, V, dt),), 0x5A,
                        dtype=torch.uint8, device=DEV)
    else:
        ws = torch.empty(max(sprint.lmhead_confidence_ws(M, H, V, dt), 256), dtype=torch.uint8,
                         device=DEV)
    states = []
    for t in range(T):
        if fused:
            sprint.lmhead_confidence_unmask(X, W, masked, tokens, tau, T - t, conf=conf,
                                            argmax=amax, n_accepted=nacc, ws=ws)
        else:
            sprint.lmhead_confidence(X, W, conf=conf, argmax=amax, ws=ws)
            sprint.unmask_select(conf.view(nseq, Lq), amax.view(nseq, Lq), masked, tokens, tau,
                                 T - t, n_accepted=nacc)
        states.append(tuple(a.clone() for a in (conf, amax, masked, tokens, nacc)))
    return states


CASES = [  # nseq, Lq, H, V, dtype, planted per sequence, tau
    (1, 32, 2048, 32768, "bf16", 10, 0.95),
    (1, 32, 2048, 163840, "bf16", 0, 0.95),
    (2, 32, 1024, 5000, "bf16", 7, 0.9),
    (1, 64, 256, 40000, "bf16", 20, 0.95),
    (4, 16, 512, 3000, "bf16", 5, 0.95),
    (3, 17, 768, 7777, "bf16", 3, 0.8),
    (64, 1, 256, 1000, "bf16", 1, 0.95),
    # the two calls' kernels in turn: fp32, H not a multiple of 256, more than 64 rows
    (1, 32, 320, 4096, "bf16", 6, 0.95),
    (2, 32, 256, 3000, "f32", 8, 0.95),
    (3, 32, 512, 2000, "bf16", 4, 0.95),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_fused_tail_equals_the_two_calls(case):
    nseq, Lq, H, V, dtype, n_planted, tau = CASES[case]
    rng = np.random.default_rng(9100 + case)
    X, W, _, _ = _inputs(rng, nseq, Lq, H, V, dtype, n_planted)
    T = 9
    ref = _walk(False, X, W, nseq, Lq, tau, T)
    for rep in range(6):
        got = _walk(True, X, W, nseq, Lq, tau, T)
        for t, (a, b) in enumerate(zip(ref, got)):
            for name, x, y in zip(("conf", "argmax", "masked", "tokens", "n_accepted"), a, b):
                assert torch.equal(x, y), (case, rep, t, name)
    # the planted positions (confidence close to 1) pass the threshold at once
    assert np.all(ref[0][4].cpu().numpy() >= n_planted)


@pytest.mark.parametrize("case", [0, 2, 5])
def test_fused_tail_follows_the_oracle_rule(case):
    """Each step's acceptances are the oracle's unmask_select fed the GPU's
    confidences and argmax."""
    nseq, Lq, H, V, dtype, n_planted, tau = CASES[case]
    rng = np.random.default_rng(9200 + case)
    X, W, _, _ = _inputs(rng, nseq, Lq, H, V, dtype, n_planted)
    T = 9
    got = _walk(True, X, W, nseq, Lq, tau, T)
    masked = np.ones((nseq, Lq), np.uint8)
    tokens = np.full((nseq, Lq), -1)
    for t, (conf, amax, m_g, tok_g, nacc_g) in enumerate(got):
        c = conf.cpu().numpy().reshape(nseq, Lq)
        a = amax.cpu().numpy().reshape(nseq, Lq)
        out = oracle.unmask_select(c, a, masked, tokens, np.float32(tau), T - t)
        masked, tokens = out[0], out[1]
        assert np.array_equal(m_g.cpu().numpy(), masked), (case, t)
        assert np.array_equal(tok_g.cpu().numpy(), tokens), (case, t)
        assert np.array_equal(nacc_g.cpu().numpy(), np.asarray(out[2])), (case, t)


def test_block_with_the_fused_tail_equals_the_unfused_block():
    """A whole SPRINT block (pass + 8 pruned steps) ends in the same state
    with either step tail, eagerly and as a replayed graph."""
    wl = synth.Workload("fused", "bf16", Hq=16, Hkv=4, D=128, Lq=32, vocab=32768,
                        segments=(((0, 1024), (1, 3072)),), r_text=1.0, r_img=0.8, tau=0.95, T=9)
    x = synth.make_inputs(wl, 3)
    a = SprintBlock(x, DEV, fused_tail=False)
    b = SprintBlock(x, DEV, fused_tail=True)
    a.run_block(8)
    b.run_block(8)
    torch.cuda.synchronize()
    for name in ("tokens", "masked", "conf_blk", "argmax_blk", "O", "kept_idx"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        b.run_block(8)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        b.run_block(8)
    for _ in range(3):
        b.tokens.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name in ("tokens", "masked", "conf_blk", "argmax_blk"):
            assert torch.equal(getattr(a, name), getattr(b, name)), name
