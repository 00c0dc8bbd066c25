"""Runtime properties the C ABI promises beyond parity: bitwise-reproducible
results, correct use of the caller's stream, and whole blocks that replay
correctly as HIP graphs (each replay checked against an eager run, with eager
work and synchronisations in between)."""
import numpy as np
import pytest
import torch

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


def _attend_inputs(kv_lens, seed):
    nseq, Lq, Hq, Hkv, D = len(kv_lens), 32, 16, 4, 128
    cu = np.concatenate([[0], np.cumsum(kv_lens)]).astype(np.int32)
    Q = _to_dev(synth.normal_array((nseq, Lq, Hq, D), seed, 1.0, "bf16"), "bf16", DEV)
    K = _to_dev(synth.normal_array((cu[-1], Hkv, D), seed + 1, 1.0, "bf16"), "bf16", DEV)
    V = _to_dev(synth.normal_array((cu[-1], Hkv, D), seed + 2, 1.0, "bf16"), "bf16", DEV)
    Kb = _to_dev(synth.normal_array((nseq, Lq, Hkv, D), seed + 3, 1.0, "bf16"), "bf16", DEV)
    Vb = _to_dev(synth.normal_array((nseq, Lq, Hkv, D), seed + 4, 1.0, "bf16"), "bf16", DEV)
    return Q, K, V, _i32(cu), int(max(kv_lens)), Kb, Vb


def test_repeated_calls_are_bitwise_identical():
    Q, K, V, cu, mx, Kb, Vb = _attend_inputs([3000, 11000], 5)
    o1 = sprint.block_attend(Q, K, V, cu, mx, Kb, Vb)
    o2 = sprint.block_attend(Q, K, V, cu, mx, Kb, Vb)
    assert torch.equal(o1, o2)
    for M, H, V_ in [(32, 2048, 32768), (4096, 2048, 4096), (40, 256, 1000)]:
        X = _to_dev(synth.normal_array((M, H), M, 1.0, "bf16"), "bf16", DEV)
        W = _to_dev(synth.normal_array((V_, H), V_, 0.02, "bf16"), "bf16", DEV)
        c1, a1 = sprint.lmhead_confidence(X, W)
        c2, a2 = sprint.lmhead_confidence(X, W)
        assert torch.equal(c1, c2) and torch.equal(a1, a2)
    lay = synth.layout_from_runs([((0, 1000), (1, 3000)), ((1, 500),)])
    Kk = _to_dev(synth.normal_array((lay.total_L, 4, 128), 9, 1.0, "bf16"), "bf16", DEV)
    conf = _f32(synth.random_scores(lay.total_L, 3, 0))
    cu_l = _i32(lay.cu_len)
    i1, s1 = sprint.sprint_score(Kk, conf, cu_l)
    i2, s2 = sprint.sprint_score(Kk, conf, cu_l)
    assert torch.equal(i1, i2) and torch.equal(s1, s2)


def test_calls_run_on_the_given_stream():
    Q, K, V, cu, mx, Kb, Vb = _attend_inputs([4000], 6)
    ref = sprint.block_attend(Q, K, V, cu, mx, Kb, Vb)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    out = torch.empty_like(ref)
    with torch.cuda.stream(side):
        # a long producer on the side stream first: the call must queue behind it
        big = torch.ones(64 << 20, device=DEV)
        big.mul_(2.0)
        sprint.block_attend(Q, K, V, cu, mx, Kb, Vb, O=out, stream=side)
    side.synchronize()
    assert torch.equal(out, ref)


@pytest.mark.parametrize("name", ["tiny", "single4k"])
def test_block_graph_replays_match_eager(name):
    x = synth.make_inputs(synth.WORKLOADS[name], 0)
    blk = SprintBlock(x, DEV)
    n_steps = (blk.T - 1) if blk.T is not None else blk.Lq - 1

    def state():
        return (blk.tokens.clone(), blk.masked.clone(), blk.kept_idx.clone(), blk.O.clone(),
                blk.conf_blk.clone())

    blk.run_block(n_steps)
    torch.cuda.synchronize()
    ref = state()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        blk.run_block(n_steps)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        blk.run_block(n_steps)
    for rep in range(3):
        blk.tokens.fill_(-7)          # eager work between replays
        blk.O.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = state()
        for a, b in zip(ref, got):
            assert torch.equal(a, b), f"replay {rep} differs"
    del g


def test_two_blocks_on_two_streams_match_serial_runs():
    """No hidden shared state: two independent blocks (different workloads,
    their own buffers and workspaces) launched on two streams at once give
    bitwise the results of running them one after the other."""
    blks = [SprintBlock(synth.make_inputs(synth.WORKLOADS[n], s), DEV)
            for n, s in (("single4k", 0), ("tiny", 3))]
    steps = [(b.T - 1) if b.T is not None else 6 for b in blks]

    def state(b):
        return [b.tokens.clone(), b.masked.clone(), b.kept_idx.clone(), b.O.clone(),
                b.conf_blk.clone(), b.score.clone()]
    ref = []
    for b, n in zip(blks, steps):
        b.run_block(n)
        torch.cuda.synchronize()
        ref.append(state(b))
    for b in blks:
        b.tokens.fill_(-7)
        b.O.zero_()
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for _ in range(3):
        for b, n, s in zip(blks, steps, streams):
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                b.run_block(n)
        for s in streams:
            torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for b, r in zip(blks, ref):
            assert all(torch.equal(u, v) for u, v in zip(state(b), r))


@pytest.mark.parametrize("name", ["tiny", "single4k"])
def test_block_graph_replay_matches_oracle(name):
    """A whole block (pruning pass + every pruned step) captured as one HIP
    graph and replayed: after each replay, every stage it leaves behind is
    checked against the oracle fed that stage's GPU inputs (prefix
    confidences on sampled rows, scores, the kept set bit for bit, the pruned
    cache, the last step's attention and confidences, the last unmask)."""
    import oracle
    x = synth.make_inputs(synth.WORKLOADS[name], 0)
    wl, lay = x.wl, x.layout
    blk = SprintBlock(x, DEV)
    n_steps = (blk.T - 1) if blk.T is not None else 6
    tol = 1e-5 if wl.dtype == "f32" else 2e-2

    def last_step():
        blk.attend(pruned=True)
        blk.block_confidence()

    def run():
        blk.run_block(n_steps - 1)
        last_step()
        blk.unmask(n_steps)

    run()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        blk.run_block(n_steps - 1)
        last_step()
    keep = np.array([[oracle.keep_count(blk.r_text, lay.n_text[i]),
                      oracle.keep_count(blk.r_img, lay.n_img[i])] for i in range(lay.nseq)])
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, lay.total_L - 1],
                                     rng.integers(0, lay.total_L, size=30)]))
    c_o, _, _ = oracle.lmhead_confidence(x.hidden[rows], x.W)
    for rep in range(3):
        blk.tokens.fill_(-7)                     # eager work between replays
        blk.O.zero_()
        blk.score.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        cp = blk.conf_prefix.cpu().numpy()
        np.testing.assert_allclose(cp[rows], c_o, rtol=1e-4, atol=1e-7)
        sc = blk.score.cpu().numpy()
        sc_o = oracle.composite_score(oracle.key_norm_importance(x.K, lay.cu_len), cp, blk.alpha)
        np.testing.assert_allclose(sc, sc_o, rtol=1e-5, atol=1e-7)
        kept = blk.kept_idx.cpu().numpy().astype(np.int64)
        np.testing.assert_array_equal(kept, oracle.select_kept(sc, lay.modality, lay.cu_len, keep))
        Kp, Vp = oracle.compact(x.K, x.V, kept)
        O_o = oracle.attention(x.Q, Kp, Vp, blk.cu_kept.cpu().numpy(), x.Kb, x.Vb)
        O_g = blk.O.float().cpu().numpy()
        assert np.max(np.abs(O_g - O_o)) <= tol, rep
        c_g = blk.conf_blk.cpu().numpy()
        c_b, a_b, _ = oracle.lmhead_confidence(O_g.reshape(lay.nseq * wl.Lq, -1), x.W)
        np.testing.assert_allclose(c_g, c_b, rtol=1e-4, atol=1e-7)
        gap = oracle.lmhead_top2_gap(O_g.reshape(lay.nseq * wl.Lq, -1), x.W)
        a_g = blk.argmax_blk.cpu().numpy()
        assert np.all((a_g == a_b) | (gap <= 1e-4))
        # the last unmask step, eager, from the replayed state
        m0, t0 = blk.masked.cpu().numpy(), blk.tokens.cpu().numpy()
        blk.unmask(n_steps)
        torch.cuda.synchronize()
        m_o, t_o, _ = oracle.unmask_select(c_g.reshape(lay.nseq, -1), a_g.reshape(lay.nseq, -1),
                                           m0, t0, np.float32(blk.tau), blk.steps_left(n_steps))
        np.testing.assert_array_equal(blk.masked.cpu().numpy(), m_o)
        np.testing.assert_array_equal(blk.tokens.cpu().numpy(), t_o)
        assert int(blk.masked.sum()) == 0 or blk.T is None
    del g
