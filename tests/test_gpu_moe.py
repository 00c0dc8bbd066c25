"""GPU parity of the MoE FFN against the oracle.

Routing decides integers (the chosen experts), so a token's experts must
equal the oracle's unless the oracle's selection scores tie within 1e-5 at
the top-k boundary; for tokens routed alike the gates and the output are
compared: fp32 to 1e-4 of the output scale, bf16 to the output's own bf16
rounding (2^-9 relative) plus fp32 accumulation (5e-3 relative, 1e-3 of the
scale absolute).
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_prefix_kv_amd import sprint, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def _np(t):
    return t.float().cpu().numpy()


def _run(M, H, E, K, inter, dtype, seed=0, residual=False, force=None):
    x = synth.normal_array((M, H), seed + 11, 1.0, dtype)
    wr, bias, wg, wu, wd = synth.make_moe_weights(H, E, inter, dtype, seed)
    if force is not None:
        bias = bias.copy()
        bias[force] = 10.0            # every token chooses this expert first
    res = synth.normal_array((M, H), seed + 12, 1.0, dtype) if residual else None
    y, ids, gates = sprint.moe_ffn(_dev(x, dtype), _dev(wr, dtype),
                                   torch.from_numpy(bias).to(DEV), _dev(wg, dtype),
                                   _dev(wu, dtype), _dev(wd, dtype), K,
                                   residual=None if res is None else _dev(res, dtype))
    torch.cuda.synchronize()
    y_o, ids_o, g_o = oracle.moe_ffn(x, wr, bias, wg, wu, wd, K, residual=res)
    _, _, s_o = oracle.moe_route(x, wr, bias, K)
    sel = s_o + bias.astype(np.float64)[None, :]
    ids_g, g_g, y_g = ids.cpu().numpy(), gates.cpu().numpy(), _np(y)
    scale = np.max(np.abs(y_o))
    rtol, atol = (1e-4, 1e-4 * scale) if dtype == "f32" else (5e-3, 1e-3 * scale)
    same = 0
    for t in range(M):
        if np.array_equal(ids_g[t], ids_o[t]):
            same += 1
            np.testing.assert_allclose(g_g[t], g_o[t], rtol=1e-5 if dtype == "f32" else 1e-4)
            np.testing.assert_allclose(y_g[t], y_o[t], rtol=rtol, atol=atol)
        else:
            # only a near-tie in the oracle's selection scores may reorder them
            srt = np.sort(sel[t])[::-1]
            assert np.min(np.abs(np.diff(srt[:K + 1]))) <= 1e-5, (t, ids_g[t], ids_o[t])
    assert same >= M - 1
    return ids_g


@pytest.mark.parametrize("M,H,E,K,inter,dtype", [
    (32, 256, 16, 4, 256, "f32"),
    (7, 512, 8, 2, 256, "f32"),
    (32, 2048, 64, 8, 512, "bf16"),
    (5, 512, 8, 2, 512, "bf16"),
    (64, 1024, 32, 8, 1024, "bf16"),
    # more experts than one selection lane group holds: 65-256 and 257-1024
    (32, 512, 100, 8, 512, "bf16"),
    (24, 256, 200, 8, 256, "f32"),
    (32, 256, 300, 16, 256, "f32"),
    (8, 256, 1024, 16, 256, "f32"),
])
def test_moe_matches_oracle(M, H, E, K, inter, dtype):
    _run(M, H, E, K, inter, dtype)


@pytest.mark.parametrize("case", range(12))
def test_moe_random_shapes(case):
    """Random supported shapes: token counts, hidden and expert widths (in
    the units the expert kernels stream), expert counts and top-k, with and
    without a residual and with one expert forced for every token."""
    rng = np.random.default_rng(9000 + case)
    dtype = ["bf16", "f32"][case % 2]
    unit = 512 if dtype == "bf16" else 256
    H = unit * int(rng.integers(1, 5))
    inter = unit * int(rng.integers(1, 3))
    E = int(rng.integers(1, 65))
    while E * inter * H > 40_000_000:          # keep the host weights small
        E = max(1, E // 2)
    K = int(rng.integers(1, min(E, 16) + 1))
    M = int(rng.integers(1, 97))
    force = int(rng.integers(0, E)) if case % 4 == 3 else None
    ids = _run(M, H, E, K, inter, dtype, seed=9100 + case, residual=bool(case % 3 == 0),
               force=force)
    if force is not None:
        assert np.all(ids[:, 0] == force)


def test_moe_residual_and_one_expert_for_all():
    # every token's first choice is expert 3: 40 tokens on one expert take
    # two LDS chunks in the expert kernels
    ids = _run(40, 2048, 16, 4, 512, "bf16", seed=1, residual=True, force=3)
    assert np.all(ids[:, 0] == 3)


def test_moe_bitwise_reproducible():
    M, H, E, K, inter = 32, 2048, 64, 8, 512
    x = _dev(synth.normal_array((M, H), 5, 1.0, "bf16"), "bf16")
    wr, bias, wg, wu, wd = (torch.from_numpy(a).to(DEV) for a in
                            synth.make_moe_weights(H, E, inter, "bf16", 5))
    args = (x, wr.to(torch.bfloat16), bias, wg.to(torch.bfloat16), wu.to(torch.bfloat16),
            wd.to(torch.bfloat16), K)
    a = sprint.moe_ffn(*args)
    b = sprint.moe_ffn(*args)
    torch.cuda.synchronize()
    assert all(torch.equal(p, q) for p, q in zip(a, b))


def test_block_with_moe_between_attention_and_lm_head():
    from sparse_prefix_kv_amd.block import SprintBlock
    wl = synth.WORKLOADS["tiny"]
    x = synth.make_inputs(wl, 0)
    lay = x.layout
    E, K, inter = 16, 4, 256
    wr, bias, wg, wu, wd = synth.make_moe_weights(wl.H, E, inter, "f32", 3)
    # W_down scaled up so that the experts visibly move the LM head's input
    wd = wd * np.float32(8.0)
    dev_moe = tuple(torch.from_numpy(a).to(DEV) for a in (wr, bias, wg, wu, wd)) + (K, 2.5)
    blk = SprintBlock(x, DEV, moe=dev_moe)
    blk.reset()
    blk.pruning_pass()
    torch.cuda.synchronize()
    c0, ids0 = blk.conf_blk.cpu().numpy(), blk.moe_ids.cpu().numpy()
    blk.pruned_step(1)
    torch.cuda.synchronize()
    c1, ids1 = blk.conf_blk.cpu().numpy(), blk.moe_ids.cpu().numpy()
    res = oracle.run_block(x.Q, x.K, x.V, x.Kb, x.Vb, x.hidden, x.W, lay.cu_len, lay.modality,
                           wl.r_text, wl.r_img, np.float32(wl.tau), wl.T, 1,
                           moe=(wr, bias, wg, wu, wd, K, 2.5), store_dtype="f32")
    same_kept = np.array_equal(blk.kept_idx.cpu().numpy(), res.kept_idx)
    for t, (c, ids) in enumerate(((c0, ids0), (c1, ids1))):
        if t == 1 and not same_kept:
            break
        agree = np.all(ids == res.moe_ids[t], axis=1)
        assert agree.sum() >= len(agree) - 1
        np.testing.assert_allclose(c[agree], res.confs[t][0][agree], rtol=1e-4)
