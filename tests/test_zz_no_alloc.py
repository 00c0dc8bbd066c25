"""block_attend_noalloc: the workspace-free variant of block_attend, whose
key-range partials live in the library's fixed device array, gives exactly
block_attend's output on consecutive calls of different sizes (the array
keeps the previous call's contents), replays correctly from a HIP graph, and
takes no memory from the caller's allocator."""
import numpy as np
import pytest
import torch

from sparse_prefix_kv_amd import sprint, synth
from sparse_prefix_kv_amd.block import _to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(kv_lens, dtype, seed, Hq=16, Hkv=4, D=128, Lq=32):
    nseq = len(kv_lens)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(kv_lens)]).astype(np.int32)).to(DEV)
    total = int(sum(kv_lens))
    Q = _to_dev(synth.normal_array((nseq, Lq, Hq, D), seed, 1.0, dtype), dtype, DEV)
    K = _to_dev(synth.normal_array((total, Hkv, D), seed + 1, 1.0, dtype), dtype, DEV)
    V = _to_dev(synth.normal_array((total, Hkv, D), seed + 2, 1.0, dtype), dtype, DEV)
    Kb = _to_dev(synth.normal_array((nseq, Lq, Hkv, D), seed + 3, 1.0, dtype), dtype, DEV)
    Vb = _to_dev(synth.normal_array((nseq, Lq, Hkv, D), seed + 4, 1.0, dtype), dtype, DEV)
    return Q, K, V, cu, max(kv_lens), Kb, Vb


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_equals_block_attend_on_consecutive_calls(dtype):
    # a split cache, then a smaller one, then one that needs no partials
    for kv_lens, seed in (([27852], 10), ([3000, 700], 20), ([100], 30)):
        Q, K, V, cu, mx, Kb, Vb = _case(kv_lens, dtype, seed)
        ref = sprint.block_attend(Q, K, V, cu, mx, Kb, Vb)
        out = torch.full_like(ref, float("nan"))
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        sprint.block_attend_noalloc(Q, K, V, cu, mx, Kb, Vb, O=out)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        assert torch.equal(out, ref), (kv_lens, dtype)


def test_noalloc_graph_replays():
    Q, K, V, cu, mx, Kb, Vb = _case([13209], "bf16", 40)
    ref = sprint.block_attend(Q, K, V, cu, mx, Kb, Vb)
    out = torch.empty_like(ref)
    sprint.block_attend_noalloc(Q, K, V, cu, mx, Kb, Vb, O=out)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        sprint.block_attend_noalloc(Q, K, V, cu, mx, Kb, Vb, O=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sprint.block_attend_noalloc(Q, K, V, cu, mx, Kb, Vb, O=out)
    for rep in range(3):
        out.zero_()                           # eager work between replays
        # another size through the same array between replays
        Q2, K2, V2, cu2, mx2, Kb2, Vb2 = _case([5000, 900], "bf16", 50 + rep)
        o2 = torch.empty_like(Q2)
        sprint.block_attend_noalloc(Q2, K2, V2, cu2, mx2, Kb2, Vb2, O=o2)
        torch.cuda.synchronize()
        assert torch.equal(o2, sprint.block_attend(Q2, K2, V2, cu2, mx2, Kb2, Vb2))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), rep
    del g
