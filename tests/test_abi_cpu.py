"""The C ABI without a GPU: the library loads, exports what the header
declares, computes its host-side keep counts, and rejects bad arguments
before any HIP call."""
import ctypes
import json
import os
import re

import pytest

from sparse_prefix_kv_amd import sprint

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sprint.h")
FAKE = 0x10000          # a 16-byte-aligned address that is never dereferenced


def _header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)
    return sorted({n for n in names if n not in ("if", "sizeof")})


def test_library_exports_every_declared_function():
    lib = sprint.lib()
    declared = _header_functions()
    assert len(declared) >= 19
    for name in declared:
        assert hasattr(lib, name), name
    assert set(declared) == set(sprint.EXPORTS)


def test_strerror_and_version():
    assert sprint.strerror(0) == "ok"
    assert "workspace" in sprint.strerror(3)
    assert sprint.lib().sprint_version() >= 100


def test_keep_count_matches_page_rule_golden():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "sprint_settings.json")))
    for row in g["keep_counts"]:
        assert sprint.sprint_keep_count(row["r"], row["n"]) == row["k"]
    assert sprint.sprint_keep_count(float("nan"), 10) == 0
    assert sprint.sprint_keep_count(2.0, 10) == 10
    assert sprint.sprint_keep_count(0.8, 0) == 0


def test_plan_keep():
    keep, cu, tot = sprint.sprint_plan_keep([1024, 512, 0], [3072, 15872, 64], 1.0, 0.8)
    assert keep == [1024, 2457, 512, 12697, 0, 51]
    assert cu == [0, 3481, 3481 + 13209, 3481 + 13209 + 51]
    assert tot == cu[-1]
    with pytest.raises(sprint.SprintError):
        sprint.sprint_plan_keep([-1], [3], 1.0, 1.0)


def test_workspace_queries_are_host_only():
    # at least one 16-byte partial per row and vocabulary tile of at most 256 entries
    assert sprint.lmhead_confidence_ws(4096, 2048, 32768, sprint.BF16) >= 4096 * 128 * 16
    assert sprint.sprint_score_ws(4096, 1) > 0
    assert sprint.sprint_prune_kv_ws(4096, 1) > 0
    assert sprint.block_attend_ws(1, 32, 16, 4, 128, 4096, 1) > 0
    assert sprint.block_attend_ws(1, 32, 16, 5, 128, 4096, 1) == 0       # Hq % Hkv != 0


def _call(name, *args):
    return getattr(sprint.lib(), name)(*args)


def test_lmhead_rejects_before_hip():
    ok = (FAKE, 32, 2048, FAKE, 32768, sprint.BF16, FAKE, FAKE, None, FAKE, 1 << 30, None)
    a = list(ok); a[0] = None
    assert _call("lmhead_confidence", *a) == 1                      # NULL hidden
    a = list(ok); a[0] = FAKE + 2
    assert _call("lmhead_confidence", *a) == 1                      # misaligned
    a = list(ok); a[2] = 100
    assert _call("lmhead_confidence", *a) == 2                      # H not a multiple of 64
    a = list(ok); a[5] = 7
    assert _call("lmhead_confidence", *a) == 1                      # bad dtype
    a = list(ok); a[10] = 16
    assert _call("lmhead_confidence", *a) == 3                      # workspace too small
    a = list(ok); a[1] = 0
    assert _call("lmhead_confidence", *a) == 1                      # M = 0


def test_score_and_prune_reject_before_hip():
    sc = [FAKE, FAKE, FAKE, 1, 4096, 4, 128, sprint.BF16, 0.5, FAKE, FAKE, FAKE, 1 << 30, None]
    a = list(sc); a[6] = 96
    assert _call("sprint_score", *a) == 2
    a = list(sc); a[3] = 0
    assert _call("sprint_score", *a) == 1
    a = list(sc); a[8] = float("inf")
    assert _call("sprint_score", *a) == 1
    a = list(sc); a[12] = 4
    assert _call("sprint_score", *a) == 3
    pr = [FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4096, 3481, FAKE, FAKE, 4, 128, sprint.BF16,
          FAKE, FAKE, FAKE, FAKE, 1 << 30, None]
    a = list(pr); a[7] = 5000
    assert _call("sprint_prune_kv", *a) == 1                        # kept > total
    a = list(pr); a[13] = None
    assert _call("sprint_prune_kv", *a) == 1                        # NULL K_out
    a = list(pr); a[17] = 1
    assert _call("sprint_prune_kv", *a) == 3


def test_per_layer_score_and_prune_reject_before_hip():
    ws = sprint.sprint_prune_kv_per_layer_ws(4096, 1, 16)
    assert ws > sprint.sprint_prune_kv_ws(4096, 1)
    assert sprint.sprint_prune_kv_per_layer_ws(4096, 1, 0) == 0
    sc = [FAKE, 16, FAKE, FAKE, 1, 4096, 4, 128, sprint.BF16, 0.5, FAKE, FAKE, FAKE, 1 << 30, None]
    a = list(sc); a[1] = 0
    assert _call("sprint_score_per_layer", *a) == 1                 # no layers
    a = list(sc); a[1] = 65536
    assert _call("sprint_score_per_layer", *a) == 1
    a = list(sc); a[13] = sprint.sprint_score_layers_ws(4096, 1, 16) - 1
    assert _call("sprint_score_per_layer", *a) == 3
    pr = [FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4096, 3481, FAKE, FAKE, 16, 4, 128, sprint.BF16,
          FAKE, FAKE, FAKE, FAKE, ws, None]
    a = list(pr); a[18] = sprint.sprint_prune_kv_ws(4096, 1)
    assert _call("sprint_prune_kv_per_layer", *a) == 3              # one layer's workspace
    a = list(pr); a[10] = 0
    assert _call("sprint_prune_kv_per_layer", *a) == 1
    a = list(pr); a[16] = None
    assert _call("sprint_prune_kv_per_layer", *a) == 1              # NULL kept_idx


def test_attend_and_unmask_reject_before_hip():
    at = [FAKE, 1, 32, 16, FAKE, FAKE, FAKE, 4096, 4096, FAKE, FAKE, 4, 128, 0.088, sprint.BF16,
          FAKE, FAKE, 1 << 30, None]
    a = list(at); a[11] = 5
    assert _call("block_attend", *a) == 1                           # Hq % Hkv
    a = list(at); a[12] = 80
    assert _call("block_attend", *a) == 2                           # head dim
    a = list(at); a[2] = 65
    assert _call("block_attend", *a) == 2                           # Lq > 64
    a = list(at); a[10] = None
    assert _call("block_attend", *a) == 1                           # Kb without Vb
    a = list(at); a[9] = None; a[10] = None; a[8] = 0
    assert _call("block_attend", *a) == 1                           # no keys at all
    a = list(at); a[13] = 0.0
    assert _call("block_attend", *a) == 1                           # scale must be > 0
    a = list(at); a[8] = 4095
    assert _call("block_attend", *a) == 1                           # one sequence longer than max_kv
    a = list(at); a[17] = 8
    assert _call("block_attend", *a) == 3
    um = [FAKE, FAKE, 1, 32, 0.9, 9, FAKE, FAKE, FAKE, None]
    a = list(um); a[3] = 65
    assert _call("unmask_select", *a) == 2
    a = list(um); a[4] = float("nan")
    assert _call("unmask_select", *a) == 1
    a = list(um); a[6] = None
    assert _call("unmask_select", *a) == 1


def test_append_rejects_before_hip():
    # old, cu_old, nseq, total_old, blk, n_blk, row_bytes, out, cu_out, stream
    ap = [FAKE, FAKE, 2, 100, FAKE + (1 << 20), 32, 1024, FAKE + (1 << 24), FAKE + 64, None]
    a = list(ap); a[2] = 0
    assert _call("sprint_append_rows", *a) == 1                     # no sequences
    a = list(ap); a[5] = -1
    assert _call("sprint_append_rows", *a) == 1                     # negative block rows
    a = list(ap); a[6] = 0
    assert _call("sprint_append_rows", *a) == 1                     # empty rows
    a = list(ap); a[8] = FAKE
    assert _call("sprint_append_rows", *a) == 1                     # cu_out aliases cu_old
    a = list(ap); a[7] = FAKE + 1024
    assert _call("sprint_append_rows", *a) == 1                     # out overlaps old
    a = list(ap); a[7] = FAKE + (1 << 20) + 64
    assert _call("sprint_append_rows", *a) == 1                     # out overlaps blk
    a = list(ap); a[0] = None
    assert _call("sprint_append_rows", *a) == 1                     # NULL old with rows
    a = list(ap); a[1] = FAKE + 2
    assert _call("sprint_append_rows", *a) == 1                     # misaligned cu_old


def test_layers_entry_points_reject_before_hip():
    # K, n_layers, conf, cu_len, nseq, total_L, Hkv, D, dtype, alpha, ibar, score, ws, ws_bytes
    sc = [FAKE, 4, FAKE, FAKE, 1, 4096, 4, 128, sprint.BF16, 0.5, FAKE, FAKE, FAKE, 1 << 30, None]
    a = list(sc); a[1] = 0
    assert _call("sprint_score_layers", *a) == 1                    # no layers
    a = list(sc); a[7] = 96
    assert _call("sprint_score_layers", *a) == 2                    # head dim
    a = list(sc); a[13] = 8
    assert _call("sprint_score_layers", *a) == 3                    # workspace
    assert sprint.sprint_score_layers_ws(4096, 1, 4) > sprint.sprint_score_ws(4096, 1)
    pr = [FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4096, 3481, FAKE, FAKE, 4, 4, 128, sprint.BF16,
          FAKE, FAKE, FAKE, FAKE, 1 << 30, None]
    a = list(pr); a[10] = 0
    assert _call("sprint_prune_kv_layers", *a) == 1                 # no layers
    a = list(pr); a[7] = 5000
    assert _call("sprint_prune_kv_layers", *a) == 1                 # kept > total
    a = list(pr); a[15] = None
    assert _call("sprint_prune_kv_layers", *a) == 1                 # NULL V_out


def test_moe_rejects_before_hip():
    # x, M, H, w_router, bias, E, top_k, scale, w_gate, w_up, w_down, inter, dtype,
    # residual, y, ids, gates, ws, ws_bytes, stream
    ok = [FAKE, 32, 2048, FAKE, FAKE, 256, 8, 2.5, FAKE, FAKE, FAKE, 512, sprint.BF16, None,
          FAKE, FAKE, FAKE, FAKE, 1 << 30, None]
    a = list(ok); a[6] = 257
    assert _call("moe_ffn", *a) == 1                                # top_k > E
    a = list(ok); a[7] = float("inf")
    assert _call("moe_ffn", *a) == 1                                # scale not finite
    a = list(ok); a[2] = 2304
    assert _call("moe_ffn", *a) == 2                                # H not supported
    a = list(ok); a[11] = 500
    assert _call("moe_ffn", *a) == 2                                # inter not supported
    a = list(ok); a[6] = 17
    assert _call("moe_ffn", *a) == 2                                # top_k > 16
    a = list(ok); a[13] = FAKE + 4
    assert _call("moe_ffn", *a) == 1                                # misaligned residual
    a = list(ok); a[18] = 64
    assert _call("moe_ffn", *a) == 3                                # workspace
    assert sprint.moe_ffn_ws(32, 2048, 256, 8, 512) >= 32 * 8 * (512 + 2048) * 4


def test_binding_checks_dtypes_and_sizes_before_the_device():
    # CPU tensors with a wrong dtype or size are rejected before the device
    # check, so a mismatched buffer never reaches a kernel
    import torch
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    Q = torch.zeros(1, 4, 4, 64, dtype=bf)
    K = torch.zeros(10, 2, 64, dtype=f32)
    with pytest.raises(TypeError):
        sprint.block_attend(Q, K, K, torch.zeros(2, dtype=i32), 10)
    X = torch.zeros(8, 64, dtype=bf)
    with pytest.raises(ValueError):
        sprint.lmhead_confidence(X, torch.zeros(16, 32, dtype=bf))          # H mismatch
    with pytest.raises(ValueError):
        sprint.lmhead_confidence(X, torch.zeros(16, 64, dtype=bf),
                                 conf=torch.zeros(4, dtype=f32))             # conf too small
    conf = torch.zeros(2, 8, dtype=f32)
    with pytest.raises(TypeError):
        sprint.unmask_select(conf, torch.zeros(2, 8, dtype=torch.int64),
                             torch.zeros(2, 8, dtype=torch.uint8), torch.zeros(2, 8, dtype=i32),
                             0.9, 4)
    Kl = torch.zeros(2, 10, 2, 64, dtype=bf)
    with pytest.raises(ValueError):
        sprint.sprint_prune_kv_layers(torch.zeros(10, dtype=f32), torch.zeros(10, dtype=torch.uint8),
                                      torch.zeros(2, dtype=i32), torch.zeros(2, dtype=i32),
                                      torch.zeros(2, dtype=i32), 11, Kl, Kl)  # kept > total
    with pytest.raises(TypeError):
        sprint.moe_ffn(X, torch.zeros(4, 64, dtype=bf), torch.zeros(4, dtype=bf),  # bias dtype
                       torch.zeros(4, 32, 64, dtype=bf), torch.zeros(4, 32, 64, dtype=bf),
                       torch.zeros(4, 64, 32, dtype=bf), 2)
    with pytest.raises(ValueError):
        sprint.sprint_append_rows(torch.zeros(5, 3, dtype=f32), torch.tensor([0, 5], dtype=i32),
                                  torch.zeros(1, 2, 3, dtype=f32),
                                  out=torch.zeros(6, 3, dtype=f32))          # out too small


def test_c_program_links_and_runs_host_checks():
    """tests/c_abi_check.cpp includes only include/sprint.h and the HIP
    runtime header: it compiling, linking and passing its host-side checks
    shows the boundary is usable from C++ without Python."""
    import subprocess
    exe = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_check")
    assert os.path.exists(exe), "tests/c_abi_check is missing: run python -m sparse_prefix_kv_amd.build"
    r = subprocess.run([exe, "--host-only"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout


def test_binding_raises_without_the_library():
    """No CPU fallback: with libsprint.so absent the binding raises at once."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("from sparse_prefix_kv_amd import sprint\n"
            "sprint.LIB_PATH = '/nonexistent/libsprint.so'\n"
            "try:\n"
            "    sprint.lib()\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=root,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    assert "raised:" in r.stdout and "missing" in r.stdout


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], capture_output=True,
                       text=True, cwd=root, timeout=120)
    assert r.returncode != 0
    assert "--gpus 2" in r.stderr and "single" in r.stderr


def test_committed_traffic_counters_match_the_kernel_source():
    """profiles/traffic.json names the source its counters were taken on.
    Counters taken on another version of that source are stale: bench.py
    then reports traffic null (and so this test skips) until they are
    re-taken."""
    import hashlib
    tj = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    for name, ent in tj.items():
        assert ent["hbm_bytes_per_launch"] > 0
        assert os.path.exists(os.path.join(ROOT, ent["summary"]))
        src = open(os.path.join(ROOT, ent["source"]), "rb").read()
        if hashlib.sha256(src).hexdigest()[:16] != ent["source_sha"]:
            pytest.skip(f"{name}: counters taken on an earlier {ent['source']}; bench.py "
                        "reports traffic null until they are re-taken")
