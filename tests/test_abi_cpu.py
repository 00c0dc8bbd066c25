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
    a = list(pr); a[6] = 1 << 22; a[7] = 1 << 21
    assert _call("sprint_prune_kv", *a) == 2                        # 2 GiB pruned cache
    a = list(pr); a[6] = 1 << 22; a[7] = (1 << 21) - 1; a[17] = 1
    assert _call("sprint_prune_kv", *a) == 3                        # just under: passes to ws


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
    a = list(at); a[7] = 1 << 21; a[8] = 1 << 21
    assert _call("block_attend", *a) == 2                           # 2 GiB of K rows
    a = list(at); a[7] = (1 << 21) - 1; a[8] = (1 << 21) - 1; a[17] = 8
    assert _call("block_attend", *a) == 3                           # just under: passes to ws
    # the workspace-free variant: same checks, and a plan whose partials
    # exceed its 16 MiB array is refused (fp32, 4 sequences of up to 2^20 keys)
    na = at[:16] + [None]
    a = list(na); a[11] = 5
    assert _call("block_attend_noalloc", *a) == 1
    a = list(na); a[1] = 4; a[8] = 1 << 20; a[14] = sprint.F32
    assert sprint.block_attend_ws(4, 32, 16, 4, 128, 1 << 20, 1) > (16 << 20)
    assert _call("block_attend_noalloc", *a) == 3
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
    """profiles/traffic.json keys each entry by call and workload and names
    the source its counters were taken on.  bench.py reports a call's
    traffic only for the workload its counters were taken on, and only while
    the source is unchanged: counters taken on another version are stale
    (bench.py then reports traffic null, and this test skips) until they are
    re-taken."""
    import hashlib
    tj = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    stale = []
    for name, ent in tj.items():
        call, workload = name.split("@")
        assert ent["workload"] == workload and call
        assert ent["hbm_bytes_per_launch"] > 0
        assert os.path.exists(os.path.join(ROOT, ent["summary"]))
        src = open(os.path.join(ROOT, ent["source"]), "rb").read()
        if hashlib.sha256(src).hexdigest()[:16] != ent["source_sha"]:
            stale.append(name)
    if stale:
        pytest.skip(f"{stale}: counters taken on an earlier source; bench.py "
                    "reports traffic null until they are re-taken")


# ---------------------------------------------------------------- argument fuzz
# Each entry point's arguments, as (kind, valid value) pairs, where a kind
# lists values that must be rejected before any HIP call when they replace
# the valid value alone ("bad"), and values that may or may not be valid
# ("alt").  The valid tuples pass every host check; with no GPU present they
# then fail at the first HIP call (SPRINT_EHIP), or succeed when they launch
# nothing.
NAN, INF = float("nan"), float("inf")
I32_MIN, I32_MAX, I64_MIN, I64_MAX = -2**31, 2**31 - 1, -2**63, 2**63 - 1
STREAM = ("stream", (), ())


def _p16(v=FAKE):
    return ("ptr16", (None, FAKE + 2, FAKE + 8), (FAKE + 16, FAKE + (1 << 20))), v


def _p4(v=FAKE):
    return ("ptr4", (None, FAKE + 1, FAKE + 2), (FAKE + 4,)), v


def _pb(v=FAKE):
    return ("bytes", (None,), (FAKE + 1, FAKE + 3)), v


def _o16(v=None):
    return ("opt16", (FAKE + 2, FAKE + 8), (None, FAKE + 32)), v


def _o4(v=None):
    return ("opt4", (FAKE + 2,), (None, FAKE + 4)), v


def _int(v, bad, alt=()):
    return ("int", tuple(bad), tuple(alt)), v


def _dt(v=None):
    return ("dtype", (2, 7, -1, 1 << 20), (sprint.F32, sprint.BF16)), sprint.BF16 if v is None else v


def _finite(v):
    return ("finite", (NAN, INF, -INF), (0.0, -3.0, 1e30)), v


def _wsb(v=1 << 30):
    return ("ws_bytes", (0, 1, 255), (1 << 40, 2**64 - 1)), v


NSEQ_BAD = (0, -1, I32_MIN, (1 << 24) + 1, I32_MAX)
HKV_BAD = (0, -1, 4097, I32_MAX)                          # 4097 * 128 * 2 bytes > 1 MiB
D_BAD = (0, -128, 80, 96, 256, I32_MAX)
NL_BAD = (0, -1, 65536, I32_MAX)


def _score_spec(n_layers=None):
    lay = [] if n_layers is None else [_int(n_layers, NL_BAD, (1, 2, 65535))]
    return [_p16()] + lay + [
        _p4(), _p4(), _int(1, NSEQ_BAD, (2, 4096)),
        _int(4096, (-1, I64_MIN, 2**31, 2**62), (0, 1, 100)),
        _int(4, HKV_BAD, (1, 8, 1024)), _int(128, D_BAD, (64,)), _dt(), _finite(0.5),
        _p4(), _p4(), _p16(), _wsb(), (STREAM, None)]


def _prune_spec(n_layers=None, ws=1 << 30):
    lay = [] if n_layers is None else [_int(n_layers, NL_BAD, (1, 2, 16))]
    return [_p4(), _pb(), _p4(), _p4(), _p4(), _int(1, NSEQ_BAD, (2,)),
            _int(4096, (-1, I64_MIN, 2**31, 2**62, 3480), (8192,)),
            _int(3481, (-1, I64_MIN, 4097, 2**62), (0, 1, 4096)), _p16(), _p16()] + lay + [
            _int(4, HKV_BAD, (1, 8)), _int(128, D_BAD, (64,)), _dt(), _p16(), _p16(), _p4(),
            _p16(), _wsb(ws), (STREAM, None)]


def _attend_spec(with_ws):
    head = [_p16(), _int(1, NSEQ_BAD, (2, 3)), _int(32, (0, -1, 65, I32_MAX), (1, 8, 64)),
            _int(16, (0, -1, 5, I32_MAX, 2**31 - 4), (4, 8, 32)), _p16(), _p16(), _p4(),
            _int(4096, (-1, I64_MIN, 2**31, 2**62, 4097), (0, 100)),
            _int(4096, (-1, I32_MIN, 4095), (I32_MAX, 8192)), _p16(), _p16(),
            _int(4, (0, -1, 1, 3, 32, I32_MAX), (2, 8, 16)), _int(128, D_BAD, (64,)),
            (("scale", (NAN, INF, -INF, 0.0, -0.0, -1.0), (1e-30, 1e30)), 0.088), _dt(), _p16()]
    return head + ([_p16(), _wsb()] if with_ws else []) + [(STREAM, None)]


FUZZ_SPECS = {
    "lmhead_confidence": [
        _p16(), _int(32, (0, -1, I64_MIN, 2**31, 2**62), (1, 4096)),
        _int(2048, (0, -1, 100, 65600, I32_MAX), (64, 65536)), _p16(),
        _int(32768, (0, -1, I32_MIN, 2**30, I32_MAX), (1, 3000)), _dt(), _p4(), _p4(), _o4(),
        _p16(), _wsb(), (STREAM, None)],
    "lmhead_confidence_unmask": [
        _p16(), _int(1, NSEQ_BAD, (2, 64)), _int(32, (0, -1, 65, I32_MAX), (1, 64)),
        _int(2048, (0, -1, 100, 65600, I32_MAX), (64, 65536)), _p16(),
        _int(32768, (0, -1, I32_MIN, 2**30, I32_MAX), (1, 3000)), _dt(), _p4(), _p4(),
        (("tau", (NAN,), (INF, -INF, 2.0, -1.0)), 0.95), _int(9, (), (0, -1, I32_MIN, I32_MAX)),
        _pb(), _p4(), _p4(), _p16(), _wsb(), (STREAM, None)],
    "sprint_score": _score_spec(),
    "sprint_score_layers": _score_spec(4),
    "sprint_score_per_layer": _score_spec(16),
    "sprint_prune_kv": _prune_spec(),
    "sprint_prune_kv_layers": _prune_spec(4),
    "sprint_prune_kv_per_layer": _prune_spec(16, sprint.sprint_prune_kv_per_layer_ws(4096, 1, 16)),
    "block_attend": _attend_spec(True),
    "block_attend_noalloc": _attend_spec(False),
    "unmask_select": [
        _p4(), _p4(), _int(1, NSEQ_BAD, (2, 1000)), _int(32, (0, -1, 65, I32_MAX), (1, 64)),
        (("tau", (NAN,), (INF, -INF, 2.0, -1.0)), 0.9), _int(9, (), (0, -1, I32_MIN, I32_MAX)),
        _pb(), _p4(), _p4(), (STREAM, None)],
    "sprint_append_rows": [
        _pb(), (("cu_old", (None, FAKE + 2), (FAKE + 4,)), FAKE),
        _int(2, NSEQ_BAD, (1, 3)), _int(100, (-1, I64_MIN, 2**31, 2**62), (0, 5)),
        _pb(FAKE + (1 << 20)), _int(32, (-1, I32_MIN), (0, 1)),
        _int(1024, (0, -1, 2**31 + 1, 2**62), (1, 3, 16)),
        (("out", (None, FAKE + 1024, FAKE + (1 << 20) + 64), (FAKE + (1 << 30),)),
         FAKE + (1 << 24)),
        (("cu_out", (FAKE, FAKE + 66), (None, FAKE + 128)), FAKE + 64), (STREAM, None)],
    "moe_ffn": [
        _p16(), _int(32, (0, -1, I32_MIN, 1025, I32_MAX), (1, 8, 1024)),
        _int(2048, (0, -1, 100, 2304, 4096, I32_MAX), (512, 1024)), _p16(), _p4(),
        _int(256, (0, -1, 7, 1025, I32_MAX), (8, 1024)),
        _int(8, (0, -1, 17, 257, I32_MAX), (1, 16)), _finite(2.5), _p16(), _p16(), _p16(),
        _int(512, (0, -1, 500, 1536, I32_MAX), (1024,)), _dt(), _o16(), _p16(), _p4(), _p4(),
        _p16(), _wsb(), (STREAM, None)],
}


def _status(name, args):
    st = _call(name, *args)
    assert isinstance(st, int)
    return st


needs_no_gpu = pytest.mark.skipif(
    os.path.exists("/dev/kfd"),
    reason="fake device pointers must never reach a kernel: runs only where no GPU exists")


@needs_no_gpu
def test_fuzz_specs_cover_every_device_entry_point():
    """Every compute call the header declares is fuzzed, with one spec entry
    per argument, and its valid tuple passes the host checks."""
    compute = [n for n in sprint.EXPORTS if not n.endswith("_ws") and n not in (
        "sprint_strerror", "sprint_version", "sprint_keep_count", "sprint_plan_keep")]
    assert sorted(compute) == sorted(FUZZ_SPECS)
    for name, spec in FUZZ_SPECS.items():
        assert len(spec) == len(sprint._SIGS[name][1]), name
        assert _status(name, [v for _, v in spec]) == 4, name        # SPRINT_EHIP: no device


@needs_no_gpu
@pytest.mark.parametrize("name", sorted(FUZZ_SPECS))
def test_abi_rejects_each_invalid_argument_before_hip(name):
    """Each argument replaced alone by an invalid value is rejected with
    EINVAL, EUNSUPPORTED or EWORKSPACE; other values never crash and give a
    documented status."""
    spec = FUZZ_SPECS[name]
    base = [v for _, v in spec]
    for i, ((kind, bad, alt), _) in enumerate(spec):
        for v in bad:
            a = list(base); a[i] = v
            assert _status(name, a) in (1, 2, 3), (name, i, kind, v)
        for v in alt:
            a = list(base); a[i] = v
            assert _status(name, a) in (0, 1, 2, 3, 4), (name, i, kind, v)


@needs_no_gpu
@pytest.mark.parametrize("seed", range(4))
def test_abi_survives_random_invalid_argument_mixes(seed):
    """Seeded fuzz: several arguments at once take bad or alternative values.
    Every call returns a documented status without crashing; when one of the
    changed arguments is a misaligned device pointer and no size was set to 0
    (an empty array's pointer is not checked), the call is rejected before
    HIP."""
    import random
    rng = random.Random(1000 + seed)
    n_calls = 0
    for name in sorted(FUZZ_SPECS):
        spec = FUZZ_SPECS[name]
        slots = [i for i, ((_, bad, alt), _) in enumerate(spec) if bad or alt]
        for _ in range(150):
            a = [v for _, v in spec]
            hard = zeroed = False
            for i in rng.sample(slots, rng.randint(2, min(5, len(slots)))):
                (kind, bad, alt), _ = spec[i]
                pool = [(v, True) for v in bad] + [(v, False) for v in alt]
                a[i], is_bad = rng.choice(pool)
                hard |= is_bad and kind in ("ptr16", "ptr4", "opt16", "opt4") and a[i] is not None
                zeroed |= kind == "int" and a[i] == 0
            st = _status(name, a)
            assert st in (0, 1, 2, 3, 4), (name, a, st)
            if hard and not zeroed:
                assert st in (1, 2, 3), (name, a, st)
            n_calls += 1
    assert n_calls == 150 * len(FUZZ_SPECS)


def test_plan_keep_random_counts_and_ratios():
    """Host-only keep planning over random counts (with negative and
    near-overflow ones) and ratios (with NaN, infinities and values outside
    [0, 1]): a valid plan keeps floor(r * n) clamped to [0, n] per sequence
    and modality, with prefix sums in cu_kept; anything else is EINVAL."""
    import math
    import random
    rng = random.Random(7)
    f = sprint.lib().sprint_plan_keep
    ratios = [0.0, 0.25, 0.5, 0.85, 1.0, 1.5, -0.5, NAN, INF, -INF, 1e-9, 0.999999]
    for trial in range(400):
        nseq = rng.randint(1, 6)
        pick = lambda: rng.choice([rng.randint(0, 5000), rng.randint(0, 2**31), 0, 1, -1,
                                   2**31 - 1, 2**62, I64_MAX])
        nt = (ctypes.c_int64 * nseq)(*[pick() for _ in range(nseq)])
        ni = (ctypes.c_int64 * nseq)(*[pick() for _ in range(nseq)])
        rt, ri = rng.choice(ratios), rng.choice(ratios)
        keep = (ctypes.c_int32 * (2 * nseq))()
        cu = (ctypes.c_int32 * (nseq + 1))()
        tot = ctypes.c_int64(-5)
        st = f(nt, ni, nseq, rt, ri, keep, cu, ctypes.byref(tot))

        def kc(r, n):
            if n <= 0 or r != r:
                return 0
            k = math.floor(r * n) if math.isfinite(r * n) else (n if r > 0 else 0)
            return max(0, min(int(k), n))
        ok = all(0 <= nt[s] and 0 <= ni[s] and nt[s] + ni[s] <= I32_MAX for s in range(nseq))
        if ok:
            ks = [(kc(rt, nt[s]), kc(ri, ni[s])) for s in range(nseq)]
            ok = sum(a + b for a, b in ks) <= I32_MAX
        if not ok:
            assert st == 1, (trial, list(nt), list(ni))
            continue
        assert st == 0, (trial, list(nt), list(ni), rt, ri)
        acc = 0
        assert cu[0] == 0
        for s, (kt, ki) in enumerate(ks):
            assert (keep[2 * s], keep[2 * s + 1]) == (kt, ki), (trial, s)
            acc += kt + ki
            assert cu[s + 1] == acc
        assert tot.value == acc
