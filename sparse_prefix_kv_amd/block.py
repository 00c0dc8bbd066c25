"""One SPRINT block on the GPU: the pruning pass plus the pruned denoising steps.

The driver only sequences calls into libsprint.so over device buffers that it
allocates once (so a timed loop allocates nothing).  The order follows the
SPRINT paragraphs of LLaDA2.0-Uni: the block's first step is the full pass
(attention over the whole prefix, block confidences and unmasking) whose
prefix confidences, with the key norms, score the prefix; the per-modality
top-k is compacted into the pruned cache; every later step attends to that
cache and unmasks by confidence.  Q and the block's own K/V stay fixed across
steps because the model that would refresh them is not part of this path.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import sprint, synth

BIG_STEPS = 1 << 30   # steps_left for "at least one acceptance per step"


class _NullCtx:
    def __enter__(self):
        return None

    def __exit__(self, *a):
        return False


def _to_dev(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    if dtype == "bf16":
        bits = synth.bf16_bits(a)
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


class SprintBlock:
    """Device state for one block of one workload."""

    def __init__(self, x: synth.Inputs, device="cuda", r_text: Optional[float] = None,
                 r_img: Optional[float] = None, tau: Optional[float] = None,
                 T: Optional[int] = "wl", alpha: Optional[float] = None, grow: int = 0,
                 moe=None, fused_tail: bool = True):
        """`grow`: rows per sequence the prefix may gain later (blocks appended
        by a generation loop); buffers and workspaces are sized for it once.
        `moe` = (w_router, bias, w_gate, w_up, w_down, top_k, route_scale) as
        device tensors puts an MoE FFN between attention and the LM head: the
        LM head then reads O + moe_ffn(O).  `fused_tail`: each step ends with
        one lmhead_confidence_unmask call instead of lmhead_confidence and
        unmask_select (bitwise the same state)."""
        wl = x.wl
        lay = x.layout
        self.wl, self.layout = wl, lay
        self.r_text = wl.r_text if r_text is None else r_text
        self.r_img = wl.r_img if r_img is None else r_img
        self.tau = wl.tau if tau is None else tau
        self.T = wl.T if T == "wl" else T
        self.alpha = wl.alpha if alpha is None else alpha
        dev = torch.device(device)
        self.device = dev
        dt = wl.dtype
        self.nseq, self.Lq, self.Hq, self.Hkv, self.D = lay.nseq, wl.Lq, wl.Hq, wl.Hkv, wl.D
        self.Q = _to_dev(x.Q, dt, dev)
        self.Kb = _to_dev(x.Kb, dt, dev)
        self.Vb = _to_dev(x.Vb, dt, dev)
        self.W = _to_dev(x.W, dt, dev)
        f32, i32, u8 = torch.float32, torch.int32, torch.uint8
        # largest prefix this object will see: every sequence grown by `grow`
        lens_max = lay.lens.astype(np.int64) + grow
        tl_max = int(lens_max.sum())
        _, cu_kept_max, kept_max = sprint.sprint_plan_keep(lay.n_text + grow, lay.n_img + grow,
                                                           self.r_text, self.r_img)
        tk_max = max(kept_max, 1)
        self._cap_L = max(tl_max, 1)
        self.conf_prefix_buf = torch.empty(self._cap_L, dtype=f32, device=dev)
        self.argmax_prefix_buf = torch.empty(self._cap_L, dtype=i32, device=dev)
        self.ibar_buf = torch.empty(self._cap_L, dtype=f32, device=dev)
        self.score_buf = torch.empty(self._cap_L, dtype=f32, device=dev)
        kdt = self.Q.dtype
        self.K_pr_buf = torch.empty((tk_max, self.Hkv, self.D), dtype=kdt, device=dev)
        self.V_pr_buf = torch.empty((tk_max, self.Hkv, self.D), dtype=kdt, device=dev)
        self.kept_idx_buf = torch.empty(tk_max, dtype=i32, device=dev)
        self.O = torch.empty_like(self.Q)
        M = self.nseq * self.Lq
        self.conf_blk = torch.empty(M, dtype=f32, device=dev)
        self.argmax_blk = torch.empty(M, dtype=i32, device=dev)
        # tokens (int32) and mask (uint8) share one buffer, so the block-start
        # state (all masked) comes back with one device copy; a copy rather
        # than a fill keeps memset nodes out of captured graphs
        n = self.nseq * self.Lq
        self._state = torch.empty(5 * n, dtype=u8, device=dev)
        self.tokens = self._state[:4 * n].view(i32).view(self.nseq, self.Lq)
        self.masked = self._state[4 * n:].view(self.nseq, self.Lq)
        self.tokens.fill_(-1)
        self.masked.fill_(1)
        self._state0 = self._state.clone()
        self.timer = None
        self.n_acc = torch.empty(self.nseq, dtype=i32, device=dev)
        dti = sprint.BF16 if dt == "bf16" else sprint.F32
        H, Vv = wl.H, wl.vocab
        self.moe = moe
        if moe is not None:
            wr, _, wg, _, _, k, _ = moe
            E, inter = wg.shape[0], wg.shape[1]
            self.moe_y = torch.empty((M, H), dtype=self.Q.dtype, device=dev)
            self.moe_ids = torch.empty((M, k), dtype=i32, device=dev)
            self.moe_gates = torch.empty((M, k), dtype=f32, device=dev)
            self.ws_moe = torch.empty(max(sprint.moe_ffn_ws(M, H, E, k, inter), 256), dtype=u8,
                                      device=dev)
        max_len_max = int(lens_max.max())
        max_kept_max = int(np.max(np.diff(cu_kept_max)))

        def ws(n):
            return torch.empty(max(int(n), 256), dtype=u8, device=dev)
        # workspace sizes grow with the sizes they are queried for
        self.ws_lm_prefix = ws(sprint.lmhead_confidence_ws(self._cap_L, H, Vv, dti))
        self.ws_lm_blk = ws(sprint.lmhead_confidence_ws(M, H, Vv, dti))
        self.fused_tail = fused_tail
        self.ws_lm_unmask = ws(sprint.lmhead_confidence_unmask_ws(self.nseq, self.Lq, H, Vv, dti))
        self.ws_score = ws(sprint.sprint_score_ws(self._cap_L, self.nseq))
        self.ws_prune = ws(sprint.sprint_prune_kv_ws(self._cap_L, self.nseq))
        # the attention split plan is not monotone in the cache length: size
        # for every length the prefix can pass through
        def att_ws(lo, hi):
            return max(sprint.block_attend_ws(self.nseq, self.Lq, self.Hq, self.Hkv, self.D, n, True)
                       for n in range(int(lo), int(hi) + 1))
        _, cu_kept0, _ = sprint.sprint_plan_keep(lay.n_text, lay.n_img, self.r_text, self.r_img)
        self.ws_att_full = ws(att_ws(lay.lens.max(), max_len_max))
        self.ws_att_pr = ws(att_ws(np.max(np.diff(cu_kept0)), max_kept_max))
        # the workload's own prefix
        K = _to_dev(x.K, dt, dev)
        V = _to_dev(x.V, dt, dev)
        hidden = _to_dev(x.hidden, dt, dev) if x.hidden is not None else None
        cu_len = torch.from_numpy(lay.cu_len.astype(np.int32)).to(dev)
        modality = torch.from_numpy(lay.modality).to(dev)
        keep, cu_kept, total_kept = sprint.sprint_plan_keep(lay.n_text, lay.n_img, self.r_text,
                                                            self.r_img)
        self.set_prefix(K, V, hidden, modality, cu_len, lay.lens,
                        torch.tensor(keep, dtype=i32, device=dev),
                        torch.tensor(cu_kept, dtype=i32, device=dev), cu_kept)

    def set_prefix(self, K, V, hidden, modality, cu_len, lens, keep, cu_kept, cu_kept_host,
                   conf=None):
        """Point the block at a (possibly grown) prefix: device K, V, hidden,
        modality and cu_len; host `lens` per sequence; device keep/cu_kept and
        the host copy of cu_kept (from sprint_plan_keep).  `conf`, if given, is
        a device array already holding the prefix confidences."""
        tl = int(K.shape[0])
        if tl > self._cap_L:
            raise ValueError(f"prefix of {tl} rows exceeds the {self._cap_L} sized for")
        self.K, self.V, self.hidden, self.modality, self.cu_len = K, V, hidden, modality, cu_len
        self.total_L = tl
        self.max_len = int(np.max(lens))
        self.keep, self.cu_kept = keep, cu_kept
        self.cu_kept_host = list(cu_kept_host)
        self.total_kept = int(cu_kept_host[-1])
        self.max_kept = int(np.max(np.diff(cu_kept_host)))
        self.conf_prefix = self.conf_prefix_buf[:tl] if conf is None else conf
        self.argmax_prefix = self.argmax_prefix_buf[:tl]
        self.ibar = self.ibar_buf[:tl]
        self.score = self.score_buf[:tl]
        self.K_pr = self.K_pr_buf[:self.total_kept]
        self.V_pr = self.V_pr_buf[:self.total_kept]
        self.kept_idx = self.kept_idx_buf[:self.total_kept]

    # ------------------------------------------------------------------ pieces
    def steps_left(self, t: int) -> int:
        return BIG_STEPS if self.T is None else self.T - t

    def reset(self):
        self._state.copy_(self._state0)

    def _t(self, name):
        """Event-timed region around one library call when a timer is set."""
        return self.timer(name) if self.timer is not None else _NullCtx()

    def prefix_confidence(self):
        with self._t("lmhead_prefix"):
            sprint.lmhead_confidence(self.hidden, self.W, conf=self.conf_prefix,
                                     argmax=self.argmax_prefix, ws=self.ws_lm_prefix)

    def score_prefix(self):
        with self._t("score"):
            sprint.sprint_score(self.K, self.conf_prefix, self.cu_len, self.alpha,
                                ibar=self.ibar, score=self.score, ws=self.ws_score)

    def prune_prefix(self):
        with self._t("prune"):
            sprint.sprint_prune_kv(self.score, self.modality, self.cu_len, self.keep,
                                   self.cu_kept, self.total_kept, self.K, self.V,
                                   K_out=self.K_pr, V_out=self.V_pr, kept_idx=self.kept_idx,
                                   ws=self.ws_prune)

    def score_and_prune(self):
        self.score_prefix()
        self.prune_prefix()

    def attend(self, pruned: bool):
        if pruned:
            with self._t("attend_pruned"):
                sprint.block_attend(self.Q, self.K_pr, self.V_pr, self.cu_kept, self.max_kept,
                                    self.Kb, self.Vb, O=self.O, ws=self.ws_att_pr)
        else:
            with self._t("attend_full"):
                sprint.block_attend(self.Q, self.K, self.V, self.cu_len, self.max_len, self.Kb,
                                    self.Vb, O=self.O, ws=self.ws_att_full)

    def moe_ffn(self):
        """y = O + moe_ffn(O), the LM head's input when an MoE FFN is set."""
        M = self.nseq * self.Lq
        wr, bias, wg, wu, wd, k, sc = self.moe
        O = self.O.view(M, self.Hq * self.D)
        with self._t("moe_ffn"):
            sprint.moe_ffn(O, wr, bias, wg, wu, wd, k, sc, residual=O, y=self.moe_y,
                           expert_ids=self.moe_ids, gates=self.moe_gates, ws=self.ws_moe)

    def block_confidence(self):
        M = self.nseq * self.Lq
        h = self.O.view(M, self.Hq * self.D)
        if self.moe is not None:
            self.moe_ffn()
            h = self.moe_y
        with self._t("lmhead_block"):
            sprint.lmhead_confidence(h, self.W, conf=self.conf_blk, argmax=self.argmax_blk,
                                     ws=self.ws_lm_blk)

    def unmask(self, t: int):
        with self._t("unmask"):
            sprint.unmask_select(self.conf_blk.view(self.nseq, self.Lq),
                                 self.argmax_blk.view(self.nseq, self.Lq), self.masked,
                                 self.tokens, self.tau, self.steps_left(t),
                                 n_accepted=self.n_acc)

    def confidence_and_unmask(self, t: int):
        if not self.fused_tail:
            self.block_confidence()
            self.unmask(t)
            return
        M = self.nseq * self.Lq
        h = self.O.view(M, self.Hq * self.D)
        if self.moe is not None:
            self.moe_ffn()
            h = self.moe_y
        with self._t("lmhead_unmask"):
            sprint.lmhead_confidence_unmask(h, self.W, self.masked, self.tokens, self.tau,
                                            self.steps_left(t), conf=self.conf_blk,
                                            argmax=self.argmax_blk, n_accepted=self.n_acc,
                                            ws=self.ws_lm_unmask)

    # ------------------------------------------------------------------ block
    def pruning_pass(self, prefix_conf: bool = True):
        """t = 0: full pass over the prefix, scoring and pruning, first unmask.
        `prefix_conf=False` takes conf_prefix as already filled (a generation
        loop that carries earlier blocks' confidences forward)."""
        if prefix_conf:
            self.prefix_confidence()
        self.score_and_prune()
        self.attend(pruned=False)
        self.confidence_and_unmask(0)

    def pruned_step(self, t: int):
        self.attend(pruned=True)
        self.confidence_and_unmask(t)

    def run_block(self, n_steps: int, prefix_conf: bool = True):
        self.reset()
        self.pruning_pass(prefix_conf)
        for t in range(1, n_steps + 1):
            self.pruned_step(t)

    def run_full_block(self, n_steps: int):
        """Baseline without SPRINT pruning: every step attends to the full prefix."""
        self.reset()
        for t in range(0, n_steps + 1):
            self.attend(pruned=False)
            self.confidence_and_unmask(t)
