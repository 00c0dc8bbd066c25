"""One SPRINT block of a several-layer stand-in on the GPU.

Every layer holds its own prefix KV cache and its own block queries and K/V;
the prefix confidences (one per position) come from the LM head over the
prefix hidden states, and each step's block confidences from the LM head over
the last layer's output.  Sparse Prefix Retention then prunes every layer's
cache, either with one kept set shared by all layers (the layer-mean of the
mean-normalised key norms: sprint_score_layers + sprint_prune_kv_layers, one
top-k and one compaction launch over all layers) or with a set per layer
(sprint_score_per_layer + sprint_prune_kv_per_layer: each layer's own scores
and kept set, still one launch of each kernel over all layers).  Steps attend layer by layer, as
a model's layers must run in order; only the layers' inputs are independent
draws here, since no layer weights are part of this path.

The driver sequences library calls over buffers it allocates once.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import sprint, synth
from .block import BIG_STEPS, _to_dev


class SprintLayers:
    MODES = ("shared", "per_layer")

    def __init__(self, x: synth.Inputs, n_layers: int, device="cuda", mode: str = "shared",
                 seed: int = 0, r_text: Optional[float] = None, r_img: Optional[float] = None,
                 tau: Optional[float] = None, T="wl", alpha: Optional[float] = None):
        if n_layers < 1:
            raise ValueError("n_layers must be >= 1")
        if mode not in self.MODES:
            raise ValueError(f"mode must be one of {self.MODES}")
        wl, lay = x.wl, x.layout
        self.wl, self.layout, self.n_layers, self.mode = wl, lay, n_layers, mode
        self.r_text = wl.r_text if r_text is None else r_text
        self.r_img = wl.r_img if r_img is None else r_img
        self.tau = wl.tau if tau is None else tau
        self.T = wl.T if T == "wl" else T
        self.alpha = wl.alpha if alpha is None else alpha
        dev = torch.device(device)
        self.device = dev
        dt = wl.dtype
        self.nseq, self.Lq, self.Hq, self.Hkv, self.D = lay.nseq, wl.Lq, wl.Hq, wl.Hkv, wl.D
        draws = [(x.Q, x.K, x.V, x.Kb, x.Vb)] + [synth.make_layer_inputs(wl, lay, l, seed)
                                                 for l in range(1, n_layers)]

        def stack(i):
            return torch.stack([_to_dev(d[i], dt, dev) for d in draws])
        # layer-major device arrays
        self.Q, self.K, self.V, self.Kb, self.Vb = (stack(i) for i in range(5))
        del draws
        self.hidden = _to_dev(x.hidden, dt, dev)
        self.W = _to_dev(x.W, dt, dev)
        self.cu_len = torch.from_numpy(lay.cu_len.astype(np.int32)).to(dev)
        self.modality = torch.from_numpy(lay.modality).to(dev)
        self.max_len = int(lay.lens.max())
        self.total_L = lay.total_L
        keep, cu_kept, total_kept = sprint.sprint_plan_keep(lay.n_text, lay.n_img, self.r_text,
                                                            self.r_img)
        self.keep = torch.tensor(keep, dtype=torch.int32, device=dev)
        self.cu_kept = torch.tensor(cu_kept, dtype=torch.int32, device=dev)
        self.total_kept = total_kept
        self.max_kept = int(np.max(np.diff(cu_kept)))
        f32, i32, u8 = torch.float32, torch.int32, torch.uint8
        tl, tk = self.total_L, max(total_kept, 1)
        n_sets = 1 if mode == "shared" else n_layers
        self.conf_prefix = torch.empty(tl, dtype=f32, device=dev)
        self.argmax_prefix = torch.empty(tl, dtype=i32, device=dev)
        self.ibar = torch.empty((n_sets, tl), dtype=f32, device=dev)
        self.score = torch.empty((n_sets, tl), dtype=f32, device=dev)
        self.kept_idx = torch.empty((n_sets, tk), dtype=i32, device=dev)[:, :total_kept]
        kshape = (n_layers, tk, self.Hkv, self.D)
        self.K_pr = torch.empty(kshape, dtype=self.K.dtype, device=dev)[:, :total_kept]
        self.V_pr = torch.empty(kshape, dtype=self.K.dtype, device=dev)[:, :total_kept]
        self.O = torch.empty_like(self.Q)
        M = self.nseq * self.Lq
        self.conf_blk = torch.empty(M, dtype=f32, device=dev)
        self.argmax_blk = torch.empty(M, dtype=i32, device=dev)
        n = self.nseq * self.Lq
        self._state = torch.empty(5 * n, dtype=u8, device=dev)   # tokens, then mask
        self.tokens = self._state[:4 * n].view(i32).view(self.nseq, self.Lq)
        self.masked = self._state[4 * n:].view(self.nseq, self.Lq)
        self.tokens.fill_(-1)
        self.masked.fill_(1)
        self._state0 = self._state.clone()
        self.n_acc = torch.empty(self.nseq, dtype=i32, device=dev)
        dti = sprint.BF16 if dt == "bf16" else sprint.F32

        def ws(n):
            return torch.empty(max(int(n), 256), dtype=u8, device=dev)
        self.ws_lm_prefix = ws(sprint.lmhead_confidence_ws(tl, wl.H, wl.vocab, dti))
        self.ws_lm_blk = ws(sprint.lmhead_confidence_unmask_ws(self.nseq, self.Lq, wl.H, wl.vocab,
                                                               dti))
        self.ws_score = ws(sprint.sprint_score_layers_ws(tl, self.nseq, n_layers))
        self.ws_prune = ws(sprint.sprint_prune_kv_ws(tl, self.nseq) if mode == "shared" else
                           sprint.sprint_prune_kv_per_layer_ws(tl, self.nseq, n_layers))
        self.ws_att_full = ws(sprint.block_attend_ws(self.nseq, self.Lq, self.Hq, self.Hkv, self.D,
                                                     self.max_len, True))
        self.ws_att_pr = ws(sprint.block_attend_ws(self.nseq, self.Lq, self.Hq, self.Hkv, self.D,
                                                   self.max_kept, True))

    # ------------------------------------------------------------------ pieces
    def reset(self):
        self._state.copy_(self._state0)

    def steps_left(self, t: int) -> int:
        return BIG_STEPS if self.T is None else self.T - t

    def prefix_confidence(self):
        sprint.lmhead_confidence(self.hidden, self.W, conf=self.conf_prefix,
                                 argmax=self.argmax_prefix, ws=self.ws_lm_prefix)

    def score_and_prune(self):
        if self.mode == "shared":
            sprint.sprint_score_layers(self.K, self.conf_prefix, self.cu_len, self.alpha,
                                       ibar=self.ibar[0], score=self.score[0], ws=self.ws_score)
            sprint.sprint_prune_kv_layers(self.score[0], self.modality, self.cu_len, self.keep,
                                          self.cu_kept, self.total_kept, self.K, self.V,
                                          K_out=self.K_pr, V_out=self.V_pr,
                                          kept_idx=self.kept_idx[0], ws=self.ws_prune)
            return
        sprint.sprint_score_per_layer(self.K, self.conf_prefix, self.cu_len, self.alpha,
                                      ibar=self.ibar, score=self.score, ws=self.ws_score)
        sprint.sprint_prune_kv_per_layer(self.score, self.modality, self.cu_len, self.keep,
                                         self.cu_kept, self.total_kept, self.K, self.V,
                                         K_out=self.K_pr, V_out=self.V_pr, kept_idx=self.kept_idx,
                                         ws=self.ws_prune)

    def attend_layers(self, pruned: bool):
        for l in range(self.n_layers):
            if pruned:
                sprint.block_attend(self.Q[l], self.K_pr[l], self.V_pr[l], self.cu_kept,
                                    self.max_kept, self.Kb[l], self.Vb[l], O=self.O[l],
                                    ws=self.ws_att_pr)
            else:
                sprint.block_attend(self.Q[l], self.K[l], self.V[l], self.cu_len, self.max_len,
                                    self.Kb[l], self.Vb[l], O=self.O[l], ws=self.ws_att_full)

    def confidence_and_unmask(self, t: int):
        """The last layer's LM-head confidences and one unmasking step, in one
        call (bitwise lmhead_confidence followed by unmask_select)."""
        M = self.nseq * self.Lq
        sprint.lmhead_confidence_unmask(self.O[-1].view(M, self.Hq * self.D), self.W,
                                        self.masked, self.tokens, self.tau, self.steps_left(t),
                                        conf=self.conf_blk, argmax=self.argmax_blk,
                                        n_accepted=self.n_acc, ws=self.ws_lm_blk)

    # ------------------------------------------------------------------ block
    def pruning_pass(self, prefix_conf: bool = True):
        """`prefix_conf=False`: the prefix confidences are already in
        conf_prefix (carried from the blocks that produced those positions,
        as in a generation after its first block), so the pass runs no
        prefix LM head."""
        if prefix_conf:
            self.prefix_confidence()
        self.score_and_prune()
        self.attend_layers(pruned=False)
        self.confidence_and_unmask(0)

    def pruned_step(self, t: int):
        self.attend_layers(pruned=True)
        self.confidence_and_unmask(t)

    def run_block(self, n_steps: int, prefix_conf: bool = True):
        self.reset()
        self.pruning_pass(prefix_conf)
        for t in range(1, n_steps + 1):
            self.pruned_step(t)

    def run_full_block(self, n_steps: int):
        """Baseline without pruning: every step attends to every layer's full prefix."""
        self.reset()
        for t in range(0, n_steps + 1):
            self.attend_layers(pruned=False)
            self.confidence_and_unmask(t)
