"""Block-wise generation with SPRINT over a growing prefix, on the GPU.

LLaDA2.0-Uni generates B blocks one after another, each with up to T
denoising steps (SPRINT introduction: B x T forward passes).  The first step
of every block sees the complete prefix, the clean earlier blocks included
("Sparse Prefix Retention"), so a finished block's rows join the prefix
before the next block starts: its own K/V rows, its final outputs (the hidden
states the next pass's LM head reads) and the generated modality.  The next
block's pass then scores and prunes the grown prefix afresh; the pruned cache
is built once per block.

Prefix confidences are carried forward instead of recomputed.  A block is
predicted from the clean earlier blocks and itself ("BDLM Loss" notation: a
block-causal mask), so once a block is finished the hidden states of its
positions, and so their LM-head confidences, never change.  The confidences
of a finished block's positions are exactly the block confidences of its
last step (the same LM head on the same outputs that become its hidden
states), so after block 0 the pass needs no prefix LM head at all: the
previous confidences plus the last step's block confidences are the grown
prefix's.  `carry_conf=False` recomputes them every block, as the page's
full forward pass does.

The driver sequences library calls only.  Buffers are sized once for the
last block: two ping-pong sets of packed prefix arrays that
sprint_append_rows grows by one block per sequence, and per-block keep
plans computed on the host up front, so the loop itself allocates nothing
and copies nothing from the host.
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np
import torch

from . import sprint, synth
from .block import SprintBlock, _to_dev


class SprintGeneration:
    """B consecutive blocks of one workload; block b >= 1 draws its own Q, Kb,
    Vb (synth.make_block_inputs) and sees the prefix grown by blocks < b."""

    def __init__(self, x: synth.Inputs, n_blocks: int, device="cuda", seed: int = 0,
                 carry_conf: bool = True, **block_kw):
        if n_blocks < 1:
            raise ValueError("n_blocks must be >= 1")
        wl, lay = x.wl, x.layout
        self.wl, self.layout, self.B = wl, lay, n_blocks
        self.carry_conf = carry_conf
        nseq, Lq = lay.nseq, wl.Lq
        self.nseq, self.Lq = nseq, Lq
        self.blk = SprintBlock(x, device, grow=(n_blocks - 1) * Lq, **block_kw)
        blk = self.blk
        dev = blk.device
        self.device = dev
        # per-block queries and block K/V
        self.Qs, self.Kbs, self.Vbs = [blk.Q], [blk.Kb], [blk.Vb]
        for b in range(1, n_blocks):
            Q, Kb, Vb = synth.make_block_inputs(wl, nseq, b, seed)
            self.Qs.append(_to_dev(Q, wl.dtype, dev))
            self.Kbs.append(_to_dev(Kb, wl.dtype, dev))
            self.Vbs.append(_to_dev(Vb, wl.dtype, dev))
        # per-block layouts and keep plans (host), uploaded once
        gm = wl.gen_modality
        self.lens: List[np.ndarray] = []
        self.cu_kept_host: List[list] = []
        self.keep_dev: List[torch.Tensor] = []
        self.cu_kept_dev: List[torch.Tensor] = []
        self.n_text: List[np.ndarray] = []
        self.n_img: List[np.ndarray] = []
        for b in range(n_blocks):
            nt = lay.n_text + (b * Lq if gm == synth.TEXT else 0)
            ni = lay.n_img + (b * Lq if gm == synth.IMAGE else 0)
            keep, cu_kept, _ = sprint.sprint_plan_keep(nt, ni, blk.r_text, blk.r_img)
            self.lens.append(lay.lens + b * Lq)
            self.n_text.append(nt)
            self.n_img.append(ni)
            self.cu_kept_host.append(cu_kept)
            self.keep_dev.append(torch.tensor(keep, dtype=torch.int32, device=dev))
            self.cu_kept_dev.append(torch.tensor(cu_kept, dtype=torch.int32, device=dev))
        # block 0's prefix is the block object's own; blocks >= 1 alternate
        # between two grown sets
        self.base = (blk.K, blk.V, blk.hidden, blk.modality, blk.cu_len)
        cap = lay.total_L + (n_blocks - 1) * nseq * Lq
        H = wl.H
        kdt = blk.K.dtype
        self.sets = []
        for _ in range(2 if n_blocks > 1 else 0):
            self.sets.append((
                torch.empty((cap, wl.Hkv, wl.D), dtype=kdt, device=dev),
                torch.empty((cap, wl.Hkv, wl.D), dtype=kdt, device=dev),
                # hidden states are only read by a recomputed prefix LM head
                (torch.empty((cap, H), dtype=kdt, device=dev)
                 if blk.hidden is not None and not carry_conf else None),
                torch.empty(cap, dtype=torch.uint8, device=dev),
                torch.empty(nseq + 1, dtype=torch.int32, device=dev),
                torch.empty(cap, dtype=torch.float32, device=dev),
            ))
        self.mod_blk = torch.full((nseq * Lq,), gm, dtype=torch.uint8, device=dev)
        self.tokens_out = torch.empty((n_blocks, nseq, Lq), dtype=torch.int32, device=dev)

    # ------------------------------------------------------------------ pieces
    def prefix(self, b: int):
        """(K, V, hidden, modality, cu_len) views of block b's prefix."""
        if b == 0:
            return self.base
        rows = int(np.sum(self.lens[b]))
        K, V, hid, mod, cu, _ = self.sets[(b - 1) % 2]
        return K[:rows], V[:rows], (hid[:rows] if hid is not None else None), mod[:rows], cu

    def conf_carried(self, b: int) -> bool:
        """Whether block b's pass takes its prefix confidences from earlier blocks."""
        return self.carry_conf and b > 0

    def begin_block(self, b: int):
        """Point the block object at block b's prefix and inputs."""
        blk = self.blk
        K, V, hid, mod, cu = self.prefix(b)
        conf = None
        if self.conf_carried(b):
            conf = self.sets[(b - 1) % 2][5][:K.shape[0]]
        blk.set_prefix(K, V, hid, mod, cu, self.lens[b], self.keep_dev[b], self.cu_kept_dev[b],
                       self.cu_kept_host[b], conf=conf)
        blk.Q, blk.Kb, blk.Vb = self.Qs[b], self.Kbs[b], self.Vbs[b]

    def finish_block(self, b: int, full: bool = False):
        """Record block b's tokens and append its rows to form block b+1's
        prefix (`full`: the block ran the unpruned baseline, which needs no
        prefix confidences)."""
        blk = self.blk
        self.tokens_out[b].copy_(blk.tokens)
        if b + 1 >= self.B:
            return
        K, V, hid, mod, cu = self.prefix(b)
        Kn, Vn, hidn, modn, cun, confn = self.sets[b % 2]
        rows = int(np.sum(self.lens[b + 1]))
        sprint.sprint_append_rows(K, cu, blk.Kb, out=Kn[:rows], cu_out=cun)
        # cu_out is written once, by the first call
        sprint.sprint_append_rows(V, cu, blk.Vb, out=Vn[:rows], cu_out=None)
        sprint.sprint_append_rows(mod, cu, self.mod_blk, out=modn[:rows], cu_out=None)
        if self.carry_conf and not full:
            # the last step's block confidences are those of the rows appended
            sprint.sprint_append_rows(blk.conf_prefix, cu, blk.conf_blk, out=confn[:rows],
                                      cu_out=None)
        if hid is not None and not self.carry_conf:
            sprint.sprint_append_rows(hid, cu, blk.O, out=hidn[:rows], cu_out=None)

    # ------------------------------------------------------------------ loop
    def run(self, n_steps: int, full: bool = False, on_block=None):
        """All B blocks: SPRINT (pass + n_steps pruned steps) or, with `full`,
        the unpruned baseline (n_steps + 1 steps over the full prefix).
        `on_block(b)` runs after each block, before its rows are appended."""
        for b in range(self.B):
            self.begin_block(b)
            if full:
                self.blk.run_full_block(n_steps)
            else:
                self.blk.run_block(n_steps, prefix_conf=not self.conf_carried(b))
            if on_block is not None:
                on_block(b)
            self.finish_block(b, full)
        return self.tokens_out
