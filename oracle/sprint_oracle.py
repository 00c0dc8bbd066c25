"""CPU oracle for the SPRINT block step -- TEST INFRASTRUCTURE ONLY.

Plain, slow, fp64 NumPy.  Only the tests, the package's ``smoke()`` entry and
the CPU-baseline leg of ``bench.py`` may import this module; the product path
never does.  It shares no code with the HIP library.

Source: "LLaDA2.0-Uni: Unifying Multimodal Understanding and Generation with
Diffusion Large Language Model" (arXiv 2604.20796, HTML version), the SPRINT
paragraphs:
  * SPRINT introduction -- B blocks x T denoising steps; two components.
  * "Sparse Prefix Retention" -- first step of a block is a full pass giving
    logits and the full KV cache; composite score of the mean-normalised key
    norm and the top-1 softmax confidence (alpha = 0.5); per-modality keep
    ratios, top-floor(r*n) kept within each modality; the pruned cache is
    built once per block and attended by every later step.
  * "Non-uniform Token Unmasking" -- per-position confidence of the predicted
    token; accept all masked positions above tau, at least ceil(m/(T-t)).
  * "BDLM Loss" notation -- a block is predicted from the clean earlier blocks
    and its own noisy block (the block's own keys are part of its context).

Readings of points the page leaves open (each is also listed in the design
notes): the score equation itself did not survive on the page, and is read as
the linear blend alpha*I + (1-alpha)*c; a position's key is the concatenation
of its KV heads; the mean runs over the sequence's prefix positions of both
modalities; ties in the top-k go to the lower position; "within each modality"
pools all runs of that modality in the sequence; GQA head h reads KV head
floor(h*Hkv/Hq); scores are scaled by 1/sqrt(D); "exceeds tau" is strict;
m is the current masked count and t the 0-based step.

Generation over several blocks (``append_block``, ``store_as``,
``run_generation``) reads the SPRINT introduction's B blocks x T steps with
the pass of "Sparse Prefix Retention" seeing the complete prefix: a finished
block's own K/V rows, its last step's outputs (as the hidden states of its
positions, stored in the workload's dtype) and the generated modality join
every sequence before the next block.

Parity status: every function below is pinned by the tests in
``tests/test_oracle_pins.py`` (closed forms, invariants, brute force).  The
one thing no pin can reach is the *reading* of the lost score equation
(``composite_score``): its arithmetic is pinned, its fidelity to the page is
"parity unpinned".
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np


# --------------------------------------------------------------------------
# Scoring (Sparse Prefix Retention)
# --------------------------------------------------------------------------

def key_norms(K) -> np.ndarray:
    """Per prefix position, the L2 norm of its key over all KV heads and dims.

    K: [total_L, Hkv, D].  Reading: the key k_i of position i is the
    concatenation of its KV heads, so ||k_i||^2 = sum_h sum_d K[i,h,d]^2.
    """
    K = np.asarray(K, dtype=np.float64)
    flat = K.reshape(K.shape[0], -1)
    return np.sqrt(np.einsum("ij,ij->i", flat, flat))


def key_norm_importance(K, cu_len) -> np.ndarray:
    """Mean-normalised key norm I_i = ||k_i|| / ((1/L) sum_j ||k_j||).

    Sparse Prefix Retention, definition of the key-norm importance.  The mean
    runs over the L prefix positions of each sequence (cu_len: [nseq+1]
    offsets).  A sequence whose keys are all zero has no defined ratio; it
    gets I_i = 1 (every position equally important).
    """
    n = key_norms(K)
    out = np.empty_like(n)
    cu = np.asarray(cu_len, dtype=np.int64)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        L = b - a
        if L == 0:
            continue
        mu = n[a:b].sum() / L
        out[a:b] = n[a:b] / mu if mu > 0.0 else 1.0
    return out


def composite_score(ibar, conf, alpha: float = 0.5) -> np.ndarray:
    """s_i = alpha * I_i + (1 - alpha) * c_i  (Sparse Prefix Retention).

    The page names the two blended terms and alpha = 0.5 but its equation was
    lost; the linear blend is the plain reading (at alpha = 0.5 the order of
    the terms does not matter).
    """
    ibar = np.asarray(ibar, dtype=np.float64)
    conf = np.asarray(conf, dtype=np.float64)
    return alpha * ibar + (1.0 - alpha) * conf


def keep_count(r: float, n: int) -> int:
    """floor(r * n), clamped to [0, n]  (Sparse Prefix Retention, keep rule)."""
    k = math.floor(float(r) * int(n))
    return max(0, min(int(n), int(k)))


def select_kept(score, modality, cu_len, keep) -> np.ndarray:
    """Global row indices kept by per-modality top-k, ascending.

    Sparse Prefix Retention: within each modality of a sequence the
    top-floor(r*n) positions by s_i are kept.  keep: [nseq, 2] counts
    (text, image).  Order is (s descending, position ascending), so an equal
    score keeps the lower position.  Returned indices are rows of the packed
    [total_L, ...] cache, ascending (sequence order, then position).
    """
    score = np.asarray(score, dtype=np.float64)
    modality = np.asarray(modality)
    cu = np.asarray(cu_len, dtype=np.int64)
    keep = np.asarray(keep, dtype=np.int64).reshape(-1, 2)
    kept: List[int] = []
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        chosen = []
        for m in (0, 1):
            pos = np.nonzero(modality[a:b] == m)[0] + a
            k = max(0, min(int(keep[s, m]), len(pos)))
            order = np.lexsort((pos, -score[pos]))      # primary: -s, then position
            chosen.extend(pos[order[:k]].tolist())
        kept.extend(sorted(chosen))
    return np.asarray(kept, dtype=np.int64)


def compact(K, V, kept_idx):
    """Pruned cache K'[j] = K[kept[j]], V'[j] = V[kept[j]] (bit copies)."""
    kept_idx = np.asarray(kept_idx, dtype=np.int64)
    return np.asarray(K)[kept_idx], np.asarray(V)[kept_idx]


# --------------------------------------------------------------------------
# Block attention (the denoising step's attention over the prefix cache)
# --------------------------------------------------------------------------

def attention(Q, Kp, Vp, cu_kv, Kb=None, Vb=None, scale: Optional[float] = None):
    """O = softmax(Q K^T * scale) V per (sequence, query head), fp64.

    Q: [nseq, Lq, Hq, D]; Kp/Vp: [total_kv, Hkv, D] packed by cu_kv;
    Kb/Vb: [nseq, Lq, Hkv, D] (the block's own keys, attended without a mask:
    the block is predicted bidirectionally from the clean prefix and its own
    noisy tokens) or None.  Query head h reads KV head floor(h*Hkv/Hq).
    Keys are [prefix ; block]; a softmax over an empty key set is undefined
    and not allowed.
    """
    Q = np.asarray(Q, dtype=np.float64)
    Kp = np.asarray(Kp, dtype=np.float64)
    Vp = np.asarray(Vp, dtype=np.float64)
    nseq, Lq, Hq, D = Q.shape
    Hkv = Kp.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    cu = np.asarray(cu_kv, dtype=np.int64)
    O = np.zeros_like(Q)
    for b in range(nseq):
        kb = Kp[cu[b]:cu[b + 1]]
        vb = Vp[cu[b]:cu[b + 1]]
        if Kb is not None:
            kb = np.concatenate([kb, np.asarray(Kb[b], dtype=np.float64)], axis=0)
            vb = np.concatenate([vb, np.asarray(Vb[b], dtype=np.float64)], axis=0)
        if kb.shape[0] == 0:
            raise ValueError("attention over an empty key set")
        for h in range(Hq):
            g = (h * Hkv) // Hq
            logits = (Q[b, :, h, :] @ kb[:, g, :].T) * scale      # [Lq, n]
            logits -= logits.max(axis=1, keepdims=True)
            p = np.exp(logits)
            p /= p.sum(axis=1, keepdims=True)
            O[b, :, h, :] = p @ vb[:, g, :]
    return O


# --------------------------------------------------------------------------
# LM-head confidence
# --------------------------------------------------------------------------

def lmhead_confidence(X, W):
    """Top-1 softmax confidence of logits z = X W^T, fp64.

    Sparse Prefix Retention defines c_i = max_v p(v | x_t); Non-uniform Token
    Unmasking uses c_n = p(x0_hat^n | x_t), read with x0_hat = argmax (greedy),
    which is the same number.  Returns (conf, argmax, lse): conf = 1 / sum_v
    exp(z_v - z*), argmax = lowest index attaining z*, lse = z* + log sum.
    """
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    Z = X @ W.T
    zmax = Z.max(axis=1)
    amax = Z.argmax(axis=1)              # first (lowest) index of the maximum
    S = np.exp(Z - zmax[:, None]).sum(axis=1)
    return 1.0 / S, amax.astype(np.int64), zmax + np.log(S)


def lmhead_top2_gap(X, W) -> np.ndarray:
    """z* minus the second largest logit of each row, fp64 (0 when the maximum
    is attained twice; V = 1 has no runner-up and gives +inf).

    Where this gap is below the GPU's fp32 rounding of the logits, two
    vocabulary entries are equally valid argmaxes of Sparse Prefix
    Retention's c_i = max_v p (the confidence is the same either way), so the
    parity tests excuse an argmax mismatch only there.
    """
    Z = np.asarray(X, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T
    if Z.shape[1] < 2:
        return np.full(Z.shape[0], np.inf)
    part = np.partition(Z, Z.shape[1] - 2, axis=1)
    return part[:, -1] - part[:, -2]


# --------------------------------------------------------------------------
# Non-uniform Token Unmasking
# --------------------------------------------------------------------------

def min_acceptances(m: int, steps_left: int) -> int:
    """ceil(m / (T - t)) with steps_left = T - t; all of m when none are left."""
    if m <= 0:
        return 0
    if steps_left <= 0:
        return m
    return min(m, -(-m // steps_left))


def fixed_schedule_count(m0: int, T: int) -> int:
    """The standard schedule's tokens per step, ceil(m0 / T)."""
    return -(-m0 // T)


def unmask_select(conf, argmax, masked, tokens, tau, steps_left: int):
    """One confidence-adaptive unmasking step (Non-uniform Token Unmasking).

    conf, argmax, masked, tokens: [nseq, Lq].  tau is compared with strict
    '>' in the precision it is given in (pass the float32 value the kernel
    uses).  For each sequence: m = #masked, q = min_acceptances(m, steps_left),
    count = max(#{masked with conf > tau}, q); the first `count` masked
    positions by (conf descending, position ascending) are accepted:
    tokens <- argmax, masked <- 0.  Returns (masked, tokens, n_accepted) as
    new arrays.
    """
    conf = np.asarray(conf, dtype=np.float64)
    argmax = np.asarray(argmax)
    masked = np.array(masked, dtype=np.uint8, copy=True)
    tokens = np.array(tokens, dtype=np.int64, copy=True)
    tau = float(tau)
    nseq, Lq = conf.shape
    n_acc = np.zeros(nseq, dtype=np.int64)
    for s in range(nseq):
        cand = np.nonzero(masked[s] == 1)[0]
        m = len(cand)
        if m == 0:
            continue
        n_hi = int(np.sum(conf[s, cand] > tau))
        count = max(n_hi, min_acceptances(m, steps_left))
        order = np.lexsort((cand, -conf[s, cand]))
        acc = cand[order[:count]]
        tokens[s, acc] = argmax[s, acc]
        masked[s, acc] = 0
        n_acc[s] = count
    return masked, tokens, n_acc


# --------------------------------------------------------------------------
# One block: the pruning pass followed by pruned denoising steps
# --------------------------------------------------------------------------

@dataclass
class BlockResult:
    conf_prefix: np.ndarray
    ibar: np.ndarray
    score: np.ndarray
    kept_idx: np.ndarray
    cu_kept: np.ndarray
    outputs: List[np.ndarray] = field(default_factory=list)    # O per step
    moe_ids: List[np.ndarray] = field(default_factory=list)    # experts per step (with an MoE)
    confs: List[np.ndarray] = field(default_factory=list)      # block conf per step
    argmaxes: List[np.ndarray] = field(default_factory=list)
    masks: List[np.ndarray] = field(default_factory=list)      # mask after each step
    tokens: List[np.ndarray] = field(default_factory=list)
    n_accepted: List[np.ndarray] = field(default_factory=list)


def run_block(Q, K, V, Kb, Vb, hidden, W, cu_len, modality, r_text, r_img,
              tau, T: Optional[int], n_steps: int, alpha: float = 0.5, moe=None,
              store_dtype: Optional[str] = None) -> BlockResult:
    """The SPRINT block as one composition (Sparse Prefix Retention +
    Non-uniform Token Unmasking).

    t = 0 is the full pass: attention over the whole prefix, block confidence
    and unmasking; the prefix confidences give the scores, which select and
    compact the pruned cache.  Steps t = 1..n_steps attend to the pruned cache.
    Q, Kb, Vb stay fixed across steps (the model that would refresh them is
    not part of this path).  T = None means at least one acceptance per step.
    `moe` = (w_router, bias, w_gate, w_up, w_down, top_k, route_scale) puts an
    MoE FFN between attention and the LM head: the LM head reads
    O + moe_ffn(O), with O stored in `store_dtype` first (the workload's
    dtype) as the FFN's input.
    """
    nseq, Lq, Hq, D = np.asarray(Q).shape
    cu = np.asarray(cu_len, dtype=np.int64)
    conf_prefix, _, _ = lmhead_confidence(hidden, W)
    ibar = key_norm_importance(K, cu)
    score = composite_score(ibar, conf_prefix, alpha)
    keep = np.zeros((nseq, 2), dtype=np.int64)
    for s in range(nseq):
        seg = np.asarray(modality)[cu[s]:cu[s + 1]]
        keep[s, 0] = keep_count(r_text, int(np.sum(seg == 0)))
        keep[s, 1] = keep_count(r_img, int(np.sum(seg == 1)))
    kept = select_kept(score, modality, cu, keep)
    cu_kept = np.zeros(nseq + 1, dtype=np.int64)
    cu_kept[1:] = np.cumsum(keep.sum(axis=1))
    Kp, Vp = compact(K, V, kept)
    res = BlockResult(conf_prefix, ibar, score, kept, cu_kept)
    masked = np.ones((nseq, Lq), dtype=np.uint8)
    tokens = np.full((nseq, Lq), -1, dtype=np.int64)
    big = 1 << 30
    for t in range(n_steps + 1):
        if t == 0:
            O = attention(Q, K, V, cu, Kb, Vb)
        else:
            O = attention(Q, Kp, Vp, cu_kept, Kb, Vb)
        h = O.reshape(nseq * Lq, Hq * D)
        if moe is not None:
            wr, mb, wg, wu, wd, k, sc = moe
            hs = store_as(h, store_dtype) if store_dtype else h
            h, ids, _ = moe_ffn(hs, wr, mb, wg, wu, wd, k, sc, residual=hs)
            res.moe_ids.append(ids)
        conf, amax, _ = lmhead_confidence(h, W)
        conf = conf.reshape(nseq, Lq)
        amax = amax.reshape(nseq, Lq)
        steps_left = big if T is None else T - t
        masked, tokens, nacc = unmask_select(conf, amax, masked, tokens, tau, steps_left)
        res.outputs.append(O)
        res.confs.append(conf)
        res.argmaxes.append(amax)
        res.masks.append(masked.copy())
        res.tokens.append(tokens.copy())
        res.n_accepted.append(nacc)
    return res


# --------------------------------------------------------------------------
# Block-wise generation: B blocks over a growing prefix
# --------------------------------------------------------------------------

def append_block(old, cu_len, blk):
    """Prefix growth between blocks (SPRINT introduction: blocks are generated
    one after another; Sparse Prefix Retention: a block's first step sees the
    complete prefix, earlier blocks included).

    old: rows [total, ...] packed by cu_len [nseq+1]; blk: [nseq, n_blk, ...].
    Sequence s of the result holds its old rows, then its block rows.
    Returns (new rows, new cu_len).
    """
    old = np.asarray(old)
    blk = np.asarray(blk)
    cu = np.asarray(cu_len, dtype=np.int64)
    nseq = len(cu) - 1
    parts = []
    for s in range(nseq):
        parts.append(old[cu[s]:cu[s + 1]])
        parts.append(blk[s])
    new = np.concatenate(parts, axis=0) if parts else old[:0]
    n_blk = blk.shape[1]
    cu_new = cu + n_blk * np.arange(nseq + 1, dtype=np.int64)
    return new, cu_new


def store_as(x, dtype: str) -> np.ndarray:
    """Values as the workload stores them: float32 ("f32") or bfloat16 ("bf16",
    round to nearest, ties to even), returned as float64."""
    x32 = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    if dtype == "f32":
        return x32.astype(np.float64)
    bits = x32.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    bits = ((bits + 0x7FFF + lsb) >> 16) << 16
    return bits.astype(np.uint32).view(np.float32).astype(np.float64)


def run_generation(blocks, K, V, hidden, W, cu_len, modality, gen_modality: int, r_text, r_img,
                   tau, T: Optional[int], n_steps: int, dtype: str, alpha: float = 0.5):
    """B SPRINT blocks one after another (SPRINT introduction; Sparse Prefix
    Retention; Non-uniform Token Unmasking).

    blocks: list of (Q, Kb, Vb) per block.  Block b runs run_block over the
    prefix grown by blocks < b; afterwards its own K/V rows, its last step's
    outputs (the hidden states of its positions, stored in `dtype`) and
    `gen_modality` are appended to every sequence.  Returns the BlockResult
    of every block and the prefix layouts (cu_len) they saw.
    """
    cu = np.asarray(cu_len, dtype=np.int64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    hidden = np.asarray(hidden, dtype=np.float64)
    modality = np.asarray(modality)
    results, layouts = [], []
    for b, (Q, Kb, Vb) in enumerate(blocks):
        res = run_block(Q, K, V, Kb, Vb, hidden, W, cu, modality, r_text, r_img, tau, T,
                        n_steps, alpha)
        results.append(res)
        layouts.append(cu.copy())
        if b + 1 == len(blocks):
            break
        nseq, Lq, Hq, D = np.asarray(Q).shape
        O = store_as(res.outputs[-1], dtype).reshape(nseq, Lq, Hq * D)
        K, _ = append_block(K, cu, Kb)
        V, _ = append_block(V, cu, Vb)
        hidden, _ = append_block(hidden, cu, O)
        modality, cu = append_block(modality, cu,
                                    np.full((nseq, Lq), gen_modality, dtype=modality.dtype))
    return results, layouts


# --------------------------------------------------------------------------
# Several layers: one kept set shared by every layer, or one set per layer
# --------------------------------------------------------------------------

def key_norm_importance_layers(K_layers, cu_len) -> np.ndarray:
    """Layer-mean key-norm importance: I_i = (1/n_layers) sum_l I_i^l, where
    I^l is the mean-normalised key norm of layer l's cache (Sparse Prefix
    Retention scores positions; with several layers the per-layer importances
    are averaged so that one kept set serves every layer)."""
    return np.mean([key_norm_importance(K, cu_len) for K in K_layers], axis=0)


@dataclass
class LayersResult:
    conf_prefix: np.ndarray
    ibars: List[np.ndarray]          # one per layer, or one (the layer mean) when shared
    scores: List[np.ndarray]
    kept: List[np.ndarray]           # kept rows per layer (all equal when shared)
    cu_kept: np.ndarray
    outputs: List[List[np.ndarray]] = field(default_factory=list)   # per step, per layer
    confs: List[np.ndarray] = field(default_factory=list)
    masks: List[np.ndarray] = field(default_factory=list)
    tokens: List[np.ndarray] = field(default_factory=list)


def run_block_layers(layers, hidden, W, cu_len, modality, r_text, r_img, tau,
                     T: Optional[int], n_steps: int, shared: bool = True,
                     alpha: float = 0.5) -> LayersResult:
    """One SPRINT block of a model with several layers, each with its own
    prefix cache and its own block queries and K/V.

    layers: list of (Q, K, V, Kb, Vb) per layer.  The prefix confidences come
    from the LM head over `hidden` (one per position, for every layer).
    shared: one kept set from the layer-mean importance, compacted in every
    layer's cache; otherwise each layer keeps the top positions of its own
    score.  Every step attends layer by layer; the LM head reads the last
    layer's output (the layers' inputs are independent draws here, standing
    in for the layers of one model).
    """
    cu = np.asarray(cu_len, dtype=np.int64)
    nseq = len(cu) - 1
    conf_prefix, _, _ = lmhead_confidence(hidden, W)
    keep = np.zeros((nseq, 2), dtype=np.int64)
    for s in range(nseq):
        seg = np.asarray(modality)[cu[s]:cu[s + 1]]
        keep[s, 0] = keep_count(r_text, int(np.sum(seg == 0)))
        keep[s, 1] = keep_count(r_img, int(np.sum(seg == 1)))
    cu_kept = np.zeros(nseq + 1, dtype=np.int64)
    cu_kept[1:] = np.cumsum(keep.sum(axis=1))
    if shared:
        ibars = [key_norm_importance_layers([l[1] for l in layers], cu)]
    else:
        ibars = [key_norm_importance(l[1], cu) for l in layers]
    scores = [composite_score(ib, conf_prefix, alpha) for ib in ibars]
    kept_sets = [select_kept(sc, modality, cu, keep) for sc in scores]
    if shared:
        kept_sets = kept_sets * len(layers)
    pruned = [compact(l[1], l[2], k) for l, k in zip(layers, kept_sets)]
    res = LayersResult(conf_prefix, ibars, scores, kept_sets, cu_kept)
    Q_last = np.asarray(layers[-1][0])
    _, Lq, Hq, D = Q_last.shape
    masked = np.ones((nseq, Lq), dtype=np.uint8)
    tokens = np.full((nseq, Lq), -1, dtype=np.int64)
    big = 1 << 30
    for t in range(n_steps + 1):
        outs = []
        for (Q, K, V, Kb, Vb), (Kp, Vp) in zip(layers, pruned):
            if t == 0:
                outs.append(attention(Q, K, V, cu, Kb, Vb))
            else:
                outs.append(attention(Q, Kp, Vp, cu_kept, Kb, Vb))
        conf, amax, _ = lmhead_confidence(outs[-1].reshape(nseq * Lq, Hq * D), W)
        conf = conf.reshape(nseq, Lq)
        amax = amax.reshape(nseq, Lq)
        steps_left = big if T is None else T - t
        masked, tokens, _ = unmask_select(conf, amax, masked, tokens, tau, steps_left)
        res.outputs.append(outs)
        res.confs.append(conf)
        res.masks.append(masked.copy())
        res.tokens.append(tokens.copy())
    return res


# --------------------------------------------------------------------------
# An MoE FFN on synthetic weights (the backbone's expert layer)
# --------------------------------------------------------------------------

def silu(z):
    """z * sigmoid(z)."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def moe_route(x, w_router, bias, top_k: int, route_scale: float = 2.5):
    """Routing of each token (LLaDA2.0-Uni, "Load Balancing Strategy").

    Affinity s_e = sigmoid(x . r_e) per expert.  The auxiliary-loss-free
    balancing bias b only steers selection: the top_k experts by s_e + b_e
    are chosen (the lower expert index wins a tie), and their gates are the
    affinities normalised over the chosen experts and scaled by route_scale
    (2.5 on the page).  Returns (expert ids [M, top_k] in selection order,
    gates [M, top_k], affinities [M, E]).
    """
    x = np.asarray(x, dtype=np.float64)
    logits = x @ np.asarray(w_router, dtype=np.float64).T
    s = 1.0 / (1.0 + np.exp(-logits))
    sel_score = s + np.asarray(bias, dtype=np.float64)[None, :]
    M, E = s.shape
    ids = np.zeros((M, top_k), dtype=np.int64)
    gates = np.zeros((M, top_k))
    for t in range(M):
        order = np.lexsort((np.arange(E), -sel_score[t]))
        ids[t] = order[:top_k]
        gates[t] = route_scale * s[t, ids[t]] / s[t, ids[t]].sum()
    return ids, gates, s


def expert_ffn(x, w_gate, w_up, w_down):
    """SwiGLU expert: W_down (silu(W_gate x) * (W_up x)).  x [n, H];
    w_gate, w_up [I, H]; w_down [H, I]."""
    x = np.asarray(x, dtype=np.float64)
    g = x @ np.asarray(w_gate, dtype=np.float64).T
    u = x @ np.asarray(w_up, dtype=np.float64).T
    return (silu(g) * u) @ np.asarray(w_down, dtype=np.float64).T


def moe_ffn(x, w_router, bias, w_gate, w_up, w_down, top_k: int, route_scale: float = 2.5,
            residual=None):
    """y_t = residual_t + sum_j gate_{t,j} * FFN_{e_{t,j}}(x_t)  (residual
    optional).  w_gate, w_up [E, I, H]; w_down [E, H, I].  Returns (y, ids,
    gates)."""
    ids, gates, _ = moe_route(x, w_router, bias, top_k, route_scale)
    x = np.asarray(x, dtype=np.float64)
    M, H = x.shape
    y = np.zeros((M, H)) if residual is None else np.asarray(residual, dtype=np.float64).copy()
    for t in range(M):
        for j in range(top_k):
            e = ids[t, j]
            y[t] += gates[t, j] * expert_ffn(x[t:t + 1], w_gate[e], w_up[e], w_down[e])[0]
    return y, ids, gates
