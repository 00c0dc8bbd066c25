"""Seeded synthetic inputs for the SPRINT block step.

This module only draws random numbers and lays them out. It holds none of the
method's arithmetic (no norms, scores, selections, softmaxes or schedules), so
both the HIP path and the CPU oracle may take their inputs from it.

Workloads are shaped like the text-plus-image prefixes that LLaDA2.0-Uni
(arXiv 2604.20796) describes: the image token counts of its training-stage
section (about 256, 1024 and 2048 tokens per image) and its 8k/16k SFT
contexts. Every value is synthetic; no dataset or trained weight is used.

Draw order (numpy ``default_rng(seed)``, one generator, in this order):
  1. ragged layouts only: per sequence, prefix length ~ U{lmin..lmax}, then
     image fraction ~ U[fmin, fmax]; n_img = floor(f * L), text run first;
  2. Q ~ N(0,1)            [nseq, Lq, Hq, D]
  3. K ~ N(0,1)            [total_L, Hkv, D]
  4. key scale ~ lognormal(0, 0.5) per prefix position, applied to K's row
  5. V ~ N(0,1)            [total_L, Hkv, D]
  6. Kb, Vb ~ N(0,1)       [nseq, Lq, Hkv, D] (the current block's own K/V)
  7. hidden ~ N(0,1)       [total_L, H] (prefix hidden states fed to the LM head)
  8. W ~ N(0, 0.02^2)      [Vocab, H]
Values are drawn in float32; bf16 workloads round them to nearest-even bf16
(the float32 arrays then hold exactly the bf16 values).

Generation over several blocks: block 0 uses the draws above; block b >= 1
draws its own Q, Kb, Vb (same shapes and laws, in that order) from
``default_rng([seed, b])``.  The rows a finished block adds to the prefix
are not drawn: they are that block's own K/V and outputs.

MoE FFN weights (``make_moe_weights``) come from ``default_rng([seed,
2**21])``.

Several layers: layer 0 uses the draws above; layer l >= 1 draws its own
Q, K (with its own key scales), V, Kb, Vb from ``default_rng([seed, 2**20,
l])``.  The prefix hidden states and the LM head are shared.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

TEXT = 0
IMAGE = 1


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                      # "f32" or "bf16"
    Hq: int
    Hkv: int
    D: int
    Lq: int                         # block length
    vocab: int
    # per-sequence runs of (modality, length); ignored when `ragged` is set
    segments: Tuple[Tuple[Tuple[int, int], ...], ...] = ()
    ragged: Optional[Tuple[int, int, int, float, float]] = None  # nseq,lmin,lmax,fmin,fmax
    r_text: float = 1.0
    r_img: float = 0.8
    tau: float = 0.95
    T: Optional[int] = 9            # steps per block incl. the pass; None: >=1 per step
    alpha: float = 0.5
    gen_modality: int = TEXT        # modality of the positions a generation appends
    desc: str = ""

    @property
    def H(self) -> int:
        return self.Hq * self.D

    @property
    def es(self) -> int:
        return 4 if self.dtype == "f32" else 2


def _interleaved(pairs: int, text: int, img: int):
    runs = []
    for _ in range(pairs):
        runs.append((TEXT, text))
        runs.append((IMAGE, img))
    return tuple(runs)


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload(
        "tiny", "f32", Hq=4, Hkv=2, D=64, Lq=32, vocab=4096,
        segments=(((TEXT, 192), (IMAGE, 64)),), r_text=1.0, r_img=0.8,
        tau=0.9, T=None,
        desc="fp32, 4/2 heads, d64, prefix 256 = 192 text + 64 image, H 256, V 4096"),
    "single4k": Workload(
        "single4k", "bf16", Hq=16, Hkv=4, D=128, Lq=32, vocab=32768,
        segments=(((TEXT, 1024), (IMAGE, 3072)),), T=9,
        desc="bf16, 16/4 heads, d128, prefix 4096 = 1024 text + 3072 image, H 2048, V 32768, "
             "pass + 8 steps"),
    "imggen16k": Workload(
        "imggen16k", "bf16", Hq=16, Hkv=4, D=128, Lq=32, vocab=32768,
        segments=(((TEXT, 512), (IMAGE, 15872)),), T=9, gen_modality=IMAGE,
        desc="bf16, prefix 16384 = 512 text + 15872 image, H 2048, V 32768, "
             "blocks of image positions"),
    "ragged8": Workload(
        "ragged8", "bf16", Hq=16, Hkv=4, D=128, Lq=32, vocab=65536,
        ragged=(8, 2048, 16384, 0.25, 0.9), T=9,
        desc="bf16, 8 sequences, L ~ U[2048,16384], image fraction ~ U[0.25,0.9], V 65536"),
    "interleaved32k": Workload(
        "interleaved32k", "bf16", Hq=16, Hkv=4, D=128, Lq=32, vocab=163840,
        segments=(_interleaved(8, 1024, 3072),), T=9,
        desc="bf16, prefix 32768 = 8 x (1024 text + 3072 image), V 163840"),
}


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bf16 patterns of float32 values that are already bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


@dataclass
class Layout:
    runs: List[Tuple[Tuple[int, int], ...]]   # per sequence
    lens: np.ndarray                           # int64 [nseq]
    cu_len: np.ndarray                         # int32 [nseq+1]
    modality: np.ndarray                       # uint8 [total_L]
    n_text: np.ndarray                         # int64 [nseq]
    n_img: np.ndarray                          # int64 [nseq]

    @property
    def nseq(self) -> int:
        return len(self.lens)

    @property
    def total_L(self) -> int:
        return int(self.cu_len[-1])


def layout_from_runs(runs) -> Layout:
    runs = [tuple((int(m), int(n)) for m, n in r) for r in runs]
    lens = np.array([sum(n for _, n in r) for r in runs], dtype=np.int64)
    cu = np.zeros(len(runs) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lens)
    mod = np.zeros(int(cu[-1]), dtype=np.uint8)
    n_text = np.zeros(len(runs), dtype=np.int64)
    n_img = np.zeros(len(runs), dtype=np.int64)
    for s, r in enumerate(runs):
        p = int(cu[s])
        for m, n in r:
            mod[p:p + n] = m
            p += n
            if m == TEXT:
                n_text[s] += n
            else:
                n_img[s] += n
    return Layout(runs, lens, cu.astype(np.int32), mod, n_text, n_img)


@dataclass
class Inputs:
    wl: Workload
    layout: Layout
    Q: np.ndarray
    K: np.ndarray
    V: np.ndarray
    Kb: np.ndarray
    Vb: np.ndarray
    hidden: Optional[np.ndarray]
    W: Optional[np.ndarray]
    key_scale: np.ndarray
    extra: dict = field(default_factory=dict)


def _ragged_runs(rng, nseq, lmin, lmax, fmin, fmax):
    runs = []
    for _ in range(nseq):
        L = int(rng.integers(lmin, lmax + 1))
        f = float(rng.uniform(fmin, fmax))
        n_img = int(np.floor(f * L))
        runs.append(((TEXT, L - n_img), (IMAGE, n_img)))
    return runs


def make_inputs(wl: Workload, seed: int = 0, with_lmhead: bool = True,
                prefix_scale: float = 1.0, length_override=None) -> Inputs:
    """Draw one block's inputs for workload `wl` (see module docstring)."""
    rng = np.random.default_rng(seed)
    if wl.ragged is not None:
        runs = _ragged_runs(rng, *wl.ragged)
    else:
        runs = list(wl.segments)
    if length_override is not None:
        runs = length_override
    lay = layout_from_runs(runs)
    nseq, tl = lay.nseq, lay.total_L
    f32 = np.float32
    Q = rng.standard_normal((nseq, wl.Lq, wl.Hq, wl.D), dtype=f32)
    K = rng.standard_normal((tl, wl.Hkv, wl.D), dtype=f32)
    ks = rng.lognormal(0.0, 0.5, size=tl).astype(f32) * f32(prefix_scale)
    K *= ks[:, None, None]
    V = rng.standard_normal((tl, wl.Hkv, wl.D), dtype=f32)
    Kb = rng.standard_normal((nseq, wl.Lq, wl.Hkv, wl.D), dtype=f32)
    Vb = rng.standard_normal((nseq, wl.Lq, wl.Hkv, wl.D), dtype=f32)
    hidden = W = None
    if with_lmhead:
        hidden = rng.standard_normal((tl, wl.H), dtype=f32)
        W = rng.standard_normal((wl.vocab, wl.H), dtype=f32)
        W *= f32(0.02)
    if wl.dtype == "bf16":
        Q, K, V, Kb, Vb = (bf16_round(a) for a in (Q, K, V, Kb, Vb))
        if with_lmhead:
            hidden = bf16_round(hidden)
            W = bf16_round(W)
    return Inputs(wl, lay, Q, K, V, Kb, Vb, hidden, W, ks)


def make_block_inputs(wl: Workload, nseq: int, b: int, seed: int = 0):
    """Q, Kb, Vb of block b >= 1 of a generation (see module docstring)."""
    if b < 1:
        raise ValueError("block 0 takes its inputs from make_inputs")
    rng = np.random.default_rng([seed, b])
    f32 = np.float32
    Q = rng.standard_normal((nseq, wl.Lq, wl.Hq, wl.D), dtype=f32)
    Kb = rng.standard_normal((nseq, wl.Lq, wl.Hkv, wl.D), dtype=f32)
    Vb = rng.standard_normal((nseq, wl.Lq, wl.Hkv, wl.D), dtype=f32)
    if wl.dtype == "bf16":
        Q, Kb, Vb = (bf16_round(a) for a in (Q, Kb, Vb))
    return Q, Kb, Vb


def make_layer_inputs(wl: Workload, layout: "Layout", l: int, seed: int = 0,
                      prefix_scale: float = 1.0):
    """Q, K, V, Kb, Vb of layer l >= 1 of a several-layer stand-in (layer 0
    uses make_inputs's draws): the same laws, drawn from
    default_rng([seed, 1 << 20, l]) in the order Q, K, key scale, V, Kb, Vb."""
    if l < 1:
        raise ValueError("layer 0 takes its inputs from make_inputs")
    rng = np.random.default_rng([seed, 1 << 20, l])
    f32 = np.float32
    nseq, tl = layout.nseq, layout.total_L
    Q = rng.standard_normal((nseq, wl.Lq, wl.Hq, wl.D), dtype=f32)
    K = rng.standard_normal((tl, wl.Hkv, wl.D), dtype=f32)
    ks = rng.lognormal(0.0, 0.5, size=tl).astype(f32) * f32(prefix_scale)
    K *= ks[:, None, None]
    V = rng.standard_normal((tl, wl.Hkv, wl.D), dtype=f32)
    Kb = rng.standard_normal((nseq, wl.Lq, wl.Hkv, wl.D), dtype=f32)
    Vb = rng.standard_normal((nseq, wl.Lq, wl.Hkv, wl.D), dtype=f32)
    if wl.dtype == "bf16":
        Q, K, V, Kb, Vb = (bf16_round(a) for a in (Q, K, V, Kb, Vb))
    return Q, K, V, Kb, Vb


def make_moe_weights(H: int, E: int, inter: int, dtype: str, seed: int = 0):
    """Synthetic MoE FFN weights, from default_rng([seed, 2**21]) in the order
    router [E, H] ~ N(0, 1/H), bias [E] ~ U(-0.05, 0.05), gate and up
    [E, inter, H] ~ N(0, 1/H), down [E, H, inter] ~ N(0, 1/inter); rounded to
    bf16 for bf16 (the bias stays float32)."""
    rng = np.random.default_rng([seed, 1 << 21])
    f32 = np.float32
    wr = rng.standard_normal((E, H), dtype=f32) * f32(H ** -0.5)
    bias = rng.uniform(-0.05, 0.05, E).astype(f32)
    wg = rng.standard_normal((E, inter, H), dtype=f32) * f32(H ** -0.5)
    wu = rng.standard_normal((E, inter, H), dtype=f32) * f32(H ** -0.5)
    wd = rng.standard_normal((E, H, inter), dtype=f32) * f32(inter ** -0.5)
    if dtype == "bf16":
        wr, wg, wu, wd = (bf16_round(a) for a in (wr, wg, wu, wd))
    return wr, bias, wg, wu, wd


# ---------------------------------------------------------------------------
# Small synthetic operands for per-call tests (random draws only).
# ---------------------------------------------------------------------------

def random_scores(n: int, seed: int, levels: int = 0) -> np.ndarray:
    """Non-negative float32 scores; `levels` > 0 quantises them to force ties."""
    rng = np.random.default_rng(seed)
    if levels > 0:
        return (rng.integers(0, levels, size=n) / float(levels)).astype(np.float32)
    return rng.uniform(0.0, 2.0, size=n).astype(np.float32)


def random_unmask_state(nseq: int, Lq: int, vocab: int, seed: int, tau: float,
                        frac_masked: float = 0.7, frac_confident: float = 0.15,
                        tie_levels: int = 0):
    """Confidences, argmax tokens, a mask and current tokens for one block."""
    rng = np.random.default_rng(seed)
    conf = rng.uniform(1.0 / vocab, 1.0, size=(nseq, Lq))
    hi = rng.uniform(0, 1, size=(nseq, Lq)) < frac_confident
    conf[hi] = rng.uniform(tau, 1.0, size=int(hi.sum()))
    if tie_levels > 0:
        conf = np.floor(conf * tie_levels) / tie_levels
    conf = conf.astype(np.float32)
    argmax = rng.integers(0, vocab, size=(nseq, Lq)).astype(np.int32)
    masked = (rng.uniform(0, 1, size=(nseq, Lq)) < frac_masked).astype(np.uint8)
    tokens = np.where(masked == 1, -1, rng.integers(0, vocab, size=(nseq, Lq))).astype(np.int32)
    return conf, argmax, masked, tokens


def normal_array(shape, seed: int, std: float = 1.0, dtype: str = "f32") -> np.ndarray:
    """N(0, std^2) float32 draws, rounded to bf16 values when dtype is "bf16"."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
    return bf16_round(a) if dtype == "bf16" else a


def lognormal_rows(a: np.ndarray, seed: int, sigma: float = 0.5) -> np.ndarray:
    """Scale each leading-axis row of `a` by its own lognormal(0, sigma) draw."""
    rng = np.random.default_rng(seed)
    f = rng.lognormal(0.0, sigma, size=a.shape[0]).astype(np.float32)
    return a * f.reshape((-1,) + (1,) * (a.ndim - 1))


def plant_rows(W: np.ndarray, X: np.ndarray, pairs, gain: float, dtype: str = "f32") -> np.ndarray:
    """Copy gain * X[r] into W[v] for each (r, v) pair, so that row r's logit
    for token v is large (a planted confident prediction)."""
    W = W.copy()
    for r, v in pairs:
        W[v] = np.float32(gain) * X[r]
    return bf16_round(W) if dtype == "bf16" else W
