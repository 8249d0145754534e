"""Seeded synthetic layers: workload definitions and input generators.

This module is shared by the tests, the bench and the smoke check. It holds
the workload parameters and draws the random inputs; it contains none of the
attention layer's arithmetic (no rotation, pooling, selection, softmax or
low-rank algebra). Both the HIP path and the CPU oracle consume exactly the
arrays produced here.

Workloads follow the pages' deployment shapes:
  * Wan2.1-1.3B at 480p, 81 frames -> latent grid 21x30x52 (RoLA,
    arXiv 2609.06712, §5.2; the 30x52 frame also appears in RoPeSLR,
    arXiv 2605.20659, Fig. 13 caption),
  * Wan2.1-14B at 720p, 81 frames -> grid 21x45x80 (RoLA abstract, §5.2),
  * HunyuanVideo-13B "100K+ token" sequences -> grid 33x45x80 (RoPeSLR
    abstract).
The pages measure on real model trajectories and VBench prompts; none of
that is available here, so seeded clustered Q/K (to create semantic spikes)
and Gaussian V stand in for them.

Random streams: every (tensor id, b, h) slice comes from its own
``numpy.random.default_rng([seed, tensor_id, b, h])`` so any slice can be
regenerated independently and in any order. For bf16 layers every tensor
that enters the layer in bf16 (Q, K, V) and the projection / embedding
tables are rounded fp32 -> bf16 with round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Tuple

import numpy as np

# tensor ids of the per-slice random streams
TID_Q, TID_K, TID_V, TID_WQ, TID_WK, TID_GATE, TID_CENT, TID_CLUSTER = 0, 1, 2, 3, 4, 5, 6, 7
TID_ET, TID_EH, TID_EW = 8, 9, 10
TID_WG, TID_BG = 11, 12
TID_DOUT = 13      # upstream gradient of the layer output (backward)
TID_OMEGA = 14     # FAVOR+ random directions
TID_SAMPLE = 99  # query-block sample for the oracle's partial coverage

N_CENTROIDS = 64
CENTROID_SCALE = 3.0
NOISE_SCALE = 0.5
EMBED_VAR = 0.02


@dataclasses.dataclass(frozen=True)
class Layer:
    """One attention-layer workload. Tensors are [B, H, L, D] contiguous,
    L = T*Hg*Wg flattened t-major, then h, then w."""
    name: str
    B: int
    H: int
    D: int
    T: int
    Hg: int
    Wg: int
    dtype: str                     # "f32" or "bf16"
    base: float                    # rotary base
    pairs: Tuple[int, int, int]    # backbone rotary pairs on t, h, w (sum = D/2)
    block: int                     # tokens per block
    keep: int                      # kept key blocks per query block
    rank: int                      # low-rank width r
    lr_mode: str                   # "rola" (rotation after phi) or "abspe"
    lr_pairs: Tuple[int, int, int] # rotary pairs the rank-r branch reuses (sum = r/2)
    seed: int
    gen: str                       # "normal", "clustered" or "zero_qk" (q = k = 0: every block score ties)
    eps: float = 1e-6
    gate: str = "head"             # combine gate: "head" (g_h) or "token" (RoLA §4.4)
    fmap: str = "elu1"             # low-rank feature map: "elu1" (elu + 1), "silu" (RoLA §5.3) or
                                   # "favor" (positive random features, RoPeSLR appendix)

    @property
    def L(self) -> int:
        return self.T * self.Hg * self.Wg

    @property
    def nblk(self) -> int:
        return -(-self.L // self.block)

    def flops(self) -> Dict[str, float]:
        """Algorithmic FLOP counts (multiply-add = 2)."""
        B, H, D, L, r = self.B, self.H, self.D, self.L, self.rank
        nb, bs, k = self.nblk, self.block, self.keep
        return {
            # QK^T and PV over the kept tiles, nominal (padded) block sizes
            "sparse": 4.0 * B * H * nb * k * bs * bs * D,
            "dense": 4.0 * B * H * L * L * D,
            # x.W (2LDr) and the summary / readout (2LrD each) for K and Q
            "lowrank": 8.0 * B * H * L * r * D,
            # block scores Qbar.Kbar^T
            "select": 2.0 * B * H * nb * nb * D,
        }


def _split_211(r: int) -> Tuple[int, int, int]:
    """Low-rank rotary pairs split 2:1:1 over t:h:w (r/2 pairs in total)."""
    p = r // 2
    return (p // 2, p // 4, p - p // 2 - p // 4)


def tiny() -> Layer:
    return Layer("tiny-fp32 4x8x8", 1, 2, 64, 4, 8, 8, "f32", 10000.0, (12, 10, 10),
                 32, 2, 8, "rola", _split_211(8), 0, "normal")


def wan13b() -> Layer:
    return Layer("wan2.1-1.3B 480p 21x30x52", 2, 12, 128, 21, 30, 52, "bf16", 10000.0,
                 (22, 21, 21), 64, 52, 32, "rola", _split_211(32), 1, "clustered")


def wan14b() -> Layer:
    return Layer("wan2.1-14B 720p 21x45x80", 2, 40, 128, 21, 45, 80, "bf16", 10000.0,
                 (22, 21, 21), 64, 119, 32, "rola", _split_211(32), 2, "clustered")


def hunyuan13b() -> Layer:
    return Layer("hunyuan-13B 33x45x80", 1, 24, 128, 33, 45, 80, "bf16", 10000.0,
                 (22, 21, 21), 64, 186, 32, "abspe", (0, 0, 0), 3, "clustered")


SWEEP_KEEP_FRACTIONS = (0.05, 0.10, 0.20, 0.50, 1.00)
SWEEP_RANKS = (16, 32, 64)


def sweep() -> List[Layer]:
    """Keep-fraction x rank sweep at the Wan2.1-1.3B shape. Kept blocks are
    ceil(fraction * nblk): 26, 52, 103, 256, 512 of 512."""
    out = []
    for f in SWEEP_KEEP_FRACTIONS:
        for r in SWEEP_RANKS:
            nb = -(-32760 // 64)
            k = int(math.ceil(round(f * nb, 9)))
            out.append(Layer(f"wan1.3B sweep keep{int(f*100)}% r{r}", 2, 12, 128, 21, 30, 52,
                             "bf16", 10000.0, (22, 21, 21), 64, k, r, "rola", _split_211(r),
                             4, "clustered"))
    return out


def by_name(name: str) -> Layer:
    table = {"tiny": tiny, "wan13b": wan13b, "wan14b": wan14b, "hunyuan13b": hunyuan13b}
    return table[name]()


# ----------------------------------------------------------------------------
# bf16 helpers (storage format only)

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even. Inputs here
    are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Values of x rounded to the nearest bf16, returned as fp32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


# ----------------------------------------------------------------------------
# per-slice generators; every array is fp32 holding the exact values the layer
# receives (bf16-representable for bf16 layers)

def _rng(seed: int, tid: int, b: int = 0, h: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, tid, b, h])


def centroids(cfg: Layer, h: int) -> np.ndarray:
    c = _rng(cfg.seed, TID_CENT, 0, h).standard_normal((N_CENTROIDS, cfg.D), dtype=np.float32)
    c /= np.linalg.norm(c, axis=1, keepdims=True).astype(np.float32)
    return c


def qkv_slice(cfg: Layer, b: int, h: int, L: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Q, K, V of one (b, h) slice as fp32 [L, D] arrays. ``L`` overrides
    the sequence length (used by edge-case tests on custom grids)."""
    L = cfg.L if L is None else L
    D = cfg.D
    if cfg.gen == "normal":
        q = _rng(cfg.seed, TID_Q, b, h).standard_normal((L, D), dtype=np.float32)
        k = _rng(cfg.seed, TID_K, b, h).standard_normal((L, D), dtype=np.float32)
    elif cfg.gen == "zero_qk":
        q = np.zeros((L, D), dtype=np.float32)
        k = np.zeros((L, D), dtype=np.float32)
    else:
        cent = centroids(cfg, h) * np.float32(CENTROID_SCALE)
        cl = _rng(cfg.seed, TID_CLUSTER, b, h).integers(0, N_CENTROIDS, size=L)
        q = _rng(cfg.seed, TID_Q, b, h).standard_normal((L, D), dtype=np.float32)
        q *= np.float32(NOISE_SCALE)
        q += cent[cl]
        k = _rng(cfg.seed, TID_K, b, h).standard_normal((L, D), dtype=np.float32)
        k *= np.float32(NOISE_SCALE)
        k += cent[cl]
    v = _rng(cfg.seed, TID_V, b, h).standard_normal((L, D), dtype=np.float32)
    if cfg.dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    return q, k, v


def dout_slice(cfg: Layer, b: int, h: int) -> np.ndarray:
    """Upstream gradient dL/dout of one (b, h) slice, fp32 [L, D] ~ N(0, 1)
    (bf16-representable for bf16 layers): the input of the backward pass."""
    g = _rng(cfg.seed, TID_DOUT, b, h).standard_normal((cfg.L, cfg.D), dtype=np.float32)
    return round_bf16(g) if cfg.dtype == "bf16" else g


def lowrank_params(cfg: Layer) -> Dict[str, np.ndarray]:
    """Per-head projections W_q, W_k [H, D, r] ~ N(0, 1/D) (variance), the
    per-head gate g [H] ~ U(0, 1), for the token gate W_g [H, D] ~ N(0, 1/D)
    and b_g [H] ~ U(-2, 0.5) (a mostly negative bias, as the pages start
    the gate), for FAVOR+ features the random directions omega [H, r, r] ~
    N(0, 1) (fp32, not rounded), and for the absolute-PE variant the axis
    tables E_t [T, r], E_h [Hg, r], E_w [Wg, r] ~ N(0, 0.02) (variance)."""
    H, D, r = cfg.H, cfg.D, cfg.rank
    std = np.float32(1.0 / math.sqrt(D))
    wq = np.stack([_rng(cfg.seed, TID_WQ, 0, h).standard_normal((D, r), dtype=np.float32) * std
                   for h in range(H)])
    wk = np.stack([_rng(cfg.seed, TID_WK, 0, h).standard_normal((D, r), dtype=np.float32) * std
                   for h in range(H)])
    g = _rng(cfg.seed, TID_GATE).uniform(0.0, 1.0, size=H).astype(np.float32)
    out = {"wq": wq, "wk": wk, "gate": g}
    if cfg.gate == "token":
        out["wg"] = _rng(cfg.seed, TID_WG).standard_normal((H, D), dtype=np.float32) * std
        out["bg"] = _rng(cfg.seed, TID_BG).uniform(-2.0, 0.5, size=H).astype(np.float32)
    if cfg.fmap == "favor":
        # FAVOR+ random directions omega [H, r, r] ~ N(0, I_r) per row (the
        # random numbers of the method, drawn here and passed in)
        out["omega"] = np.stack([_rng(cfg.seed, TID_OMEGA, 0, h).standard_normal((r, r), dtype=np.float32)
                                 for h in range(H)])
    if cfg.lr_mode == "abspe":
        es = np.float32(math.sqrt(EMBED_VAR))
        out["et"] = _rng(cfg.seed, TID_ET).standard_normal((cfg.T, r), dtype=np.float32) * es
        out["eh"] = _rng(cfg.seed, TID_EH).standard_normal((cfg.Hg, r), dtype=np.float32) * es
        out["ew"] = _rng(cfg.seed, TID_EW).standard_normal((cfg.Wg, r), dtype=np.float32) * es
    if cfg.dtype == "bf16":
        for key in ("wq", "wk", "et", "eh", "ew"):
            if key in out:
                out[key] = round_bf16(out[key])
    return out


def sample_query_blocks(cfg: Layer, b: int, h: int, n_extra: int = 6) -> np.ndarray:
    """Query blocks the oracle checks when a full sparse pass is too slow:
    the first and last block plus ``n_extra`` seeded others, ascending."""
    nb = cfg.nblk
    rest = _rng(cfg.seed, TID_SAMPLE, b, h).choice(np.arange(1, max(nb - 1, 1)),
                                                   size=min(n_extra, max(nb - 2, 0)), replace=False)
    return np.unique(np.concatenate([[0, nb - 1], rest])).astype(np.int32)
