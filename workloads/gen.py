"""Seeded synthetic inputs for the load-balanced MoE token path.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no routing, no counting, no planning).  Both the CPU
oracle's tests and the GPU path take their inputs from here.

Workloads (the shapes come from the MoonEP article's benchmark description --
TWO DOTS, "MoonEP: πώς η εξισορρόπηση των AI experts ...", section "Τι δείχνουν
— και τι δεν αποδεικνύουν — τα benchmarks" -- and from the WideEP EP8->64 DP
claim on the research-vault page, section "WideEP"):

  tiny     E=8   K=2 R=4  S=64   H=128  B=2  blk=16  softmax, Zipf s=1.2, unpermuted
  dsv3     E=256 K=8 R=8  S=4096 H=7168 B=32 blk=128 sigmoid, Zipf s=1.1, permuted per layer
  wideep   E=256 K=8 R=64 S=512  H=7168 B=4  blk=64  sigmoid, Zipf s=1.3, permuted per layer
  kimi     E=384 K=8 R=32 S=8192 H=7168 B=4  blk=128 sigmoid, 5% hot experts draw ~30%
  decodeS  E=256 K=8 R=8  S in {1,16,128} H=7168 B=3 blk=128 sigmoid, Zipf s=1.1
  moonep   E=384 K=8 R=8  S=8192 H=7168 B=48 blk=128 sigmoid, routing built for a
           given max_vio (MoonEP's sweep over max_vio in {0.2, 1, 10, 20})

Router logits are fp32 z + bias[e] with z ~ N(0,1) (numpy PCG64, drawn in
fp32) and bias the log of a Zipf pmf p_i ∝ i^-s over i=1..E, mapped to experts
through a per-layer random permutation (so the hot experts move between
layers).  The add is one fp32 round-to-nearest-even operation.  Activations x
are N(0,1) rounded to bf16 (round to nearest even) and returned as the raw
uint16 bit patterns; they are drawn in independent chunks of ``X_CHUNK`` rows
so any row can be regenerated on its own.
"""
from __future__ import annotations

import dataclasses
import numpy as np

X_CHUNK = 1024  # rows of x drawn per independent random stream

# Offset for the hot experts of the Kimi-K3-scale workload.  Chosen so that
# the realised share of (token, expert) assignments that land on the 19 hot
# experts (5% of 384) is 0.30; tests/calibrate_kimi_delta.py recomputes it
# with the oracle's router and prints the share it reaches.
KIMI_DELTA = 1.0263671875


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    E: int
    K: int
    R: int
    S: int
    H: int
    B: int
    blk: int
    score: str            # "softmax" | "sigmoid"
    skew: str             # "zipf" | "hot"
    zipf_s: float = 0.0
    permute: bool = True
    hot_frac: float = 0.0
    seed: int = 0
    vio: float = 0.0      # target max_vio of the "maxvio" skew

    @property
    def N(self) -> int:
        return self.R * self.S

    @property
    def P(self) -> int:
        return self.R * self.S * self.K

    @property
    def SK(self) -> int:
        return self.S * self.K

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 8, 2, 4, 64, 128, 2, 16, "softmax", "zipf", 1.2, False, seed=0),
    "dsv3": Workload("dsv3", 256, 8, 8, 4096, 7168, 32, 128, "sigmoid", "zipf", 1.1, True, seed=1),
    "wideep": Workload("wideep", 256, 8, 64, 512, 7168, 4, 64, "sigmoid", "zipf", 1.3, True, seed=2),
    "kimi": Workload("kimi", 384, 8, 32, 8192, 7168, 4, 128, "sigmoid", "hot", 0.0, True,
                     hot_frac=0.05, seed=3),
    "decode1": Workload("decode1", 256, 8, 8, 1, 7168, 3, 128, "sigmoid", "zipf", 1.1, True, seed=4),
    "decode16": Workload("decode16", 256, 8, 8, 16, 7168, 3, 128, "sigmoid", "zipf", 1.1, True, seed=4),
    "decode128": Workload("decode128", 256, 8, 8, 128, 7168, 3, 128, "sigmoid", "zipf", 1.1, True, seed=4),
    "moonep": Workload("moonep", 384, 8, 8, 8192, 7168, 48, 128, "sigmoid", "maxvio", seed=5, vio=20.0),
}

MAXVIO_SWEEP = (0.2, 1.0, 10.0, 20.0)


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def zipf_log_pmf(E: int, s: float) -> np.ndarray:
    """log p_i for p_i ∝ i^-s, i = 1..E (fp64)."""
    i = np.arange(1, E + 1, dtype=np.float64)
    w = i ** (-s)
    return np.log(w / w.sum())


def n_hot(w: Workload) -> int:
    return int(round(w.hot_frac * w.E))


def expert_bias(w: Workload, layer: int = 0, delta: float | None = None) -> np.ndarray:
    """fp32 per-expert logit offset for one layer (or decode step)."""
    rng = _rng(w.seed, layer, 0)
    perm = rng.permutation(w.E) if w.permute else np.arange(w.E)
    if w.skew == "zipf":
        logp = zipf_log_pmf(w.E, w.zipf_s)
        bias = np.empty(w.E, np.float64)
        bias[perm] = logp            # expert perm[i] gets the i-th hottest weight
    elif w.skew == "hot":
        bias = np.zeros(w.E, np.float64)
        bias[perm[: n_hot(w)]] = KIMI_DELTA if delta is None else delta
    else:
        raise ValueError(w.skew)
    return bias.astype(np.float32)


def hot_pair_count(w: Workload) -> int:
    """Pairs the hot expert of the "maxvio" skew receives: (1 + vio) times
    the mean per-expert load N*K/E, rounded to the nearest integer."""
    return int(round((1.0 + w.vio) * w.N * w.K / w.E))


def maxvio_choice(w: Workload, layer: int = 0) -> tuple[int, np.ndarray]:
    """(hot expert, bool [N, E] choice matrix) of the "maxvio" skew.

    A seeded random set of hot_pair_count(w) tokens picks the hot expert;
    every other (token, slot) is dealt round-robin over a seeded random cyclic
    order of the remaining E-1 experts, token by token, so those experts'
    loads differ by at most one and each token's experts are distinct."""
    if not (0.0 <= w.vio <= w.E / w.K - 1.0):
        raise ValueError("vio must lie in [0, E/K - 1]")
    rng = _rng(w.seed, layer, 4)
    hot = int(rng.integers(w.E))
    n_hot = hot_pair_count(w)
    if n_hot > w.N:
        raise ValueError("too few tokens for this vio")
    is_hot = np.zeros(w.N, bool)
    is_hot[rng.choice(w.N, n_hot, replace=False)] = True
    others = np.delete(np.arange(w.E), hot)
    cyc = others[rng.permutation(w.E - 1)]
    k_t = w.K - is_hot.astype(np.int64)                  # non-hot picks per token
    start = np.concatenate([[0], np.cumsum(k_t)[:-1]])
    choice = np.zeros((w.N, w.E), bool)
    for j in range(w.K):
        sel = j < k_t
        choice[np.nonzero(sel)[0], cyc[(start[sel] + j) % (w.E - 1)]] = True
    choice[is_hot, hot] = True
    return hot, choice


def maxvio_logits(w: Workload, layer: int = 0) -> np.ndarray:
    """fp32 [N, E] logits whose K largest per row are maxvio_choice's experts:
    chosen experts get 1 + u, the others -u, u ~ U[0, 1) drawn in fp32."""
    _, choice = maxvio_choice(w, layer)
    u = _rng(w.seed, layer, 5).random((w.N, w.E), dtype=np.float32)
    return np.where(choice, np.float32(1.0) + u, -u).astype(np.float32)


def router_logits(w: Workload, layer: int = 0, delta: float | None = None,
                  rows: slice | None = None) -> np.ndarray:
    """fp32 [N, E] router logits z + bias for one layer."""
    if w.skew == "maxvio":
        lg = maxvio_logits(w, layer)
        return lg if rows is None else lg[rows]
    z = _rng(w.seed, layer, 1).standard_normal((w.N, w.E), dtype=np.float32)
    if rows is not None:
        z = z[rows]
    return z + expert_bias(w, layer, delta)[None, :]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest even) and return the uint16 bit patterns.
    Inputs are finite."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def x_chunk(w: Workload, layer: int, chunk: int, H: int | None = None) -> np.ndarray:
    """bf16 bits of rows [chunk*X_CHUNK, (chunk+1)*X_CHUNK) of x (clipped to N)."""
    H = w.H if H is None else H
    lo = chunk * X_CHUNK
    n = min(X_CHUNK, w.N - lo)
    v = _rng(w.seed, layer, 2, chunk).standard_normal((n, H), dtype=np.float32)
    return f32_to_bf16_bits(v)


def activations(w: Workload, layer: int = 0, H: int | None = None) -> np.ndarray:
    """bf16 bits [N, H] of the token activations."""
    H = w.H if H is None else H
    out = np.empty((w.N, H), np.uint16)
    for c in range((w.N + X_CHUNK - 1) // X_CHUNK):
        lo = c * X_CHUNK
        blk = x_chunk(w, layer, c, H)
        out[lo: lo + blk.shape[0]] = blk
    return out


def activation_rows(w: Workload, rows: np.ndarray, layer: int = 0, H: int | None = None) -> np.ndarray:
    """bf16 bits of selected rows of x, regenerated chunk by chunk."""
    H = w.H if H is None else H
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, H), np.uint16)
    for c in np.unique(rows // X_CHUNK):
        blk = x_chunk(w, layer, int(c), H)
        sel = np.nonzero(rows // X_CHUNK == c)[0]
        out[sel] = blk[rows[sel] - c * X_CHUNK]
    return out


def random_expert_out(w: Workload, n_rows: int, H: int | None = None, seed: int = 7) -> np.ndarray:
    """bf16 bits of a random stand-in for an expert's output buffer."""
    H = w.H if H is None else H
    return f32_to_bf16_bits(_rng(w.seed, seed, 3).standard_normal((n_rows, H), dtype=np.float32))


def device_normal_bf16(shape, seed: int, device):
    """bf16 bits (as int16) of N(0,1) values drawn on the device with torch's
    seeded generator and rounded to nearest even: a stand-in for buffers too
    large to draw on the host (a full-size expert-output buffer)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = torch.empty(shape, dtype=torch.int16, device=device)
    flat = out.view(-1)
    step = 1 << 26
    for lo in range(0, flat.numel(), step):
        n = min(step, flat.numel() - lo)
        v = torch.randn(n, generator=g, device=device, dtype=torch.float32)
        flat[lo: lo + n] = v.to(torch.bfloat16).view(torch.int16)
    return out
