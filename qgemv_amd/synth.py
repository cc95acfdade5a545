"""Seeded synthetic inputs for the five workloads (no method arithmetic here).

Every array is drawn with numpy's PCG64 (`numpy.random.default_rng(seed)`);
the same generators feed the oracle and the GPU library, so both consume
identical inputs.  Nothing here rotates, encodes, decodes or multiplies:
weights that need encoding are handed to an encoder by the caller.

Workloads (the pages measure Qwen3-4B and Llama-3.1-8B; no weights or
datasets are available, so these shapes and distributions stand in for them):
  single   512 x 2048 layer, W ~ N(0,1) fp32 (seed 0), batch-1 fp16 N(0,1)
  qwen1    one Qwen3-4B-shaped layer (q,k,v,o,gate,up,down), W ~ 0.02 N(0,1)
           with 0.1% of entries x20, batch-1 fp16 N(0,1) activations
  qwen36   36 Qwen3-4B-shaped layers, uniform random code bytes,
           scales fp16(U(0.005, 0.05)), fp16 N(0,1) input fed layer to layer
  llama32  32 Llama-3.1-8B-shaped layers, same generators, batch 1 and 4
  prompt   qgemm on the Qwen3-4B layer shapes, M = 512 / 4096 bf16 N(0,1) rows

Seeds: C0's W uses 0; matrix i (q,k,v,o,gate,up,down = 0..6) of layer l uses
1000*l + 10*i for W or codes, +1 for scales, +2 for outlier positions; the
sign vector of input site t (qkv=0, o=1, gate/up=2, down=3) of layer l uses
900000 + 10*l + t; activations use 7.
"""

from __future__ import annotations

import numpy as np

MATS = ("q", "k", "v", "o", "gate", "up", "down")
SITES = ("qkv", "o", "gu", "down")
SITE_OF = {"q": 0, "k": 0, "v": 0, "o": 1, "gate": 2, "up": 2, "down": 3}


def qwen3_4b_shapes():
    """(name -> (N out, K in)) of one Qwen3-4B decoder layer's linears."""
    h, q, kv, ff = 2560, 4096, 1024, 9728
    return {"q": (q, h), "k": (kv, h), "v": (kv, h), "o": (h, q),
            "gate": (ff, h), "up": (ff, h), "down": (h, ff)}


def llama31_8b_shapes():
    h, q, kv, ff = 4096, 4096, 1024, 14336
    return {"q": (q, h), "k": (kv, h), "v": (kv, h), "o": (h, q),
            "gate": (ff, h), "up": (ff, h), "down": (h, ff)}


def merged_shapes(shapes):
    """Launch groups sharing one input: qkv and gate/up are stacked by rows."""
    return {
        "qkv": (shapes["q"][0] + shapes["k"][0] + shapes["v"][0], shapes["q"][1]),
        "o": shapes["o"],
        "gu": (shapes["gate"][0] + shapes["up"][0], shapes["gate"][1]),
        "down": shapes["down"],
    }


def mat_seed(layer: int, name: str) -> int:
    return 1000 * layer + 10 * MATS.index(name)


def site_sign_bits(layer: int, site: int, k: int) -> np.ndarray:
    """Random sign vector of one input site, packed: bit (k & 7) of byte
    (k >> 3), 1 meaning -1."""
    return np.random.default_rng(900000 + 10 * layer + site).integers(0, 256, k // 8, dtype=np.uint8)


def activations_fp16(rows: int, k: int, seed: int = 7) -> np.ndarray:
    """fp16 N(0,1) activations [rows][K] (returned as float16)."""
    return np.random.default_rng(seed).standard_normal((rows, k), dtype=np.float32).astype(np.float16)


def activations_f32(rows: int, k: int, seed: int = 7) -> np.ndarray:
    return np.random.default_rng(seed).standard_normal((rows, k), dtype=np.float32)


def single_layer_weights():
    """512 x 2048 W ~ N(0,1) fp32 from seed 0."""
    return np.random.default_rng(0).standard_normal((512, 2048), dtype=np.float32)


def qwen_layer_weights(name: str, layer: int = 0):
    """0.02 N(0,1) fp32 with round(0.001 N K) distinct entries scaled by 20."""
    n, k = qwen3_4b_shapes()[name]
    seed = mat_seed(layer, name)
    w = (0.02 * np.random.default_rng(seed).standard_normal((n, k), dtype=np.float32)).astype(np.float32)
    count = int(round(0.001 * n * k))
    pos = np.random.default_rng(seed + 2).choice(n * k, size=count, replace=False)
    flat = w.reshape(-1)
    flat[pos] = flat[pos] * np.float32(20.0)
    return w


def random_codes(n: int, k: int, seed: int) -> np.ndarray:
    """Uniform random code bytes u8 [N][K/4] (every byte string is a valid
    trellis path in this format)."""
    return np.random.default_rng(seed).integers(0, 256, (n, k // 4), dtype=np.uint8)


def random_codebook_table(seed: int, dist: str = "uniform") -> np.ndarray:
    """A swappable codebook for the table-driven variant: int8 [8][256][4]
    (four levels per state and code byte).  "uniform": every int8 value
    equally likely, -128 and 127 included; "gauss": round(N(0, 24^2))
    clipped to [-127, 127], a non-uniform value set of the kind a learned
    codebook has."""
    rng = np.random.default_rng(seed)
    if dist == "uniform":
        return rng.integers(-128, 128, (8, 256, 4), dtype=np.int16).astype(np.int8)
    if dist == "gauss":
        return np.clip(np.rint(rng.normal(0.0, 24.0, (8, 256, 4))), -127, 127).astype(np.int8)
    raise ValueError(f"unknown table distribution {dist!r}")


def random_scale_bits(n: int, k: int, seed: int, lo: float = 0.005, hi: float = 0.05) -> np.ndarray:
    """fp16 bits of U(lo, hi) scales [N][K/128] (numpy's float16 cast rounds
    to nearest even)."""
    v = np.random.default_rng(seed).uniform(lo, hi, (n, k // 128))
    return v.astype(np.float16).view(np.uint16)


def random_matrix(layer: int, name: str, shapes):
    n, k = shapes[name]
    s = mat_seed(layer, name)
    return random_codes(n, k, s), random_scale_bits(n, k, s + 1)


def random_layer_merged(layer: int, shapes):
    """Codes/scales of one layer stacked into its four launch groups."""
    m = {nm: random_matrix(layer, nm, shapes) for nm in MATS}
    out = {
        "qkv": (np.concatenate([m["q"][0], m["k"][0], m["v"][0]]),
                np.concatenate([m["q"][1], m["k"][1], m["v"][1]])),
        "o": m["o"],
        "gu": (np.concatenate([m["gate"][0], m["up"][0]]),
               np.concatenate([m["gate"][1], m["up"][1]])),
        "down": m["down"],
    }
    return out


def bf16_activations_bits(rows: int, k: int, seed: int = 7) -> np.ndarray:
    """bf16 bits of N(0,1) activations [rows][K] (fp32 draw, RNE to bf16)."""
    f = np.random.default_rng(seed).standard_normal((rows, k), dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
