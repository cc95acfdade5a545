"""Shared test helpers: device transfer, cached oracle encodings, metrics.

Encoded matrices are produced by the oracle's encoder only (never by the
library) and cached under .p8f_cache/ (git-ignored)."""
from __future__ import annotations

import os

import numpy as np

from oracle import p8f
from qgemv_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CACHE = os.path.join(ROOT, ".p8f_cache")
TOL = 1e-3          # relative error bar for products (fp64 oracle reference)


def dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def rel_err(y, y_ref) -> float:
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    return float(np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref))


def rel_err_rows(y, y_ref) -> np.ndarray:
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    return np.linalg.norm(y - y_ref, axis=-1) / np.linalg.norm(y_ref, axis=-1)


def _cached(name: str, fn):
    os.makedirs(CACHE, exist_ok=True)
    path = os.path.join(CACHE, f"v1_{name}.npz")
    if os.path.exists(path):
        d = np.load(path)
        return d["codes"], d["scales"]
    codes, scales = fn()
    np.savez(path + ".tmp.npz", codes=codes, scales=scales)
    os.replace(path + ".tmp.npz", path)
    return codes, scales


def encoded_single():
    """The 512 x 2048 N(0,1) layer, Viterbi-encoded by the oracle."""
    return _cached("single", lambda: p8f.encode_matrix(synth.single_layer_weights(),
                                                        synth.site_sign_bits(0, 0, 2048)))


def encoded_qwen(name: str):
    """One Qwen3-4B-shaped matrix (0.02 N(0,1) + 0.1% x20 outliers), encoded
    by the oracle with its input site's signs."""
    def run():
        w = synth.qwen_layer_weights(name)
        sb = synth.site_sign_bits(0, synth.SITE_OF[name], w.shape[1])
        return p8f.encode_matrix(w, sb)
    return _cached(f"qwen_{name}", run)


def oracle_chain(codes, scales, signs, shapes, h0, layers, carry=False, table=None, rate23=False):
    """The stack driver's chain (qgemv_amd.stack) written with the oracle's
    fp64 functions: rotate, RMS-normalise with fp16 rounding, product
    (carry: codes of the carried-state variant; table: levels read through
    that codebook table)."""
    from qgemv_amd.stack import ORDER
    merged = synth.merged_shapes(shapes)
    h = np.asarray(h0, dtype=np.float64)
    out = {}
    for layer in range(layers):
        for site in ORDER:
            n, k = merged[site]
            if site == "qkv":
                src = h if layer == 0 else p8f.rmsnorm16(out["down"])
            else:
                prev = {"o": "qkv", "gu": "o", "down": "gu"}[site]
                src = p8f.rmsnorm16(out[prev][:, :k])
            xr = p8f.rotate(src[:, :k], signs[layer][site])
            if table is None:
                out[site] = p8f.gemv_ref(codes[layer][site], scales[layer][site], xr, carry)
            else:
                out[site] = p8f.gemv_table_ref(codes[layer][site], scales[layer][site], table, xr, carry, rate23)
    return out["down"]


def assert_codes_equivalent(w, sb, codes, oracle_codes, scales):
    """Codes must be equal, except on blocks where the two searches are tied
    (their rotated inputs differ by rounding order): there both paths must
    reach the optimum distortion to 1e-12 relative."""
    n, k = w.shape
    diff = np.nonzero((codes != oracle_codes).reshape(n, k // 128, 32).any(axis=2))
    wr = p8f.rotate(w, sb).reshape(n, k // 128, 128)
    for r, b in zip(*diff):
        d_lib = p8f.block_distortion(wr[r, b][None], codes[r, 32 * b:32 * b + 32][None], scales[r, b:b + 1])[0]
        d_orc = p8f.block_distortion(wr[r, b][None], oracle_codes[r, 32 * b:32 * b + 32][None], scales[r, b:b + 1])[0]
        assert abs(d_lib - d_orc) <= 1e-12 * d_orc
    assert len(diff[0]) <= max(1, n * (k // 128) // 10000)
