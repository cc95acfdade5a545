"""GPU parity of pg_qgemm (the prompt path on the matrix cores) against the
oracle's fp64 product on the same bf16 activations.  Bar: relative error
<= 1e-3 per output row."""
import numpy as np
import pytest

import qgemv_amd as q
from oracle import p8f
from qgemv_amd import synth
from tests.helpers import TOL, dev, encoded_qwen, host, rel_err_rows

pytestmark = pytest.mark.gpu


def _qgemm(codes, scales, xb):
    import torch
    n, kg = codes.shape
    k = 4 * kg
    m = xb.shape[0]
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    if _kernel[0] is None:
        q.pg_qgemm(dev(codes), dev(scales), n, k, dev(xb), m, y)
    else:
        q.pg_qgemm_tune(dev(codes), dev(scales), n, k, dev(xb), m, y, None, 0, _kernel[0], 0, 0)
    torch.cuda.synchronize()
    return host(y)


_kernel = [None]


@pytest.fixture(params=["auto", "1", "2", "3", "4", "5", "6", "7", "8", "9"])
def kernel(request):
    """Which product kernel runs: pg_qgemm's own, or one selected through
    pg_qgemm_tune (1: the 128x128-tile one-buffer kernel, 2: the pipelined
    256x128-tile kernel with per-block partial sums, 3: the same tile with
    producer and consumer waves, 4: the same in 1024 threads with the block
    scales carried in the running sums, 5: the library's choice through
    pg_qgemm_tune, 6: 256x256 tiles with carried block scales, 7: the same
    with the weight operands decoded in registers, 8: as 7 with 256x32 wave
    tiles, 9: 256x128 tiles of four waves with register-decoded operands,
    the library's choice)."""
    _kernel[0] = {"auto": None, "1": 1, "2": 4, "3": 2, "4": 3, "5": 0, "6": 5, "7": 6, "8": 7, "9": 8}[request.param]
    yield request.param
    _kernel[0] = None


@pytest.mark.parametrize("m,n,k", [(128, 128, 128), (256, 384, 512), (77, 130, 640), (1, 5, 256), (300, 1024, 2560),
                                   (513, 257, 1152)])
def test_small_and_ragged(m, n, k, kernel):
    rng = np.random.default_rng(m * n + k)
    codes = rng.integers(0, 256, (n, k // 4), dtype=np.uint8)
    scales = synth.random_scale_bits(n, k, m + n)
    xb = synth.bf16_activations_bits(m, k, seed=m)
    y = _qgemm(codes, scales, xb)
    ref = p8f.gemm_ref(codes, scales, p8f.bf16_bits_to_float(xb))
    assert np.max(rel_err_rows(y, ref)) <= TOL


def test_encoded_matrix_m512(kernel):
    codes, scales = encoded_qwen("k")
    xb = synth.bf16_activations_bits(512, codes.shape[1] * 4)
    y = _qgemm(codes, scales, xb)
    ref = p8f.gemm_ref(codes, scales, p8f.bf16_bits_to_float(xb))
    assert np.max(rel_err_rows(y, ref)) <= TOL


@pytest.mark.parametrize("m", [512, 4096])
def test_prompt_shapes_sampled_rows(m):
    """Full-size Qwen3-4B-shaped launches (merged qkv and gate/up), checked on
    32 sampled activation rows against the oracle."""
    merged = synth.random_layer_merged(0, synth.qwen3_4b_shapes())
    rng = np.random.default_rng(m)
    for site, (codes, scales) in merged.items():
        k = codes.shape[1] * 4
        xb = synth.bf16_activations_bits(m, k, seed=m + k)
        y = _qgemm(codes, scales, xb)
        rows = np.sort(rng.choice(m, 32, replace=False))
        ref = p8f.gemm_ref(codes, scales, p8f.bf16_bits_to_float(xb[rows]))
        assert np.max(rel_err_rows(y[rows], ref)) <= TOL, site


def test_one_hot_column(kernel):
    codes, scales = encoded_qwen("v")
    n, kg = codes.shape
    k = 4 * kg
    w = p8f.decode_weights(codes, scales)
    xb = np.zeros((128, k), np.uint16)
    cols = [0, 5, 127, 128, 1000, 2559]
    for i, c in enumerate(cols):
        xb[i, c] = 0x3F80            # bf16 1.0
    y = _qgemm(codes, scales, xb)
    for i, c in enumerate(cols):
        if _kernel[0] in (None, 0, 3, 5, 6, 7, 8):
            # the carried-scale kernels (the library's among them) rescale
            # their sums once per later block
            # (one rounding each): within nbk * 2^-24 of the value
            assert np.max(np.abs(y[i] - w[:, c]) / np.maximum(np.abs(w[:, c]), 1e-30)) <= (k // 128) * 2.0 ** -23
        else:
            assert np.array_equal(y[i].astype(np.float64), w[:, c])
    assert not y[len(cols):].any()


# ----------------------------------------------------------------- split K
def _qgemm_ex(codes, scales, xb, ws_bytes=None, guard=0, plan=None, kern=0):
    """pg_qgemm_ex with a workspace of ws_bytes (default: the full split)
    followed by `guard` float32 values that must stay untouched; with a plan
    "S" or "S:T", pg_qgemm_tune with that split."""
    import torch
    n, kg = codes.shape
    k = 4 * kg
    m = xb.shape[0]
    if ws_bytes is None:
        ws_bytes = q.pg_qgemm_workspace_bytes(n, k, m)
    ws = torch.full((ws_bytes // 4 + guard + 4,), 7.0, dtype=torch.float32, device="cuda")
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    if plan is None:
        q.pg_qgemm_ex(dev(codes), dev(scales), n, k, dev(xb), m, y, ws, ws_bytes)
    else:
        sp, _, t = plan.partition(":")
        q.pg_qgemm_tune(dev(codes), dev(scales), n, k, dev(xb), m, y, ws, ws_bytes, kern, int(sp), int(t or 0))
    torch.cuda.synchronize()
    if guard:
        assert (host(ws[ws_bytes // 4:]) == 7.0).all(), "workspace written past workspace_bytes"
    return host(y)


def _case(m, n, k):
    rng = np.random.default_rng(m * n + k + 1)
    codes = rng.integers(0, 256, (n, k // 4), dtype=np.uint8)
    scales = synth.random_scale_bits(n, k, m + n + 1)
    xb = synth.bf16_activations_bits(m, k, seed=m + 1)
    return codes, scales, xb


@pytest.mark.parametrize("m,n,k", [(100, 256, 2048), (300, 1024, 2560), (1, 5, 640), (512, 2560, 4096)])
def test_split_k_matches_oracle(m, n, k):
    """Shapes whose tiles leave compute units idle: pg_qgemm_ex splits K on
    its own (nonzero workspace) and matches the oracle."""
    codes, scales, xb = _case(m, n, k)
    assert q.pg_qgemm_workspace_bytes(n, k, m) > 0
    y = _qgemm_ex(codes, scales, xb)
    rows = np.arange(m) if m <= 128 else np.sort(np.random.default_rng(k).choice(m, 64, replace=False))
    ref = p8f.gemm_ref(codes, scales, p8f.bf16_bits_to_float(xb[rows]))
    assert np.max(rel_err_rows(y[rows], ref)) <= TOL


TILE_BYTES = 256 * 128 * 4


@pytest.mark.parametrize("kern", [0, 2, 3, 4, 8])
@pytest.mark.parametrize("plan", ["2", "3", "8", "2:1", "3:5"])
@pytest.mark.parametrize("m,n,k", [(77, 130, 1152), (256, 384, 512), (3, 1, 1024), (300, 1024, 2560),
                                   (513, 1030, 1152)])
def test_forced_splits_ragged(m, n, k, plan, kern):
    """Split plans given to pg_qgemm_tune: S (every tile split S ways,
    capped at the number of 128-blocks) or S:T (tiles T.. split, the others
    whole), on ragged tiles and odd n (the sum kernel's scalar edge); the
    workspace past the parts stays untouched."""
    codes, scales, xb = _case(m, n, k)
    tiles = -(-n // 128) * -(-m // 256)
    y = _qgemm_ex(codes, scales, xb, ws_bytes=7 * tiles * TILE_BYTES, guard=64, plan=plan, kern=kern)
    ref = p8f.gemm_ref(codes, scales, p8f.bf16_bits_to_float(xb))
    assert np.max(rel_err_rows(y, ref)) <= TOL


def test_split_k_small_workspace_and_none():
    """Fewer workspace bytes give fewer splits (one part: two splits) and
    still the product; too little for a part is pg_qgemm, bit for bit."""
    codes, scales, xb = _case(512, 2560, 4096)
    m, n = xb.shape[0], codes.shape[0]
    ref = p8f.gemm_ref(codes, scales, p8f.bf16_bits_to_float(xb[:64]))
    y1 = _qgemm_ex(codes, scales, xb, ws_bytes=m * n * 4, guard=64)   # 40 tiles: one part
    assert np.max(rel_err_rows(y1[:64], ref)) <= TOL
    y0 = _qgemm_ex(codes, scales, xb, ws_bytes=m * n * 4 - 16)   # less than one part: no split
    assert np.array_equal(y0, _qgemm(codes, scales, xb))


def test_split_k_deterministic_and_close_to_unsplit():
    codes, scales, xb = _case(512, 2560, 9728)
    a = _qgemm_ex(codes, scales, xb)
    b = _qgemm_ex(codes, scales, xb)
    assert np.array_equal(a, b)
    c = _qgemm(codes, scales, xb)
    scale = np.max(np.abs(c), axis=1, keepdims=True)
    assert np.max(np.abs(a - c) / scale) <= 1e-5                 # only the summation order differs


def test_split_k_graph_replays():
    """pg_qgemm_ex (product + split sum, two launches) captured in a HIP graph
    and replayed three times, eager work between the replays; every replay
    equals the eager call."""
    import torch
    codes, scales, xb = _case(512, 2560, 4096)
    n, k, m = codes.shape[0], 4 * codes.shape[1], xb.shape[0]
    cd, sc, xd = dev(codes), dev(scales), dev(xb)
    wsb = q.pg_qgemm_workspace_bytes(n, k, m)
    ws = torch.empty((wsb // 4,), dtype=torch.float32, device="cuda")
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    q.pg_qgemm_ex(cd, sc, n, k, xd, m, y, ws, wsb)
    torch.cuda.synchronize()
    eager = host(y)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        q.pg_qgemm_ex(cd, sc, n, k, xd, m, y, ws, wsb)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q.pg_qgemm_ex(cd, sc, n, k, xd, m, y, ws, wsb)
    for i in range(3):
        y.fill_(float(i + 1))
        ws.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(y), eager), i


@pytest.mark.parametrize("m", [512, 4096])
def test_prompt_shapes_split_sampled_rows(m):
    """The full-size Qwen3-4B-shaped launches through pg_qgemm_ex with the
    workspace it asks for (the 2560-row shapes split at m = 512)."""
    merged = synth.random_layer_merged(0, synth.qwen3_4b_shapes())
    rng = np.random.default_rng(m + 1)
    for site, (codes, scales) in merged.items():
        k = codes.shape[1] * 4
        xb = synth.bf16_activations_bits(m, k, seed=m + k)
        y = _qgemm_ex(codes, scales, xb)
        rows = np.sort(rng.choice(m, 32, replace=False))
        ref = p8f.gemm_ref(codes, scales, p8f.bf16_bits_to_float(xb[rows]))
        assert np.max(rel_err_rows(y[rows], ref)) <= TOL, site


def test_zero_and_wide_scales(kernel):
    """Blocks of zero scale (first, middle, last, whole rows) and scales that
    span eight decades within a row: every kernel matches the oracle (the
    carried-scale kernel rescales its running sums by ratios of consecutive
    non-zero scales and decodes zero-scale blocks as zero levels)."""
    rng = np.random.default_rng(77)
    m, n, k = 300, 384, 1280
    codes = rng.integers(0, 256, (n, k // 4), dtype=np.uint8)
    sc = rng.uniform(0.005, 0.05, (n, k // 128))
    sc[0, 0] = 0.0
    sc[1, 4:7] = 0.0
    sc[2, -1] = 0.0
    sc[3, :] = 0.0
    sc[4, :3] = 0.0
    sc[5] = 10.0 ** rng.uniform(-4, 4, k // 128)
    scales = sc.astype(np.float16).view(np.uint16)
    xb = synth.bf16_activations_bits(m, k, seed=78)
    y = _qgemm(codes, scales, xb)
    ref = p8f.gemm_ref(codes, scales, p8f.bf16_bits_to_float(xb))
    assert np.all(y[:, 3] == 0.0)
    live = [c for c in range(n) if c != 3]
    assert np.max(rel_err_rows(y[:, live].T, ref[:, live].T)) <= TOL


def test_wide_tiles_equal_carried_scale_kernel_and_library_choice():
    """Kernels that sum every output in the same order give equal results:
    the LDS-staged 256x256 tiles and the 1024-thread carried-scale kernel;
    the register-decoded kernels with 128x64 and 256x32 wave tiles and the
    4-wave 256x128 tiles (which pg_qgemm runs, unsplit without a workspace).
    On ragged and whole tiles, each also against the oracle."""
    import torch
    rng = np.random.default_rng(91)
    for (m, n, k) in [(300, 390, 384), (2048, 8192, 256)]:
        codes = rng.integers(0, 256, (n, k // 4), dtype=np.uint8)
        sc = rng.uniform(0.005, 0.05, (n, k // 128))
        sc[1, 0] = 0.0
        scales = sc.astype(np.float16).view(np.uint16)
        xb = synth.bf16_activations_bits(m, k, seed=m + n)
        ys = {}
        for kern in (3, 4, 5, 6, 7, 8, None):
            y = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
            if kern is None:
                q.pg_qgemm(dev(codes), dev(scales), n, k, dev(xb), m, y)
            else:
                q.pg_qgemm_tune(dev(codes), dev(scales), n, k, dev(xb), m, y, None, 0, kern, 0, 0)
            torch.cuda.synchronize()
            ys[kern] = host(y)
        assert np.array_equal(ys[5], ys[3]), (m, n, k)
        assert np.array_equal(ys[7], ys[6]), (m, n, k)
        assert np.array_equal(ys[8], ys[7]), (m, n, k)
        assert np.array_equal(ys[None], ys[8]), (m, n, k)
        rows = np.sort(rng.choice(m, 16, replace=False))
        ref = p8f.gemm_ref(codes, scales, p8f.bf16_bits_to_float(xb[rows]))
        for kern in (4, 5, 6):
            assert np.max(rel_err_rows(ys[kern][rows], ref)) <= TOL, kern
