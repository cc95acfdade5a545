"""End-to-end parity of the per-token stack driver (rotation + RMS norm +
qgemv, chained layer to layer as in a decoder's linear stack) against the
same chain computed by the oracle in fp64, at full layer sizes."""
import numpy as np
import pytest

from qgemv_amd import synth
from qgemv_amd.stack import Stack
from tests.helpers import TOL, host, oracle_chain, rel_err

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("shapes_fn,layers", [(synth.qwen3_4b_shapes, 2), (synth.llama31_8b_shapes, 2)])
def test_chain_matches_oracle(shapes_fn, layers, fused):
    import torch
    shapes = shapes_fn()
    st = Stack(shapes, layers, fused=fused)
    d = st.token()
    torch.cuda.synchronize()
    got = host(d)
    codes, scales, signs = zip(*[st.host_arrays(l) for l in range(layers)])
    ref = oracle_chain(list(codes), list(scales), list(signs), shapes, host(st.h0).astype(np.float64), layers)
    assert rel_err(got, ref) <= TOL
    # a second token from the same input is bitwise identical
    d2 = host(st.token())
    assert np.array_equal(d2.view(np.uint32), got.view(np.uint32))


PATHS = {"fused": dict(fused=True), "split": dict(fused=False), "hybrid": dict(fused=True, split_above=4096)}


@pytest.mark.parametrize("path", ["fused", "split", "hybrid"])
@pytest.mark.parametrize("batch", [2, 3, 4, 8])
def test_chain_batched_matches_oracle(batch, path):
    """Batched decode, through the fused stage (several activation rows per
    launch), the rotation + matrix-core product, or both (fused where
    k <= 4096, the default batched path of the benchmark), against the
    oracle's chain, row by row."""
    import torch
    from tests.helpers import rel_err_rows
    shapes = synth.llama31_8b_shapes()
    st = Stack(shapes, 2, batch=batch, **PATHS[path])
    got = host(st.token())
    torch.cuda.synchronize()
    codes, scales, signs = zip(*[st.host_arrays(l) for l in range(2)])
    ref = oracle_chain(list(codes), list(scales), list(signs), shapes, host(st.h0).astype(np.float64), 2)
    assert got.shape == ref.shape == (batch, shapes["down"][0])
    assert np.max(rel_err_rows(got, ref)) <= TOL


@pytest.mark.parametrize("batch,path", [(1, "split"), (8, "split"), (2, "hybrid"), (8, "hybrid")])
def test_graph_replays_match_eager(batch, path):
    """A captured token replays bitwise-identically to the eager token, on
    every replay, with eager work and synchronisations in between (batch
    2..8: the matrix-core kernels)."""
    import torch
    st = Stack(synth.qwen3_4b_shapes(), 3, batch=batch, **PATHS[path])
    eager = host(st.token()).copy()
    st.capture()
    for i in range(4):
        st.out["down"].zero_()
        torch.cuda.synchronize()
        got = host(st.replay())
        torch.cuda.synchronize()
        assert np.array_equal(got.view(np.uint32), eager.view(np.uint32)), i
        e2 = host(st.token())                 # eager work between replays
        assert np.array_equal(e2.view(np.uint32), eager.view(np.uint32))


def test_chain_f32_path_matches_q16_path():
    """The fp32-activation path and the PG_Q16 path agree to well within the
    bar on the same stack (they differ only in the 16-bit activation rounding)."""
    import qgemv_amd as q
    shapes = synth.qwen3_4b_shapes()
    a = host(Stack(shapes, 2, x_dtype=q.PG_Q16, fused=False).token())
    b = host(Stack(shapes, 2, x_dtype=q.PG_F32, fused=False).token())
    assert rel_err(a, b) <= 1e-3
