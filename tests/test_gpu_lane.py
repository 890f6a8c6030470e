"""The lane-scan path of the bidirectional scan (chunk_len = CHUNK_LANE_SCAN) against the fp64 oracle.

That path spreads each sequence over the lanes, 16 positions per lane and 1024 per wave segment,
and carries the state between lanes by an associative scan of (decay, state) pairs instead of
splitting the sequence into chunks.  The shapes put the sequence end at every place that matters:
inside a lane's run, at a run boundary, at a segment boundary (1023, 1024, 1025), with one or many
segments, an odd or even number of them (the two directions' halves), and the longest sequence
the path takes (8192).  Same tolerances as the other paths (1e-5 float32, 2e-2 bfloat16)."""
import numpy as np
import pytest

import oracle as O
import synth
from gpu_common import TOL, oracle_vim, oracle_vim_v2, run_vim, run_vim_v2

pytestmark = pytest.mark.gpu

LANE = -1  # VMSCAN_CHUNK_LANE_SCAN


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import selective_state_space_41_amd as V
    assert V.CHUNK_LANE_SCAN == LANE


def _report(name, err, tol):
    print(f"[parity] {name}: err {err:.3e} (tol {tol:.0e})", flush=True)
    assert err <= tol, f"{name}: err {err:.3e} > {tol:.0e}"


LANE_SHAPES = [(1, 1, 1), (2, 5, 7), (1, 16, 16), (1, 17, 17), (2, 20, 197), (1, 9, 1023), (1, 8, 1024),
               (1, 8, 1025), (1, 6, 2049), (2, 3, 3000), (1, 2, 5121), (1, 2, 8192)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", LANE_SHAPES, ids=[f"b{b}d{d}l{l}" for b, d, l in LANE_SHAPES])
def test_lane_small(shape, dtype):
    nb, nd, L = shape
    p = synth.make_vim_inputs(0, layer=4000 + L, batch=nb, dim=nd, seqlen=L, dtype=dtype)
    _report(f"lane {shape} {dtype}", O.rel_err(run_vim(p, chunk_len=LANE), oracle_vim(p)), TOL[dtype])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(1, 5, 1500), (2, 3, 4100)], ids=["b1d5l1500", "b2d3l4100"])
def test_lane_v2_indep(shape, dtype):
    """Separate backward branch and independent per-channel, per-branch parameters."""
    nb, nd, L = shape
    p = synth.make_vim_v2_inputs(0, layer=4100 + L, batch=nb, dim=nd, seqlen=L, dtype=dtype, params="indep")
    _report(f"lane v2 indep {shape} {dtype}", O.rel_err(run_vim_v2(p, chunk_len=LANE), oracle_vim_v2(p)), TOL[dtype])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_lane_d_state32(dtype):
    p = synth.make_vim_inputs(0, layer=4200, batch=2, dim=5, seqlen=2100, d_state=32, dtype=dtype, params="indep")
    _report(f"lane d_state 32 {dtype}", O.rel_err(run_vim(p, chunk_len=LANE), oracle_vim(p)), TOL[dtype])


def test_lane_v1_aliasing():
    """v1 by aliasing (B_b = B, C_b = C, D_b = D) through the lane path."""
    p = synth.make_vim_inputs(0, layer=4300, batch=1, dim=6, seqlen=1300, dtype="f32", params="indep")
    _report("lane v1 aliasing", O.rel_err(run_vim(p, chunk_len=LANE, alias_v1=True), oracle_vim(p, alias_v1=True)),
            1e-5)


def test_lane_deterministic():
    """Fixed combination orders: two calls give the same bits."""
    p = synth.make_vim_inputs(0, layer=4400, batch=2, dim=7, seqlen=3333, dtype="bf16")
    assert np.array_equal(run_vim(p, chunk_len=LANE), run_vim(p, chunk_len=LANE))


def test_lane_too_long():
    """Sequences past 8192 positions are refused (the chunked path takes them)."""
    import torch
    import selective_state_space_41_amd as V
    L = 8193
    u = torch.zeros(1, 1, L, device="cuda")
    bc = torch.zeros(1, 16, L, device="cuda")
    a = torch.zeros(1, 16, device="cuda")
    d = torch.zeros(1, device="cuda")
    with pytest.raises(RuntimeError, match="UNSUPPORTED"):
        V.vmscan_fwd_bidir(u, u, u, a, a, bc, bc, bc, bc, d, d, d, chunk_len=LANE)
    assert V.lib.vmscan_fwd_bidir_workspace_bytes_ex(1, 1, L, 16, 0, LANE) == 0


def test_config3_lane_sampled():
    """The 1248-pixel Vim-Ti workload (B8 D384 L6085, bf16) through the lane path, batches 0 and 7."""
    p = synth.make_vim_inputs(3)
    bsel = np.array([0, 7])
    _report("config 3 lane (batches 0,7)", O.rel_err(run_vim(p, chunk_len=LANE)[bsel], oracle_vim(p, batches=bsel)),
            2e-2)
