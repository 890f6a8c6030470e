"""Front convolutions on the GPU against the fp64 oracle: the Vim conv1d + SiLU (both branches)
and the SS2D 3 x 3 conv2d (+ SiLU) with its transposed copy, alone and followed by the scans.
Tolerances as for the scans: 1e-5 (float32 inputs), 2e-2 (bfloat16 inputs; the fronts round
their outputs to bfloat16 once)."""
import numpy as np
import pytest

import oracle as O
import synth
from gpu_common import TOL, pdev, tdev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import selective_state_space_41_amd  # noqa: F401


def _report(name, err, tol):
    print(f"[parity] {name}: err {err:.3e} (tol {tol:.0e})", flush=True)
    assert err <= tol, f"{name}: err {err:.3e} > {tol:.0e}"


def _np(t):
    import torch
    torch.cuda.synchronize()
    return t.float().cpu().numpy()


def run_conv1d(p, both=True, alias_v1=False):
    import selective_state_space_41_amd as V
    x = tdev(p["x"], p["dtype"])
    w, b = pdev(p["conv_w"]), pdev(p["conv_b"])
    if not both:
        u, ub = V.conv1d_silu_fwd(x, w, b)
        return _np(u), None
    wb, bb = (w, b) if alias_v1 else (pdev(p["conv_w_b"]), pdev(p["conv_b_b"]))
    u, ub = V.conv1d_silu_fwd(x, w, b, wb, bb)
    return _np(u), _np(ub)


def oracle_conv1d(p, batches=None, alias_v1=False):
    x = p["x"] if batches is None else p["x"][batches]
    wb, bb = (p["conv_w"], p["conv_b"]) if alias_v1 else (p["conv_w_b"], p["conv_b_b"])
    return O.conv1d_silu(x, p["conv_w"], p["conv_b"]), O.conv1d_silu(x, wb, bb, reverse=True)


# a thread takes 8 consecutive elements of the flat [rows][L] tensor: rows shorter than 8 go element
# by element (the first three and (1, 300, 3)); 8 and 9 put the window's far end two rows on; the
# others put row boundaries at every offset inside a run
CONV1D = [(1, 1, 1), (1, 3, 2), (2, 5, 7), (1, 16, 8), (2, 17, 9), (1, 6, 10), (2, 9, 16), (1, 5, 17), (2, 3, 23),
          (1, 16, 197), (3, 40, 100), (1, 7, 1000), (1, 300, 3), (1, 3, 2049), (1, 2, 4100)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("K", [1, 2, 3, 4])
@pytest.mark.parametrize("shape", CONV1D, ids=[f"b{b}d{d}l{l}" for b, d, l in CONV1D])
def test_conv1d_front(shape, K, dtype):
    nb, nd, L = shape
    p = synth.make_conv1d_inputs(1, layer=10 * L + K, batch=nb, dim=nd, seqlen=L, d_conv=K, dtype=dtype)
    u, ub = run_conv1d(p)
    ru, rub = oracle_conv1d(p)
    _report(f"conv1d {shape} K={K} {dtype} u", O.rel_err(u, ru), TOL[dtype])
    _report(f"conv1d {shape} K={K} {dtype} u_b", O.rel_err(ub, rub), TOL[dtype])


def test_conv1d_front_one_branch_and_v1():
    """Without the backward branch only u is written (and equals the two-branch u); with the
    forward weights passed for both branches (v1) u_b is the mirrored convolution."""
    p = synth.make_conv1d_inputs(1, layer=3, batch=2, dim=24, seqlen=77, dtype="f32")
    u1, none = run_conv1d(p, both=False)
    assert none is None
    u2, _ = run_conv1d(p)
    assert np.array_equal(u1, u2)
    u, ub = run_conv1d(p, alias_v1=True)
    ru, rub = oracle_conv1d(p, alias_v1=True)
    _report("conv1d v1 u_b", O.rel_err(ub, rub), 1e-5)


@pytest.mark.parametrize("cfg", [0, 1, 2, 3])
def test_conv1d_front_config_sampled(cfg):
    """The Vim fronts of the bench's workloads (d_conv 4): float32 B1 D384 L197, Vim-Ti bf16 B128
    D384 L197, Vim-S bf16 B128 D768 L197 and 1248-pixel bf16 B8 D384 L6085; first and last batch."""
    p = synth.make_conv1d_inputs(cfg)
    u, ub = run_conv1d(p)
    nb = p["x"].shape[0]
    bsel = np.array(sorted({0, nb - 1}))
    ru, rub = oracle_conv1d(p, batches=bsel)
    tol = TOL[p["dtype"]]
    _report(f"conv1d config {cfg} u (batches {bsel.tolist()})", O.rel_err(u[bsel], ru), tol)
    _report(f"conv1d config {cfg} u_b (batches {bsel.tolist()})", O.rel_err(ub[bsel], rub), tol)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_vim_front_then_scan(dtype):
    """x -> (u, u_b) by the front -> the bidirectional scan with a separate backward branch,
    against the oracle's composition of the same steps."""
    import selective_state_space_41_amd as V
    nb, nd, L = 2, 40, 150
    c = synth.make_conv1d_inputs(1, layer=21, batch=nb, dim=nd, seqlen=L, dtype=dtype)
    p = synth.make_vim_v2_inputs(0, layer=21, batch=nb, dim=nd, seqlen=L, dtype=dtype)
    x = tdev(c["x"], dtype)
    u, ub = V.conv1d_silu_fwd(x, pdev(c["conv_w"]), pdev(c["conv_b"]), pdev(c["conv_w_b"]), pdev(c["conv_b_b"]))
    act = {k: tdev(p[k], dtype) for k in ("delta_raw", "delta_raw_b", "z", "B", "C", "B_b", "C_b")}
    par = {k: pdev(p[k]) for k in ("A_log", "A_b_log", "D", "D_b", "delta_bias", "delta_bias_b")}
    out = V.vmscan_fwd_bidir_v2(u, act["delta_raw"], par["delta_bias"], ub, act["delta_raw_b"], par["delta_bias_b"],
                                act["z"], par["A_log"], par["A_b_log"], act["B"], act["C"], act["B_b"], act["C_b"],
                                par["D"], par["D_b"])
    ru, rub = oracle_conv1d(c)
    ref = O.vim_bidir_v2(ru, p["delta_raw"], p["delta_bias"], rub, p["delta_raw_b"], p["delta_bias_b"], p["z"],
                         p["A_log"], p["A_b_log"], p["B"], p["C"], p["B_b"], p["C_b"], p["D"], p["D_b"])
    _report(f"vim front + scan {dtype}", O.rel_err(_np(out), ref), TOL[dtype])


def run_conv2d(p, act=True, transposed=True):
    import selective_state_space_41_amd as V
    xo, xt = V.ss2d_conv2d_silu_fwd(tdev(p["x"], p["dtype"]), pdev(p["conv_w"]), pdev(p["conv_b"]), act=act,
                                    transposed=transposed)
    return _np(xo), (None if xt is None else _np(xt))


CONV2D = [(1, 1, 1, 1), (2, 3, 5, 7), (1, 2, 1, 9), (1, 4, 56, 56), (1, 2, 67, 70), (2, 3, 129, 3), (1, 1, 64, 64),
          (1, 2, 65, 1)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("act", [True, False])
@pytest.mark.parametrize("shape", CONV2D, ids=[f"b{b}d{d}h{h}w{w}" for b, d, h, w in CONV2D])
def test_conv2d_front(shape, act, dtype):
    nb, nd, H, W = shape
    p = synth.make_conv2d_inputs(4, layer=H * 131 + W, batch=nb, dim=nd, H=H, W=W, dtype=dtype)
    xo, xt = run_conv2d(p, act=act)
    _report(f"conv2d {shape} act={act} {dtype}", O.rel_err(xo, O.conv2d_silu(p["x"], p["conv_w"], p["conv_b"], act)),
            TOL[dtype])
    assert np.array_equal(xt, np.swapaxes(xo, -1, -2)), "transposed copy differs from the row-major result"


def test_conv2d_front_row_major_only():
    p = synth.make_conv2d_inputs(4, layer=5, batch=2, dim=3, H=9, W=11, dtype="f32")
    xo1, none = run_conv2d(p, transposed=False)
    assert none is None
    xo2, _ = run_conv2d(p)
    assert np.array_equal(xo1, xo2)


def test_conv2d_front_config4_sampled():
    """The VMamba front (bf16, batch 32, 512 channels, 56 x 56), batches 0 and 31."""
    p = synth.make_conv2d_inputs(4)
    xo, xt = run_conv2d(p)
    bsel = np.array([0, 31])
    _report("conv2d config 4 (batches 0,31)",
            O.rel_err(xo[bsel], O.conv2d_silu(p["x"][bsel], p["conv_w"], p["conv_b"])), 2e-2)
    assert np.array_equal(xt, np.swapaxes(xo, -1, -2))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ss2d_front_then_scan(dtype):
    """x -> (x', x'^T) by the front -> the cross-scan reading the transposed copy, gated, against
    the oracle's composition; and the scan given x'^T equals the scan that transposes itself."""
    import torch
    import selective_state_space_41_amd as V
    nb, nd, H, W = 2, 20, 9, 13
    c = synth.make_conv2d_inputs(4, layer=31, batch=nb, dim=nd, H=H, W=W, dtype=dtype)
    p = synth.make_ss2d_inputs(4, layer=31, batch=nb, dim=nd, H=H, W=W, dtype=dtype, with_z=True)
    xo, xt = V.ss2d_conv2d_silu_fwd(tdev(c["x"], dtype), pdev(c["conv_w"]), pdev(c["conv_b"]))
    args = (tdev(p["delta_raw"], dtype), pdev(p["A_log"]), tdev(p["B"], dtype), tdev(p["C"], dtype), pdev(p["D"]),
            pdev(p["delta_bias"]))
    z = tdev(p["z"], dtype)
    for K in (0, 16):
        out = V.ss2d_cross_scan_fwd(xo, *args, z=z, chunk_len=K, xT=xt)
        ref = O.ss2d_cross_scan(O.conv2d_silu(c["x"], c["conv_w"], c["conv_b"]), p["delta_raw"], p["A_log"], p["B"],
                                p["C"], p["D"], p["delta_bias"], p["z"])
        _report(f"ss2d front + scan {dtype} K={K}", O.rel_err(_np(out), ref), TOL[dtype])
        own = V.ss2d_cross_scan_fwd(xo, *args, z=z, chunk_len=K)
        torch.cuda.synchronize()
        assert torch.equal(out, own)
