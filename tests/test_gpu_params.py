"""HIP path vs the fp64 oracle with independent parameters and at the method's limits.

Independent parameters: every channel has its own A_log row, the backward branch its own A_b_log
and D_b, and every SS2D direction its own A_log[k], D[k] and Δ bias[k] (the v2 parameter sets of
"Vision Mamba的双向SSM" §2.1; the per-direction projections of "VMamba的SS2D模块" §3.1).  With the
pages' shared initial values (A_log = log(1..N) everywhere, D = 1) a kernel that read A_log
without the channel index, swapped the two branches' parameter sets, used one SS2D direction's
parameters for all four, or dropped the D·u term would still agree with the oracle; here each of
those mistakes moves the output far beyond the tolerance (``tests/test_synth_params.py`` checks
that on the oracle).

Limits ("Vision Mamba实战 双向SSM Encoder核心代码解析与实现" §4 bounds Δ only through softplus):
Δ -> 0 (bias -40: the output tends to D·u·silu(z)), Δ|A| large (bias +30: softplus(x) = x to
float32 resolution, the decay underflows), a bias sweep over [-40, 30] across the channels (every
softplus regime in one call, including arguments just below 20 where a softplus evaluated as
log(1 + e^x) with a compensation term meant for small e^x goes wrong), and z = 0 (the output is
exactly zero; in the backward pass only dz survives).

Same metric and tolerances as the other parity tests: max_i |y_i - r_i| / max(|r_i|, rms(r))
<= 1e-5 (float32 inputs) or 2e-2 (bfloat16 inputs, float32 state); the backward's cancelling
sums take the rounding allowance of ``gpu_common.grad_err``, and dA_log at Δ|A| large the
conditioning allowance below."""
import numpy as np
import pytest

import oracle as O
import synth
from gpu_common import (GRADS, PER_BATCH, SS2D_GRADS, TOL, _dout, grad_err, oracle_bwd, oracle_ss2d, oracle_ss2d_bwd,
                        oracle_vim, oracle_vim_v2, run_bwd, run_ss2d, run_ss2d_bwd, run_vim, run_vim_v2, shared_ref)

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


def _finite(name, *arrays):
    for a in arrays:
        if a is not None:
            assert np.all(np.isfinite(a)), f"{name}: non-finite output"


# ---------------------------------------------------------------------------------------------
# forward, independent parameters

VIM_SHAPES = [(1, 16, 1), (2, 17, 15), (1, 40, 33), (2, 24, 197), (1, 70, 130), (3, 130, 64)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", VIM_SHAPES, ids=[f"b{b}d{d}l{l}" for b, d, l in VIM_SHAPES])
def test_vim_indep(shape, dtype):
    """vmscan_fwd_bidir, library-chosen and forced chunking (split sequences carry each channel's
    own decays across the chunks)."""
    nb, nd, L = shape
    p = synth.make_vim_inputs(0, layer=2000 + L, batch=nb, dim=nd, seqlen=L, dtype=dtype, params="indep")
    ref = oracle_vim(p)
    _report(f"vim indep {shape} {dtype}", O.rel_err(run_vim(p), ref), TOL[dtype])
    if L > 20:
        for K in (16, 41):
            _report(f"vim indep {shape} {dtype} K={K}", O.rel_err(run_vim(p, chunk_len=K), ref), TOL[dtype])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(1, 16, 1), (2, 17, 15), (2, 24, 197), (1, 40, 300)], ids=str)
def test_vim_v2_indep(shape, dtype):
    """vmscan_fwd_bidir_v2: the backward branch's own u_b, Δ_raw_b, bias_b, A_b_log, B_b, C_b, D_b."""
    nb, nd, L = shape
    p = synth.make_vim_v2_inputs(0, layer=2100 + L, batch=nb, dim=nd, seqlen=L, dtype=dtype, params="indep")
    ref = oracle_vim_v2(p)
    _report(f"vim v2 indep {shape} {dtype}", O.rel_err(run_vim_v2(p), ref), TOL[dtype])
    if L > 20:
        _report(f"vim v2 indep {shape} {dtype} K=24", O.rel_err(run_vim_v2(p, chunk_len=24), ref), TOL[dtype])


def test_vim_v1_aliasing_indep():
    """v1: B_b = B, C_b = C, D_b = D passed as the same tensors, while A_b_log stays the backward
    branch's own (per-channel) matrix."""
    p = synth.make_vim_inputs(0, layer=2200, batch=2, dim=40, seqlen=90, dtype="f32", params="indep")
    ref = oracle_vim(p, alias_v1=True)
    _report("vim v1 aliasing indep", O.rel_err(run_vim(p, alias_v1=True), ref), 1e-5)
    _report("vim v1 aliasing indep K=32", O.rel_err(run_vim(p, chunk_len=32, alias_v1=True), ref), 1e-5)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(1, 16, 1), (2, 17, 15), (1, 40, 33), (2, 24, 197)], ids=str)
def test_vim_d_state32_indep(shape, dtype):
    nb, nd, L = shape
    p = synth.make_vim_v2_inputs(0, layer=2300 + L, batch=nb, dim=nd, seqlen=L, d_state=32, dtype=dtype,
                                 params="indep")
    ref = oracle_vim_v2(p)
    _report(f"vim v2 N=32 indep {shape} {dtype}", O.rel_err(run_vim_v2(p), ref), TOL[dtype])
    if L > 20:
        _report(f"vim v2 N=32 indep {shape} {dtype} K=16", O.rel_err(run_vim_v2(p, chunk_len=16), ref), TOL[dtype])


def test_config1_indep_sampled():
    """The Vim-Ti workload (bf16, B128 D384 L197) in the bench's launch configuration, with
    independent parameters and a separate backward branch: sampled batches."""
    p = synth.make_vim_v2_inputs(1, layer=1, params="indep")
    bsel = np.array([0, 50, 127])
    _report("config 1 v2 indep (batches 0,50,127)", O.rel_err(run_vim_v2(p)[bsel], oracle_vim_v2(p, batches=bsel)),
            2e-2)


def test_config3_indep_sampled():
    """The 1248-pixel workload (L 6085, split into chunks) with independent parameters."""
    p = synth.make_vim_inputs(3, layer=1, params="indep")
    bsel = np.array([2])
    _report("config 3 indep (batch 2)", O.rel_err(run_vim(p)[bsel], oracle_vim(p, batches=bsel)), 2e-2)


SS2D_SHAPES = [(1, 16, 1, 1), (2, 5, 3, 7), (1, 20, 7, 9), (1, 16, 23, 19), (2, 3, 67, 5), (1, 70, 12, 12)]


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SS2D_SHAPES, ids=[f"b{b}d{d}h{h}w{w}" for b, d, h, w in SS2D_SHAPES])
def test_ss2d_indep(shape, dtype, gated):
    """Every direction with its own A_log[k], D[k], bias[k]; library-chosen and forced chunks."""
    nb, nd, H, W = shape
    p = synth.make_ss2d_inputs(4, layer=2400 + H * 31 + W, batch=nb, dim=nd, H=H, W=W, dtype=dtype, with_z=gated,
                               params="indep")
    ref = oracle_ss2d(p)
    _report(f"ss2d indep {shape} {dtype} gated={gated}", O.rel_err(run_ss2d(p), ref), TOL[dtype])
    if H * W > 40:
        _report(f"ss2d indep {shape} {dtype} gated={gated} K=24", O.rel_err(run_ss2d(p, chunk_len=24), ref),
                TOL[dtype])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ss2d_d_state32_indep(dtype):
    p = synth.make_ss2d_inputs(4, layer=2500, batch=2, dim=20, H=9, W=11, d_state=32, dtype=dtype, with_z=True,
                               params="indep")
    ref = oracle_ss2d(p)
    _report(f"ss2d N=32 indep {dtype}", O.rel_err(run_ss2d(p), ref), TOL[dtype])
    _report(f"ss2d N=32 indep {dtype} K=16", O.rel_err(run_ss2d(p, chunk_len=16), ref), TOL[dtype])


def test_config4_indep_sampled():
    """The 56 x 56 SS2D workload with every direction's own parameters: one sampled batch."""
    p = synth.make_ss2d_inputs(4, layer=1, params="indep")
    bsel = np.array([9])
    _report("config 4 indep (batch 9)", O.rel_err(run_ss2d(p)[bsel], oracle_ss2d(p, batches=bsel)), 2e-2)


# ---------------------------------------------------------------------------------------------
# forward, limits of the method

def _limit_vim(kind, dtype, L, nb=2, nd=40, layer=0):
    p = synth.make_vim_v2_inputs(0, layer=2600 + layer, batch=nb, dim=nd, seqlen=L, dtype=dtype, params="indep")
    if kind == "delta0":
        p["delta_bias"] = np.full(nd, -40.0, np.float32)
        p["delta_bias_b"] = np.full(nd, -40.0, np.float32)
    elif kind == "delta_large":
        # |A| >= 1 in every state: the decay exp(Δ A) underflows and each step forgets the past
        p["A_log"] = np.maximum(p["A_log"], 0.0).astype(np.float32)
        p["A_b_log"] = np.maximum(p["A_b_log"], 0.0).astype(np.float32)
        p["delta_bias"] = np.full(nd, 30.0, np.float32)
        p["delta_bias_b"] = np.full(nd, 30.0, np.float32)
    elif kind == "bias_sweep":
        # every regime in one call: vanishing steps, the usual range, and arguments past 20
        p["delta_bias"] = np.linspace(-40.0, 30.0, nd).astype(np.float32)
        p["delta_bias_b"] = np.linspace(30.0, -40.0, nd).astype(np.float32)
    elif kind == "z0":
        p["z"] = np.zeros_like(p["z"])
    else:
        raise ValueError(kind)
    return p


LIMITS = ["delta0", "delta_large", "bias_sweep", "z0"]


@pytest.mark.parametrize("L,K", [(197, 0), (150, 32), (1100, -1)], ids=["whole", "split", "lanescan"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kind", LIMITS)
def test_vim_limits(kind, dtype, L, K):
    p = _limit_vim(kind, dtype, L, layer=LIMITS.index(kind))
    out = run_vim_v2(p, chunk_len=K)
    _finite(f"vim limit {kind}", out)
    ref = oracle_vim_v2(p)
    if kind == "z0":
        assert np.all(out == 0.0), "z = 0 must give an output of exactly zero"
        assert np.all(ref == 0.0)
    if kind == "delta0":
        # the limit itself: (D u + D_b u_b) / 2 · silu(z), to within the vanishing Δ terms
        lim = 0.5 * (p["D"][None, :, None] * p["u"] + p["D_b"][None, :, None] * p["u_b"]) * O.silu(p["z"])
        _report(f"vim limit {kind} {dtype} vs D·u·silu(z)", O.rel_err(out, lim), TOL[dtype])
    _report(f"vim limit {kind} {dtype} L={L} K={K}", O.rel_err(out, ref), TOL[dtype])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kind", ["delta0", "delta_large", "bias_sweep", "z0"])
def test_ss2d_limits(kind, dtype):
    nd = 24
    p = synth.make_ss2d_inputs(4, layer=2700 + len(kind), batch=2, dim=nd, H=9, W=13, dtype=dtype, with_z=True,
                               params="indep")
    if kind == "delta0":
        p["delta_bias"] = np.full((4, nd), -40.0, np.float32)
    elif kind == "delta_large":
        p["A_log"] = np.maximum(p["A_log"], 0.0).astype(np.float32)
        p["delta_bias"] = np.full((4, nd), 30.0, np.float32)
    elif kind == "bias_sweep":
        p["delta_bias"] = np.stack([np.roll(np.linspace(-40.0, 30.0, nd), 5 * k) for k in range(4)]).astype(np.float32)
    else:
        p["z"] = np.zeros_like(p["z"])
    ref = oracle_ss2d(p)
    for K in (0, 24):
        out = run_ss2d(p, chunk_len=K)
        _finite(f"ss2d limit {kind}", out)
        if kind == "z0":
            assert np.all(out == 0.0), "z = 0 must give an output of exactly zero"
        _report(f"ss2d limit {kind} {dtype} K={K}", O.rel_err(out, ref), TOL[dtype])


# ---------------------------------------------------------------------------------------------
# backward pass, independent parameters and limits

BWD_SHAPES = [(1, 16, 1), (2, 17, 9), (1, 40, 33), (2, 24, 197), (1, 24, 300), (3, 70, 64)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", BWD_SHAPES, ids=[f"b{b}d{d}l{l}" for b, d, l in BWD_SHAPES])
def test_bwd_indep(shape, dtype):
    """All 15 gradients of vmscan_fwd_bidir_v2 (a sequence of 300 steps on 24 channels is split by
    the backward pass)."""
    nb, nd, L = shape
    p = synth.make_vim_v2_inputs(0, layer=2800 + L, batch=nb, dim=nd, seqlen=L, dtype=dtype, params="indep")
    dout = _dout(p, L + 21)
    got, ref = run_bwd(p, dout), oracle_bwd(p, dout)
    for k in GRADS:
        _report(f"bwd indep {shape} {dtype} {k}", grad_err(got[k], ref, k, TOL[dtype]), TOL[dtype])


def test_bwd_shared_inputs_indep():
    p = synth.make_vim_v2_inputs(0, layer=2900, batch=2, dim=48, seqlen=77, dtype="f32", params="indep")
    dout = _dout(p, 29)
    got, ref = run_bwd(p, dout, shared=True), oracle_bwd(p, dout, shared=True)
    for k, rk in (("du", ("du", "du_b")), ("ddelta_raw", ("ddelta_raw", "ddelta_raw_b")),
                  ("ddelta_bias", ("ddelta_bias", "ddelta_bias_b"))):
        _report(f"bwd shared indep {k}", grad_err(got[k], shared_ref(ref, k, rk), k, 1e-5), 1e-5)
    for k in ("dz", "dA_log", "dA_b_log", "dB", "dC", "dB_b", "dC_b", "dD", "dD_b"):
        _report(f"bwd shared indep {k}", grad_err(got[k], ref, k, 1e-5), 1e-5)


@pytest.mark.parametrize("L", [40, 65, 1001])
def test_bwd_d_state32_indep(L):
    p = synth.make_vim_v2_inputs(0, layer=3000 + L, batch=1, dim=24, seqlen=L, d_state=32, dtype="f32",
                                 params="indep")
    dout = _dout(p, L + 5)
    got, ref = run_bwd(p, dout), oracle_bwd(p, dout)
    for k in GRADS:
        _report(f"bwd n32 indep L={L} {k}", grad_err(got[k], ref, k, 1e-5), 1e-5)


def test_bwd_config1_indep_sampled():
    """The Vim-Ti workload's backward pass with independent parameters: per-batch gradients on
    sampled batches; the batch-summed parameter gradients on those batches run as a batch."""
    p = synth.make_vim_v2_inputs(1, layer=2, params="indep")
    dout = _dout(p, 31)
    got = run_bwd(p, dout)
    bsel = np.array([1, 64, 126])
    ref = oracle_bwd(p, dout, batches=bsel)
    for k in PER_BATCH:
        _report(f"bwd config 1 indep {k} (batches 1,64,126)", grad_err(got[k][bsel], ref, k, 2e-2), 2e-2)
    per = ("u", "delta_raw", "u_b", "delta_raw_b", "z", "B", "C", "B_b", "C_b")
    sub = {k: (v[bsel] if k in per else v) for k, v in p.items()}
    gsub = run_bwd(sub, np.ascontiguousarray(dout[bsel]))
    for k in ("ddelta_bias", "ddelta_bias_b", "dA_log", "dA_b_log", "dD", "dD_b"):
        _report(f"bwd config 1 indep, batches as a batch: {k}", grad_err(gsub[k], ref, k, 2e-2), 2e-2)


# With Δ|A| large the decay exp(Δ A) is ill-conditioned: its relative error is |Δ A| times that
# of its exponent, so dA = Σ λ Δ a h moves by about 2e-6 of its scale when Δ's bias (30.0) moves
# by one float32 ulp.  A float32 evaluation rounds that exponent several times (the bias and the
# raw input scaled to base 2, their sum, the product with A), so dA_log there is held to the
# exact result of inputs moved by a few ulps: |y - r| <= tol max(|r|, rms(r)) + COND_ULPS S, with
# S the sum over the inputs that set the exponent (bias, Δ_raw, A_log of that branch) of the
# oracle's change for a one-ulp change of that input.
COND_ULPS = 8
COND_INPUTS = {"dA_log": ("delta_bias", "delta_raw", "A_log"), "dA_b_log": ("delta_bias_b", "delta_raw_b", "A_b_log")}


def _cond_err(p, dout, ref, got, k, tol):
    s = np.zeros_like(ref[k], dtype=np.float64)
    for name in COND_INPUTS[k]:
        q = dict(p)
        q[name] = (p[name] + np.spacing(np.abs(p[name]).astype(np.float32))).astype(np.float32)
        s += np.abs(oracle_bwd(q, dout)[k] - ref[k])
    r = np.asarray(ref[k], np.float64)
    scale = np.maximum(np.abs(r), np.sqrt(np.mean(r * r)))
    print(f"[parity]   {k}: one-ulp input sensitivity, max relative {np.max(s / scale):.2e}", flush=True)
    return float(np.max(np.abs(np.asarray(got, np.float64) - r) / (scale + COND_ULPS * s / tol)))


@pytest.mark.parametrize("L", [197, 300], ids=["whole", "split"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kind", LIMITS)
def test_bwd_limits(kind, dtype, L):
    """The backward pass at the limits; bias +30 takes the large-argument side of softplus, where
    its derivative is 1.  With z = 0 only dz is nonzero."""
    p = _limit_vim(kind, dtype, L, nb=1, nd=24, layer=10 + LIMITS.index(kind))
    dout = _dout(p, L + LIMITS.index(kind))
    got, ref = run_bwd(p, dout), oracle_bwd(p, dout)
    _finite(f"bwd limit {kind}", *got.values())
    for k in GRADS:
        if kind == "z0" and k != "dz":
            assert np.all(got[k] == 0.0), f"z = 0: {k} must be exactly zero"
        if kind == "delta_large" and k in COND_INPUTS:
            err = _cond_err(p, dout, ref, got[k], k, TOL[dtype])
        else:
            err = grad_err(got[k], ref, k, TOL[dtype])
        _report(f"bwd limit {kind} {dtype} L={L} {k}", err, TOL[dtype])


SS2D_BWD_SHAPES = [(1, 16, 1, 1), (2, 5, 3, 4), (1, 17, 7, 9), (1, 4, 67, 70)]


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SS2D_BWD_SHAPES, ids=[f"b{b}d{d}h{h}w{w}" for b, d, h, w in SS2D_BWD_SHAPES])
def test_ss2d_bwd_indep(shape, dtype, gated):
    nb, nd, H, W = shape
    p = synth.make_ss2d_inputs(4, layer=3100 + H * 31 + W, batch=nb, dim=nd, H=H, W=W, dtype=dtype, with_z=gated,
                               params="indep")
    dout = _dout(dict(u=p["x"], dtype=dtype), H * W + 41)
    got, ref = run_ss2d_bwd(p, dout), oracle_ss2d_bwd(p, dout)
    for k in SS2D_GRADS:
        if ref[k] is None:
            assert got[k] is None
            continue
        _report(f"ss2d bwd indep {shape} {dtype} gated={gated} {k}", grad_err(got[k], ref, k, TOL[dtype]), TOL[dtype])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kind", LIMITS)
def test_ss2d_bwd_limits(kind, dtype):
    nd = 20
    p = synth.make_ss2d_inputs(4, layer=3200 + len(kind), batch=1, dim=nd, H=7, W=9, dtype=dtype, with_z=True,
                               params="indep")
    if kind == "delta0":
        p["delta_bias"] = np.full((4, nd), -40.0, np.float32)
    elif kind == "delta_large":
        p["A_log"] = np.maximum(p["A_log"], 0.0).astype(np.float32)
        p["delta_bias"] = np.full((4, nd), 30.0, np.float32)
    elif kind == "bias_sweep":
        p["delta_bias"] = np.stack([np.roll(np.linspace(-40.0, 30.0, nd), 3 * k) for k in range(4)]).astype(np.float32)
    else:
        p["z"] = np.zeros_like(p["z"])
    dout = _dout(dict(u=p["x"], dtype=dtype), 77)
    got, ref = run_ss2d_bwd(p, dout), oracle_ss2d_bwd(p, dout)
    _finite(f"ss2d bwd limit {kind}", *got.values())
    for k in SS2D_GRADS:
        if kind == "z0" and k != "dz":
            assert np.all(got[k] == 0.0), f"z = 0: {k} must be exactly zero"
        _report(f"ss2d bwd limit {kind} {dtype} {k}", grad_err(got[k], ref, k, TOL[dtype]), TOL[dtype])
