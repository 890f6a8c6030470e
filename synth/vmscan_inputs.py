"""Seeded synthetic inputs for the Vim bidirectional scan and the VMamba SS2D cross-scan.

Every tensor is drawn from its own stream,
``numpy.random.Generator(PCG64(SeedSequence([41, cfg, layer, tensor_id])))``, so any tensor of
any layer can be regenerated independently.  Distributions follow the workloads:

* u, z, Δ_raw, B, C ~ N(0, 1), drawn in float32; the bf16 workloads round them to bf16 with
  round-to-nearest-even, so the GPU and the oracle read identical values.
* A_log = log(1..N) broadcast over channels (the A/A_b initialisation of the pages).
* D = 1.
* Δ bias = inverse softplus of dt, dt log-uniform on [1e-3, 1e-1], computed in float64 and
  stored as float32 (the dt initialisation range stated for SS2D).

* Front convolutions: the pre-convolution activation x ~ N(0, 1) like the others; weights and
  bias uniform on [-1/sqrt(fan_in), 1/sqrt(fan_in)] with fan_in = d_conv (conv1d) or d_conv^2
  (depthwise conv2d), the default initialisation of a convolution layer.

Tensor ids: Vim u=0, z=1, Δ_raw=2, B=3, C=4, B_b=5, C_b=6, dt=7 and, for a separate backward
branch, u_b=8, Δ_raw_b=9, dt_b=17; SS2D x=0, z=1 and, for direction k, Δ_raw=10k+2, B=10k+3,
C=10k+4, dt=10k+7.  Front convolutions: x=50, conv_w=51, conv_b=52, conv_w_b=53, conv_b_b=54.

Independent parameters (``params="indep"``): the parity tests also draw the parameters the
pages initialise to shared constants, so that every per-channel, per-direction and per-branch
parameter differs from every other (v2 gives the backward branch its own parameter set; SS2D
gives each direction its own projections).  A_log = log(1..N) + U[-0.5, 0.5] per (channel,
state), D ~ U[-1.5, 1.5] per channel, each tensor from its own stream: Vim A_log=20, A_b_log=21,
D=22, D_b=23; SS2D direction k A_log=10k+5, D=10k+6 (its Δ bias already has its own draw).
"""
import numpy as np

# name -> workload description
CONFIGS = {
    0: dict(kind="vim", name="vim_bidir_fp32_b1_d384_l197", batch=1, dim=384, seqlen=197, d_state=16, dtype="f32", layers=1),
    1: dict(kind="vim", name="vim_ti_bidir_bf16_b128_d384_l197", batch=128, dim=384, seqlen=197, d_state=16, dtype="bf16", layers=1),
    2: dict(kind="vim", name="vim_s_bidir_bf16_b128_d768_l197_x24", batch=128, dim=768, seqlen=197, d_state=16, dtype="bf16", layers=24),
    3: dict(kind="vim", name="vim_ti_1248px_bidir_bf16_b8_d384_l6085", batch=8, dim=384, seqlen=6085, d_state=16, dtype="bf16", layers=1),
    4: dict(kind="ss2d", name="vmamba_ss2d_bf16_b32_d512_56x56", batch=32, dim=512, H=56, W=56, d_state=16, dtype="bf16", layers=1),
}


def _rng(cfg, layer, tensor_id):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([41, int(cfg), int(layer), int(tensor_id)])))


def round_bf16(x):
    """Round float32 values to the nearest bfloat16 (ties to even); returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    out = (rounded & 0xFFFFFFFF).astype(np.uint32).view(np.float32)
    # keep NaN payloads quiet (inputs here are finite; this only guards the helper)
    return np.where(np.isnan(x), x, out).astype(np.float32)


def _normal(cfg, layer, tid, shape, dtype):
    a = _rng(cfg, layer, tid).standard_normal(size=shape, dtype=np.float32)
    return round_bf16(a) if dtype == "bf16" else a


def dt_bias(cfg, layer, tid, dim, dt_min=1e-3, dt_max=1e-1):
    """Δ bias = log(expm1(dt)) with dt log-uniform on [dt_min, dt_max] (float64 -> float32)."""
    r = _rng(cfg, layer, tid).random(size=dim)
    dt = np.exp(np.log(dt_min) + r * (np.log(dt_max) - np.log(dt_min)))
    return np.log(np.expm1(dt)).astype(np.float32)


def a_log_init(dim, d_state):
    """A_log = log(arange(1..d_state)) repeated over channels (float32)."""
    return np.tile(np.log(np.arange(1, d_state + 1, dtype=np.float64)), (dim, 1)).astype(np.float32)


def a_log_indep(cfg, layer, tid, dim, d_state):
    """A_log = log(1..d_state) + U[-0.5, 0.5], drawn per (channel, state) (float32)."""
    jitter = _rng(cfg, layer, tid).uniform(-0.5, 0.5, size=(dim, d_state))
    return (np.log(np.arange(1, d_state + 1, dtype=np.float64))[None, :] + jitter).astype(np.float32)


def d_indep(cfg, layer, tid, dim):
    """D ~ U[-1.5, 1.5] per channel (float32)."""
    return _rng(cfg, layer, tid).uniform(-1.5, 1.5, size=dim).astype(np.float32)


def make_vim_inputs(cfg, layer=0, batch=None, dim=None, seqlen=None, d_state=None, dtype=None, params="init"):
    """Inputs of one bidirectional Vim scan call as a dict of float32 numpy arrays.

    Defaults come from ``CONFIGS[cfg]``; the overrides give smaller or ragged shapes with the
    same distributions (used by the parity tests).  Values of bf16 workloads are already
    rounded to bf16.  ``params="indep"`` draws A_log, A_b_log, D and D_b independently (see the
    module docstring) instead of the shared initial values."""
    c = CONFIGS.get(cfg, CONFIGS[0])
    nb = c["batch"] if batch is None else batch
    nd = c["dim"] if dim is None else dim
    L = c["seqlen"] if seqlen is None else seqlen
    N = c["d_state"] if d_state is None else d_state
    dt = c["dtype"] if dtype is None else dtype
    if params not in ("init", "indep"):
        raise ValueError(f"params must be 'init' or 'indep', not {params!r}")
    if params == "indep":
        al, alb = a_log_indep(cfg, layer, 20, nd, N), a_log_indep(cfg, layer, 21, nd, N)
        dd, ddb = d_indep(cfg, layer, 22, nd), d_indep(cfg, layer, 23, nd)
    else:
        al = a_log_init(nd, N)
        alb = al.copy()
        dd, ddb = np.ones(nd, dtype=np.float32), np.ones(nd, dtype=np.float32)
    return dict(
        u=_normal(cfg, layer, 0, (nb, nd, L), dt),
        z=_normal(cfg, layer, 1, (nb, nd, L), dt),
        delta_raw=_normal(cfg, layer, 2, (nb, nd, L), dt),
        B=_normal(cfg, layer, 3, (nb, N, L), dt),
        C=_normal(cfg, layer, 4, (nb, N, L), dt),
        B_b=_normal(cfg, layer, 5, (nb, N, L), dt),
        C_b=_normal(cfg, layer, 6, (nb, N, L), dt),
        A_log=al,
        A_b_log=alb,
        D=dd,
        D_b=ddb,
        delta_bias=dt_bias(cfg, layer, 7, nd),
        dtype=dt,
    )


def make_vim_v2_inputs(cfg, layer=0, batch=None, dim=None, seqlen=None, d_state=None, dtype=None, params="init"):
    """``make_vim_inputs`` plus a separate backward branch: u_b, delta_raw_b (same distributions)
    and delta_bias_b (its own dt draw), for the bidirectional scan with v2 parameter sets."""
    p = make_vim_inputs(cfg, layer, batch, dim, seqlen, d_state, dtype, params)
    nb, nd, L = p["u"].shape
    p["u_b"] = _normal(cfg, layer, 8, (nb, nd, L), p["dtype"])
    p["delta_raw_b"] = _normal(cfg, layer, 9, (nb, nd, L), p["dtype"])
    p["delta_bias_b"] = dt_bias(cfg, layer, 17, nd)
    return p


def make_ss2d_inputs(cfg=4, layer=0, batch=None, dim=None, H=None, W=None, d_state=None, dtype=None, with_z=False,
                     params="init"):
    """Inputs of one SS2D cross-scan call: x [batch, dim, H, W]; delta_raw [batch, 4, dim, H*W];
    B, C [batch, 4, N, H*W] (scan order of each direction); A_log [4, dim, N]; D, delta_bias
    [4, dim]; z [batch, dim, H, W] only when ``with_z``.  ``params="indep"`` draws every
    direction's A_log and D independently (see the module docstring)."""
    c = CONFIGS.get(cfg, CONFIGS[4])
    nb = c["batch"] if batch is None else batch
    nd = c["dim"] if dim is None else dim
    h = c["H"] if H is None else H
    w = c["W"] if W is None else W
    N = c["d_state"] if d_state is None else d_state
    dt = c["dtype"] if dtype is None else dtype
    L = h * w
    if params not in ("init", "indep"):
        raise ValueError(f"params must be 'init' or 'indep', not {params!r}")
    if params == "indep":
        al = np.stack([a_log_indep(cfg, layer, 10 * k + 5, nd, N) for k in range(4)], axis=0)
        dd = np.stack([d_indep(cfg, layer, 10 * k + 6, nd) for k in range(4)], axis=0)
    else:
        al = np.stack([a_log_init(nd, N) for _ in range(4)], axis=0)
        dd = np.ones((4, nd), dtype=np.float32)
    out = dict(
        x=_normal(cfg, layer, 0, (nb, nd, h, w), dt),
        delta_raw=np.stack([_normal(cfg, layer, 10 * k + 2, (nb, nd, L), dt) for k in range(4)], axis=1),
        B=np.stack([_normal(cfg, layer, 10 * k + 3, (nb, N, L), dt) for k in range(4)], axis=1),
        C=np.stack([_normal(cfg, layer, 10 * k + 4, (nb, N, L), dt) for k in range(4)], axis=1),
        A_log=al,
        D=dd,
        delta_bias=np.stack([dt_bias(cfg, layer, 10 * k + 7, nd) for k in range(4)], axis=0),
        z=_normal(cfg, layer, 1, (nb, nd, h, w), dt) if with_z else None,
        dtype=dt,
    )
    return out


def _uniform(cfg, layer, tid, shape, bound):
    return _rng(cfg, layer, tid).uniform(-bound, bound, size=shape).astype(np.float32)


def make_conv1d_inputs(cfg=1, layer=0, batch=None, dim=None, seqlen=None, d_conv=4, dtype=None):
    """Inputs of the Vim front convolution: x [batch, dim, L] (pre-convolution activation) and
    both branches' depthwise weights [dim, d_conv] and biases [dim]."""
    c = CONFIGS[cfg]
    nb = c["batch"] if batch is None else batch
    nd = c["dim"] if dim is None else dim
    L = c["seqlen"] if seqlen is None else seqlen
    dt = c["dtype"] if dtype is None else dtype
    bound = 1.0 / np.sqrt(d_conv)
    return dict(
        x=_normal(cfg, layer, 50, (nb, nd, L), dt),
        conv_w=_uniform(cfg, layer, 51, (nd, d_conv), bound),
        conv_b=_uniform(cfg, layer, 52, (nd,), bound),
        conv_w_b=_uniform(cfg, layer, 53, (nd, d_conv), bound),
        conv_b_b=_uniform(cfg, layer, 54, (nd,), bound),
        dtype=dt,
    )


def make_conv2d_inputs(cfg=4, layer=0, batch=None, dim=None, H=None, W=None, d_conv=3, dtype=None):
    """Inputs of the SS2D front convolution: x [batch, dim, H, W] (pre-convolution activation),
    depthwise weights [dim, d_conv, d_conv] and bias [dim]."""
    c = CONFIGS[cfg]
    nb = c["batch"] if batch is None else batch
    nd = c["dim"] if dim is None else dim
    h = c["H"] if H is None else H
    w = c["W"] if W is None else W
    dt = c["dtype"] if dtype is None else dtype
    bound = 1.0 / d_conv
    return dict(
        x=_normal(cfg, layer, 50, (nb, nd, h, w), dt),
        conv_w=_uniform(cfg, layer, 51, (nd, d_conv, d_conv), bound),
        conv_b=_uniform(cfg, layer, 52, (nd,), bound),
        dtype=dt,
    )

