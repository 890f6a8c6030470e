"""fp64 reference ("oracle") for the selective scan path.

TEST INFRASTRUCTURE: plain, slow and written to be checked by eye against the pages.  Only
``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use it; the
HIP library never imports it and it never imports the HIP library.

Pages cited (short keys used throughout this repository):

* [P1] "状态空间模型如何重塑视觉序列处理 Vision Mamba的技术突破与应用价值",
  sumeiyu.com/news/203653.  Section "选择性扫描机制的计算效率优势" states the linear
  recurrence h_t = A h_{t-1} + B x_t, y_t = C h_t + D x_t.
* [P3] "Vision Mamba的双向SSM 计算机视觉模型架构的下一代突破", aitangshan.cn/news/1404048.
  §2.1 (A/A_b initialisation, v1/v2 parameter sets), §2.2 (backward scan runs on the reversed
  sequence and is reversed back; fusion by averaging), §4.3 (v2 fast path averages the two
  directions).
* [P4] "VMamba的SS2D模块 状态空间模型在视觉领域的革新设计", lpnh.cn/news/670717.
  §2.1 (forward: x, z split; y * act(z)), §2.2 (the four cross-scan orders X_s), §3.1 (Δ is
  softplus of a projection; per-direction projections), §3.2 (A = -exp(A_log); fp32 for the
  critical parts).
* [P5] "Vision Mamba实战 双向SSM Encoder核心代码解析与实现", lpnh.cn/news/710454.
  §1 table (shapes: A/A_b [d_inner, d_state], B/C [batch, d_state, seq_len], D/D_b [d_inner]),
  §2.1 (A_log = log(arange(1..d_state)), D = 1), §2.2 (bidirectional scan = forward scan plus
  the reversed scan of the reversed input), §4 (delta = softplus(dt_proj(.))).

Readings where the pages are silent or garbled (each is also listed in the design notes):

* Discretisation: zero-order hold for A (a = exp(Δ·A)) and Euler for B (b = Δ·B·u).  The pages
  say only that the state equation is discretised ([P4] §3.2); the cumsum formula printed there
  has no decay term and is not followed.
* Initial state h_{-1} = 0 for every direction.
* Vim backward direction shares u, Δ_raw, z and the Δ bias with the forward direction and has
  its own A_b_log, B_b, C_b, D_b; B_b and C_b are stored in ORIGINAL token order.
* Fusion is the average (y_f + y_b) / 2 ([P3] §2.2, §4.3), each direction gated by silu(z)
  with z reversed together with x ([P3] §2.2 flips ``xz`` as one tensor).
* SS2D: per-direction Δ_raw, B, C are stored in that direction's scan order; the four outputs
  are mapped back to row-major pixel order and summed with no scale; the gate silu(z) is
  applied to the sum only when z is given.
"""
import numpy as np
from scipy.special import expit


def softplus(x):
    """softplus(x) = log(1 + exp(x)), evaluated without overflow ([P5] §4, [P4] §3.1)."""
    return np.logaddexp(0.0, np.asarray(x, dtype=np.float64))


def silu(v):
    """silu(v) = v * sigmoid(v), the activation applied to the gate z ([P4] §2.1)."""
    v = np.asarray(v, dtype=np.float64)
    return v * expit(v)


def scan_1d(u, delta_raw, A_log, B, C, D, delta_bias):
    """One direction of the selective scan, ungated.

    Shapes: u, delta_raw [batch, dim, L]; A_log [dim, N]; B, C [batch, N, L]; D, delta_bias [dim].
    Returns s[batch, dim, L] with, per (b, d):

        A_n   = -exp(A_log[d, n])                            [P4] §3.2
        Δ_t   = softplus(delta_raw[b, d, t] + delta_bias[d])  [P4] §3.1, [P5] §4
        h_t,n = exp(Δ_t A_n) h_{t-1},n + Δ_t B[b, n, t] u[b, d, t],  h_{-1} = 0   [P1]
        s_t   = Σ_n C[b, n, t] h_t,n + D[d] u[b, d, t]        [P1]

    The loop over t is the recurrence as written; batch, channel and state are vectorised.
    """
    u = np.asarray(u, dtype=np.float64)
    delta_raw = np.asarray(delta_raw, dtype=np.float64)
    A = -np.exp(np.asarray(A_log, dtype=np.float64))            # [dim, N]
    B = np.asarray(B, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    D = np.asarray(D, dtype=np.float64)
    bias = np.asarray(delta_bias, dtype=np.float64)
    nb, nd, L = u.shape
    N = A.shape[1]
    delta = softplus(delta_raw + bias[None, :, None])           # [batch, dim, L]
    h = np.zeros((nb, nd, N), dtype=np.float64)
    s = np.empty((nb, nd, L), dtype=np.float64)
    for t in range(L):
        dt = delta[:, :, t][:, :, None]                          # [batch, dim, 1]
        a = np.exp(dt * A[None, :, :])                           # [batch, dim, N]
        b = dt * B[:, None, :, t] * u[:, :, t][:, :, None]       # [batch, dim, N]
        h = a * h + b
        s[:, :, t] = np.sum(h * C[:, None, :, t], axis=2) + D[None, :] * u[:, :, t]
    return s


def scan_1d_semiseparable(u, delta_raw, A_log, B, C, D, delta_bias, reverse=False):
    """The same scan written as a dense L x L matrix (brute force, small L only).

    Unrolling the recurrence gives s = (M + diag(D)) u per (b, d) with
        forward:  M[t, s] = Δ_s Σ_n C_t,n B_s,n exp(A_n Σ_{r=s+1..t} Δ_r)    for s <= t
        backward: M[t, s] = Δ_s Σ_n C_t,n B_s,n exp(A_n Σ_{r=t..s-1} Δ_r)    for s >= t
    i.e. the decay covers the receiving token and excludes the source token.  The backward form
    is the reversed scan of [P3] §2.2 written directly in original token order.  This uses sums
    of Δ inside one exponential instead of a running product, so it is an independent check.
    """
    u = np.asarray(u, dtype=np.float64)
    A = -np.exp(np.asarray(A_log, dtype=np.float64))
    B = np.asarray(B, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    D = np.asarray(D, dtype=np.float64)
    delta = softplus(np.asarray(delta_raw, dtype=np.float64) + np.asarray(delta_bias, dtype=np.float64)[None, :, None])
    nb, nd, L = u.shape
    out = np.empty((nb, nd, L), dtype=np.float64)
    for b in range(nb):
        for d in range(nd):
            dl = delta[b, d]
            M = np.zeros((L, L), dtype=np.float64)
            for t in range(L):
                srange = range(0, t + 1) if not reverse else range(t, L)
                for s in srange:
                    if not reverse:
                        seg = dl[s + 1:t + 1].sum()
                    else:
                        seg = dl[t:s].sum()
                    M[t, s] = dl[s] * np.sum(C[b, :, t] * B[b, :, s] * np.exp(A[d] * seg))
            out[b, d] = M @ u[b, d] + D[d] * u[b, d]
    return out


def vim_bidir(u, delta_raw, z, A_log, A_b_log, B, C, B_b, C_b, D, D_b, delta_bias):
    """Vision Mamba bidirectional (v2 scan inputs) selective scan with the silu(z) gate.

        y_f = scan(u, Δ_raw; A_log, B, C, D) * silu(z)
        y_b = flip( scan(flip u, flip Δ_raw; A_b_log, flip B_b, flip C_b, D_b) * silu(flip z) )
        out = (y_f + y_b) / 2

    [P3] §2.2 (reverse, scan, reverse back; average fusion), [P3] §4.3 and [P5] §2.2 (the
    backward branch is the forward branch applied to the flipped tensors).  Shapes as in
    ``scan_1d``; A_log, A_b_log [dim, N]; B, C, B_b, C_b [batch, N, L] in original order.
    """
    f = lambda x: np.flip(np.asarray(x, dtype=np.float64), axis=-1)
    g = silu(z)
    y_f = scan_1d(u, delta_raw, A_log, B, C, D, delta_bias) * g
    y_b_rev = scan_1d(f(u), f(delta_raw), A_b_log, f(B_b), f(C_b), D_b, delta_bias) * silu(f(z))
    y_b = f(y_b_rev)
    return (y_f + y_b) / 2.0


def vim_bidir_v2(u, delta_raw, delta_bias, u_b, delta_raw_b, delta_bias_b, z, A_log, A_b_log, B, C, B_b, C_b,
                 D, D_b):
    """Vision Mamba bidirectional scan with a fully separate backward branch (v2 parameter sets).

    In v2 the backward branch has its own convolution, input projection and Δ projection
    ([P3] §2.1: conv1d_b, x_proj_b, dt_proj_b, D_b), so besides A_b_log, B_b, C_b, D_b it has its
    own scan input u_b, Δ_raw_b and Δ bias delta_bias_b, all given in ORIGINAL token order.  The
    gate z is shared.

        y_f = scan(u, Δ_raw; A_log, B, C, D, bias) * silu(z)
        y_b = flip( scan(flip u_b, flip Δ_raw_b; A_b_log, flip B_b, flip C_b, D_b, bias_b) * silu(flip z) )
        out = (y_f + y_b) / 2                                   [P3] §2.2, §4.3

    ``vim_bidir`` is the case u_b = u, Δ_raw_b = Δ_raw, bias_b = bias.
    """
    f = lambda x: np.flip(np.asarray(x, dtype=np.float64), axis=-1)
    y_f = scan_1d(u, delta_raw, A_log, B, C, D, delta_bias) * silu(z)
    y_b_rev = scan_1d(f(u_b), f(delta_raw_b), A_b_log, f(B_b), f(C_b), D_b, delta_bias_b) * silu(f(z))
    return (y_f + f(y_b_rev)) / 2.0


def scan_1d_bwd(u, delta_raw, A_log, B, C, D, delta_bias, g):
    """Gradients of one ungated direction (``scan_1d``) given g = dL/ds [batch, dim, L].

    The pages give the forward only and ask that its gradient be checked numerically ([P5] §4
    runs torch.autograd.gradcheck on the bidirectional scan); this is the exact derivative of
    ``scan_1d``, by the adjoint of its recurrence.  With a_t,n = exp(Δ_t A_n) and
    h_t = a_t h_{t-1} + Δ_t B_t u_t, the adjoint state λ_t = dL/dh_t (h_t reaches s_t directly
    and h_{t+1} through a_{t+1}) runs backwards:

        λ_t,n = g_t C_t,n + a_{t+1},n λ_{t+1},n,   λ_L = 0
        dL/dC_t,n     = g_t h_t,n
        dL/dB_t,n     = λ_t,n Δ_t u_t
        dL/du_t       = g_t D + Δ_t Σ_n λ_t,n B_t,n
        dL/dΔ_t       = Σ_n λ_t,n (A_n a_t,n h_{t-1},n + B_t,n u_t)
        dL/dΔ_raw_t   = dL/dΔ_t sigmoid(Δ_raw_t + bias)          (softplus' = sigmoid)
        dL/dbias      = Σ_{b,t} dL/dΔ_raw_t
        dL/dA_n       = Σ_{b,t} λ_t,n Δ_t a_t,n h_{t-1},n,  dL/dA_log = dL/dA * A   (A = -exp(A_log))
        dL/dD         = Σ_{b,t} g_t u_t

    Returns dict(s, du, ddelta_raw, dA_log [dim, N], dB, dC [batch, N, L], dD, ddelta_bias [dim]),
    and du_abs, ddelta_raw_abs: the same sums with every term replaced by its absolute value
    (|g D| + Δ Σ_n |λ B|, and sigmoid · Σ_n |λ| (|A a h| + |B u|)).  They are not gradients but the
    scale of the rounding error of a finite-precision evaluation of those sums (which can cancel
    heavily), used by the tests' error bound.
    The forward states are recomputed and kept for every t (fine at oracle sizes).
    """
    u = np.asarray(u, dtype=np.float64)
    x = np.asarray(delta_raw, dtype=np.float64) + np.asarray(delta_bias, dtype=np.float64)[None, :, None]
    A = -np.exp(np.asarray(A_log, dtype=np.float64))            # [dim, N]
    B = np.asarray(B, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    D = np.asarray(D, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    nb, nd, L = u.shape
    N = A.shape[1]
    delta = softplus(x)
    # forward, keeping h_t (index t + 1; index 0 is h_{-1} = 0) and a_t
    hs = np.zeros((L + 1, nb, nd, N))
    av = np.empty((L, nb, nd, N))
    s = np.empty((nb, nd, L))
    for t in range(L):
        av[t] = np.exp(delta[:, :, t][:, :, None] * A[None])
        hs[t + 1] = av[t] * hs[t] + delta[:, :, t][:, :, None] * B[:, None, :, t] * u[:, :, t][:, :, None]
        s[:, :, t] = np.sum(hs[t + 1] * C[:, None, :, t], axis=2) + D[None, :] * u[:, :, t]
    du = g * D[None, :, None]
    du_abs = np.abs(du)
    ddelta = np.zeros((nb, nd, L))
    ddelta_abs = np.zeros((nb, nd, L))
    dA = np.zeros((nd, N))
    dB = np.zeros((nb, N, L))
    dC = np.zeros((nb, N, L))
    lam = np.zeros((nb, nd, N))
    for t in range(L - 1, -1, -1):
        carry = av[t + 1] * lam if t + 1 < L else 0.0
        lam = g[:, :, t][:, :, None] * C[:, None, :, t] + carry
        dl = delta[:, :, t][:, :, None]
        dC[:, :, t] = np.sum(g[:, :, t][:, :, None] * hs[t + 1], axis=1)
        dB[:, :, t] = np.sum(lam * dl * u[:, :, t][:, :, None], axis=1)
        du[:, :, t] += delta[:, :, t] * np.sum(lam * B[:, None, :, t], axis=2)
        du_abs[:, :, t] += delta[:, :, t] * np.sum(np.abs(lam * B[:, None, :, t]), axis=2)
        decay_term = A[None] * av[t] * hs[t]
        input_term = B[:, None, :, t] * u[:, :, t][:, :, None]
        ddelta[:, :, t] = np.sum(lam * (decay_term + input_term), axis=2)
        ddelta_abs[:, :, t] = np.sum(np.abs(lam) * (np.abs(decay_term) + np.abs(input_term)), axis=2)
        dA += np.sum(lam * dl * av[t] * hs[t], axis=0)
    ddr = ddelta * expit(x)
    return dict(s=s, du=du, ddelta_raw=ddr, ddelta_bias=ddr.sum(axis=(0, 2)), dA_log=dA * A, dB=dB, dC=dC,
                dD=np.sum(g * u, axis=(0, 2)), du_abs=du_abs, ddelta_raw_abs=ddelta_abs * expit(x))


def vim_bidir_v2_bwd(u, delta_raw, delta_bias, u_b, delta_raw_b, delta_bias_b, z, A_log, A_b_log, B, C, B_b, C_b,
                     D, D_b, dout):
    """Gradients of ``vim_bidir_v2`` for the upstream gradient dout = dL/dout [batch, dim, L].

    out = (s_f + flip s_b') silu(z) / 2, so with σ = sigmoid(z):
        dL/dz  = dout (s_f + s_b) / 2 * σ (1 + z (1 - σ))           (silu' = σ (1 + z (1 - σ)))
        dL/ds  = dout silu(z) / 2 for both branches (flipped for the backward one)
    and each branch's gradients come from ``scan_1d_bwd``; the backward branch's per-position
    gradients are flipped back to original token order.  For shared inputs (``vim_bidir``) the
    two branches' du, dΔ_raw and dbias add up.
    """
    f = lambda x: np.flip(np.asarray(x, dtype=np.float64), axis=-1)
    z = np.asarray(z, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    gs = dout * silu(z) / 2.0
    fw = scan_1d_bwd(u, delta_raw, A_log, B, C, D, delta_bias, gs)
    bw = scan_1d_bwd(f(u_b), f(delta_raw_b), A_b_log, f(B_b), f(C_b), D_b, delta_bias_b, f(gs))
    sig = expit(z)
    dz = dout * (fw["s"] + f(bw["s"])) / 2.0 * sig * (1.0 + z * (1.0 - sig))
    return dict(du=fw["du"], ddelta_raw=fw["ddelta_raw"], ddelta_bias=fw["ddelta_bias"],
                du_b=f(bw["du"]), ddelta_raw_b=f(bw["ddelta_raw"]), ddelta_bias_b=bw["ddelta_bias"], dz=dz,
                dA_log=fw["dA_log"], dA_b_log=bw["dA_log"], dB=fw["dB"], dC=fw["dC"], dB_b=f(bw["dB"]),
                dC_b=f(bw["dC"]), dD=fw["dD"], dD_b=bw["dD"],
                du_abs=fw["du_abs"], ddelta_raw_abs=fw["ddelta_raw_abs"], du_b_abs=f(bw["du_abs"]),
                ddelta_raw_b_abs=f(bw["ddelta_raw_abs"]))


def ss2d_orders(x):
    """The four cross-scan sequences of [P4] §2.2 for x[batch, dim, H, W]:
    row-major flatten, column-major flatten (transpose then flatten), and each reversed."""
    x = np.asarray(x, dtype=np.float64)
    nb, nd, H, W = x.shape
    row = x.reshape(nb, nd, H * W)
    col = np.swapaxes(x, 2, 3).reshape(nb, nd, H * W)
    return [row, col, np.flip(row, axis=-1), np.flip(col, axis=-1)]


def ss2d_cross_scan(x, delta_raw, A_log, B, C, D, delta_bias, z=None):
    """VMamba SS2D cross-scan + cross-merge ([P4] §2.1, §2.2, §3.1).

    x [batch, dim, H, W]; delta_raw [batch, 4, dim, H*W] and B, C [batch, 4, N, H*W], each in
    its own direction's scan order; A_log [4, dim, N]; D, delta_bias [4, dim]; z optional
    [batch, dim, H, W].  For k = 0..3 the ungated scan of the k-th sequence is mapped back to
    row-major pixel order and the four are summed; silu(z) multiplies the sum when z is given.
    """
    x = np.asarray(x, dtype=np.float64)
    nb, nd, H, W = x.shape
    L = H * W
    seqs = ss2d_orders(x)
    ys = [scan_1d(seqs[k], np.asarray(delta_raw)[:, k], np.asarray(A_log)[k], np.asarray(B)[:, k],
                  np.asarray(C)[:, k], np.asarray(D)[k], np.asarray(delta_bias)[k]) for k in range(4)]
    # inverse maps: row order is already row-major; column order is transposed back;
    # reversed orders are flipped back first.
    col_back = lambda y: np.swapaxes(y.reshape(nb, nd, W, H), 2, 3).reshape(nb, nd, L)
    out = ys[0] + col_back(ys[1]) + np.flip(ys[2], axis=-1) + col_back(np.flip(ys[3], axis=-1))
    out = out.reshape(nb, nd, H, W)
    if z is not None:
        out = out * silu(z)
    return out


def ss2d_cross_scan_bwd(x, delta_raw, A_log, B, C, D, delta_bias, z, dout):
    """Gradients of ``ss2d_cross_scan`` for dout = dL/dout [batch, dim, H, W] (z may be None).

    out = silu(z) Σ_k back_k(y_k) with y_k the scan of the k-th ordering of x, so the gradient
    reaching direction k's outputs is the same ordering applied to dL/d(Σ) = dout silu(z) (or
    dout without a gate); ``scan_1d_bwd`` gives that direction's gradients, and its du, in
    direction k's scan order, is mapped back to pixels and summed into dx.  Per-direction
    tensors (Δ_raw, B, C) keep their scan order.  dz = dout Σ_k back_k(y_k) silu'(z).
    Returns dict(dx, ddelta_raw [batch,4,dim,L], dA_log [4,dim,N], dB, dC [batch,4,N,L],
    dD, ddelta_bias [4,dim], dz (None without z)), and dx_abs, ddelta_raw_abs (the absolute-value
    sums of ``scan_1d_bwd``, mapped and added the same way).
    """
    x = np.asarray(x, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    nb, nd, H, W = x.shape
    L = H * W
    seqs = ss2d_orders(x)
    col_back = lambda y: np.swapaxes(y.reshape(nb, nd, W, H), 2, 3).reshape(nb, nd, L)
    backs = [lambda y: y, col_back, lambda y: np.flip(y, axis=-1), lambda y: col_back(np.flip(y, axis=-1))]
    if z is not None:
        z = np.asarray(z, dtype=np.float64)
        gsum = dout * silu(z)
    else:
        gsum = dout
    gorders = ss2d_orders(gsum)       # dL/dy_k: the k-th ordering of the merged gradient
    dx = np.zeros((nb, nd, L))
    dx_abs = np.zeros((nb, nd, L))
    ysum = np.zeros((nb, nd, L))
    res = dict(ddelta_raw=np.zeros((nb, 4, nd, L)), dA_log=np.zeros(np.asarray(A_log).shape),
               dB=np.zeros((nb, 4) + np.asarray(B).shape[2:]), dC=np.zeros((nb, 4) + np.asarray(C).shape[2:]),
               dD=np.zeros(np.asarray(D).shape), ddelta_bias=np.zeros(np.asarray(delta_bias).shape),
               ddelta_raw_abs=np.zeros((nb, 4, nd, L)))
    for k in range(4):
        r = scan_1d_bwd(seqs[k], np.asarray(delta_raw)[:, k], np.asarray(A_log)[k], np.asarray(B)[:, k],
                        np.asarray(C)[:, k], np.asarray(D)[k], np.asarray(delta_bias)[k], gorders[k])
        dx += backs[k](r["du"])
        dx_abs += backs[k](r["du_abs"])
        ysum += backs[k](r["s"])
        res["ddelta_raw"][:, k] = r["ddelta_raw"]
        res["ddelta_raw_abs"][:, k] = r["ddelta_raw_abs"]
        res["dA_log"][k] = r["dA_log"]
        res["dB"][:, k] = r["dB"]
        res["dC"][:, k] = r["dC"]
        res["dD"][k] = r["dD"]
        res["ddelta_bias"][k] = r["ddelta_bias"]
    res["dx"] = dx.reshape(nb, nd, H, W)
    res["dx_abs"] = dx_abs.reshape(nb, nd, H, W)
    if z is not None:
        sig = expit(z)
        res["dz"] = dout * ysum.reshape(nb, nd, H, W) * sig * (1.0 + z * (1.0 - sig))
    else:
        res["dz"] = None
    return res


def ss2d_cross_scan_pathwalk(x, delta_raw, A_log, B, C, D, delta_bias, z=None):
    """SS2D by walking each direction's path pixel by pixel with explicit (h, w) coordinates
    (pure Python loops; tiny inputs only).  Independent of the reshape/transpose/flip code in
    ``ss2d_cross_scan``: direction 0 visits (i div W, i mod W), direction 1 visits
    (i mod H, i div H), directions 2 and 3 visit the same paths from the other end."""
    x = np.asarray(x, dtype=np.float64)
    nb, nd, H, W = x.shape
    L = H * W
    A = -np.exp(np.asarray(A_log, dtype=np.float64))
    out = np.zeros((nb, nd, H, W), dtype=np.float64)

    def pixel(k, i):
        if k == 0:
            return divmod(i, W)
        if k == 1:
            return (i % H, i // H)
        if k == 2:
            return divmod(L - 1 - i, W)
        j = L - 1 - i
        return (j % H, j // H)

    for b in range(nb):
        for d in range(nd):
            for k in range(4):
                h = np.zeros(A.shape[2])
                for i in range(L):
                    ph, pw = pixel(k, i)
                    xv = x[b, d, ph, pw]
                    dl = float(softplus(float(delta_raw[b, k, d, i]) + float(delta_bias[k, d])))
                    h = np.exp(dl * A[k, d]) * h + dl * np.asarray(B[b, k, :, i], dtype=np.float64) * xv
                    out[b, d, ph, pw] += float(np.dot(np.asarray(C[b, k, :, i], dtype=np.float64), h)) + float(D[k, d]) * xv
    if z is not None:
        out = out * silu(z)
    return out


def conv1d_silu(x, w, b, reverse=False):
    """The local mixing in front of the Vim scan: u = silu(conv1d(x) + b), depthwise over channels.

    x: [batch, dim, L]; w: [dim, K] (K = d_conv); b: [dim].  [P3] §2.1 gives each branch a
    Conv1d of kernel size d_conv over d_inner channels (v2 has its own conv1d_b) and §2.2 runs
    the backward branch on the flipped sequence.  Readings: one filter per channel (depthwise);
    causal, i.e. K - 1 zeros in front and the first L outputs kept, so
        pre[t] = b + sum_k w[k] x[t - (K - 1) + k];
    SiLU after the convolution.  ``reverse`` is the backward branch expressed in original token
    order: the same convolution applied to the flipped sequence, flipped back (anti-causal)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if reverse:
        return np.flip(conv1d_silu(np.flip(x, axis=-1), w, b), axis=-1)
    K = w.shape[1]
    L = x.shape[-1]
    padded = np.concatenate([np.zeros(x.shape[:-1] + (K - 1,)), x], axis=-1)
    pre = np.broadcast_to(b[None, :, None], x.shape).copy()
    for k in range(K):
        pre += w[None, :, k, None] * padded[..., k:k + L]
    return silu(pre)


def conv2d_silu(x, w, b, act=True):
    """The local mixing in front of SS2D: x' = silu(conv2d(x) + b), depthwise, K x K.

    x: [batch, dim, H, W]; w: [dim, K, K] (K = d_conv, odd); b: [dim].  [P4] §2.1 applies a
    depthwise conv2d when d_conv > 1 (3 in its table) before the core.  Readings: zero padding
    (K - 1) / 2 on every side so the image keeps its size, cross-correlation as in the usual
    conv layer,
        pre[i, j] = b + sum_{a, c} w[a, c] x[i - (K - 1) / 2 + a, j - (K - 1) / 2 + c];
    SiLU after it when ``act`` (the snippet on the page shows the convolution only; the module's
    activation is SiLU)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    K = w.shape[1]
    assert K % 2 == 1 and w.shape[2] == K
    p = (K - 1) // 2
    H, W = x.shape[-2:]
    padded = np.pad(x, ((0, 0), (0, 0), (p, p), (p, p)))
    pre = np.broadcast_to(b[None, :, None, None], x.shape).copy()
    for a in range(K):
        for c in range(K):
            pre += w[None, :, a, c, None, None] * padded[..., a:a + H, c:c + W]
    return silu(pre) if act else pre


def rel_err(y, r):
    """Parity error: max_i |y_i - r_i| / max(|r_i|, rms(r)).

    A plain elementwise relative error is undefined where r_i ~ 0 (silu(z) ~ 0 or C.h cancelling
    D.u), so each element is normalised by max(|r_i|, rms over the whole output)."""
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if r.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(r * r)))
    denom = np.maximum(np.abs(r), rms)
    denom = np.where(denom > 0, denom, 1.0)
    return float(np.max(np.abs(y - r) / denom))
