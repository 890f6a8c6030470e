"""Plant one plausible mistake at a time in a copy of the oracle (on the CPU) and require that
at least one pin in ``oracle_pins`` catches it.  This shows the pins constrain every step:
softplus, the decay, the input term, the readout, the skip term, the flip handling, the fusion,
the gate and the SS2D index maps."""
import types

import numpy as np
import pytest

import oracle as O
from oracle_pins import ALL_PINS


def _scan(u, delta_raw, A_log, B, C, D, bias, bug=None):
    u = np.asarray(u, dtype=np.float64)
    A = -np.exp(np.asarray(A_log, dtype=np.float64))
    if bug == "A_not_exp":
        A = np.asarray(A_log, dtype=np.float64)
    if bug == "A_sign":
        A = np.exp(np.asarray(A_log, dtype=np.float64))
    B = np.asarray(B, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    if bug == "swap_BC":
        B, C = C, B
    D = np.asarray(D, dtype=np.float64)
    x = np.asarray(delta_raw, dtype=np.float64) + np.asarray(bias, dtype=np.float64)[None, :, None]
    delta = x if bug == "no_softplus" else np.logaddexp(0.0, x)
    if bug == "exp_not_softplus":
        delta = np.exp(x)
    nb, nd, L = u.shape
    h = np.zeros((nb, nd, A.shape[1]))
    s = np.empty((nb, nd, L))
    for t in range(L):
        dt = delta[:, :, t][:, :, None]
        dprev = delta[:, :, max(t - 1, 0)][:, :, None]
        a = np.exp((dprev if bug == "decay_prev_delta" else dt) * A[None])
        if bug == "euler_A":
            a = 1.0 + dt * A[None]
        uu = u[:, :, max(t - 1, 0)] if bug == "input_prev_u" else u[:, :, t]
        b = (1.0 if bug == "no_delta_in_b" else dt) * B[:, None, :, t] * uu[:, :, None]
        if bug == "readout_before_update":
            s[:, :, t] = np.sum(h * C[:, None, :, t], axis=2) + D[None, :] * u[:, :, t]
            h = a * h + b
            continue
        h = a * h + b
        y = np.sum(h * C[:, None, :, t], axis=2)
        if bug != "drop_D":
            y = y + D[None, :] * u[:, :, t]
        s[:, :, t] = y
    return s


def _vim(u, dr, z, Al, Abl, B, C, Bb, Cb, D, Db, bias, bug=None, scan_bug=None):
    f = lambda a: np.flip(np.asarray(a, dtype=np.float64), axis=-1)
    sc = lambda *a: _scan(*a, bug=scan_bug)
    g = O.silu(z)
    yf = sc(u, dr, Al, B, C, D, bias) * g
    if bug == "bwd_uses_fwd_BC":
        rev = sc(f(u), f(dr), Abl, f(B), f(C), Db, bias)
    elif bug == "bwd_uses_fwd_A":
        rev = sc(f(u), f(dr), Al, f(Bb), f(Cb), Db, bias)
    elif bug == "bwd_BC_not_flipped":
        rev = sc(f(u), f(dr), Abl, Bb, Cb, Db, bias)
    elif bug == "bwd_delta_not_flipped":
        rev = sc(f(u), dr, Abl, f(Bb), f(Cb), Db, bias)
    elif bug == "bwd_D_is_fwd_D":
        rev = sc(f(u), f(dr), Abl, f(Bb), f(Cb), D, bias)
    else:
        rev = sc(f(u), f(dr), Abl, f(Bb), f(Cb), Db, bias)
    if bug == "gate_not_flipped":
        yb = f(rev * O.silu(z))
    else:
        yb = f(rev * O.silu(f(z)))
    if bug == "no_flip_back":
        yb = rev * O.silu(z)
    if bug == "sum_not_avg":
        return yf + yb
    if bug == "gate_silu_is_sigmoid":
        g2 = 1.0 / (1.0 + np.exp(-np.asarray(z, dtype=np.float64)))
        return 0.5 * (yf / np.where(g == 0, 1, g) * g2 + yb / np.where(g == 0, 1, g) * g2)
    return 0.5 * (yf + yb)


def _v2(u, dr, bias, ub, drb, biasb, z, Al, Abl, B, C, Bb, Cb, D, Db, bug=None, scan_bug=None):
    f = lambda a: np.flip(np.asarray(a, dtype=np.float64), axis=-1)
    sc = lambda *a: _scan(*a, bug=scan_bug)
    yf = sc(u, dr, Al, B, C, D, bias) * O.silu(z)
    if bug == "v2_bwd_uses_fwd_u":
        ub = u
    if bug == "v2_bwd_uses_fwd_delta":
        drb = dr
    if bug == "v2_bwd_uses_fwd_bias":
        biasb = bias
    if bug == "v2_fwd_uses_bwd_bias":
        yf = sc(u, dr, Al, B, C, D, biasb) * O.silu(z)
    rev_u = ub if bug == "v2_ub_not_flipped" else f(ub)
    rev = sc(rev_u, f(drb), Abl, f(Bb), f(Cb), Db, biasb)
    return 0.5 * (yf + f(rev * O.silu(f(z))))


def _scan_bwd(u, dr, Al, B, C, D, bias, g, bug=None):
    from scipy.special import expit
    u = np.asarray(u, dtype=np.float64)
    x = np.asarray(dr, dtype=np.float64) + np.asarray(bias, dtype=np.float64)[None, :, None]
    A = -np.exp(np.asarray(Al, dtype=np.float64))
    B, C, D = (np.asarray(v, dtype=np.float64) for v in (B, C, D))
    nb, nd, L = u.shape
    N = A.shape[1]
    delta = np.logaddexp(0.0, x)
    hs = np.zeros((L + 1, nb, nd, N))
    av = np.empty((L, nb, nd, N))
    s = np.empty((nb, nd, L))
    for t in range(L):
        av[t] = np.exp(delta[:, :, t][:, :, None] * A[None])
        hs[t + 1] = av[t] * hs[t] + delta[:, :, t][:, :, None] * B[:, None, :, t] * u[:, :, t][:, :, None]
        s[:, :, t] = np.sum(hs[t + 1] * C[:, None, :, t], axis=2) + D[None, :] * u[:, :, t]
    du = np.zeros_like(u) if bug == "du_no_D" else g * D[None, :, None]
    ddelta = np.zeros((nb, nd, L))
    dA = np.zeros((nd, N))
    dB = np.zeros((nb, N, L))
    dC = np.zeros((nb, N, L))
    lam = np.zeros((nb, nd, N))
    for t in range(L - 1, -1, -1):
        at = av[t] if bug == "lambda_same_step_decay" else (av[t + 1] if t + 1 < L else 0.0)
        lam = g[:, :, t][:, :, None] * C[:, None, :, t] + at * lam
        dl = delta[:, :, t][:, :, None]
        hc = hs[t] if bug == "dC_prev_state" else hs[t + 1]
        dC[:, :, t] = np.sum(g[:, :, t][:, :, None] * hc, axis=1)
        dB[:, :, t] = np.sum(lam * (1.0 if bug == "dB_no_delta" else dl) * u[:, :, t][:, :, None], axis=1)
        du[:, :, t] += delta[:, :, t] * np.sum(lam * B[:, None, :, t], axis=2)
        hp = hs[t + 1] if bug == "ddelta_next_state" else hs[t]
        ddelta[:, :, t] = np.sum(lam * (A[None] * av[t] * hp + B[:, None, :, t] * u[:, :, t][:, :, None]), axis=2)
        dA += np.sum(lam * dl * av[t] * hs[t], axis=0)
    ddr = ddelta if bug == "no_sigmoid" else ddelta * expit(x)
    return dict(s=s, du=du, ddelta_raw=ddr, ddelta_bias=ddr.sum(axis=(0, 2)),
                dA_log=dA if bug == "dA_log_no_chain" else dA * A, dB=dB, dC=dC, dD=np.sum(g * u, axis=(0, 2)))


def _v2_bwd(u, dr, bias, ub, drb, biasb, z, Al, Abl, B, C, Bb, Cb, D, Db, dout, bug=None):
    from scipy.special import expit
    f = lambda x: np.flip(np.asarray(x, dtype=np.float64), axis=-1)
    z = np.asarray(z, dtype=np.float64)
    gs = dout * O.silu(z) / 2.0
    fw = _scan_bwd(u, dr, Al, B, C, D, bias, gs, bug=bug)
    bw = _scan_bwd(f(ub), f(drb), Abl, f(Bb), f(Cb), Db, biasb, gs if bug == "bwd_g_not_flipped" else f(gs), bug=bug)
    sig = expit(z)
    dsilu = O.silu(z) if bug == "dz_silu_not_derivative" else sig * (1.0 + z * (1.0 - sig))
    dz = dout * (fw["s"] + f(bw["s"])) / 2.0 * dsilu
    back = (lambda a: a) if bug == "bwd_grads_not_flipped" else f
    return dict(du=fw["du"], ddelta_raw=fw["ddelta_raw"], ddelta_bias=fw["ddelta_bias"], du_b=back(bw["du"]),
                ddelta_raw_b=back(bw["ddelta_raw"]), ddelta_bias_b=bw["ddelta_bias"], dz=dz, dA_log=fw["dA_log"],
                dA_b_log=bw["dA_log"], dB=fw["dB"], dC=fw["dC"], dB_b=back(bw["dB"]), dC_b=back(bw["dC"]),
                dD=fw["dD"], dD_b=bw["dD"])


def _ss2d_bwd(x, dr, Al, B, C, D, bias, z, dout, bug=None):
    """A copy of the oracle's SS2D gradient with an optional planted mistake."""
    r = O.ss2d_cross_scan_bwd(x, dr, Al, B, C, D, bias, z, dout)
    if bug is None:
        return r
    x = np.asarray(x, dtype=np.float64)
    nb, nd, H, W = x.shape
    L = H * W
    seqs = O.ss2d_orders(x)
    gsum = np.asarray(dout, dtype=np.float64) * (O.silu(z) if z is not None else 1.0)
    gord = O.ss2d_orders(gsum)
    if bug == "g_not_reordered":
        gord = [gsum.reshape(nb, nd, L)] * 4
    col_back = lambda y: np.swapaxes(y.reshape(nb, nd, W, H), 2, 3).reshape(nb, nd, L)
    backs = [lambda y: y, col_back, lambda y: np.flip(y, axis=-1), lambda y: col_back(np.flip(y, axis=-1))]
    if bug == "du_not_mapped_back":
        backs = [lambda y: y] * 4
    dx = np.zeros((nb, nd, L))
    out = dict(r)
    for k in range(4):
        rk = O.scan_1d_bwd(seqs[k], np.asarray(dr)[:, k], np.asarray(Al)[k], np.asarray(B)[:, k], np.asarray(C)[:, k],
                           np.asarray(D)[k], np.asarray(bias)[k], gord[k])
        dx += backs[k](rk["du"])
    out["dx"] = dx.reshape(nb, nd, H, W)
    if bug == "dz_missing_silu_derivative" and z is not None:
        out["dz"] = np.asarray(dout) * O.ss2d_cross_scan(x, dr, Al, B, C, D, bias)  # silu'(z) factor dropped
    return out


def _ss2d(x, dr, Al, B, C, D, bias, z=None, bug=None, scan_bug=None):
    x = np.asarray(x, dtype=np.float64)
    nb, nd, H, W = x.shape
    L = H * W
    row = x.reshape(nb, nd, L)
    col = np.swapaxes(x, 2, 3).reshape(nb, nd, L)
    if bug == "col_as_reshape":
        col = x.reshape(nb, nd, W, H).reshape(nb, nd, L)
    seqs = [row, col, np.flip(row, -1), np.flip(col, -1)]
    dr = np.asarray(dr)
    ys = [_scan(seqs[k], dr[:, k], np.asarray(Al)[k], np.asarray(B)[:, k], np.asarray(C)[:, k],
                np.asarray(D)[k], np.asarray(bias)[k], bug=scan_bug) for k in range(4)]
    back = lambda y: np.swapaxes(y.reshape(nb, nd, W, H), 2, 3).reshape(nb, nd, L)
    if bug == "col_not_transposed_back":
        back = lambda y: y
    flipk = (lambda y: y) if bug == "rev_not_flipped_back" else (lambda y: np.flip(y, -1))
    out = ys[0] + back(ys[1]) + flipk(ys[2]) + back(flipk(ys[3]))
    if bug == "avg4":
        out = out / 4.0
    out = out.reshape(nb, nd, H, W)
    if z is not None:
        out = out * O.silu(z)
    return out


def _conv1d(x, w, b, reverse=False, bug=None):
    """Front conv1d + SiLU written per output element, with a planted mistake."""
    x = np.asarray(x, dtype=np.float64)
    nb, nd, L = x.shape
    K = w.shape[1]
    out = np.empty_like(x)
    for bb in range(nb):
        for d in range(nd):
            for t in range(L):
                acc = 0.0 if bug == "conv1d_no_bias" else b[d]
                for k in range(K):
                    if bug == "conv1d_drop_tap" and k == 0 and K > 1:
                        continue
                    wk = w[d, K - 1 - k] if bug == "conv1d_convolution" else w[d, k]
                    if reverse and bug != "conv1d_rev_causal":
                        src = t + (K - 1) - k
                    elif bug == "conv1d_anticausal":
                        src = t + k
                    else:
                        src = t - (K - 1) + k
                    if 0 <= src < L:
                        acc += wk * x[bb, d, src]
                out[bb, d, t] = acc if bug == "conv1d_no_silu" else acc / (1.0 + np.exp(-acc))
    return out


def _conv2d(x, w, b, act=True, bug=None):
    """Front conv2d (+ SiLU) written per output pixel, with a planted mistake."""
    x = np.asarray(x, dtype=np.float64)
    nb, nd, H, W = x.shape
    K = w.shape[1]
    p = (K - 1) // 2
    out = np.empty_like(x)
    for bb in range(nb):
        for d in range(nd):
            for i in range(H):
                for j in range(W):
                    acc = 0.0 if bug == "conv2d_no_bias" else b[d]
                    for a in range(K):
                        for c in range(K):
                            wac = {"conv2d_w_transposed": w[d, c, a],
                                   "conv2d_convolution": w[d, K - 1 - a, K - 1 - c]}.get(bug, w[d, a, c])
                            off = 0 if bug == "conv2d_pad_offset" else p
                            si, sj = i - off + a, j - off + c
                            if 0 <= si < H and 0 <= sj < W:
                                acc += wac * x[bb, d, si, sj]
                    out[bb, d, i, j] = acc / (1.0 + np.exp(-acc)) if act else acc
    return out


def _impl(scan_bug=None, vim_bug=None, ss2d_bug=None, v2_bug=None, bwd_bug=None, ss2d_bwd_bug=None, conv_bug=None):
    return types.SimpleNamespace(
        conv1d_silu=lambda x, w, b, reverse=False: _conv1d(x, w, b, reverse, bug=conv_bug),
        conv2d_silu=lambda x, w, b, act=True: _conv2d(x, w, b, act, bug=conv_bug),
        ss2d_cross_scan_bwd=lambda *a: _ss2d_bwd(*a, bug=ss2d_bwd_bug),
        vim_bidir_v2_bwd=lambda *a: _v2_bwd(*a, bug=bwd_bug),
        softplus=O.softplus,
        silu=O.silu,
        scan_1d=lambda *a: _scan(*a, bug=scan_bug),
        vim_bidir=lambda *a: _vim(*a, bug=vim_bug, scan_bug=scan_bug),
        vim_bidir_v2=lambda *a: _v2(*a, bug=v2_bug, scan_bug=scan_bug),
        ss2d_cross_scan=lambda x, dr, Al, B, C, D, bias, z=None: _ss2d(x, dr, Al, B, C, D, bias, z, bug=ss2d_bug, scan_bug=scan_bug),
    )


SCAN_BUGS = ["A_not_exp", "A_sign", "swap_BC", "no_softplus", "exp_not_softplus", "decay_prev_delta", "euler_A",
             "input_prev_u", "no_delta_in_b", "readout_before_update", "drop_D"]
VIM_BUGS = ["bwd_uses_fwd_BC", "bwd_uses_fwd_A", "bwd_BC_not_flipped", "bwd_delta_not_flipped", "bwd_D_is_fwd_D",
            "gate_not_flipped", "no_flip_back", "sum_not_avg", "gate_silu_is_sigmoid"]
SS2D_BUGS = ["col_as_reshape", "col_not_transposed_back", "rev_not_flipped_back", "avg4"]
SS2D_BWD_BUGS = ["g_not_reordered", "du_not_mapped_back", "dz_missing_silu_derivative"]
BWD_BUGS = ["du_no_D", "lambda_same_step_decay", "dC_prev_state", "dB_no_delta", "ddelta_next_state", "no_sigmoid",
            "dA_log_no_chain", "bwd_g_not_flipped", "dz_silu_not_derivative", "bwd_grads_not_flipped"]
CONV_BUGS = ["conv1d_no_bias", "conv1d_drop_tap", "conv1d_convolution", "conv1d_rev_causal", "conv1d_anticausal",
             "conv1d_no_silu", "conv2d_no_bias", "conv2d_w_transposed", "conv2d_convolution", "conv2d_pad_offset"]
V2_BUGS = ["v2_bwd_uses_fwd_u", "v2_bwd_uses_fwd_delta", "v2_bwd_uses_fwd_bias", "v2_fwd_uses_bwd_bias", "v2_ub_not_flipped"]


def _caught(impl):
    failures = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                msgs = pin(impl)
        except Exception as e:  # a crash or NaN check also counts as caught
            msgs = [f"{pin.__name__} raised {type(e).__name__}"]
        if msgs:
            failures.append(pin.__name__)
    return failures


def test_unmutated_copy_passes():
    assert _caught(_impl()) == []


@pytest.mark.parametrize("bug", SCAN_BUGS)
def test_scan_mutant_caught(bug):
    assert _caught(_impl(scan_bug=bug)), f"planted mistake {bug} passes every pin"


@pytest.mark.parametrize("bug", VIM_BUGS)
def test_vim_mutant_caught(bug):
    assert _caught(_impl(vim_bug=bug)), f"planted mistake {bug} passes every pin"


@pytest.mark.parametrize("bug", SS2D_BUGS)
def test_ss2d_mutant_caught(bug):
    assert _caught(_impl(ss2d_bug=bug)), f"planted mistake {bug} passes every pin"


@pytest.mark.parametrize("bug", V2_BUGS)
def test_v2_mutant_caught(bug):
    assert _caught(_impl(v2_bug=bug)), f"planted mistake {bug} passes every pin"


@pytest.mark.parametrize("bug", BWD_BUGS)
def test_bwd_mutant_caught(bug):
    assert _caught(_impl(bwd_bug=bug)), f"planted mistake {bug} passes every pin"


@pytest.mark.parametrize("bug", SS2D_BWD_BUGS)
def test_ss2d_bwd_mutant_caught(bug):
    assert _caught(_impl(ss2d_bwd_bug=bug)), f"planted mistake {bug} passes every pin"


@pytest.mark.parametrize("bug", CONV_BUGS)
def test_conv_mutant_caught(bug):
    assert _caught(_impl(conv_bug=bug)), f"planted mistake {bug} passes every pin"

