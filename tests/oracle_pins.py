"""Pins for the fp64 oracle: each ``pin_*`` takes an implementation namespace (with
``scan_1d``, ``vim_bidir``, ``vim_bidir_v2``, ``vim_bidir_v2_bwd``, ``ss2d_cross_scan``,
``ss2d_cross_scan_bwd``, ``conv1d_silu``, ``conv2d_silu``) and returns the list of failure messages
(empty = pass).  They check the oracle against facts fixed by the mathematics, not against the
oracle itself: hand-derived closed forms, brute force on tiny inputs, linearity, the flip
identity, limits and the SS2D reductions.  ``test_oracle_pins`` runs them on the oracle;
``test_oracle_mutants`` runs them on copies of the oracle with a planted mistake and requires
that every mistake is caught by at least one pin."""
import math
import os

import numpy as np

import oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rich_vim(rng, nb=2, nd=3, L=7, N=4, bias_lo=-2.0, bias_hi=0.5):
    """Random small inputs with non-trivial A, A_b, D, D_b (so swapped or dropped parameters show)."""
    r = rng
    return dict(
        u=r.standard_normal((nb, nd, L)),
        delta_raw=r.standard_normal((nb, nd, L)),
        z=r.standard_normal((nb, nd, L)),
        A_log=r.uniform(-1.0, 1.5, (nd, N)),
        A_b_log=r.uniform(-1.0, 1.5, (nd, N)),
        B=r.standard_normal((nb, N, L)),
        C=r.standard_normal((nb, N, L)),
        B_b=r.standard_normal((nb, N, L)),
        C_b=r.standard_normal((nb, N, L)),
        D=r.uniform(0.5, 1.5, nd),
        D_b=r.uniform(-1.5, -0.5, nd),
        delta_bias=r.uniform(bias_lo, bias_hi, nd),
    )


def rich_ss2d(rng, nb=2, nd=2, H=3, W=4, N=3):
    r = rng
    L = H * W
    return dict(
        x=r.standard_normal((nb, nd, H, W)),
        delta_raw=r.standard_normal((nb, 4, nd, L)),
        A_log=r.uniform(-1.0, 1.5, (4, nd, N)),
        B=r.standard_normal((nb, 4, N, L)),
        C=r.standard_normal((nb, 4, N, L)),
        D=r.uniform(-1.5, 1.5, (4, nd)),
        delta_bias=r.uniform(-2.0, 0.5, (4, nd)),
    )


def _vim(impl, p, **over):
    q = dict(p)
    q.update(over)
    return impl.vim_bidir(q["u"], q["delta_raw"], q["z"], q["A_log"], q["A_b_log"], q["B"], q["C"],
                          q["B_b"], q["C_b"], q["D"], q["D_b"], q["delta_bias"])


def _ss2d(impl, p, **over):
    q = dict(p)
    q.update(over)
    return impl.ss2d_cross_scan(q["x"], q["delta_raw"], q["A_log"], q["B"], q["C"], q["D"], q["delta_bias"], q.get("z"))


def _check(msgs, name, err, tol):
    if not (err <= tol):
        msgs.append(f"{name}: err {err:.3e} > {tol:.1e}")


def pin_softplus_silu(impl):
    """softplus and silu against math.log1p/math.exp evaluated one value at a time."""
    msgs = []
    xs = [-40.0, -20.0, -6.9, -3.0, -1e-3, 0.0, 1e-3, 0.7, 3.0, 19.0, 25.0, 60.0]
    for x in xs:
        ref = x + math.log1p(math.exp(-x)) if x > 0 else math.log1p(math.exp(x))
        _check(msgs, f"softplus({x})", abs(float(impl.softplus(x)) - ref) / max(abs(ref), 1e-300), 1e-14)
        sref = x / (1.0 + math.exp(-x)) if x > -700 else 0.0
        _check(msgs, f"silu({x})", abs(float(impl.silu(x)) - sref) / max(abs(sref), 1e-300), 1e-14)
    return msgs


def pin_golden_single_token(impl):
    """Hand-derived L = 1 cases stored in tests/golden/closed_forms.txt."""
    msgs = []
    env = {"log": math.log, "exp": math.exp, "log1p": math.log1p}
    with open(os.path.join(GOLDEN, "closed_forms.txt")) as f:
        for ln in f:
            ln = ln.strip()
            if not ln or ln.startswith("#"):
                continue
            lhs, rhs = ln.split("|")
            v = [float(t) for t in lhs.split()]
            u, dr, bias, B0, B1, C0, C1, D, Bb0, Bb1, Cb0, Cb1, Db, z = v
            expect = eval(rhs, {"__builtins__": {}}, env)
            a = lambda x: np.array(x, dtype=np.float64)
            got = impl.vim_bidir(a([[[u]]]), a([[[dr]]]), a([[[z]]]), a([[0.3, 0.9]]), a([[-0.2, 0.1]]),
                                 a([[[B0], [B1]]]), a([[[C0], [C1]]]), a([[[Bb0], [Bb1]]]), a([[[Cb0], [Cb1]]]),
                                 a([D]), a([Db]), a([bias]))
            err = abs(float(got[0, 0, 0]) - expect) / max(abs(expect), 1.0)
            _check(msgs, f"golden[{ln[:30]}...]", err, 1e-13)
    return msgs


def pin_single_token_closed_form(impl, seed=0):
    """L = 1: s_0 = u (Δ Σ_n B_n C_n + D) for each direction; both directions see the one token."""
    msgs = []
    rng = np.random.default_rng(seed)
    p = rich_vim(rng, nb=3, nd=4, L=1, N=5)
    dl = np.logaddexp(0.0, p["delta_raw"][:, :, 0] + p["delta_bias"][None, :])
    bc_f = np.einsum("bn,bn->b", p["B"][:, :, 0], p["C"][:, :, 0])[:, None]
    bc_b = np.einsum("bn,bn->b", p["B_b"][:, :, 0], p["C_b"][:, :, 0])[:, None]
    u = p["u"][:, :, 0]
    zz = p["z"][:, :, 0]
    g = zz / (1.0 + np.exp(-zz))
    expect = 0.5 * (u * (dl * bc_f + p["D"][None]) + u * (dl * bc_b + p["D_b"][None])) * g
    _check(msgs, "L=1 closed form", O.rel_err(_vim(impl, p)[:, :, 0], expect), 1e-13)
    return msgs


def pin_geometric_series(impl):
    """Constant Δ=δ, B=β, C=γ, u=υ, z over t: with a_n = exp(δ A_n) the forward state is
    h_t,n = δ β_n υ (1 - a_n^{t+1}) / (1 - a_n) and the backward state at original position t has
    absorbed L - t tokens: h^b_t,n = δ β^b_n υ (1 - (a^b_n)^{L-t}) / (1 - a^b_n)."""
    msgs = []
    rng = np.random.default_rng(1)
    nb, nd, L, N = 1, 3, 23, 4
    p = rich_vim(rng, nb=nb, nd=nd, L=L, N=N)
    dr = rng.standard_normal(nd)
    ups = rng.standard_normal(nd)
    zc = rng.standard_normal(nd)
    beta, gamma = rng.standard_normal(N), rng.standard_normal(N)
    beta_b, gamma_b = rng.standard_normal(N), rng.standard_normal(N)
    p["u"] = np.broadcast_to(ups[None, :, None], (nb, nd, L)).copy()
    p["delta_raw"] = np.broadcast_to(dr[None, :, None], (nb, nd, L)).copy()
    p["z"] = np.broadcast_to(zc[None, :, None], (nb, nd, L)).copy()
    p["B"] = np.broadcast_to(beta[None, :, None], (nb, N, L)).copy()
    p["C"] = np.broadcast_to(gamma[None, :, None], (nb, N, L)).copy()
    p["B_b"] = np.broadcast_to(beta_b[None, :, None], (nb, N, L)).copy()
    p["C_b"] = np.broadcast_to(gamma_b[None, :, None], (nb, N, L)).copy()
    delta = np.logaddexp(0.0, dr + p["delta_bias"])            # [nd]
    A = -np.exp(p["A_log"])
    Ab = -np.exp(p["A_b_log"])
    t = np.arange(L)
    expect = np.empty((nd, L))
    for d in range(nd):
        a = np.exp(delta[d] * A[d])
        ab = np.exp(delta[d] * Ab[d])
        hf = delta[d] * beta[None, :] * ups[d] * (1 - a[None, :] ** (t[:, None] + 1)) / (1 - a[None, :])
        hb = delta[d] * beta_b[None, :] * ups[d] * (1 - ab[None, :] ** (L - t[:, None])) / (1 - ab[None, :])
        sf = hf @ gamma + p["D"][d] * ups[d]
        sb = hb @ gamma_b + p["D_b"][d] * ups[d]
        expect[d] = 0.5 * (sf + sb) * zc[d] / (1 + np.exp(-zc[d]))
    _check(msgs, "geometric series", O.rel_err(_vim(impl, p)[0], expect), 1e-12)
    return msgs


def pin_semiseparable(impl):
    """Brute force: out = silu(z) * ((M_f + diag D) u + (M_b + diag D_b) u) / 2 with the L x L
    matrices built from exponentials of partial sums of Δ (oracle.scan_1d_semiseparable)."""
    msgs = []
    rng = np.random.default_rng(2)
    for L in (1, 2, 5, 12):
        p = rich_vim(rng, nb=2, nd=2, L=L, N=3)
        sf = O.scan_1d_semiseparable(p["u"], p["delta_raw"], p["A_log"], p["B"], p["C"], p["D"], p["delta_bias"])
        sb = O.scan_1d_semiseparable(p["u"], p["delta_raw"], p["A_b_log"], p["B_b"], p["C_b"], p["D_b"], p["delta_bias"], reverse=True)
        g = p["z"] / (1 + np.exp(-p["z"]))
        expect = 0.5 * (sf + sb) * g
        _check(msgs, f"semiseparable L={L}", O.rel_err(_vim(impl, p), expect), 1e-12)
        # the forward direction alone through scan_1d
        s1 = impl.scan_1d(p["u"], p["delta_raw"], p["A_log"], p["B"], p["C"], p["D"], p["delta_bias"])
        _check(msgs, f"semiseparable scan_1d L={L}", O.rel_err(s1, sf), 1e-12)
    return msgs


def pin_semiseparable_closed(impl):
    """The brute-force matrices themselves, at L = 1 and for constant inputs (geometric sums)."""
    msgs = []
    rng = np.random.default_rng(3)
    p = rich_vim(rng, nb=1, nd=2, L=6, N=3)
    for k in ("u", "delta_raw"):
        p[k] = np.broadcast_to(p[k][:, :, :1], p[k].shape).copy()
    for k in ("B", "C"):
        p[k] = np.broadcast_to(p[k][:, :, :1], p[k].shape).copy()
    sf = O.scan_1d_semiseparable(p["u"], p["delta_raw"], p["A_log"], p["B"], p["C"], p["D"], p["delta_bias"])
    sb = O.scan_1d_semiseparable(p["u"], p["delta_raw"], p["A_log"], p["B"], p["C"], p["D"], p["delta_bias"], reverse=True)
    L = 6
    t = np.arange(L)
    for d in range(2):
        dl = float(np.logaddexp(0.0, p["delta_raw"][0, d, 0] + p["delta_bias"][d]))
        a = np.exp(dl * -np.exp(p["A_log"][d]))
        bc = p["B"][0, :, 0] * p["C"][0, :, 0]
        uu = p["u"][0, d, 0]
        ef = ((dl * uu * (1 - a[None] ** (t[:, None] + 1)) / (1 - a[None])) @ bc) + p["D"][d] * uu
        eb = ((dl * uu * (1 - a[None] ** (L - t[:, None])) / (1 - a[None])) @ bc) + p["D"][d] * uu
        _check(msgs, "semiseparable fwd closed", O.rel_err(sf[0, d], ef), 1e-12)
        _check(msgs, "semiseparable bwd closed", O.rel_err(sb[0, d], eb), 1e-12)
    return msgs


def pin_linearity(impl):
    """out is linear in u for fixed Δ_raw, B, C, z."""
    msgs = []
    rng = np.random.default_rng(4)
    p = rich_vim(rng, nb=2, nd=3, L=9, N=4)
    u2 = rng.standard_normal(p["u"].shape)
    al, be = 0.7, -1.3
    lhs = _vim(impl, p, u=al * p["u"] + be * u2)
    rhs = al * _vim(impl, p) + be * _vim(impl, p, u=u2)
    _check(msgs, "linearity in u", O.rel_err(lhs, rhs), 1e-12)
    return msgs


def pin_flip_identity(impl):
    """Running the bidirectional scan on reversed inputs with the forward and backward parameter
    sets exchanged gives the reversed output ([P3] §2.2: the backward scan is the forward scan of
    the reversed sequence)."""
    msgs = []
    rng = np.random.default_rng(5)
    p = rich_vim(rng, nb=2, nd=3, L=11, N=4)
    f = lambda a: np.flip(a, axis=-1)
    lhs = _vim(impl, p, u=f(p["u"]), delta_raw=f(p["delta_raw"]), z=f(p["z"]), A_log=p["A_b_log"], A_b_log=p["A_log"],
               B=f(p["B_b"]), C=f(p["C_b"]), B_b=f(p["B"]), C_b=f(p["C"]), D=p["D_b"], D_b=p["D"])
    _check(msgs, "flip identity", O.rel_err(lhs, f(_vim(impl, p))), 1e-12)
    return msgs


def pin_limits(impl):
    """Δ -> 0 (bias -40): out -> (D + D_b) u silu(z) / 2.  Δ|A| large (bias +30, A_n <= -1):
    memoryless, s_t = u_t (Δ_t Σ_n B C + D).  z = 0: out = 0."""
    msgs = []
    rng = np.random.default_rng(6)
    p = rich_vim(rng, nb=2, nd=3, L=8, N=4)
    g = p["z"] / (1 + np.exp(-p["z"]))
    small = _vim(impl, p, delta_bias=np.full(3, -40.0))
    expect = 0.5 * (p["D"][None, :, None] + p["D_b"][None, :, None]) * p["u"] * g
    _check(msgs, "delta->0", O.rel_err(small, expect), 1e-12)
    q = dict(p)
    q["A_log"] = np.abs(p["A_log"])
    q["A_b_log"] = np.abs(p["A_b_log"])
    q["delta_raw"] = 0.1 * p["delta_raw"]
    big = _vim(impl, q, delta_bias=np.full(3, 30.0))
    dl = np.logaddexp(0.0, q["delta_raw"] + 30.0)
    bcf = np.einsum("bnt,bnt->bt", q["B"], q["C"])[:, None, :]
    bcb = np.einsum("bnt,bnt->bt", q["B_b"], q["C_b"])[:, None, :]
    expect = 0.5 * (q["u"] * (dl * bcf + q["D"][None, :, None]) + q["u"] * (dl * bcb + q["D_b"][None, :, None])) * g
    _check(msgs, "memoryless", O.rel_err(big, expect), 1e-9)
    zero = _vim(impl, p, z=np.zeros_like(p["z"]))
    if np.max(np.abs(zero)) != 0.0:
        msgs.append("z=0 does not give 0")
    return msgs


def pin_ss2d_pathwalk(impl):
    """SS2D against the pixel-by-pixel path walk (explicit coordinates, no reshape/flip)."""
    msgs = []
    rng = np.random.default_rng(7)
    for (H, W) in ((1, 1), (2, 3), (3, 2), (4, 4)):
        p = rich_ss2d(rng, nb=2, nd=2, H=H, W=W, N=3)
        walk = O.ss2d_cross_scan_pathwalk(p["x"], p["delta_raw"], p["A_log"], p["B"], p["C"], p["D"], p["delta_bias"])
        _check(msgs, f"ss2d pathwalk {H}x{W}", O.rel_err(_ss2d(impl, p), walk), 1e-12)
    p = rich_ss2d(rng, nb=1, nd=2, H=3, W=2, N=3)
    z = rng.standard_normal(p["x"].shape)
    walk = O.ss2d_cross_scan_pathwalk(p["x"], p["delta_raw"], p["A_log"], p["B"], p["C"], p["D"], p["delta_bias"], z)
    _check(msgs, "ss2d pathwalk gated", O.rel_err(_ss2d(impl, p, z=z), walk), 1e-12)
    return msgs


def pin_ss2d_single_pixel(impl):
    """H = W = 1: out = x Σ_k (Δ_k Σ_n B_k,n C_k,n + D_k)."""
    msgs = []
    rng = np.random.default_rng(8)
    p = rich_ss2d(rng, nb=3, nd=2, H=1, W=1, N=4)
    dl = np.logaddexp(0.0, p["delta_raw"][:, :, :, 0] + p["delta_bias"][None])      # [nb, 4, nd]
    bc = np.einsum("bkn,bkn->bk", p["B"][..., 0], p["C"][..., 0])                 # [nb, 4]
    expect = p["x"][:, :, 0, 0] * np.sum(dl * bc[:, :, None] + p["D"][None], axis=1)
    _check(msgs, "ss2d 1x1", O.rel_err(_ss2d(impl, p)[:, :, 0, 0], expect), 1e-13)
    return msgs


def pin_ss2d_one_row(impl):
    """H = 1: column order equals row order, so with direction 1 = direction 0 and direction 3 =
    direction 2, and direction 2 set up as the Vim backward branch (its scan-order Δ_raw = flip Δ_raw,
    B = flip B_b, C = flip C_b), SS2D = 2 (s_f + s_b) = 4 vim_bidir / silu(z) (ungated Vim sum)."""
    msgs = []
    rng = np.random.default_rng(9)
    W = 9
    p = rich_vim(rng, nb=2, nd=3, L=W, N=4)
    p["z"] = np.full(p["z"].shape, 3.0)
    f = lambda a: np.flip(a, axis=-1)
    vim = _vim(impl, p)
    g = 3.0 / (1 + math.exp(-3.0))
    q = dict(
        x=p["u"][:, :, None, :],
        delta_raw=np.stack([p["delta_raw"], p["delta_raw"], f(p["delta_raw"]), f(p["delta_raw"])], axis=1),
        A_log=np.stack([p["A_log"], p["A_log"], p["A_b_log"], p["A_b_log"]]),
        B=np.stack([p["B"], p["B"], f(p["B_b"]), f(p["B_b"])], axis=1),
        C=np.stack([p["C"], p["C"], f(p["C_b"]), f(p["C_b"])], axis=1),
        D=np.stack([p["D"], p["D"], p["D_b"], p["D_b"]]),
        delta_bias=np.stack([p["delta_bias"]] * 4),
    )
    _check(msgs, "ss2d one row = 2 x bidir", O.rel_err(_ss2d(impl, q)[:, :, 0, :], 4.0 * vim / g), 1e-12)
    return msgs


def pin_ss2d_transpose(impl):
    """ss2d(x^T, directions 0<->1 and 2<->3 exchanged) = ss2d(x)^T."""
    msgs = []
    rng = np.random.default_rng(10)
    p = rich_ss2d(rng, nb=2, nd=2, H=3, W=5, N=3)
    perm = [1, 0, 3, 2]
    q = dict(x=np.swapaxes(p["x"], 2, 3), delta_raw=p["delta_raw"][:, perm], A_log=p["A_log"][perm],
             B=p["B"][:, perm], C=p["C"][:, perm], D=p["D"][perm], delta_bias=p["delta_bias"][perm])
    _check(msgs, "ss2d transpose", O.rel_err(_ss2d(impl, q), np.swapaxes(_ss2d(impl, p), 2, 3)), 1e-12)
    return msgs


def rich_v2(rng, nb=2, nd=3, L=7, N=4):
    """rich_vim plus a backward branch with its own u_b, Δ_raw_b and bias_b."""
    p = rich_vim(rng, nb=nb, nd=nd, L=L, N=N)
    p["u_b"] = rng.standard_normal((nb, nd, L))
    p["delta_raw_b"] = rng.standard_normal((nb, nd, L))
    p["delta_bias_b"] = rng.uniform(-2.5, 0.0, nd)
    return p


def _v2(impl, p, **over):
    q = dict(p)
    q.update(over)
    return impl.vim_bidir_v2(q["u"], q["delta_raw"], q["delta_bias"], q["u_b"], q["delta_raw_b"], q["delta_bias_b"],
                             q["z"], q["A_log"], q["A_b_log"], q["B"], q["C"], q["B_b"], q["C_b"], q["D"], q["D_b"])


def pin_v2_single_token(impl):
    """L = 1 with a separate backward branch: out = silu(z) (u (Δ Σ B C + D) + u_b (Δ_b Σ B_b C_b + D_b)) / 2
    with Δ = softplus(Δ_raw + bias) and Δ_b = softplus(Δ_raw_b + bias_b)."""
    msgs = []
    rng = np.random.default_rng(11)
    p = rich_v2(rng, nb=3, nd=4, L=1, N=5)
    dl = np.logaddexp(0.0, p["delta_raw"][:, :, 0] + p["delta_bias"][None, :])
    dlb = np.logaddexp(0.0, p["delta_raw_b"][:, :, 0] + p["delta_bias_b"][None, :])
    bc_f = np.einsum("bn,bn->b", p["B"][:, :, 0], p["C"][:, :, 0])[:, None]
    bc_b = np.einsum("bn,bn->b", p["B_b"][:, :, 0], p["C_b"][:, :, 0])[:, None]
    zz = p["z"][:, :, 0]
    g = zz / (1.0 + np.exp(-zz))
    expect = 0.5 * (p["u"][:, :, 0] * (dl * bc_f + p["D"][None]) + p["u_b"][:, :, 0] * (dlb * bc_b + p["D_b"][None])) * g
    _check(msgs, "v2 L=1 closed form", O.rel_err(_v2(impl, p)[:, :, 0], expect), 1e-13)
    return msgs


def pin_v2_semiseparable(impl):
    """Brute force with a separate backward branch: out = silu(z) ((M_f + diag D) u + (M_b + diag D_b) u_b) / 2,
    M_b built from Δ_b = softplus(Δ_raw_b + bias_b)."""
    msgs = []
    rng = np.random.default_rng(12)
    for L in (1, 3, 8):
        p = rich_v2(rng, nb=2, nd=2, L=L, N=3)
        sf = O.scan_1d_semiseparable(p["u"], p["delta_raw"], p["A_log"], p["B"], p["C"], p["D"], p["delta_bias"])
        sb = O.scan_1d_semiseparable(p["u_b"], p["delta_raw_b"], p["A_b_log"], p["B_b"], p["C_b"], p["D_b"],
                                     p["delta_bias_b"], reverse=True)
        expect = 0.5 * (sf + sb) * (p["z"] / (1 + np.exp(-p["z"])))
        _check(msgs, f"v2 semiseparable L={L}", O.rel_err(_v2(impl, p), expect), 1e-12)
    return msgs


def pin_v2_flip_identity(impl):
    """Exchanging the two branches (all of their inputs) and reversing every sequence reverses the output."""
    msgs = []
    rng = np.random.default_rng(13)
    p = rich_v2(rng, nb=2, nd=3, L=10, N=4)
    f = lambda a: np.flip(a, axis=-1)
    lhs = _v2(impl, p, u=f(p["u_b"]), delta_raw=f(p["delta_raw_b"]), delta_bias=p["delta_bias_b"],
              u_b=f(p["u"]), delta_raw_b=f(p["delta_raw"]), delta_bias_b=p["delta_bias"], z=f(p["z"]),
              A_log=p["A_b_log"], A_b_log=p["A_log"], B=f(p["B_b"]), C=f(p["C_b"]), B_b=f(p["B"]), C_b=f(p["C"]),
              D=p["D_b"], D_b=p["D"])
    _check(msgs, "v2 flip identity", O.rel_err(lhs, f(_v2(impl, p))), 1e-12)
    return msgs


V2_NAMES = ("u", "delta_raw", "delta_bias", "u_b", "delta_raw_b", "delta_bias_b", "z", "A_log", "A_b_log", "B", "C",
            "B_b", "C_b", "D", "D_b")
V2_GRADS = dict(u="du", delta_raw="ddelta_raw", delta_bias="ddelta_bias", u_b="du_b", delta_raw_b="ddelta_raw_b",
                delta_bias_b="ddelta_bias_b", z="dz", A_log="dA_log", A_b_log="dA_b_log", B="dB", C="dC", B_b="dB_b",
                C_b="dC_b", D="dD", D_b="dD_b")


def pin_bwd_finite_differences(impl):
    """Every gradient of the bidirectional scan (separate backward branch) against central finite
    differences of the forward, element by element, on a tiny input: the numerical gradient check
    the pages run on the bidirectional scan ([P5] §4).  With step 1e-6 in fp64 the difference
    quotient is accurate to about 1e-9 relative; a wrong index, sign, factor or a dropped term in
    any gradient shows up at the 1e-2 level or above."""
    msgs = []
    rng = np.random.default_rng(14)
    p = rich_v2(rng, nb=2, nd=2, L=5, N=3)
    dout = rng.standard_normal(p["u"].shape)
    loss = lambda q: float(np.sum(O.vim_bidir_v2(*[q[k] for k in V2_NAMES]) * dout))
    grads = impl.vim_bidir_v2_bwd(*[p[k] for k in V2_NAMES], dout)
    eps = 1e-6
    for k in V2_NAMES:
        x = np.asarray(p[k], dtype=np.float64)
        fd = np.zeros_like(x)
        for i in np.ndindex(x.shape):
            q = dict(p)
            xp = x.copy()
            xp[i] += eps
            q[k] = xp
            lp = loss(q)
            xm = x.copy()
            xm[i] -= eps
            q[k] = xm
            fd[i] = (lp - loss(q)) / (2 * eps)
        got = np.asarray(grads[V2_GRADS[k]], dtype=np.float64)
        if got.shape != fd.shape:
            msgs.append(f"d{k}: shape {got.shape} != {fd.shape}")
            continue
        _check(msgs, f"d{k} vs finite differences", float(np.max(np.abs(got - fd)) / max(np.max(np.abs(fd)), 1e-12)), 1e-6)
    return msgs


def pin_bwd_shared_inputs(impl):
    """With the backward branch's u, Δ_raw, bias equal to the forward branch's, the gradient of the
    shared-input scan is the sum of the two branches' gradients (finite differences of vim_bidir)."""
    msgs = []
    rng = np.random.default_rng(15)
    p = rich_vim(rng, nb=1, nd=2, L=4, N=3)
    dout = rng.standard_normal(p["u"].shape)
    g = impl.vim_bidir_v2_bwd(p["u"], p["delta_raw"], p["delta_bias"], p["u"], p["delta_raw"], p["delta_bias"], p["z"],
                              p["A_log"], p["A_b_log"], p["B"], p["C"], p["B_b"], p["C_b"], p["D"], p["D_b"], dout)
    loss = lambda q: float(np.sum(O.vim_bidir(q["u"], q["delta_raw"], q["z"], q["A_log"], q["A_b_log"], q["B"], q["C"],
                                              q["B_b"], q["C_b"], q["D"], q["D_b"], q["delta_bias"]) * dout))
    eps = 1e-6
    for k, gk in (("u", g["du"] + g["du_b"]), ("delta_raw", g["ddelta_raw"] + g["ddelta_raw_b"]),
                  ("delta_bias", g["ddelta_bias"] + g["ddelta_bias_b"])):
        x = np.asarray(p[k], dtype=np.float64)
        fd = np.zeros_like(x)
        for i in np.ndindex(x.shape):
            q = dict(p)
            xp = x.copy()
            xp[i] += eps
            q[k] = xp
            lp = loss(q)
            xm = x.copy()
            xm[i] -= eps
            q[k] = xm
            fd[i] = (lp - loss(q)) / (2 * eps)
        _check(msgs, f"shared d{k}", float(np.max(np.abs(gk - fd)) / max(np.max(np.abs(fd)), 1e-12)), 1e-6)
    return msgs


SS2D_NAMES = ("x", "delta_raw", "A_log", "B", "C", "D", "delta_bias")
SS2D_GRADS = dict(x="dx", delta_raw="ddelta_raw", A_log="dA_log", B="dB", C="dC", D="dD", delta_bias="ddelta_bias",
                  z="dz")


def pin_ss2d_bwd_finite_differences(impl):
    """Every SS2D gradient, with and without the gate, against central finite differences of the
    forward on a tiny non-square image (so the row and column orders differ)."""
    msgs = []
    rng = np.random.default_rng(16)
    for gated in (False, True):
        p = rich_ss2d(rng, nb=1, nd=2, H=2, W=3, N=2)
        p["z"] = rng.standard_normal(p["x"].shape) if gated else None
        dout = rng.standard_normal(p["x"].shape)
        names = SS2D_NAMES + (("z",) if gated else ())
        loss = lambda q: float(np.sum(O.ss2d_cross_scan(*[q[k] for k in SS2D_NAMES], q["z"]) * dout))
        grads = impl.ss2d_cross_scan_bwd(*[p[k] for k in SS2D_NAMES], p["z"], dout)
        if not gated and grads["dz"] is not None:
            msgs.append("ungated dz is not None")
        eps = 1e-6
        for k in names:
            x = np.asarray(p[k], dtype=np.float64)
            fd = np.zeros_like(x)
            for i in np.ndindex(x.shape):
                q = dict(p)
                xp = x.copy()
                xp[i] += eps
                q[k] = xp
                lp = loss(q)
                xm = x.copy()
                xm[i] -= eps
                q[k] = xm
                fd[i] = (lp - loss(q)) / (2 * eps)
            got = np.asarray(grads[SS2D_GRADS[k]], dtype=np.float64)
            if got.shape != fd.shape:
                msgs.append(f"ss2d d{k}: shape {got.shape} != {fd.shape}")
                continue
            err = float(np.max(np.abs(got - fd)) / max(np.max(np.abs(fd)), 1e-12))
            _check(msgs, f"ss2d d{k} vs finite differences (gated={gated})", err, 1e-6)
    return msgs


def _conv1d_impulse_pre(K, w, b, L, j, reverse):
    """Pre-activation of the depthwise conv1d for a unit impulse at position j, written from the
    tap arithmetic: causally the impulse reaches t = j .. j + K - 1 with weight w[K - 1 - (t - j)];
    the reversed branch mirrors that to t = j - K + 1 .. j with weight w[K - 1 - (j - t)]."""
    pre = np.full(L, b)
    for t in range(L):
        lag = (j - t) if reverse else (t - j)
        if 0 <= lag <= K - 1:
            pre[t] += w[K - 1 - lag]
    return pre


def pin_conv1d_impulse(impl):
    """Unit impulses through the front convolution, both branches, every width 1-4, and a
    random input as the superposition of its impulses (the pre-activation is affine)."""
    msgs = []
    rng = np.random.default_rng(11)
    L = 9
    for K in (1, 2, 3, 4):
        nd = 3
        w = rng.standard_normal((nd, K))
        b = rng.standard_normal(nd)
        for reverse in (False, True):
            for j in (0, 4, L - 1):
                x = np.zeros((1, nd, L))
                x[0, :, j] = 1.0
                got = np.asarray(impl.conv1d_silu(x, w, b, reverse), dtype=np.float64)
                exp = np.stack([O.silu(_conv1d_impulse_pre(K, w[d], b[d], L, j, reverse)) for d in range(nd)])
                _check(msgs, f"conv1d impulse K={K} rev={reverse} j={j}", O.rel_err(got[0], exp), 1e-14)
            x = rng.standard_normal((2, nd, L))
            pre = np.zeros((2, nd, L))
            for bb in range(2):
                for d in range(nd):
                    pre[bb, d] = b[d] + sum(x[bb, d, j] * (_conv1d_impulse_pre(K, w[d], b[d], L, j, reverse) - b[d])
                                            for j in range(L))
            got = np.asarray(impl.conv1d_silu(x, w, b, reverse), dtype=np.float64)
            _check(msgs, f"conv1d superposition K={K} rev={reverse}", O.rel_err(got, O.silu(pre)), 1e-13)
    return msgs


def pin_conv1d_numpy(impl):
    """The causal branch against numpy's full convolution with the kernel reversed (numpy
    convolves; the layer correlates), truncated to the first L outputs."""
    msgs = []
    rng = np.random.default_rng(12)
    x = rng.standard_normal((2, 3, 13))
    w = rng.standard_normal((3, 4))
    b = rng.standard_normal(3)
    exp = np.empty_like(x)
    for bb in range(2):
        for d in range(3):
            exp[bb, d] = O.silu(b[d] + np.convolve(x[bb, d], w[d][::-1])[:13])
    _check(msgs, "conv1d vs np.convolve", O.rel_err(impl.conv1d_silu(x, w, b, False), exp), 1e-13)
    return msgs


def pin_conv2d_scipy(impl):
    """The SS2D front against scipy's 2-D correlation with zero fill and 'same' output size,
    with and without the activation."""
    from scipy.signal import correlate2d
    msgs = []
    rng = np.random.default_rng(13)
    x = rng.standard_normal((2, 3, 5, 7))
    w = rng.standard_normal((3, 3, 3))
    b = rng.standard_normal(3)
    pre = np.empty_like(x)
    for bb in range(2):
        for d in range(3):
            pre[bb, d] = b[d] + correlate2d(x[bb, d], w[d], mode="same", boundary="fill")
    _check(msgs, "conv2d vs correlate2d", O.rel_err(impl.conv2d_silu(x, w, b, True), O.silu(pre)), 1e-13)
    _check(msgs, "conv2d no act vs correlate2d", O.rel_err(impl.conv2d_silu(x, w, b, False), pre), 1e-13)
    return msgs


def pin_conv2d_impulse(impl):
    """A unit impulse at (i0, j0) reaches (i, j) with weight w[i0 - i + 1, j0 - j + 1] (3 x 3
    correlation, one pixel of zero padding), including at the image corners."""
    msgs = []
    rng = np.random.default_rng(14)
    H, W = 4, 5
    w = rng.standard_normal((2, 3, 3))
    b = rng.standard_normal(2)
    for i0, j0 in ((0, 0), (2, 3), (H - 1, W - 1), (0, W - 1)):
        x = np.zeros((1, 2, H, W))
        x[0, :, i0, j0] = 1.0
        exp = np.empty((2, H, W))
        for d in range(2):
            for i in range(H):
                for j in range(W):
                    a, c = i0 - i + 1, j0 - j + 1
                    exp[d, i, j] = b[d] + (w[d, a, c] if 0 <= a < 3 and 0 <= c < 3 else 0.0)
        _check(msgs, f"conv2d impulse ({i0},{j0})", O.rel_err(impl.conv2d_silu(x, w, b, False)[0], exp), 1e-14)
        _check(msgs, f"conv2d impulse act ({i0},{j0})", O.rel_err(impl.conv2d_silu(x, w, b, True)[0], O.silu(exp)),
               1e-14)
    return msgs


def pin_bwd_abs_sums(impl):
    """The absolute-value sums that scale the parity bound of du, dΔ_raw and dx: each bounds its
    gradient (triangle inequality), and with a single term (one state, D = 0; for dΔ_raw also
    u = 0, which removes the input term) it equals the gradient's magnitude.  These sums are a
    diagnostic of the oracle; a copy that does not produce them (the planted-mistake copies of
    the gradients) is not checked here."""
    msgs = []
    rng = np.random.default_rng(15)
    p = rich_v2(rng, nb=2, nd=3, L=6, N=4)
    dout = rng.standard_normal(p["u"].shape)
    gr = impl.vim_bidir_v2_bwd(*[p[k] for k in V2_NAMES], dout)
    if "du_abs" not in gr:
        return msgs
    for k in ("du", "ddelta_raw", "du_b", "ddelta_raw_b"):
        over = float(np.max(np.abs(gr[k]) - gr[k + "_abs"]))
        _check(msgs, f"|{k}| <= {k}_abs", max(over, 0.0), 1e-12)
        _check(msgs, f"{k}_abs not a plain copy of |{k}|", 1.0 if np.allclose(np.abs(gr[k]), gr[k + "_abs"]) else 0.0, 0.0)
    q = rich_v2(rng, nb=2, nd=3, L=6, N=1)
    q["D"] = np.zeros_like(q["D"])
    q["D_b"] = np.zeros_like(q["D_b"])
    g1 = impl.vim_bidir_v2_bwd(*[q[k] for k in V2_NAMES], dout)
    for k in ("du", "du_b"):
        _check(msgs, f"single-term {k}_abs = |{k}|", float(np.max(np.abs(np.abs(g1[k]) - g1[k + "_abs"]))), 1e-12)
    q["u"] = np.zeros_like(q["u"])
    g0 = impl.vim_bidir_v2_bwd(*[q[k] for k in V2_NAMES], dout)
    _check(msgs, "single-term ddelta_raw_abs = |ddelta_raw|",
           float(np.max(np.abs(np.abs(g0["ddelta_raw"]) - g0["ddelta_raw_abs"]))), 1e-12)
    s2 = rich_ss2d(rng, nb=1, nd=2, H=3, W=4, N=3)
    d2 = rng.standard_normal(s2["x"].shape)
    gs = impl.ss2d_cross_scan_bwd(s2["x"], s2["delta_raw"], s2["A_log"], s2["B"], s2["C"], s2["D"],
                                  s2["delta_bias"], None, d2)
    for k in ("dx", "ddelta_raw"):
        over = float(np.max(np.abs(gs[k]) - gs[k + "_abs"]))
        _check(msgs, f"ss2d |{k}| <= {k}_abs", max(over, 0.0), 1e-12)
    return msgs


ALL_PINS = [
    pin_softplus_silu,
    pin_golden_single_token,
    pin_single_token_closed_form,
    pin_geometric_series,
    pin_semiseparable,
    pin_semiseparable_closed,
    pin_linearity,
    pin_flip_identity,
    pin_limits,
    pin_ss2d_pathwalk,
    pin_ss2d_single_pixel,
    pin_ss2d_one_row,
    pin_ss2d_transpose,
    pin_v2_single_token,
    pin_v2_semiseparable,
    pin_v2_flip_identity,
    pin_bwd_finite_differences,
    pin_bwd_shared_inputs,
    pin_ss2d_bwd_finite_differences,
    pin_bwd_abs_sums,
    pin_conv1d_impulse,
    pin_conv1d_numpy,
    pin_conv2d_scipy,
    pin_conv2d_impulse,
]
