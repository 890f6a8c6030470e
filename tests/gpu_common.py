"""Helpers for the GPU parity tests: move seeded numpy inputs to the device, run the HIP entry
points through the binding, and compare with the fp64 oracle on the same (rounded) inputs."""
import numpy as np
import torch

import oracle as O
import synth

TOL = {"f32": 1e-5, "bf16": 2e-2}


def tdev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)  # exact: the values are already bf16
    return t.cuda()


def pdev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def vim_device(p):
    dt = p["dtype"]
    act = {k: tdev(p[k], dt) for k in ("u", "delta_raw", "z", "B", "C", "B_b", "C_b")}
    par = {k: pdev(p[k]) for k in ("A_log", "A_b_log", "D", "D_b", "delta_bias")}
    return act, par


def run_vim(p, chunk_len=0, alias_v1=False):
    import selective_state_space_41_amd as V
    act, par = vim_device(p)
    B_b, C_b, D_b = (act["B"], act["C"], par["D"]) if alias_v1 else (act["B_b"], act["C_b"], par["D_b"])
    out = V.vmscan_fwd_bidir(act["u"], act["delta_raw"], act["z"], par["A_log"], par["A_b_log"], act["B"], act["C"],
                             B_b, C_b, par["D"], D_b, par["delta_bias"], chunk_len=chunk_len)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def oracle_vim(p, batches=None, alias_v1=False):
    sel = (lambda a: a) if batches is None else (lambda a: a[batches])
    B_b, C_b, D_b = (p["B"], p["C"], p["D"]) if alias_v1 else (p["B_b"], p["C_b"], p["D_b"])
    return O.vim_bidir(sel(p["u"]), sel(p["delta_raw"]), sel(p["z"]), p["A_log"], p["A_b_log"], sel(p["B"]),
                       sel(p["C"]), sel(B_b), sel(C_b), p["D"], D_b, p["delta_bias"])


def run_vim_v2(p, chunk_len=0, alias=()):
    """vmscan_fwd_bidir_v2 on the device; names in ``alias`` (u_b, delta_raw_b, delta_bias_b) pass the
    forward branch's tensor instead of the backward one."""
    import selective_state_space_41_amd as V
    dt = p["dtype"]
    act = {k: tdev(p[k], dt) for k in ("u", "delta_raw", "u_b", "delta_raw_b", "z", "B", "C", "B_b", "C_b")}
    par = {k: pdev(p[k]) for k in ("A_log", "A_b_log", "D", "D_b", "delta_bias", "delta_bias_b")}
    fwd_of = {"u_b": act["u"], "delta_raw_b": act["delta_raw"], "delta_bias_b": par["delta_bias"]}
    pick = lambda k, t: fwd_of[k] if k in alias else t
    out = V.vmscan_fwd_bidir_v2(act["u"], act["delta_raw"], par["delta_bias"], pick("u_b", act["u_b"]),
                                pick("delta_raw_b", act["delta_raw_b"]), pick("delta_bias_b", par["delta_bias_b"]),
                                act["z"], par["A_log"], par["A_b_log"], act["B"], act["C"], act["B_b"], act["C_b"],
                                par["D"], par["D_b"], chunk_len=chunk_len)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def oracle_vim_v2(p, batches=None, alias=()):
    sel = (lambda a: a) if batches is None else (lambda a: a[batches])
    fwd_of = {"u_b": "u", "delta_raw_b": "delta_raw", "delta_bias_b": "delta_bias"}
    g = lambda k: p[fwd_of[k]] if k in alias else p[k]
    return O.vim_bidir_v2(sel(p["u"]), sel(p["delta_raw"]), p["delta_bias"], sel(g("u_b")), sel(g("delta_raw_b")),
                          g("delta_bias_b"), sel(p["z"]), p["A_log"], p["A_b_log"], sel(p["B"]), sel(p["C"]),
                          sel(p["B_b"]), sel(p["C_b"]), p["D"], p["D_b"])


def run_ss2d(p, chunk_len=0):
    import selective_state_space_41_amd as V
    dt = p["dtype"]
    x = tdev(p["x"], dt)
    z = tdev(p["z"], dt) if p.get("z") is not None else None
    out = V.ss2d_cross_scan_fwd(x, tdev(p["delta_raw"], dt), pdev(p["A_log"]), tdev(p["B"], dt), tdev(p["C"], dt),
                                pdev(p["D"]), pdev(p["delta_bias"]), z=z, chunk_len=chunk_len)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def oracle_ss2d(p, batches=None):
    sel = (lambda a: a) if batches is None else (lambda a: a[batches])
    z = p.get("z")
    return O.ss2d_cross_scan(sel(p["x"]), sel(p["delta_raw"]), p["A_log"], sel(p["B"]), sel(p["C"]), p["D"],
                             p["delta_bias"], None if z is None else sel(z))


# ---- backward pass helpers

GRADS = ("du", "ddelta_raw", "ddelta_bias", "du_b", "ddelta_raw_b", "ddelta_bias_b", "dz", "dA_log", "dA_b_log", "dB",
         "dC", "dB_b", "dC_b", "dD", "dD_b")
PER_BATCH = ("du", "ddelta_raw", "du_b", "ddelta_raw_b", "dz", "dB", "dC", "dB_b", "dC_b")


# Rounding allowed per unit of a gradient's absolute-value sum S_i, for the sums over the states
# whose terms can cancel (du, dΔ_raw, SS2D dx): a float32 evaluation whose decays carry the
# hardware exp2's rounding (one ulp) through the adjoint is good to a few units of 2^-24 S_i; the
# worst case measured over the parity suite is about 5 units.
ROUND_UNITS = 8
ROUND = ROUND_UNITS * 2.0 ** -24
ABS = {"du": "du_abs", "ddelta_raw": "ddelta_raw_abs", "du_b": "du_b_abs", "ddelta_raw_b": "ddelta_raw_b_abs",
       "dx": "dx_abs"}


def grad_err(y, ref, k, tol):
    """O.rel_err, or for the sums in ABS max_i |y - r| / (max(|r_i|, rms(r)) + ROUND S_i / tol),
    so that err <= tol is the bound in the module docstring."""
    r = ref[k]
    s_abs = ref.get(ABS.get(k, ""))
    if s_abs is None:
        return O.rel_err(y, r)
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    s_abs = np.asarray(s_abs, dtype=np.float64)
    scale = np.maximum(np.abs(r), np.sqrt(np.mean(r * r)))
    excess = np.abs(y - r) - tol * scale
    used = float(np.max(np.where(s_abs > 0, excess / np.where(s_abs > 0, s_abs * 2.0 ** -24, 1.0), 0.0)))
    if used > 0:
        print(f"[parity]   {k}: rounding units of 2^-24 S used {used:.2f} (allowed {ROUND_UNITS})", flush=True)
    den = scale + (ROUND / tol) * s_abs
    den = np.where(den > 0, den, 1.0)  # an all-zero reference (z = 0): the absolute error
    return float(np.max(np.abs(y - r) / den))


def shared_ref(ref, k, pair):
    """The reference (and absolute-value sum) of a gradient summed over both branches."""
    out = {k: ref[pair[0]] + ref[pair[1]]}
    if pair[0] in ABS:
        out[ABS[k]] = ref[ABS[pair[0]]] + ref[ABS[pair[1]]]
    return out


def _dout(p, seed):
    rng = np.random.default_rng(seed)
    d = rng.standard_normal(p["u"].shape).astype(np.float32)
    return synth.round_bf16(d) if p["dtype"] == "bf16" else d


def run_bwd(p, dout, shared=False):
    import torch
    import selective_state_space_41_amd as V
    dt = p["dtype"]
    act = {k: tdev(p[k], dt) for k in ("u", "delta_raw", "u_b", "delta_raw_b", "z", "B", "C", "B_b", "C_b")}
    par = {k: pdev(p[k]) for k in ("A_log", "A_b_log", "D", "D_b", "delta_bias", "delta_bias_b")}
    if shared:
        act["u_b"], act["delta_raw_b"], par["delta_bias_b"] = act["u"], act["delta_raw"], par["delta_bias"]
    g = V.vmscan_bwd_bidir_v2(act["u"], act["delta_raw"], par["delta_bias"], act["u_b"], act["delta_raw_b"],
                              par["delta_bias_b"], act["z"], par["A_log"], par["A_b_log"], act["B"], act["C"],
                              act["B_b"], act["C_b"], par["D"], par["D_b"], tdev(dout, dt), shared=shared)
    torch.cuda.synchronize()
    return {k: (None if v is None else v.float().cpu().numpy()) for k, v in g.items()}


def oracle_bwd(p, dout, batches=None, shared=False):
    sel = (lambda a: a) if batches is None else (lambda a: a[batches])
    q = dict(p)
    if shared:
        q["u_b"], q["delta_raw_b"], q["delta_bias_b"] = p["u"], p["delta_raw"], p["delta_bias"]
    return O.vim_bidir_v2_bwd(sel(q["u"]), sel(q["delta_raw"]), q["delta_bias"], sel(q["u_b"]), sel(q["delta_raw_b"]),
                              q["delta_bias_b"], sel(q["z"]), q["A_log"], q["A_b_log"], sel(q["B"]), sel(q["C"]),
                              sel(q["B_b"]), sel(q["C_b"]), q["D"], q["D_b"], sel(dout))


SS2D_GRADS = ("dx", "ddelta_raw", "dA_log", "dB", "dC", "dD", "ddelta_bias", "dz")


def run_ss2d_bwd(p, dout):
    import torch
    import selective_state_space_41_amd as V
    dt = p["dtype"]
    z = tdev(p["z"], dt) if p.get("z") is not None else None
    g = V.ss2d_cross_scan_bwd(tdev(p["x"], dt), tdev(p["delta_raw"], dt), pdev(p["A_log"]), tdev(p["B"], dt),
                              tdev(p["C"], dt), pdev(p["D"]), pdev(p["delta_bias"]), z, tdev(dout, dt))
    torch.cuda.synchronize()
    return {k: (None if v is None else v.float().cpu().numpy()) for k, v in g.items()}


def oracle_ss2d_bwd(p, dout, batches=None):
    sel = (lambda a: a) if batches is None else (lambda a: a[batches])
    z = p.get("z")
    return O.ss2d_cross_scan_bwd(sel(p["x"]), sel(p["delta_raw"]), p["A_log"], sel(p["B"]), sel(p["C"]), p["D"],
                                 p["delta_bias"], None if z is None else sel(z), sel(dout))
