"""Helpers for the GPU parity tests: move seeded numpy inputs to the device, run the HIP entry
points through the binding, and compare with the fp64 oracle on the same (rounded) inputs."""
import numpy as np
import torch

import oracle as O

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
