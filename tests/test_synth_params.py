"""The independent-parameter inputs make parameter-indexing mistakes visible (CPU, oracle only).

With the pages' shared initial values (A_log = log(1..N) for every channel and both branches,
D = D_b = 1, the same A_log and D for all four SS2D directions) a kernel that read A_log without
the channel index, swapped the two branches' parameter sets, used one SS2D direction's
parameters for every direction or dropped the D·u term could not be told apart from a correct
one.  Each test below plants one such mistake in the arguments given to the oracle and checks
that the independent parameters of ``synth`` move the result far beyond the parity tolerance
(and, for the first three, that the shared initial values do not: the blind spot they close)."""
import numpy as np
import pytest

import oracle as O
import synth

TOL_F32 = 1e-5


def _vim(p, **over):
    q = dict(p)
    q.update(over)
    return O.vim_bidir_v2(q["u"], q["delta_raw"], q["delta_bias"], q["u_b"], q["delta_raw_b"], q["delta_bias_b"],
                          q["z"], q["A_log"], q["A_b_log"], q["B"], q["C"], q["B_b"], q["C_b"], q["D"], q["D_b"])


def _mistakes(p):
    nd = p["A_log"].shape[0]
    return {
        "A_log without the channel index": dict(A_log=np.repeat(p["A_log"][:1], nd, axis=0),
                                                A_b_log=np.repeat(p["A_b_log"][:1], nd, axis=0)),
        "A_log and A_b_log swapped": dict(A_log=p["A_b_log"], A_b_log=p["A_log"]),
        "D and D_b swapped": dict(D=p["D_b"], D_b=p["D"]),
        "D·u term dropped": dict(D=np.zeros_like(p["D"]), D_b=np.zeros_like(p["D_b"])),
    }


@pytest.mark.parametrize("params", ["init", "indep"])
def test_vim_parameter_mistakes(params):
    p = synth.make_vim_v2_inputs(0, layer=5, batch=2, dim=24, seqlen=40, dtype="f32", params=params)
    ref = _vim(p)
    for name, over in _mistakes(p).items():
        err = O.rel_err(_vim(p, **over), ref)
        print(f"{params}: {name}: {err:.3e}")
        if params == "indep" or name == "D·u term dropped":
            assert err > 100 * TOL_F32, (name, err)
        else:
            assert err < TOL_F32, (name, err)  # invisible with the shared initial values


def test_ss2d_direction_parameter_mistake():
    """Direction 0's A_log, D and bias used for all four directions."""
    for params, visible in (("init", False), ("indep", True)):
        p = synth.make_ss2d_inputs(4, layer=6, batch=1, dim=12, H=5, W=6, dtype="f32", params=params)
        ref = O.ss2d_cross_scan(p["x"], p["delta_raw"], p["A_log"], p["B"], p["C"], p["D"], p["delta_bias"])
        bad_a = np.repeat(p["A_log"][:1], 4, axis=0)
        bad_d = np.repeat(p["D"][:1], 4, axis=0)
        err = O.rel_err(O.ss2d_cross_scan(p["x"], p["delta_raw"], bad_a, p["B"], p["C"], bad_d, p["delta_bias"]), ref)
        print(f"{params}: direction 0's A_log, D for all: {err:.3e}")
        assert (err > 100 * TOL_F32) == visible, (params, err)


def test_indep_params_ranges():
    """A_log stays within 0.5 of log(1..N) (so A = -exp(A_log) keeps the pages' scale), D within
    [-1.5, 1.5], and the drawn tensors all differ from each other."""
    p = synth.make_vim_v2_inputs(0, layer=1, batch=1, dim=64, seqlen=4, d_state=32, params="indep")
    base = np.log(np.arange(1, 33, dtype=np.float64))
    for k in ("A_log", "A_b_log"):
        assert p[k].shape == (64, 32) and p[k].dtype == np.float32
        assert np.max(np.abs(p[k] - base)) <= 0.5 + 1e-6
        assert len(np.unique(p[k][:, 0])) == 64  # per channel
    assert not np.array_equal(p["A_log"], p["A_b_log"])
    for k in ("D", "D_b"):
        assert p[k].shape == (64,) and np.max(np.abs(p[k])) <= 1.5
    assert not np.array_equal(p["D"], p["D_b"])
    q = synth.make_ss2d_inputs(4, layer=1, batch=1, dim=16, H=2, W=3, params="indep")
    for k in range(4):
        for j in range(k):
            assert not np.array_equal(q["A_log"][k], q["A_log"][j])
            assert not np.array_equal(q["D"][k], q["D"][j])
            assert not np.array_equal(q["delta_bias"][k], q["delta_bias"][j])
    # the default stays the pages' initialisation
    r = synth.make_vim_inputs(0, batch=1, dim=3, seqlen=2)
    assert np.all(r["D"] == 1) and np.array_equal(r["A_log"], r["A_b_log"])
    with pytest.raises(ValueError):
        synth.make_vim_inputs(0, batch=1, dim=3, seqlen=2, params="other")
