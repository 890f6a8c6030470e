"""vmscan_fwd_bidir_noalloc (the entry point for callers that cannot allocate) against
vmscan_fwd_bidir: the same kernels on the library's fixed scratch buffer instead of a caller's
workspace, so the outputs must be identical bit for bit; both are also checked against the fp64
oracle.  Two calls in a row, the second with a smaller input, so the second runs on a buffer that
still holds the first call's contents."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from gpu_common import TOL, oracle_vim, vim_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import selective_state_space_41_amd  # noqa: F401


def _both(p):
    import selective_state_space_41_amd as V
    act, par = vim_device(p)
    args = (act["u"], act["delta_raw"], act["z"], par["A_log"], par["A_b_log"], act["B"], act["C"], act["B_b"],
            act["C_b"], par["D"], par["D_b"], par["delta_bias"])
    out = torch.empty_like(act["u"])
    V.vmscan_fwd_bidir_noalloc(*args, out=out)
    ref = V.vmscan_fwd_bidir(*args)
    torch.cuda.synchronize()
    return out, ref


def test_noalloc_two_calls():
    cases = [
        # the Vim-Ti workload (bf16, B128 D384 L197), independent parameters
        (synth.make_vim_inputs(1, layer=11, params="indep"), np.array([0, 127])),
        # then a smaller float32 call whose sequence the library splits (chunk carries in the scratch)
        (synth.make_vim_inputs(0, layer=12, batch=2, dim=40, seqlen=1000, dtype="f32", params="indep"), None),
    ]
    for i, (p, bsel) in enumerate(cases):
        shape = p["u"].shape
        print(f"[no-alloc] call {i + 1}: {shape} {p['dtype']}", flush=True)
        out, ref = _both(p)
        assert torch.equal(out, ref), f"call {i + 1}: no-alloc output differs from vmscan_fwd_bidir"
        got = out.float().cpu().numpy()
        r = oracle_vim(p, batches=bsel)
        err = O.rel_err(got if bsel is None else got[bsel], r)
        print(f"[no-alloc] call {i + 1} vs oracle: err {err:.3e} (tol {TOL[p['dtype']]:.0e})", flush=True)
        assert err <= TOL[p["dtype"]]


def test_noalloc_rejects_oversized():
    """A shape whose workspace exceeds the fixed scratch buffer is refused before any launch."""
    import selective_state_space_41_amd as V
    p = synth.make_vim_inputs(0, layer=13, batch=1, dim=16, seqlen=8, dtype="bf16")
    act, par = vim_device(p)
    lib = V.load()
    big = (4096, 384, 197)
    assert lib.vmscan_fwd_bidir_workspace_bytes(*big, 16, 1) > V.SCRATCH_BYTES
    out = torch.empty_like(act["u"])
    ptrs = [V._ptr(t) for t in (act["u"], act["delta_raw"], act["z"], par["A_log"], par["A_b_log"], act["B"],
                                act["C"], act["B_b"], act["C_b"], par["D"], par["D_b"], par["delta_bias"], out)]
    assert lib.vmscan_fwd_bidir_noalloc(*ptrs, *big, 16, 1, None) == 7  # VMSCAN_ERR_SCRATCH
