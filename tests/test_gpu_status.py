"""The wait status word: every workspace starts with an int32 that the call's first kernel sets to
0 and that a bounded wait between the state parts of a direction sets to 1 if it gives up (which
no correct run does).  Each entry point is called on a workspace whose bytes all start as 0xFF;
after the call the word must read 0, for the unsplit and split Vim scans, the separate-branch
scan, the chunked and whole-sequence SS2D cross-scans and both backward passes."""
import numpy as np
import pytest
import torch

import synth
from gpu_common import _dout, pdev, tdev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    import selective_state_space_41_amd  # noqa: F401


def _ws(nbytes):
    return torch.full((max(nbytes, 4),), 255, dtype=torch.uint8, device="cuda")


def _word(ws):
    torch.cuda.synchronize()
    return int(ws[:4].cpu().numpy().view(np.int32)[0])


@pytest.mark.parametrize("L,K", [(197, 0), (300, 40)], ids=["whole", "split"])
def test_status_word_vim(L, K):
    import selective_state_space_41_amd as V
    p = synth.make_vim_v2_inputs(0, layer=5000 + L, batch=2, dim=40, seqlen=L, dtype="bf16", params="indep")
    a = {k: tdev(p[k], "bf16") for k in ("u", "delta_raw", "u_b", "delta_raw_b", "z", "B", "C", "B_b", "C_b")}
    q = {k: pdev(p[k]) for k in ("A_log", "A_b_log", "D", "D_b", "delta_bias", "delta_bias_b")}
    ws = _ws(V.lib.vmscan_fwd_bidir_workspace_bytes_ex(2, 40, L, 16, 1, K))
    V.vmscan_fwd_bidir(a["u"], a["delta_raw"], a["z"], q["A_log"], q["A_b_log"], a["B"], a["C"], a["B_b"], a["C_b"],
                       q["D"], q["D_b"], q["delta_bias"], chunk_len=K, workspace=ws)
    assert _word(ws) == 0
    ws.fill_(255)
    V.vmscan_fwd_bidir_v2(a["u"], a["delta_raw"], q["delta_bias"], a["u_b"], a["delta_raw_b"], q["delta_bias_b"],
                          a["z"], q["A_log"], q["A_b_log"], a["B"], a["C"], a["B_b"], a["C_b"], q["D"], q["D_b"],
                          chunk_len=K, workspace=ws)
    assert _word(ws) == 0
    wb = _ws(V.lib.vmscan_bwd_bidir_v2_workspace_bytes(2, 40, L, 16, 1))
    V.vmscan_bwd_bidir_v2(a["u"], a["delta_raw"], q["delta_bias"], a["u_b"], a["delta_raw_b"], q["delta_bias_b"],
                          a["z"], q["A_log"], q["A_b_log"], a["B"], a["C"], a["B_b"], a["C_b"], q["D"], q["D_b"],
                          tdev(_dout(p, 3), "bf16"), workspace=wb)
    assert _word(wb) == 0


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("walk", [False, True])
def test_status_word_ss2d(walk, gated):
    import selective_state_space_41_amd as V
    H, W = 13, 17
    p = synth.make_ss2d_inputs(4, layer=5100, batch=2, dim=40, H=H, W=W, dtype="bf16", with_z=gated, params="indep")
    K = H * W if walk else 0
    args = (tdev(p["x"], "bf16"), tdev(p["delta_raw"], "bf16"), pdev(p["A_log"]), tdev(p["B"], "bf16"),
            tdev(p["C"], "bf16"), pdev(p["D"]), pdev(p["delta_bias"]))
    z = tdev(p["z"], "bf16") if gated else None
    ws = _ws(V.lib.ss2d_cross_scan_workspace_bytes_ex(2, 40, H, W, 16, 1, K))
    V.ss2d_cross_scan_fwd(*args, z=z, chunk_len=K, workspace=ws)
    assert _word(ws) == 0
    if not walk:
        wb = _ws(V.lib.ss2d_cross_scan_bwd_workspace_bytes(2, 40, H, W, 16, 1))
        V.ss2d_cross_scan_bwd(*args, z, tdev(_dout(dict(u=p["x"], dtype="bf16"), 1), "bf16"), workspace=wb)
        assert _word(wb) == 0
