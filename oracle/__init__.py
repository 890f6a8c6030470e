"""Plain fp64 CPU oracle for the Vision Mamba bidirectional selective scan and the VMamba
SS2D cross-scan.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or execute this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library in
``selective_state_space_41_amd/``.
"""
from .vmscan_oracle import (  # noqa: F401
    softplus,
    silu,
    scan_1d,
    scan_1d_semiseparable,
    vim_bidir,
    vim_bidir_v2,
    scan_1d_bwd,
    vim_bidir_v2_bwd,
    ss2d_orders,
    ss2d_cross_scan,
    ss2d_cross_scan_bwd,
    ss2d_cross_scan_pathwalk,
    conv1d_silu,
    conv2d_silu,
    rel_err,
)
