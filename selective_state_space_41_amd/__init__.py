"""vmscan: MI355X (gfx950) Vision Mamba bidirectional selective scan and VMamba SS2D cross-scan.

Thin ctypes binding over ``libvmscan.so`` (C ABI in ``include/vmscan.h``).  The functions below
only check and marshal arguments (torch tensors -> device pointers, the current HIP stream, a
workspace from torch's allocator); every step of the scan runs in the library's HIP kernels.
There is no fallback: the library is loaded on first use (``load()``), and if it is missing or
cannot be loaded that raises.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libvmscan.so")

VMSCAN_F32 = 0
VMSCAN_BF16 = 1
CHUNK_LANE_SCAN = -1  # VMSCAN_CHUNK_LANE_SCAN: chunk_len that selects the lane-scan path (seqlen <= 8192)
D_STATE = 16          # the usual state size; the forward entry points also take 32
D_STATES_FWD = (16, 32)

_c_void_p = ctypes.c_void_p
_i64 = ctypes.c_int64


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m selective_state_space_41_amd.build` "
                          "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    lib.vmscan_status_string.restype = ctypes.c_char_p
    lib.vmscan_status_string.argtypes = [ctypes.c_int]
    lib.vmscan_last_hip_error.restype = ctypes.c_int
    lib.vmscan_last_hip_error.argtypes = []
    lib.vmscan_fwd_bidir_chunk_len.restype = _i64
    lib.vmscan_fwd_bidir_chunk_len.argtypes = [_i64, _i64, _i64, ctypes.c_int]
    lib.vmscan_fwd_bidir_workspace_bytes.restype = ctypes.c_size_t
    lib.vmscan_fwd_bidir_workspace_bytes.argtypes = [_i64, _i64, _i64, ctypes.c_int, ctypes.c_int]
    lib.vmscan_fwd_bidir_workspace_bytes_ex.restype = ctypes.c_size_t
    lib.vmscan_fwd_bidir_workspace_bytes_ex.argtypes = [_i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _i64]
    fwd_args = [_c_void_p] * 13 + [_i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _c_void_p, ctypes.c_size_t]
    lib.vmscan_fwd_bidir.restype = ctypes.c_int
    lib.vmscan_fwd_bidir.argtypes = fwd_args + [_c_void_p]
    lib.vmscan_fwd_bidir_ex.restype = ctypes.c_int
    lib.vmscan_fwd_bidir_ex.argtypes = fwd_args + [_i64, _c_void_p]
    lib.vmscan_fwd_bidir_stage.restype = ctypes.c_int
    lib.vmscan_fwd_bidir_stage.argtypes = fwd_args + [_i64, ctypes.c_int, _c_void_p]
    lib.vmscan_fwd_bidir_noalloc.restype = ctypes.c_int
    lib.vmscan_fwd_bidir_noalloc.argtypes = [_c_void_p] * 13 + [_i64, _i64, _i64, ctypes.c_int, ctypes.c_int,
                                                                 _c_void_p]
    v2_args = [_c_void_p] * 16 + [_i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _c_void_p, ctypes.c_size_t, _i64]
    lib.vmscan_fwd_bidir_v2.restype = ctypes.c_int
    lib.vmscan_fwd_bidir_v2.argtypes = v2_args + [_c_void_p]
    lib.vmscan_fwd_bidir_v2_stage.restype = ctypes.c_int
    lib.vmscan_fwd_bidir_v2_stage.argtypes = v2_args + [ctypes.c_int, _c_void_p]
    lib.vmscan_bwd_bidir_v2_workspace_bytes.restype = ctypes.c_size_t
    lib.vmscan_bwd_bidir_v2_workspace_bytes.argtypes = [_i64, _i64, _i64, ctypes.c_int, ctypes.c_int]
    lib.vmscan_bwd_bidir_v2.restype = ctypes.c_int
    lib.vmscan_bwd_bidir_v2.argtypes = ([_c_void_p] * 31 + [_i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _c_void_p,
                                                           ctypes.c_size_t, _c_void_p])
    lib.ss2d_cross_scan_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.ss2d_cross_scan_bwd_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int]
    lib.ss2d_cross_scan_bwd.restype = ctypes.c_int
    lib.ss2d_cross_scan_bwd.argtypes = ([_c_void_p] * 17 + [_i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int,
                                                           _c_void_p, ctypes.c_size_t, _c_void_p])
    lib.ss2d_cross_scan_workspace_bytes.restype = ctypes.c_size_t
    lib.ss2d_cross_scan_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int]
    lib.ss2d_cross_scan_workspace_bytes_ex.restype = ctypes.c_size_t
    lib.ss2d_cross_scan_workspace_bytes_ex.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _i64]
    ss_args = [_c_void_p] * 9 + [_i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _c_void_p, ctypes.c_size_t]
    lib.ss2d_cross_scan_fwd.restype = ctypes.c_int
    lib.ss2d_cross_scan_fwd.argtypes = ss_args + [_c_void_p]
    lib.ss2d_cross_scan_fwd_ex.restype = ctypes.c_int
    lib.ss2d_cross_scan_fwd_ex.argtypes = ss_args + [_i64, _c_void_p]
    lib.ss2d_cross_scan_fwd_xt.restype = ctypes.c_int
    lib.ss2d_cross_scan_fwd_xt.argtypes = [_c_void_p] + ss_args + [_i64, _c_void_p]
    lib.vmscan_conv1d_silu_fwd.restype = ctypes.c_int
    lib.vmscan_conv1d_silu_fwd.argtypes = [_c_void_p] * 7 + [_i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _c_void_p]
    lib.ss2d_conv2d_silu_fwd.restype = ctypes.c_int
    lib.ss2d_conv2d_silu_fwd.argtypes = ([_c_void_p] * 3 + [ctypes.c_int] + [_c_void_p] * 2 +
                                         [_i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _c_void_p])
    return lib


_LIB = None


def load():
    """Load libvmscan.so (once) and return the ctypes handle; raises if it is not built."""
    global _LIB
    if _LIB is None:
        _LIB = _load()
    return _LIB


def __getattr__(name):
    if name == "lib":
        return load()
    raise AttributeError(name)


def status_string(code):
    return load().vmscan_status_string(int(code)).decode()


def _check(code):
    if code != 0:
        msg = status_string(code)
        if code == 6:
            msg += f" (hipError_t {load().vmscan_last_hip_error()})"
        raise RuntimeError(msg)


def _call(fn, args, prepare, keep):
    """Make the C call now, or with ``prepare`` return a callable that makes it again with the same
    validated and marshalled arguments (no per-call checks: for timing and serving loops that
    repeat one call on the same tensors, which ``keep`` holds alive)."""
    if prepare:
        def run(_keep=keep):
            _check(fn(*args))
        return run
    _check(fn(*args))
    return None


def _act_dtype(t):
    if t.dtype == torch.float32:
        return VMSCAN_F32
    if t.dtype == torch.bfloat16:
        return VMSCAN_BF16
    raise TypeError(f"activation dtype must be float32 or bfloat16, got {t.dtype}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(t, name, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(stream, device):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _workspace(ws, nbytes, dev):
    """The caller's workspace if it is a large enough uint8 device tensor; a new one when none
    was given and the call needs one (None when it needs none).  A workspace that is given but
    too small is an error, not silently replaced: the stages of one call must see the same
    buffer."""
    if ws is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes > 0 else None
    if ws.dtype != torch.uint8 or ws.device != dev or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor on the inputs' device")
    if ws.numel() < nbytes:
        raise ValueError(f"workspace holds {ws.numel()} bytes, {nbytes} needed")
    return ws


def _nbytes(t):
    return t.numel() if t is not None else 0


def _d_state(A_log):
    """d_state from the last dimension of A_log (the library rejects sizes it does not take)."""
    if A_log.dim() < 1:
        raise ValueError("A_log must have a state dimension")
    return int(A_log.shape[-1])


def vmscan_fwd_bidir(u, delta_raw, z, A_log, A_b_log, B, C, B_b, C_b, D, D_b, delta_bias,
                     out=None, chunk_len=0, workspace=None, stream=None, stage=3, prepare=False):
    """Bidirectional selective scan with the silu(z) gate; returns ``out`` [batch, dim, L].

    u, delta_raw, z: [batch, dim, L]; A_log, A_b_log: [dim, N] float32 (d_state N = 16 or 32,
    taken from A_log); B, C, B_b, C_b: [batch, N, L] (original token order); D, D_b, delta_bias:
    [dim] float32.  Activations are
    float32 or bfloat16 (all the same).  ``chunk_len`` 0 lets the library choose;
    ``CHUNK_LANE_SCAN`` selects the lane-scan path (no chunks, seqlen <= 8192).  ``stage``
    1 / 2 runs only the preparation (B/C copy, chunk carries) / the fused scan
    (vmscan_fwd_bidir_stage); 3 runs both.  ``prepare=True`` validates once and returns a callable
    that repeats the call on the same tensors and stream."""
    if u.dim() != 3:
        raise ValueError("u must be [batch, dim, L]")
    nb, nd, L = u.shape
    ns = _d_state(A_log)
    dev = u.device
    adt = u.dtype
    dt = _act_dtype(u)
    for name, t in (("u", u), ("delta_raw", delta_raw), ("z", z)):
        _need(t, name, (nb, nd, L), adt, dev)
    for name, t in (("B", B), ("C", C), ("B_b", B_b), ("C_b", C_b)):
        _need(t, name, (nb, ns, L), adt, dev)
    for name, t in (("A_log", A_log), ("A_b_log", A_b_log)):
        _need(t, name, (nd, ns), torch.float32, dev)
    for name, t in (("D", D), ("D_b", D_b), ("delta_bias", delta_bias)):
        _need(t, name, (nd,), torch.float32, dev)
    if out is None:
        out = torch.empty_like(u)
    else:
        _need(out, "out", (nb, nd, L), adt, dev)
    lib = load()
    wsb = lib.vmscan_fwd_bidir_workspace_bytes_ex(nb, nd, L, ns, dt, int(chunk_len))
    workspace = _workspace(workspace, wsb, dev)
    args = (_ptr(u), _ptr(delta_raw), _ptr(z), _ptr(A_log), _ptr(A_b_log), _ptr(B), _ptr(C), _ptr(B_b), _ptr(C_b),
            _ptr(D), _ptr(D_b), _ptr(delta_bias), _ptr(out), nb, nd, L, ns, dt,
            _ptr(workspace), _nbytes(workspace), int(chunk_len), int(stage), _stream(stream, dev))
    run = _call(lib.vmscan_fwd_bidir_stage, args, prepare, (u, delta_raw, z, A_log, A_b_log, B, C, B_b, C_b, D, D_b,
                                                            delta_bias, out, workspace))
    return run if prepare else out


SCRATCH_BYTES = 64 << 20  # VMSCAN_SCRATCH_BYTES: the no-allocation entry point's fixed scratch


def vmscan_fwd_bidir_noalloc(u, delta_raw, z, A_log, A_b_log, B, C, B_b, C_b, D, D_b, delta_bias, out,
                             stream=None):
    """vmscan_fwd_bidir without any device allocation: the library's fixed per-GPU scratch buffer
    stands in for the workspace, and the caller passes ``out``.  Same arguments and result as
    ``vmscan_fwd_bidir`` (bit for bit); raises for shapes whose workspace would exceed
    ``SCRATCH_BYTES``.  Calls that overlap on one GPU share that buffer and race."""
    if u.dim() != 3:
        raise ValueError("u must be [batch, dim, L]")
    nb, nd, L = u.shape
    ns = _d_state(A_log)
    dev = u.device
    adt = u.dtype
    dt = _act_dtype(u)
    for name, t in (("u", u), ("delta_raw", delta_raw), ("z", z), ("out", out)):
        _need(t, name, (nb, nd, L), adt, dev)
    for name, t in (("B", B), ("C", C), ("B_b", B_b), ("C_b", C_b)):
        _need(t, name, (nb, ns, L), adt, dev)
    for name, t in (("A_log", A_log), ("A_b_log", A_b_log)):
        _need(t, name, (nd, ns), torch.float32, dev)
    for name, t in (("D", D), ("D_b", D_b), ("delta_bias", delta_bias)):
        _need(t, name, (nd,), torch.float32, dev)
    _check(load().vmscan_fwd_bidir_noalloc(
        _ptr(u), _ptr(delta_raw), _ptr(z), _ptr(A_log), _ptr(A_b_log), _ptr(B), _ptr(C), _ptr(B_b), _ptr(C_b),
        _ptr(D), _ptr(D_b), _ptr(delta_bias), _ptr(out), nb, nd, L, ns, dt, _stream(stream, dev)))
    return out


def vmscan_fwd_bidir_v2(u, delta_raw, delta_bias, u_b, delta_raw_b, delta_bias_b, z, A_log, A_b_log, B, C, B_b,
                        C_b, D, D_b, out=None, chunk_len=0, workspace=None, stream=None, stage=3, prepare=False):
    """Bidirectional scan whose backward branch has its own u_b, delta_raw_b and delta_bias_b
    (vmscan_fwd_bidir_v2_stage); the other arguments as for ``vmscan_fwd_bidir``.  u_b and
    delta_raw_b are [batch, dim, L] in original token order, delta_bias_b is [dim] float32; any
    of them may be the forward branch's tensor.  ``prepare`` as for ``vmscan_fwd_bidir``."""
    if u.dim() != 3:
        raise ValueError("u must be [batch, dim, L]")
    nb, nd, L = u.shape
    ns = _d_state(A_log)
    dev = u.device
    adt = u.dtype
    dt = _act_dtype(u)
    for name, t in (("u", u), ("delta_raw", delta_raw), ("u_b", u_b), ("delta_raw_b", delta_raw_b), ("z", z)):
        _need(t, name, (nb, nd, L), adt, dev)
    for name, t in (("B", B), ("C", C), ("B_b", B_b), ("C_b", C_b)):
        _need(t, name, (nb, ns, L), adt, dev)
    for name, t in (("A_log", A_log), ("A_b_log", A_b_log)):
        _need(t, name, (nd, ns), torch.float32, dev)
    for name, t in (("D", D), ("D_b", D_b), ("delta_bias", delta_bias), ("delta_bias_b", delta_bias_b)):
        _need(t, name, (nd,), torch.float32, dev)
    if out is None:
        out = torch.empty_like(u)
    else:
        _need(out, "out", (nb, nd, L), adt, dev)
    lib = load()
    wsb = lib.vmscan_fwd_bidir_workspace_bytes_ex(nb, nd, L, ns, dt, int(chunk_len))
    workspace = _workspace(workspace, wsb, dev)
    args = (_ptr(u), _ptr(delta_raw), _ptr(delta_bias), _ptr(u_b), _ptr(delta_raw_b), _ptr(delta_bias_b), _ptr(z),
            _ptr(A_log), _ptr(A_b_log), _ptr(B), _ptr(C), _ptr(B_b), _ptr(C_b), _ptr(D), _ptr(D_b), _ptr(out),
            nb, nd, L, ns, dt, _ptr(workspace), _nbytes(workspace), int(chunk_len), int(stage),
            _stream(stream, dev))
    run = _call(lib.vmscan_fwd_bidir_v2_stage, args, prepare, (u, delta_raw, delta_bias, u_b, delta_raw_b,
                                                               delta_bias_b, z, A_log, A_b_log, B, C, B_b, C_b, D,
                                                               D_b, out, workspace))
    return run if prepare else out


def vmscan_bwd_bidir_v2(u, delta_raw, delta_bias, u_b, delta_raw_b, delta_bias_b, z, A_log, A_b_log, B, C, B_b, C_b,
                        D, D_b, dout, shared=False, workspace=None, stream=None, prepare=False):
    """Gradients of ``vmscan_fwd_bidir_v2`` for ``dout`` (vmscan_bwd_bidir_v2); returns a dict with
    du, ddelta_raw, ddelta_bias, du_b, ddelta_raw_b, ddelta_bias_b, dz, dA_log, dA_b_log, dB, dC,
    dB_b, dC_b, dD, dD_b.  With ``shared=True`` (u_b is u, delta_raw_b is delta_raw, delta_bias_b
    is delta_bias, i.e. ``vmscan_fwd_bidir``) the backward branch's du, ddelta_raw and ddelta_bias
    are added into the forward ones and the ``_b`` entries are None.  d_state 16 or 32.  With
    ``prepare`` it returns (callable, gradient dict): each call rewrites the same gradient tensors."""
    if u.dim() != 3:
        raise ValueError("u must be [batch, dim, L]")
    nb, nd, L = u.shape
    ns = _d_state(A_log)
    dev = u.device
    adt = u.dtype
    dt = _act_dtype(u)
    for name, t in (("u", u), ("delta_raw", delta_raw), ("u_b", u_b), ("delta_raw_b", delta_raw_b), ("z", z),
                    ("dout", dout)):
        _need(t, name, (nb, nd, L), adt, dev)
    for name, t in (("B", B), ("C", C), ("B_b", B_b), ("C_b", C_b)):
        _need(t, name, (nb, ns, L), adt, dev)
    for name, t in (("A_log", A_log), ("A_b_log", A_b_log)):
        _need(t, name, (nd, ns), torch.float32, dev)
    for name, t in (("D", D), ("D_b", D_b), ("delta_bias", delta_bias), ("delta_bias_b", delta_bias_b)):
        _need(t, name, (nd,), torch.float32, dev)
    act = lambda: torch.empty_like(u)
    bcs = lambda: torch.empty_like(B)
    par = lambda *s: torch.empty(*s, dtype=torch.float32, device=dev)
    g = dict(du=act(), ddelta_raw=act(), ddelta_bias=par(nd), dz=act(), dA_log=par(nd, ns),
             dA_b_log=par(nd, ns), dB=bcs(), dC=bcs(), dB_b=bcs(), dC_b=bcs(), dD=par(nd), dD_b=par(nd))
    g["du_b"], g["ddelta_raw_b"], g["ddelta_bias_b"] = (None, None, None) if shared else (act(), act(), par(nd))
    lib = load()
    wsb = lib.vmscan_bwd_bidir_v2_workspace_bytes(nb, nd, L, ns, dt)
    workspace = _workspace(workspace, wsb, dev)
    args = (_ptr(u), _ptr(delta_raw), _ptr(delta_bias), _ptr(u_b), _ptr(delta_raw_b), _ptr(delta_bias_b), _ptr(z),
            _ptr(A_log), _ptr(A_b_log), _ptr(B), _ptr(C), _ptr(B_b), _ptr(C_b), _ptr(D), _ptr(D_b), _ptr(dout),
            *[_ptr(g[k]) for k in ("du", "ddelta_raw", "ddelta_bias", "du_b", "ddelta_raw_b", "ddelta_bias_b", "dz",
                                   "dA_log", "dA_b_log", "dB", "dC", "dB_b", "dC_b", "dD", "dD_b")],
            nb, nd, L, ns, dt, _ptr(workspace), _nbytes(workspace), _stream(stream, dev))
    run = _call(lib.vmscan_bwd_bidir_v2, args, prepare, (u, delta_raw, delta_bias, u_b, delta_raw_b, delta_bias_b, z,
                                                         A_log, A_b_log, B, C, B_b, C_b, D, D_b, dout, g, workspace))
    return (run, g) if prepare else g


def ss2d_cross_scan_fwd(x, delta_raw, A_log, B, C, D, delta_bias, z=None, out=None, chunk_len=0,
                        workspace=None, stream=None, xT=None, prepare=False):
    """SS2D four-direction cross-scan with cross-merge; returns ``out`` [batch, dim, H, W].

    x: [batch, dim, H, W]; delta_raw: [batch, 4, dim, H*W]; A_log: [4, dim, N] float32 (d_state
    N = 16 or 32); B, C: [batch, 4, N, H*W] (each direction's scan order); D, delta_bias: [4, dim]
    float32; z: optional [batch, dim, H, W] gate; xT: optional [batch, dim, W, H], x transposed
    (as written by ``ss2d_conv2d_silu_fwd``), read instead of a copy made by the call
    (ss2d_cross_scan_fwd_xt).  ``prepare`` as for ``vmscan_fwd_bidir``."""
    if x.dim() != 4:
        raise ValueError("x must be [batch, dim, H, W]")
    nb, nd, H, W = x.shape
    L = H * W
    ns = _d_state(A_log)
    dev = x.device
    adt = x.dtype
    dt = _act_dtype(x)
    _need(x, "x", (nb, nd, H, W), adt, dev)
    _need(delta_raw, "delta_raw", (nb, 4, nd, L), adt, dev)
    _need(B, "B", (nb, 4, ns, L), adt, dev)
    _need(C, "C", (nb, 4, ns, L), adt, dev)
    _need(A_log, "A_log", (4, nd, ns), torch.float32, dev)
    _need(D, "D", (4, nd), torch.float32, dev)
    _need(delta_bias, "delta_bias", (4, nd), torch.float32, dev)
    if z is not None:
        _need(z, "z", (nb, nd, H, W), adt, dev)
    if out is None:
        out = torch.empty_like(x)
    else:
        _need(out, "out", (nb, nd, H, W), adt, dev)
    lib = load()
    wsb = lib.ss2d_cross_scan_workspace_bytes_ex(nb, nd, H, W, ns, dt, int(chunk_len))
    workspace = _workspace(workspace, wsb, dev)
    args = (_ptr(delta_raw), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D), _ptr(delta_bias), _ptr(z), _ptr(out),
            nb, nd, H, W, ns, dt, _ptr(workspace), _nbytes(workspace), int(chunk_len), _stream(stream, dev))
    keep = (x, xT, delta_raw, A_log, B, C, D, delta_bias, z, out, workspace)
    if xT is None:
        run = _call(lib.ss2d_cross_scan_fwd_ex, (_ptr(x),) + args, prepare, keep)
    else:
        _need(xT, "xT", (nb, nd, W, H), adt, dev)
        run = _call(lib.ss2d_cross_scan_fwd_xt, (_ptr(x), _ptr(xT)) + args, prepare, keep)
    return run if prepare else out


def ss2d_cross_scan_bwd(x, delta_raw, A_log, B, C, D, delta_bias, z, dout, workspace=None, stream=None,
                        prepare=False):
    """Gradients of ``ss2d_cross_scan_fwd`` for ``dout`` (ss2d_cross_scan_bwd); returns a dict with
    dx, ddelta_raw, dA_log, dB, dC, dD, ddelta_bias and dz (None when z is None).  d_state 16 or 32.
    ``prepare`` as for ``vmscan_bwd_bidir_v2``."""
    if x.dim() != 4:
        raise ValueError("x must be [batch, dim, H, W]")
    nb, nd, H, W = x.shape
    L = H * W
    ns = _d_state(A_log)
    dev = x.device
    adt = x.dtype
    dt = _act_dtype(x)
    _need(x, "x", (nb, nd, H, W), adt, dev)
    _need(dout, "dout", (nb, nd, H, W), adt, dev)
    _need(delta_raw, "delta_raw", (nb, 4, nd, L), adt, dev)
    _need(B, "B", (nb, 4, ns, L), adt, dev)
    _need(C, "C", (nb, 4, ns, L), adt, dev)
    _need(A_log, "A_log", (4, nd, ns), torch.float32, dev)
    _need(D, "D", (4, nd), torch.float32, dev)
    _need(delta_bias, "delta_bias", (4, nd), torch.float32, dev)
    if z is not None:
        _need(z, "z", (nb, nd, H, W), adt, dev)
    g = dict(dx=torch.empty_like(x), ddelta_raw=torch.empty_like(delta_raw), dA_log=torch.empty_like(A_log),
             dB=torch.empty_like(B), dC=torch.empty_like(C), dD=torch.empty_like(D),
             ddelta_bias=torch.empty_like(delta_bias), dz=torch.empty_like(x) if z is not None else None)
    lib = load()
    wsb = lib.ss2d_cross_scan_bwd_workspace_bytes(nb, nd, H, W, ns, dt)
    workspace = _workspace(workspace, wsb, dev)
    args = (_ptr(x), _ptr(delta_raw), _ptr(A_log), _ptr(B), _ptr(C), _ptr(D), _ptr(delta_bias), _ptr(z), _ptr(dout),
            *[_ptr(g[k]) for k in ("dx", "ddelta_raw", "dA_log", "dB", "dC", "dD", "ddelta_bias", "dz")],
            nb, nd, H, W, ns, dt, _ptr(workspace), _nbytes(workspace), _stream(stream, dev))
    run = _call(lib.ss2d_cross_scan_bwd, args, prepare, (x, delta_raw, A_log, B, C, D, delta_bias, z, dout, g,
                                                         workspace))
    return (run, g) if prepare else g


def conv1d_silu_fwd(x, conv_w, conv_b, conv_w_b=None, conv_b_b=None, u=None, u_b=None, stream=None):
    """Front of the Vim scan (vmscan_conv1d_silu_fwd): u = silu(causal depthwise conv1d(x) + conv_b)
    and, when conv_w_b / conv_b_b are given, u_b = the flipped branch's convolution in original
    token order.  x: [batch, dim, L] float32 or bfloat16; conv_w(_b): [dim, d_conv] float32
    (d_conv 1..4); conv_b(_b): [dim] float32.  Returns (u, u_b), u_b None for one branch."""
    if x.dim() != 3:
        raise ValueError("x must be [batch, dim, L]")
    nb, nd, L = x.shape
    dev, adt, dt = x.device, x.dtype, _act_dtype(x)
    if conv_w.dim() != 2:
        raise ValueError("conv_w must be [dim, d_conv]")
    K = int(conv_w.shape[1])
    _need(conv_w, "conv_w", (nd, K), torch.float32, dev)
    _need(conv_b, "conv_b", (nd,), torch.float32, dev)
    two = conv_w_b is not None or conv_b_b is not None
    if two:
        _need(conv_w_b, "conv_w_b", (nd, K), torch.float32, dev)
        _need(conv_b_b, "conv_b_b", (nd,), torch.float32, dev)
    if u is None:
        u = torch.empty_like(x)
    _need(u, "u", (nb, nd, L), adt, dev)
    if two:
        if u_b is None:
            u_b = torch.empty_like(x)
        _need(u_b, "u_b", (nb, nd, L), adt, dev)
    else:
        u_b = None
    _check(load().vmscan_conv1d_silu_fwd(_ptr(x), _ptr(conv_w), _ptr(conv_b), _ptr(conv_w_b), _ptr(conv_b_b),
                                         _ptr(u), _ptr(u_b), nb, nd, L, K, dt, _stream(stream, dev)))
    return u, u_b


def ss2d_conv2d_silu_fwd(x, conv_w, conv_b, act=True, transposed=True, x_out=None, xT_out=None, stream=None):
    """Front of SS2D (ss2d_conv2d_silu_fwd): depthwise 3 x 3 convolution (+ SiLU when ``act``) of
    x [batch, dim, H, W]; conv_w [dim, 3, 3], conv_b [dim] float32.  Returns (x_out, xT_out):
    the result row-major and, when ``transposed``, also as [batch, dim, W, H]."""
    if x.dim() != 4:
        raise ValueError("x must be [batch, dim, H, W]")
    nb, nd, H, W = x.shape
    dev, adt, dt = x.device, x.dtype, _act_dtype(x)
    if conv_w.dim() != 3:
        raise ValueError("conv_w must be [dim, K, K]")
    K = int(conv_w.shape[1])
    _need(conv_w, "conv_w", (nd, K, K), torch.float32, dev)
    _need(conv_b, "conv_b", (nd,), torch.float32, dev)
    if x_out is None:
        x_out = torch.empty_like(x)
    _need(x_out, "x_out", (nb, nd, H, W), adt, dev)
    if transposed:
        if xT_out is None:
            xT_out = torch.empty((nb, nd, W, H), dtype=adt, device=dev)
        _need(xT_out, "xT_out", (nb, nd, W, H), adt, dev)
    else:
        xT_out = None
    _check(load().ss2d_conv2d_silu_fwd(_ptr(x), _ptr(conv_w), _ptr(conv_b), int(bool(act)), _ptr(x_out),
                                       _ptr(xT_out), nb, nd, H, W, K, dt, _stream(stream, dev)))
    return x_out, xT_out


def fwd_bidir_chunk_len(batch, dim, seqlen, d_state=D_STATE):
    return int(load().vmscan_fwd_bidir_chunk_len(batch, dim, seqlen, d_state))
