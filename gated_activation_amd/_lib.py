"""ctypes binding of libga.so.  Argument marshalling only."""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(HERE, "libga.so")

GA_F32, GA_F16, GA_BF16 = 0, 1, 2
GA_OK, GA_EINVAL, GA_EUNSUPPORTED, GA_EHIP = 0, 1, 2, 3
GA_MAX_D = 65536
GA_ROUND_INTERMEDIATES = 1
# Phi^-1(0.95): the cutoff multiplier for a target sparsity of 95%.
Z_SPARSITY_095 = 1.6448536

_TORCH_DTYPE = {torch.float32: GA_F32, torch.float16: GA_F16, torch.bfloat16: GA_BF16}


class Plan(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("waves_per_row", ctypes.c_int32),
                ("per_lane", ctypes.c_int32), ("up_late", ctypes.c_int32),
                ("block", ctypes.c_int32), ("splits", ctypes.c_int32),
                ("grid", ctypes.c_int64), ("spin_limit", ctypes.c_uint32),
                ("flags", ctypes.c_int32), ("lanes_per_row", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]

    def __init__(self, **kw):
        kw.setdefault("splits", 1)
        kw.setdefault("spin_limit", 1 << 16)
        super().__init__(**kw)

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


GA_DOWN_DECODE, GA_DOWN_STAGED, GA_DOWN_TILED = 1, 2, 3


class DownPlan(ctypes.Structure):
    """Geometry of the activation fused with the down projection."""
    _fields_ = [("rows_per_block", ctypes.c_int32), ("features_per_block", ctypes.c_int32),
                ("waves", ctypes.c_int32), ("k_step", ctypes.c_int32), ("k_chunk", ctypes.c_int32),
                ("splits", ctypes.c_int32), ("form", ctypes.c_int32), ("depth", ctypes.c_int32),
                ("grid", ctypes.c_int64)]

    @classmethod
    def tiled(cls, T, d, H, rows_per_block, features_per_block, waves, k_step, k_chunk, depth):
        """The tiled form's plan of one geometry (the activation stored into
        the workspace, then a matrix-core product over slices of k_chunk with
        `depth` steps of weights in flight)."""
        splits = -(-d // k_chunk)
        return cls(rows_per_block=rows_per_block, features_per_block=features_per_block, waves=waves,
                   k_step=k_step, k_chunk=k_chunk, splits=splits, form=GA_DOWN_TILED, depth=depth,
                   grid=-(-T // rows_per_block) * -(-H // features_per_block) * splits)

    @classmethod
    def _whole(cls, form, d, H, rows_per_block, features_per_block, waves):
        return cls(rows_per_block=rows_per_block, features_per_block=features_per_block, waves=waves, k_step=0,
                   k_chunk=d, splits=1, form=form, grid=-(-H // features_per_block))

    @classmethod
    def decode(cls, T, d, H, rows_per_block, features_per_block, waves):
        """The decode form: rows_per_block (1 or 2) >= T tokens,
        features_per_block output features per workgroup over all of d."""
        return cls._whole(GA_DOWN_DECODE, d, H, rows_per_block, features_per_block, waves)

    @classmethod
    def staged(cls, T, d, H, rows_per_block, features_per_block, waves):
        """The staged form: rows_per_block (2 or 4) >= T tokens; the
        activation is stored into the workspace, then multiplied."""
        return cls._whole(GA_DOWN_STAGED, d, H, rows_per_block, features_per_block, waves)

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


class GaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{status}: {message}")
        self.status = status


def _load():
    if not os.path.exists(library_path):
        raise ImportError(
            f"{library_path} is not built; run `python -m gated_activation_amd.build` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(library_path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    pplan = ctypes.POINTER(Plan)
    sigs = {
        "ga_gelu_and_mul_sparse": [vp, vp, i64, i64, i32, ctypes.c_float, vp, vp],
        "ga_silu_and_mul_bounded": [vp, vp, i64, i64, i32, vp, vp],
        "ga_gelu_and_mul_sparse_with_plan": [vp, vp, i64, i64, i32, ctypes.c_float, vp, pplan, vp,
                                             ctypes.c_size_t, vp],
        "ga_gelu_and_mul_sparse_ws": [vp, vp, i64, i64, i32, ctypes.c_float, vp, vp, ctypes.c_size_t, vp],
        "ga_gelu_and_mul_sparse_ex": [vp, vp, i64, i64, i32, ctypes.c_float, vp, i32, vp, ctypes.c_size_t, vp],
        "ga_gelu_and_mul_sparse_noalloc": [vp, vp, i64, i64, i32, ctypes.c_float, vp, vp],
        "ga_silu_and_mul_bounded_with_plan": [vp, vp, i64, i64, i32, vp, pplan, vp],
        "ga_plan_gelu_and_mul_sparse": [i64, i64, i32, i32, i32, i32, pplan],
        "ga_plan_silu_and_mul_bounded": [i64, i64, i32, i32, i32, pplan],
        "ga_stream_xor_rows": [vp, vp, i64, i64, vp],
        "ga_gelu_and_mul": [vp, vp, i64, i64, i32, i32, vp, vp],
        "ga_squared_relu_bounded": [vp, vp, i64, i64, i32, vp, vp],
        "ga_gelu_and_mul_sparse_down": [vp, vp, vp, i64, i64, i64, i32, ctypes.c_float, vp, vp,
                                        ctypes.c_size_t, vp],
        "ga_gelu_and_mul_sparse_down_with_plan": [vp, vp, vp, i64, i64, i64, i32, ctypes.c_float, vp,
                                                  ctypes.POINTER(DownPlan), vp, ctypes.c_size_t, vp],
        "ga_plan_gelu_and_mul_sparse_down": [i64, i64, i64, i32, ctypes.POINTER(DownPlan)],
    }
    for name, args in sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.ga_status_str.argtypes = [i32]
    lib.ga_status_str.restype = ctypes.c_char_p
    lib.ga_last_error.argtypes = []
    lib.ga_last_error.restype = ctypes.c_char_p
    lib.ga_version.argtypes = []
    lib.ga_version.restype = i32
    lib.ga_z_from_sparsity.argtypes = [ctypes.c_double]
    lib.ga_z_from_sparsity.restype = ctypes.c_double
    lib.ga_gelu_and_mul_sparse_workspace_bytes.argtypes = [i64]
    lib.ga_gelu_and_mul_sparse_workspace_bytes.restype = ctypes.c_size_t
    lib.ga_gelu_and_mul_sparse_down_workspace_bytes.argtypes = [i64, i64, i64, ctypes.POINTER(DownPlan)]
    lib.ga_gelu_and_mul_sparse_down_workspace_bytes.restype = ctypes.c_size_t
    return lib


lib = _load()
# Calls of more rows than this are never split over workgroups, so a workspace
# of WORKSPACE_BYTES serves every call.
GA_SPLIT_PLAN_ROWS = 256
WORKSPACE_BYTES = int(lib.ga_gelu_and_mul_sparse_workspace_bytes(GA_SPLIT_PLAN_ROWS))


def _check(status):
    if status != GA_OK:
        raise GaError(lib.ga_status_str(status).decode(), lib.ga_last_error().decode())


def _stream_of(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _prep(x, out, name, gated=True):
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise ValueError(f"{name}: x must be a CUDA (HIP) tensor")
    cols = 2 if gated else 1
    if x.dim() != 2 or x.shape[1] % cols != 0 or x.shape[1] == 0:
        raise ValueError(f"{name}: x must be [rows, {cols}d] with d >= 1, got {tuple(x.shape)}")
    if not x.is_contiguous():
        raise ValueError(f"{name}: x must be contiguous")
    if x.dtype not in _TORCH_DTYPE:
        raise ValueError(f"{name}: unsupported dtype {x.dtype}")
    rows, d = x.shape[0], x.shape[1] // cols
    if out is None:
        out = torch.empty((rows, d), dtype=x.dtype, device=x.device)
    elif (out.shape != (rows, d) or out.dtype != x.dtype or out.device != x.device
          or not out.is_contiguous()):
        raise ValueError(f"{name}: out must be a contiguous [{rows}, {d}] {x.dtype} tensor on {x.device}")
    return rows, d, out


def _live_ptr(live_rows, x, name):
    if live_rows is None:
        return None
    if (not isinstance(live_rows, torch.Tensor) or live_rows.dtype != torch.int32
            or live_rows.device != x.device or live_rows.numel() < 1):
        raise ValueError(f"{name}: live_rows must be an int32 tensor on {x.device}")
    return ctypes.c_void_p(live_rows.data_ptr())


# Split-row workspaces: one per (device index, stream handle), of a fixed size
# that covers every call the planner splits (it splits only calls of at most
# GA_SPLIT_PLAN_ROWS rows), zero-filled once and then kept for the life of the
# process.  A workspace is never replaced or released, so a graph captured
# with one keeps a valid pointer for as long as it can be replayed.  Calls
# that share a workspace must not overlap in time: calls on one stream are
# serialised by the stream, and each stream has its own workspace.
_WORKSPACES = {}


def _workspace_key(device, stream):
    return (device.index, stream.cuda_stream)


def reserve_workspace(device=None, stream=None):
    """Create the split-row workspace of `stream` (default: the current stream
    of `device`) now, if it does not exist yet, and return it.  Call this
    before capturing a graph on a stream that has not run a call yet, so the
    workspace is allocated (and zeroed) outside the graph; otherwise the first
    call inside the capture allocates it from the graph's memory pool and
    records its zero fill into the graph, which then re-zeroes it on every
    replay."""
    device = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    if device.index is None:
        device = torch.device("cuda", torch.cuda.current_device())
    stream = torch.cuda.current_stream(device) if stream is None else stream
    key = _workspace_key(device, stream)
    ws = _WORKSPACES.get(key)
    if ws is None:
        with torch.cuda.device(device), torch.cuda.stream(stream):
            ws = torch.zeros(WORKSPACE_BYTES, dtype=torch.uint8, device=device)
        _WORKSPACES[key] = ws
    return ws


def workspace_for(x, T):
    """The split-row workspace for x's device and current stream, or None when
    a call of T rows is never split (T > GA_SPLIT_PLAN_ROWS) and the stream
    has none yet.  Created on first use (see reserve_workspace for graph
    capture) and kept for the life of the process."""
    stream = torch.cuda.current_stream(x.device)
    ws = _WORKSPACES.get(_workspace_key(x.device, stream))
    if ws is None and 0 < T <= GA_SPLIT_PLAN_ROWS:
        ws = reserve_workspace(x.device, stream)
    return ws


def held_workspaces():
    """{(device index, stream handle): data_ptr} of every workspace the
    binding holds."""
    return {k: v.data_ptr() for k, v in _WORKSPACES.items()}


def gelu_and_mul_sparse(x, z=Z_SPARSITY_095, out=None, live_rows=None, plan=None, workspace=None,
                        round_intermediates=False):
    """Sparse GELU-and-multiply of x = [gate | up] ([T, 2d]) -> [T, d].
    z = Phi^-1(target sparsity); live_rows (optional int32 device tensor)
    limits the rows written; plan (optional Plan) forces a launch geometry
    (its `flags` then select the form).  workspace: None = the binding's
    workspace of the current stream (lets few rows split over several
    workgroups; see reserve_workspace), False = none, or a zero-filled uint8
    tensor owned by the caller.  round_intermediates: the
    round-trip form, which rounds each intermediate to the input dtype as an
    eager PyTorch composition does (never split, no workspace)."""
    T, d, out = _prep(x, out, "gelu_and_mul_sparse")
    live = _live_ptr(live_rows, x, "gelu_and_mul_sparse")
    with torch.cuda.device(x.device):
        if round_intermediates:
            if plan is not None:
                raise ValueError("gelu_and_mul_sparse: pass round_intermediates through plan.flags")
            _check(lib.ga_gelu_and_mul_sparse_ex(
                ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(out.data_ptr()), T, d,
                _TORCH_DTYPE[x.dtype], ctypes.c_float(z), live, GA_ROUND_INTERMEDIATES, None, 0,
                _stream_of(x)))
            return out
        if workspace is None:
            workspace = workspace_for(x, T) if T > 0 else None
        elif workspace is False:
            workspace = None
        ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else None
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        args = (ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(out.data_ptr()), T, d,
                _TORCH_DTYPE[x.dtype], ctypes.c_float(z), live)
        if plan is not None:
            _check(lib.ga_gelu_and_mul_sparse_with_plan(*args, ctypes.byref(plan), ws_ptr, ws_bytes,
                                                        _stream_of(x)))
        elif ws_ptr is not None:
            _check(lib.ga_gelu_and_mul_sparse_ws(*args, ws_ptr, ws_bytes, _stream_of(x)))
        else:
            _check(lib.ga_gelu_and_mul_sparse(*args, _stream_of(x)))
    return out


# Workspaces of the fused down projection: per (device index, stream handle),
# zero-filled when created and grown (never shrunk) to the largest size a call
# on that stream has needed.  A grown workspace replaces the old one for later
# calls, but every one ever made is kept for the life of the process, so a
# graph captured with an older one can still be replayed.
GA_DOWN_MAX_ROWS = 256
_DOWN_WORKSPACES = {}


def reserve_down_workspace(nbytes, device=None, stream=None):
    """The fused down projection's workspace of `stream` (default: the current
    stream of `device`), grown to at least `nbytes` if it is smaller (a new
    zero-filled buffer of at least twice the size).  Call it before capturing
    a graph so the buffer is allocated outside the capture."""
    device = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    if device.index is None:
        device = torch.device("cuda", torch.cuda.current_device())
    stream = torch.cuda.current_stream(device) if stream is None else stream
    held = _DOWN_WORKSPACES.setdefault(_workspace_key(device, stream), [])
    if not held or held[-1].numel() < nbytes:
        size = max(int(nbytes), 2 * held[-1].numel() if held else 0, 1 << 20)
        with torch.cuda.device(device), torch.cuda.stream(stream):
            held.append(torch.zeros(size, dtype=torch.uint8, device=device))
    return held[-1]


def plan_gelu_and_mul_sparse_down(T, d, H, dtype=GA_BF16):
    p = DownPlan()
    _check(lib.ga_plan_gelu_and_mul_sparse_down(T, d, H, dtype, ctypes.byref(p)))
    return p


def gelu_and_mul_sparse_down_workspace_bytes(T, d, H, plan=None):
    return int(lib.ga_gelu_and_mul_sparse_down_workspace_bytes(T, d, H, None if plan is None else ctypes.byref(plan)))


def gelu_and_mul_sparse_down(x, w, z=Z_SPARSITY_095, out=None, live_rows=None, plan=None, workspace=None):
    """Sparse GELU-and-multiply of x = [gate | up] ([T, 2d]) fused with the
    down projection: out[T, H] = a . w^T with w [H, d] (a linear layer's
    weight) and a the activation as gelu_and_mul_sparse stores it.  bf16 or
    fp16; T <= GA_DOWN_MAX_ROWS, d a multiple of 8, H a multiple of 16.
    workspace: None = the binding's workspace of the current stream (grown as
    needed, see reserve_down_workspace), or a zero-filled uint8 tensor owned
    by the caller."""
    name = "gelu_and_mul_sparse_down"
    if not isinstance(x, torch.Tensor) or not x.is_cuda or x.dim() != 2 or x.shape[1] % 2 != 0:
        raise ValueError(f"{name}: x must be a [T, 2d] CUDA (HIP) tensor")
    if (not isinstance(w, torch.Tensor) or w.dim() != 2 or w.shape[1] * 2 != x.shape[1]
            or w.dtype != x.dtype or w.device != x.device):
        raise ValueError(f"{name}: w must be a [H, d] tensor of x's dtype on x's device")
    if not x.is_contiguous() or not w.is_contiguous():
        raise ValueError(f"{name}: x and w must be contiguous")
    if x.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError(f"{name}: bf16 or fp16 only, got {x.dtype}")
    T, d, H = x.shape[0], x.shape[1] // 2, w.shape[0]
    if out is None:
        out = torch.empty((T, H), dtype=x.dtype, device=x.device)
    elif (out.shape != (T, H) or out.dtype != x.dtype or out.device != x.device
          or not out.is_contiguous()):
        raise ValueError(f"{name}: out must be a contiguous [{T}, {H}] {x.dtype} tensor on {x.device}")
    live = _live_ptr(live_rows, x, name)
    with torch.cuda.device(x.device):
        p = plan if plan is not None else plan_gelu_and_mul_sparse_down(T, d, H, _TORCH_DTYPE[x.dtype])
        need = gelu_and_mul_sparse_down_workspace_bytes(T, d, H, p)
        if workspace is None and T > 0 and need > 0:
            workspace = reserve_down_workspace(need, x.device)
        ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else None
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        _check(lib.ga_gelu_and_mul_sparse_down_with_plan(
            ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(w.data_ptr()), ctypes.c_void_p(out.data_ptr()),
            T, d, H, _TORCH_DTYPE[x.dtype], ctypes.c_float(z), live, ctypes.byref(p), ws_ptr, ws_bytes,
            _stream_of(x)))
    return out


def gelu_and_mul_sparse_noalloc(x, z=Z_SPARSITY_095, out=None, live_rows=None):
    """gelu_and_mul_sparse for at most GA_SPLIT_PLAN_ROWS rows that uses the
    library's own static split-row array instead of a workspace, for code
    that must not allocate (pass `out` too).  Calls on one device share that
    array: they must not overlap in time."""
    T, d, out = _prep(x, out, "gelu_and_mul_sparse_noalloc")
    live = _live_ptr(live_rows, x, "gelu_and_mul_sparse_noalloc")
    with torch.cuda.device(x.device):
        _check(lib.ga_gelu_and_mul_sparse_noalloc(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                                  T, d, _TORCH_DTYPE[x.dtype], ctypes.c_float(z), live,
                                                  _stream_of(x)))
    return out


def silu_and_mul_bounded(x, live_rows, out=None, plan=None):
    """silu(gate) * up on rows [0, clamp(live_rows[0], 0, M)) of x = [gate | up]
    ([M, 2d]); other rows of `out` are left as they are."""
    M, d, out = _prep(x, out, "silu_and_mul_bounded")
    live = _live_ptr(live_rows, x, "silu_and_mul_bounded")
    if live is None:
        raise ValueError("silu_and_mul_bounded: live_rows is required")
    with torch.cuda.device(x.device):
        args = (ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(out.data_ptr()), M, d,
                _TORCH_DTYPE[x.dtype], live)
        if plan is None:
            _check(lib.ga_silu_and_mul_bounded(*args, _stream_of(x)))
        else:
            _check(lib.ga_silu_and_mul_bounded_with_plan(*args, ctypes.byref(plan), _stream_of(x)))
    return out


def gelu_and_mul(x, approximate="tanh", out=None, live_rows=None):
    """gelu(gate) * up of x = [gate | up] ([T, 2d]) -> [T, d]; approximate
    "tanh" or "none" (the exact erf form); live_rows optional."""
    if approximate not in ("tanh", "none"):
        raise ValueError("gelu_and_mul: approximate must be 'tanh' or 'none'")
    T, d, out = _prep(x, out, "gelu_and_mul")
    live = _live_ptr(live_rows, x, "gelu_and_mul")
    with torch.cuda.device(x.device):
        _check(lib.ga_gelu_and_mul(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(out.data_ptr()), T, d,
                                   _TORCH_DTYPE[x.dtype], 1 if approximate == "tanh" else 0, live,
                                   _stream_of(x)))
    return out


def squared_relu_bounded(x, live_rows, out=None):
    """max(x, 0)^2 on rows [0, clamp(live_rows[0], 0, M)) of x ([M, d], not
    gated); other rows of `out` are left as they are."""
    M, d, out = _prep(x, out, "squared_relu_bounded", gated=False)
    live = _live_ptr(live_rows, x, "squared_relu_bounded")
    if live is None:
        raise ValueError("squared_relu_bounded: live_rows is required")
    with torch.cuda.device(x.device):
        _check(lib.ga_squared_relu_bounded(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(out.data_ptr()), M, d,
                                           _TORCH_DTYPE[x.dtype], live, _stream_of(x)))
    return out


def z_from_sparsity(target_sparsity):
    """Phi^-1(target_sparsity): the cutoff multiplier for a target fraction of
    zeros (0.95 -> 1.6448536...)."""
    return float(lib.ga_z_from_sparsity(float(target_sparsity)))


def stream_xor_rows(x, out=None):
    """Measurement aid: out = first half XOR second half of each row of x,
    16 bytes at a time (the streaming ceiling of this access pattern)."""
    rows, d, out = _prep(x, out, "stream_xor_rows")
    with torch.cuda.device(x.device):
        _check(lib.ga_stream_xor_rows(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                      rows, d * x.element_size(), _stream_of(x)))
    return out


def plan_gelu_and_mul_sparse(T, d, dtype=GA_BF16, aligned=True, num_cus=256, with_workspace=True):
    p = Plan()
    _check(lib.ga_plan_gelu_and_mul_sparse(T, d, dtype, int(aligned), num_cus, int(with_workspace),
                                           ctypes.byref(p)))
    return p


def plan_silu_and_mul_bounded(M, d, dtype=GA_BF16, aligned=True, num_cus=256):
    p = Plan()
    _check(lib.ga_plan_silu_and_mul_bounded(M, d, dtype, int(aligned), num_cus, ctypes.byref(p)))
    return p
