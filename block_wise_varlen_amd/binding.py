"""ctypes binding of libfcp.so: argument marshalling only.

Every function has the name of the C entry point it wraps and does no arithmetic of
its own: it checks dtypes and shapes, fills ``fcp_dims_t``, allocates outputs and the
workspace with torch when the caller passes none, and passes device pointers and
torch's current stream to the library. If libfcp.so is missing the import of any
entry point raises; there is no fallback.
"""
import ctypes
import os

import numpy as np

from .descriptors import PAIR_DTYPE, PAIR_FIELDS, COPY_DTYPE, STAGE_DTYPE

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfcp.so")

FCP_OK, FCP_ERR_INVALID_ARG, FCP_ERR_UNSUPPORTED, FCP_ERR_WORKSPACE, FCP_ERR_HIP, \
    FCP_ERR_INTERNAL = range(6)
FCP_OP_FWD, FCP_OP_MERGE, FCP_OP_BWD, FCP_OP_FWD_FUSED = range(4)

# Every symbol include/fcp.h declares.
SYMBOLS = ("fcp_abi_version", "fcp_status_string", "fcp_last_error", "fcp_validate",
           "fcp_workspace_bytes", "fcp_block_attn_fwd", "fcp_merge_partials",
           "fcp_block_attn_fwd_fused", "fcp_block_attn_fwd_fused_noalloc",
           "fcp_block_attn_bwd", "fcp_timing_enable",
           "fcp_timing_read", "fcp_kernel_name", "fcp_comm_plan", "fcp_pipeline_fwd",
           "fcp_pipeline_workspace_bytes", "fcp_plan_info", "fcp_timing_read_clock",
           "fcp_block_attn_fwd_ex", "fcp_merge_partials_ex", "fcp_block_attn_bwd_ex")
FCP_KERNEL_COUNT = 8
FCP_PIPE_COPY_SHADER = 1
FCP_PIPE_PART_BF16 = 2
FCP_BWD_OVERWRITE = 1
FCP_PART_F32, FCP_PART_BF16 = 0, 1


class FcpError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("%s (%d): %s" % (_status_text(status), status, msg))
        self.status = status


class FcpPair(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int32) for f in PAIR_FIELDS]


class FcpDims(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("q_rows", ctypes.c_int64), ("kv_rows", ctypes.c_int64),
                ("part_rows", ctypes.c_int64)]


assert ctypes.sizeof(FcpPair) == PAIR_DTYPE.itemsize == 32
assert ctypes.sizeof(FcpDims) == 40

_lib = None


def load():
    """Loads libfcp.so once; raises FileNotFoundError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise FileNotFoundError(
            "libfcp.so not built at %s (run python -m block_wise_varlen_amd.build)" % LIB_PATH)
    # torch first: its HIP runtime (soname libamdhip64.so.7) is then the one libfcp.so
    # binds to, so the process has a single runtime. Loaded the other way round, the
    # library would bring in its own copy beside torch's, and the second runtime finds
    # no device.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    D = ctypes.POINTER(FcpDims)
    sig = {
        "fcp_abi_version": (ctypes.c_int, []),
        "fcp_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "fcp_last_error": (ctypes.c_char_p, []),
        "fcp_validate": (ctypes.c_int, [D, P, I32, ctypes.c_int]),
        "fcp_workspace_bytes": (SZ, [D, P, I32, ctypes.c_int]),
        "fcp_block_attn_fwd": (ctypes.c_int, [D, P, P, P, P, I32, P, P, P, SZ, P]),
        "fcp_merge_partials": (ctypes.c_int, [D, P, I32, P, P, P, P, P, SZ, P]),
        "fcp_block_attn_fwd_ex": (ctypes.c_int, [D, P, P, P, P, I32, P, P, I32, P, SZ, P]),
        "fcp_merge_partials_ex": (ctypes.c_int, [D, P, I32, P, P, I32, P, P, P, SZ, P]),
        "fcp_block_attn_fwd_fused": (ctypes.c_int, [D, P, P, P, P, I32, P, P, P, SZ, P]),
        "fcp_block_attn_fwd_fused_noalloc": (ctypes.c_int, [D, P, P, P, P, I32, P, P, P]),
        "fcp_block_attn_bwd": (ctypes.c_int, [D, P, P, P, P, P, P, P, I32, P, P, P, P, SZ,
                                              P]),
        "fcp_block_attn_bwd_ex": (ctypes.c_int, [D, P, P, P, P, P, P, P, I32, P, P, P, I32, P,
                                                 SZ, P]),
        "fcp_timing_enable": (ctypes.c_int, [ctypes.c_int]),
        "fcp_timing_read": (ctypes.c_int, [P, P, I32]),
        "fcp_timing_read_clock": (ctypes.c_int, [P, P, P, I32]),
        "fcp_kernel_name": (ctypes.c_char_p, [ctypes.c_int]),
        "fcp_comm_plan": (ctypes.c_int, [I32, I32, P, P, P, P]),
        "fcp_pipeline_fwd": (ctypes.c_int, [D, P, P, P, P, P, ctypes.c_int64, P, I32, P, P,
                                            I32, P, P, P, P, I32, P, SZ, P, P]),
        "fcp_pipeline_workspace_bytes": (SZ, [D, P, I32, P, P, I32, ctypes.c_int64]),
        "fcp_plan_info": (ctypes.c_int, [D, P, I32, ctypes.c_int, P, I32]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    _lib = lib
    return lib


def _status_text(status):
    try:
        return load().fcp_status_string(status).decode()
    except Exception:
        return "status"


def _check(status):
    if status != FCP_OK:
        raise FcpError(status, load().fcp_last_error().decode())


def _pairs_arg(pairs):
    arr = np.ascontiguousarray(np.asarray(pairs, dtype=PAIR_DTYPE))
    return arr, arr.ctypes.data_as(ctypes.c_void_p), len(arr)


def make_dims(num_q_heads, num_kv_heads, head_dim, q_rows, kv_rows, part_rows=0,
              softmax_scale=0.0):
    return FcpDims(num_q_heads, num_kv_heads, head_dim, float(softmax_scale), int(q_rows),
                   int(kv_rows), int(part_rows))


def _dims_from(q, k, part_rows=0, scale=0.0):
    return make_dims(q.shape[1], k.shape[1], q.shape[2], q.shape[0], k.shape[0], part_rows,
                     scale)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(t, stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, dtype, name):
    import torch
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_contiguous() \
            or t.device.type != "cuda":
        raise TypeError("%s must be a contiguous %s CUDA tensor" % (name, dtype))


def _workspace(size_fn, like, ws, stream=None):
    """The caller's workspace as given (the library checks its size), or a new one of
    size_fn() bytes. A new one is freed when the wrapper returns, while the call may
    still be reading it on ``stream``: it is recorded on that stream, so torch's caching
    allocator hands its memory out again only once the stream has passed the call."""
    import torch
    if ws is not None:
        return ws, ws.numel() * ws.element_size()
    nbytes = size_fn()
    if nbytes == 0:
        return None, 0
    ws = torch.empty(nbytes, dtype=torch.uint8, device=like.device)
    if stream is not None:
        ws.record_stream(stream)
    return ws, nbytes


# ---- host-only entry points -------------------------------------------------------

def fcp_abi_version():
    return load().fcp_abi_version()


def fcp_status_string(status):
    return load().fcp_status_string(status).decode()


def fcp_last_error():
    return load().fcp_last_error().decode()


def fcp_validate(dims, pairs, op):
    arr, p, n = _pairs_arg(pairs)
    return load().fcp_validate(ctypes.byref(dims), p, n, op)


def fcp_workspace_bytes(dims, pairs, op):
    arr, p, n = _pairs_arg(pairs)
    return load().fcp_workspace_bytes(ctypes.byref(dims), p, n, op)


# ---- device entry points ----------------------------------------------------------

PLAN_INFO_FIELDS = ("qitems", "kvitems", "split_tiles", "slots", "multihead_parts",
                    "multihead_offset_parts", "ws_bytes", "q_workgroups", "kv_workgroups",
                    "empty_workgroups", "q_kvheads_per_xcd", "kv_kvheads_per_xcd")


def fcp_plan_info(dims, pairs, op):
    """{field: int} summary of the work lists ``op`` builds (host only)."""
    arr, p, n = _pairs_arg(pairs)
    out = (ctypes.c_int64 * len(PLAN_INFO_FIELDS))()
    _check(load().fcp_plan_info(ctypes.byref(dims), p, n, op, out, len(PLAN_INFO_FIELDS)))
    return dict(zip(PLAN_INFO_FIELDS, (int(x) for x in out)))


def _part_format(o_part):
    import torch
    if o_part.dtype == torch.float32:
        return FCP_PART_F32
    if o_part.dtype == torch.bfloat16:
        return FCP_PART_BF16
    raise TypeError("o_part must be float32 or bfloat16")


def fcp_block_attn_fwd(q, k, v, pairs, o_part=None, lse_part=None, part_rows=None,
                       softmax_scale=0.0, ws=None, stream=None, part_dtype=None):
    """Per-pair partials. Returns (o_part [part_rows, Hq, D], lse_part fp32 [part_rows,
    Hq]); o_part is fp32 (fcp_block_attn_fwd) or, with part_dtype=torch.bfloat16 or a
    bf16 o_part, bf16 (fcp_block_attn_fwd_ex, FCP_PART_BF16)."""
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, torch.bfloat16, n)
    arr, p, n = _pairs_arg(pairs)
    if part_rows is None:
        part_rows = o_part.shape[0] if o_part is not None else \
            int((arr["out_row"] + arr["q_len"]).max()) if n else 0
    if o_part is None:
        o_part = torch.empty((part_rows, q.shape[1], q.shape[2]),
                             dtype=part_dtype or torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((part_rows, q.shape[1]), dtype=torch.float32, device=q.device)
    fmt = _part_format(o_part)
    _need(o_part, o_part.dtype, "o_part")
    _need(lse_part, torch.float32, "lse_part")
    dims = _dims_from(q, k, part_rows, softmax_scale)
    lib = load()
    ws, wsb = _workspace(lambda: lib.fcp_workspace_bytes(ctypes.byref(dims), p, n, FCP_OP_FWD),
                         q, ws, stream)
    if fmt == FCP_PART_F32:
        _check(lib.fcp_block_attn_fwd(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), p, n,
                                      _ptr(o_part), _ptr(lse_part), _ptr(ws), wsb,
                                      _stream(q, stream)))
    else:
        _check(lib.fcp_block_attn_fwd_ex(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), p, n,
                                         _ptr(o_part), _ptr(lse_part), fmt, _ptr(ws), wsb,
                                         _stream(q, stream)))
    return o_part, lse_part


def fcp_merge_partials(pairs, o_part, lse_part, q_rows, num_kv_heads=1, o=None, lse=None,
                       ws=None, stream=None):
    """LSE merge of fp32 or bf16 partials into bf16 o [q_rows, Hq, D] and fp32 lse
    [q_rows, Hq]. Rows no pair covers keep their previous contents (zeros when allocated
    here)."""
    import torch
    fmt = _part_format(o_part)
    _need(o_part, o_part.dtype, "o_part")
    _need(lse_part, torch.float32, "lse_part")
    hq, d = o_part.shape[1], o_part.shape[2]
    if o is None:
        o = torch.zeros((q_rows, hq, d), dtype=torch.bfloat16, device=o_part.device)
    if lse is None:
        lse = torch.zeros((q_rows, hq), dtype=torch.float32, device=o_part.device)
    _need(o, torch.bfloat16, "o")
    _need(lse, torch.float32, "lse")
    arr, p, n = _pairs_arg(pairs)
    dims = make_dims(hq, num_kv_heads, d, q_rows, 0, o_part.shape[0])
    lib = load()
    ws, wsb = _workspace(
        lambda: lib.fcp_workspace_bytes(ctypes.byref(dims), p, n, FCP_OP_MERGE), o_part, ws,
        stream)
    _check(lib.fcp_merge_partials_ex(ctypes.byref(dims), p, n, _ptr(o_part), _ptr(lse_part),
                                     fmt, _ptr(o), _ptr(lse), _ptr(ws), wsb,
                                     _stream(o_part, stream)))
    return o, lse


def fcp_block_attn_fwd_fused(q, k, v, pairs, o=None, lse=None, softmax_scale=0.0, ws=None,
                             stream=None):
    """Forward with the merge folded in: bf16 o [q_rows, Hq, D], fp32 lse [q_rows, Hq]."""
    import torch
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, torch.bfloat16, nm)
    if o is None:
        o = torch.zeros_like(q)
    if lse is None:
        lse = torch.zeros((q.shape[0], q.shape[1]), dtype=torch.float32, device=q.device)
    _need(o, torch.bfloat16, "o")
    _need(lse, torch.float32, "lse")
    arr, p, n = _pairs_arg(pairs)
    dims = _dims_from(q, k, 0, softmax_scale)
    lib = load()
    ws, wsb = _workspace(
        lambda: lib.fcp_workspace_bytes(ctypes.byref(dims), p, n, FCP_OP_FWD_FUSED), q, ws,
        stream)
    _check(lib.fcp_block_attn_fwd_fused(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), p, n,
                                        _ptr(o), _ptr(lse), _ptr(ws), wsb, _stream(q, stream)))
    return o, lse


def fcp_block_attn_fwd_fused_noalloc(q, k, v, pairs, o=None, lse=None, softmax_scale=0.0,
                                     stream=None):
    """fcp_block_attn_fwd_fused with its work lists in the library's static device array
    (no workspace argument; the library allocates nothing). Outputs are allocated here
    only when not given."""
    import torch
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, torch.bfloat16, nm)
    if o is None:
        o = torch.zeros_like(q)
    if lse is None:
        lse = torch.zeros((q.shape[0], q.shape[1]), dtype=torch.float32, device=q.device)
    _need(o, torch.bfloat16, "o")
    _need(lse, torch.float32, "lse")
    arr, p, n = _pairs_arg(pairs)
    dims = _dims_from(q, k, 0, softmax_scale)
    _check(load().fcp_block_attn_fwd_fused_noalloc(ctypes.byref(dims), _ptr(q), _ptr(k),
                                                   _ptr(v), p, n, _ptr(o), _ptr(lse),
                                                   _stream(q, stream)))
    return o, lse


def fcp_block_attn_bwd(q, k, v, o, lse, dout, pairs, dq=None, dk=None, dv=None,
                       softmax_scale=0.0, ws=None, stream=None, overwrite=False):
    """Adds gradients into fp32 dq, dk, dv (allocated zeroed here when not given); with
    overwrite=True (fcp_block_attn_bwd_ex, FCP_BWD_OVERWRITE) writes them instead, in
    the rows the pairs cover, leaving other rows as they were."""
    import torch
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _need(t, torch.bfloat16, nm)
    _need(lse, torch.float32, "lse")
    if dq is None:
        dq = torch.zeros(q.shape, dtype=torch.float32, device=q.device)
    if dk is None:
        dk = torch.zeros(k.shape, dtype=torch.float32, device=q.device)
    if dv is None:
        dv = torch.zeros(v.shape, dtype=torch.float32, device=q.device)
    for t, nm in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _need(t, torch.float32, nm)
    arr, p, n = _pairs_arg(pairs)
    dims = _dims_from(q, k, 0, softmax_scale)
    lib = load()
    ws, wsb = _workspace(lambda: lib.fcp_workspace_bytes(ctypes.byref(dims), p, n, FCP_OP_BWD),
                         q, ws, stream)
    if overwrite:
        _check(lib.fcp_block_attn_bwd_ex(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                         _ptr(lse), _ptr(dout), p, n, _ptr(dq), _ptr(dk),
                                         _ptr(dv), FCP_BWD_OVERWRITE, _ptr(ws), wsb,
                                         _stream(q, stream)))
    else:
        _check(lib.fcp_block_attn_bwd(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                      _ptr(lse), _ptr(dout), p, n, _ptr(dq), _ptr(dk),
                                      _ptr(dv), _ptr(ws), wsb, _stream(q, stream)))
    return dq, dk, dv


def _table(x, dtype):
    arr = np.ascontiguousarray(np.asarray(x, dtype=dtype))
    return arr, arr.ctypes.data_as(ctypes.c_void_p), len(arr)


def fcp_pipeline_workspace_bytes(dims, stages, copies, pairs, src_rows, depth=2):
    st, sp, ns = _table(stages, STAGE_DTYPE)
    cp, cpp, _ = _table(copies, COPY_DTYPE)
    pr, pp, _ = _table(pairs, PAIR_DTYPE)
    return load().fcp_pipeline_workspace_bytes(ctypes.byref(dims), sp, ns, cpp, pp, int(depth),
                                               int(src_rows))


def fcp_pipeline_fwd(q, k, v, k_src, v_src, stages, copies, pairs, o_part, lse_part, o=None,
                     lse=None, depth=2, flags=0, softmax_scale=0.0, ws=None, stream=None,
                     copy_stream=None):
    """Pipelined forward: per stage, copies from k_src/v_src into k/v on ``copy_stream``
    (after stage s-depth has computed) overlapping the pairs of earlier stages on
    ``stream``; then the merge into o/lse. ``copy_stream=None`` uses ``stream`` (no
    overlap). k and v are written."""
    import torch
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (k_src, "k_src"), (v_src, "v_src")):
        _need(t, torch.bfloat16, nm)
    if _part_format(o_part) == FCP_PART_BF16:
        flags = int(flags) | FCP_PIPE_PART_BF16
    _need(o_part, o_part.dtype, "o_part")
    _need(lse_part, torch.float32, "lse_part")
    if o is None:
        o = torch.zeros_like(q)
    if lse is None:
        lse = torch.zeros((q.shape[0], q.shape[1]), dtype=torch.float32, device=q.device)
    _need(o, torch.bfloat16, "o")
    _need(lse, torch.float32, "lse")
    if k_src.shape[1:] != k.shape[1:] or v_src.shape != k_src.shape or v.shape != k.shape:
        raise ValueError("k/v and k_src/v_src must have matching row layouts")
    st, sp, ns = _table(stages, STAGE_DTYPE)
    cp, cpp, _ = _table(copies, COPY_DTYPE)
    pr, pp, _ = _table(pairs, PAIR_DTYPE)
    dims = _dims_from(q, k, o_part.shape[0], softmax_scale)
    lib = load()
    src_rows = k_src.shape[0]
    ws, wsb = _workspace(lambda: lib.fcp_pipeline_workspace_bytes(ctypes.byref(dims), sp, ns,
                                                                  cpp, pp, int(depth), src_rows),
                         q, ws, stream)
    s = _stream(q, stream)
    cs = s if copy_stream is None else ctypes.c_void_p(copy_stream.cuda_stream)
    _check(lib.fcp_pipeline_fwd(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(k_src),
                                _ptr(v_src), src_rows, sp, ns, cpp, pp, int(depth), _ptr(o_part),
                                _ptr(lse_part), _ptr(o), _ptr(lse), int(flags), _ptr(ws), wsb,
                                s, cs))
    return o, lse


# ---- per-kernel timing ------------------------------------------------------------

def fcp_timing_enable(on=True):
    _check(load().fcp_timing_enable(1 if on else 0))


def fcp_kernel_name(kid):
    return load().fcp_kernel_name(kid).decode()


def fcp_timing_read():
    """{kernel name: (total ms, launches)} since the last read (waits for the events)."""
    tot = (ctypes.c_double * FCP_KERNEL_COUNT)()
    cnt = (ctypes.c_int32 * FCP_KERNEL_COUNT)()
    _check(load().fcp_timing_read(ctypes.cast(tot, ctypes.c_void_p),
                                  ctypes.cast(cnt, ctypes.c_void_p), FCP_KERNEL_COUNT))
    return {fcp_kernel_name(i): (tot[i], cnt[i]) for i in range(FCP_KERNEL_COUNT) if cnt[i]}


def fcp_timing_read_clock():
    """{kernel name: (total ms, launches, average shader clock in MHz or 0)} since the last
    read (waits for the events)."""
    tot = (ctypes.c_double * FCP_KERNEL_COUNT)()
    cnt = (ctypes.c_int32 * FCP_KERNEL_COUNT)()
    mhz = (ctypes.c_double * FCP_KERNEL_COUNT)()
    _check(load().fcp_timing_read_clock(ctypes.cast(tot, ctypes.c_void_p),
                                        ctypes.cast(cnt, ctypes.c_void_p),
                                        ctypes.cast(mhz, ctypes.c_void_p), FCP_KERNEL_COUNT))
    return {fcp_kernel_name(i): (tot[i], cnt[i], mhz[i]) for i in range(FCP_KERNEL_COUNT)
            if cnt[i]}


# ---- congestion-free communication plan (host only) --------------------------------

def fcp_comm_plan(n_workers, src, dst):
    """(stage per edge as int32 ndarray, number of stages) for the transfers src[e] -> dst[e]."""
    src = np.ascontiguousarray(src, dtype=np.int32)
    dst = np.ascontiguousarray(dst, dtype=np.int32)
    if src.shape != dst.shape or src.ndim != 1:
        raise ValueError("src and dst must be 1-D arrays of equal length")
    stage = np.empty_like(src)
    n = ctypes.c_int32(0)
    _check(load().fcp_comm_plan(int(n_workers), int(src.size), src.ctypes.data_as(ctypes.c_void_p),
                                dst.ctypes.data_as(ctypes.c_void_p),
                                stage.ctypes.data_as(ctypes.c_void_p),
                                ctypes.cast(ctypes.byref(n), ctypes.c_void_p)))
    return stage, n.value
