"""Python binding of libmoe_route_sort.so: argument marshalling only.

Every step of the route-sort path (FP32 conversion, bias, grouped top-k,
histogram, prefix, scatter) runs in the HIP kernels behind the C ABI declared
in include/moe_route_sort.h.  This module checks tensors, allocates outputs
when the caller gives none, and forwards raw device pointers and the current
HIP stream.  It fails loudly when the library is not built; there is no
fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple, Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_route_sort.so")

MRS_OK = 0
MRS_ERR_INVALID_ARG = -1
MRS_ERR_NULL_POINTER = -2
MRS_ERR_MISALIGNED = -3
MRS_ERR_WORKSPACE = -4
MRS_ERR_OVERFLOW = -5
MRS_ERR_LAUNCH = -6
MRS_ERR_SCRATCH = -7
MRS_DTYPE_F32 = 0
MRS_DTYPE_BF16 = 1
FLAG_FORCE_SINGLE_WG = 1
FLAG_FORCE_MULTI_WG = 2
FLAG_FORCE_EXACT = 4

EXPORTED = [
    "moe_route_sort",
    "moe_route_sort_ex",
    "moe_route_sort_profiled",
    "moe_route_sort_local",
    "moe_route_sort_static",
    "moe_sort_from_ids",
    "moe_sort_from_ids_counters",
    "moe_route_sort_max_rows",
    "moe_route_sort_max_blocks",
    "moe_route_sort_workspace_bytes",
    "moe_route_sort_strerror",
    "moe_route_sort_sigmoid_probe",
    "moe_route_sort_sigmoid_table_probe",
    "moe_grouped_gemm1",
    "moe_grouped_gemm1_profiled",
    "moe_gate_route_sort",
]

_lib = None


class RouteSortError(RuntimeError):
    def __init__(self, code: int):
        super().__init__(f"moe_route_sort failed ({code}): {strerror(code)}")
        self.code = code


def lib() -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "or python align_moe_route_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    common = [vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, i32, vp, sz, vp]
    L.moe_route_sort.argtypes = common
    L.moe_route_sort.restype = i32
    L.moe_route_sort_ex.argtypes = common + [ctypes.c_uint, vp]
    L.moe_route_sort_ex.restype = i32
    L.moe_route_sort_profiled.argtypes = common + [ctypes.c_uint, vp, vp, vp]
    L.moe_route_sort_profiled.restype = i32
    L.moe_route_sort_local.argtypes = common[:8] + [i32, i32] + common[8:]
    L.moe_route_sort_local.restype = i32
    L.moe_route_sort_static.argtypes = common[:14] + [vp]
    L.moe_route_sort_static.restype = i32
    L.moe_sort_from_ids.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    L.moe_sort_from_ids.restype = i32
    L.moe_sort_from_ids_counters.argtypes = [vp, i32, i32, i32, i32, vp, ctypes.c_int64, vp, vp, vp, vp, sz, vp]
    L.moe_sort_from_ids_counters.restype = i32
    for name in ("moe_route_sort_max_rows", "moe_route_sort_max_blocks"):
        getattr(L, name).argtypes = [i32, i32, i32, i32]
        getattr(L, name).restype = ctypes.c_int64
    L.moe_route_sort_workspace_bytes.argtypes = [i32, i32, i32, i32]
    L.moe_route_sort_workspace_bytes.restype = sz
    L.moe_route_sort_strerror.argtypes = [i32]
    L.moe_route_sort_strerror.restype = ctypes.c_char_p
    L.moe_route_sort_sigmoid_probe.argtypes = [vp, i32, vp, vp, vp]
    L.moe_route_sort_sigmoid_probe.restype = i32
    L.moe_route_sort_sigmoid_table_probe.argtypes = [vp, i32, vp, vp, vp]
    L.moe_route_sort_sigmoid_table_probe.restype = i32
    L.moe_grouped_gemm1.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp]
    L.moe_grouped_gemm1.restype = i32
    L.moe_grouped_gemm1_profiled.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp]
    L.moe_grouped_gemm1_profiled.restype = i32
    L.moe_gate_route_sort.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
    L.moe_gate_route_sort.restype = i32
    _lib = L
    return L


def strerror(code: int) -> str:
    return lib().moe_route_sort_strerror(int(code)).decode()


def max_rows(M: int, E: int, k: int, block: int) -> int:
    return int(lib().moe_route_sort_max_rows(M, E, k, block))


def max_blocks(M: int, E: int, k: int, block: int) -> int:
    return int(lib().moe_route_sort_max_blocks(M, E, k, block))


def workspace_bytes(M: int, E: int, k: int, block: int) -> int:
    v = int(lib().moe_route_sort_workspace_bytes(M, E, k, block))
    if v == ctypes.c_size_t(-1).value:
        raise ValueError("invalid sizes")
    return v


def raw_call(logits_ptr, bias_ptr, M, E, k, n_group, topk_group, block, out_ids_ptr, out_w_ptr,
             sorted_ids_ptr, eob_ptr, npp_ptr, dtype, ws_ptr, ws_bytes, stream_ptr,
             flags: int = 0, stats_ptr=None) -> int:
    """Direct C-ABI call with integer device pointers; returns the MRS code."""
    return int(lib().moe_route_sort_ex(logits_ptr, bias_ptr, M, E, k, n_group, topk_group, block,
                                       out_ids_ptr, out_w_ptr, sorted_ids_ptr, eob_ptr, npp_ptr,
                                       dtype, ws_ptr, ws_bytes, stream_ptr, flags, stats_ptr))


class RouteSortOutput(NamedTuple):
    ids: "torch.Tensor"              # [M, k] int32, ascending expert ids per token
    weights: "torch.Tensor"          # [M, k] float32
    sorted_ids: "torch.Tensor"       # [max_rows] int32; [0, num_post_pad) defined
    expert_of_block: "torch.Tensor"  # [max_blocks] int32; [0, num_post_pad/block) defined
    num_post_pad: "torch.Tensor"     # [1] int32 (device)


# (device, stream handle) -> the workspaces made for that stream, the last the
# largest.  No call reads workspace words that an earlier call left, so one
# buffer serves every shape that fits in it.
_ws_cache = {}


def _workspace(device, stream_handle: int, nbytes: int):
    """A zeroed workspace of at least nbytes for calls on one stream.

    Calls on one stream run in order and share a buffer; calls on different
    streams may overlap in time and each stream gets buffers of its own.  An
    outgrown buffer is kept, not freed, since a captured graph may still hold
    its address; sizes are powers of two, so a stream's buffers add up to less
    than twice the largest."""
    import torch
    bufs = _ws_cache.setdefault((str(device), int(stream_handle)), [])
    if bufs and bufs[-1].numel() >= nbytes:
        return bufs[-1]
    size = 256
    while size < nbytes:
        size *= 2
    bufs.append(torch.zeros(size, dtype=torch.uint8, device=device))
    return bufs[-1]


def _check_tensor(t, dev, dtype, n: int, name: str):
    """t is a contiguous tensor of dtype (any dtype when None) with at least n
    elements on dev; every pointer handed to the library comes through here or
    through a check of the same kind, so no host address reaches a kernel."""
    import torch
    if not (isinstance(t, torch.Tensor) and t.device == dev and (dtype is None or t.dtype == dtype)
            and t.is_contiguous() and t.numel() >= n):
        what = "a" if dtype is None else f"a {dtype}"
        raise ValueError(f"{name} must be {what} contiguous tensor of at least {n} elements on {dev}")


def _check_metadata(sorted_ids, expert_of_block, num_post_pad, rows: int, blocks: int, dev):
    import torch
    for t, n, name in ((sorted_ids, rows, "sorted_ids"), (expert_of_block, blocks, "expert_of_block"),
                       (num_post_pad, 1, "num_post_pad")):
        _check_tensor(t, dev, torch.int32, n, name)


def _check_route_output(out, M: int, k: int, rows: int, blocks: int, dev):
    """A caller's RouteSortOutput: ids and weights exactly [M, k], the metadata
    buffers at least their capacities, all contiguous on dev."""
    import torch
    for t, dtype, name in ((out.ids, torch.int32, "out.ids"), (out.weights, torch.float32, "out.weights")):
        _check_tensor(t, dev, dtype, M * k, name)
        if tuple(t.shape) != (M, k):
            raise ValueError(f"{name} must have shape ({M}, {k})")
    _check_metadata(out.sorted_ids, out.expert_of_block, out.num_post_pad, rows, blocks, dev)


def route_sort(logits, bias, k: int, n_group: int, topk_group: int, block: int, *,
               out: Optional[RouteSortOutput] = None, workspace=None, flags: int = 0,
               stats=None, stream=None, events=None, local=None) -> RouteSortOutput:
    """Run the route-sort path on the GPU.

    logits: [M, E] float32 or bfloat16 CUDA/HIP tensor, contiguous.
    bias:   [E] float32 tensor on the same device.
    out:    optional preallocated RouteSortOutput (reused, nothing else written).
    workspace: optional uint8 tensor of at least workspace_bytes() bytes that
            was zeroed once; by default a cached buffer of the call's stream
            (calls on different streams may then overlap in time).  Make the
            first call on a stream before capturing a graph on it, or the
            allocation and zero fill of that buffer join the graph.
    stats:  optional int32 [3] device tensor (tokens decided by the workgroup-wide
            exact selection / by one wave / with group scores made exact by one wave).
    events: optional list of 6 torch.cuda.Event(enable_timing=True); events
            2i and 2i+1 take the start and end of the call's kernel i (pairs
            past the last kernel are recorded after it); returns
            (output, launches) then.
    local:  optional (begin, count): metadata only for experts
            [begin, begin + count), numbered from 0 (moe_route_sort_local);
            ids and weights stay global.  Not combined with flags, stats or
            events.
    """
    import torch
    if not (isinstance(logits, torch.Tensor) and logits.is_cuda):
        raise ValueError("logits must be a GPU tensor")
    if logits.dim() != 2 or not logits.is_contiguous():
        raise ValueError("logits must be a contiguous [M, E] tensor")
    if logits.dtype == torch.float32:
        dt = MRS_DTYPE_F32
    elif logits.dtype == torch.bfloat16:
        dt = MRS_DTYPE_BF16
    else:
        raise NotImplementedError(f"logits dtype {logits.dtype} (float32 or bfloat16 only)")
    M, E = logits.shape
    if not (isinstance(bias, torch.Tensor) and bias.device == logits.device and
            bias.dtype == torch.float32 and bias.shape == (E,) and bias.is_contiguous()):
        raise ValueError("bias must be a contiguous float32 [E] tensor on the logits' device")
    dev = logits.device
    if local is not None:
        lb, lc = (int(v) for v in local)
        if not (0 <= lb and 1 <= lc and lb + lc <= E):
            raise ValueError("local range must lie inside [0, E) and hold at least one expert")
        if flags or stats is not None or events is not None:
            raise ValueError("a local range is not combined with flags, stats or events")
    EL = E if local is None else lc
    rows = max_rows(M, EL, k, block)
    blocks = max_blocks(M, EL, k, block)
    if rows < 0:
        raise ValueError("invalid sizes or row capacity overflow")
    if out is None:
        out = RouteSortOutput(
            torch.empty((M, k), dtype=torch.int32, device=dev),
            torch.empty((M, k), dtype=torch.float32, device=dev),
            torch.empty((max(rows, 1),), dtype=torch.int32, device=dev),
            torch.empty((max(blocks, 1),), dtype=torch.int32, device=dev),
            torch.empty((1,), dtype=torch.int32, device=dev),
        )
    else:
        _check_route_output(out, M, k, rows, blocks, dev)
    if stats is not None:
        _check_tensor(stats, dev, torch.int32, 3, "stats")
    nbytes = workspace_bytes(M, E, k, block)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    if workspace is None:
        workspace = _workspace(dev, stream.cuda_stream, nbytes) if nbytes else None
    else:
        _check_tensor(workspace, dev, None, 0, "workspace")
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if local is not None:
        rc = int(lib().moe_route_sort_local(
            logits.data_ptr(), bias.data_ptr(), M, E, k, n_group, topk_group, block, lb, lc,
            out.ids.data_ptr(), out.weights.data_ptr(), out.sorted_ids.data_ptr(),
            out.expert_of_block.data_ptr(), out.num_post_pad.data_ptr(), dt, ws_ptr, ws_len, stream.cuda_stream))
        if rc != MRS_OK:
            raise RouteSortError(rc)
        return out
    args = (logits.data_ptr(), bias.data_ptr(), M, E, k, n_group, topk_group, block,
            out.ids.data_ptr(), out.weights.data_ptr(), out.sorted_ids.data_ptr(),
            out.expert_of_block.data_ptr(), out.num_post_pad.data_ptr(), dt, ws_ptr, ws_len,
            stream.cuda_stream, flags, stats.data_ptr() if stats is not None else None)
    if events is not None:
        if len(events) != 6:
            raise ValueError("events must hold 6 torch.cuda.Event objects")
        for ev in events:
            if not ev.cuda_event:
                ev.record(stream)  # torch creates the HIP event on its first record
        handles = (ctypes.c_void_p * 6)(*[ev.cuda_event for ev in events])
        n = ctypes.c_int(0)
        rc = int(lib().moe_route_sort_profiled(*args, handles, ctypes.byref(n)))
        if rc != MRS_OK:
            raise RouteSortError(rc)
        return out, n.value
    rc = int(lib().moe_route_sort_ex(*args))
    if rc != MRS_OK:
        raise RouteSortError(rc)
    return out


def route_sort_static(logits, bias, k: int, n_group: int, topk_group: int, block: int, *,
                      out: Optional[RouteSortOutput] = None, stream=None) -> RouteSortOutput:
    """moe_route_sort_static: the route-sort path with the library's own
    static scratch instead of a workspace (for callers that cannot allocate;
    concurrent calls on one GPU race).  Arguments as for route_sort."""
    import torch
    if not (isinstance(logits, torch.Tensor) and logits.is_cuda and logits.dim() == 2 and logits.is_contiguous()):
        raise ValueError("logits must be a contiguous [M, E] GPU tensor")
    if logits.dtype == torch.float32:
        dt = MRS_DTYPE_F32
    elif logits.dtype == torch.bfloat16:
        dt = MRS_DTYPE_BF16
    else:
        raise NotImplementedError(f"logits dtype {logits.dtype} (float32 or bfloat16 only)")
    M, E = logits.shape
    dev = logits.device
    _check_tensor(bias, dev, torch.float32, E, "bias")
    if bias.shape != (E,):
        raise ValueError("bias must be a float32 [E] tensor")
    rows, blocks = max_rows(M, E, k, block), max_blocks(M, E, k, block)
    if rows < 0:
        raise ValueError("invalid sizes or row capacity overflow")
    if out is None:
        out = RouteSortOutput(torch.empty((M, k), dtype=torch.int32, device=dev),
                              torch.empty((M, k), dtype=torch.float32, device=dev),
                              torch.empty((max(rows, 1),), dtype=torch.int32, device=dev),
                              torch.empty((max(blocks, 1),), dtype=torch.int32, device=dev),
                              torch.empty((1,), dtype=torch.int32, device=dev))
    else:
        _check_route_output(out, M, k, rows, blocks, dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    rc = int(lib().moe_route_sort_static(logits.data_ptr(), bias.data_ptr(), M, E, k, n_group, topk_group, block,
                                         out.ids.data_ptr(), out.weights.data_ptr(), out.sorted_ids.data_ptr(),
                                         out.expert_of_block.data_ptr(), out.num_post_pad.data_ptr(), dt,
                                         stream.cuda_stream))
    if rc != MRS_OK:
        raise RouteSortError(rc)
    return out


def sigmoid_probe(x):
    """Both sigmoid forms of the kernels on a float32 GPU tensor (diagnostics)."""
    import torch
    if not (isinstance(x, torch.Tensor) and x.is_cuda and x.dtype == torch.float32):
        raise ValueError("x must be a float32 GPU tensor")
    x = x.contiguous()
    f = torch.empty_like(x)
    e = torch.empty_like(x)
    rc = lib().moe_route_sort_sigmoid_probe(x.data_ptr(), x.numel(), f.data_ptr(), e.data_ptr(),
                                            torch.cuda.current_stream(x.device).cuda_stream)
    if rc != MRS_OK:
        raise RouteSortError(rc)
    return f, e


def sigmoid_table_probe(bits):
    """Sigmoid of BF16 bit patterns (an int16/uint16-valued GPU tensor) through
    the kernels' LDS table: (single-value form, packed-pair form)."""
    import torch
    if not (isinstance(bits, torch.Tensor) and bits.is_cuda):
        raise ValueError("bits must be a GPU tensor")
    h = bits.contiguous().to(torch.int16)
    o1 = torch.empty(h.shape, dtype=torch.float32, device=h.device)
    o2 = torch.empty_like(o1)
    rc = lib().moe_route_sort_sigmoid_table_probe(h.data_ptr(), h.numel(), o1.data_ptr(), o2.data_ptr(),
                                                  torch.cuda.current_stream(h.device).cuda_stream)
    if rc != MRS_OK:
        raise RouteSortError(rc)
    return o1, o2


class SortOutput(NamedTuple):
    sorted_ids: "torch.Tensor"       # [max_rows] int32; [0, num_post_pad) defined
    expert_of_block: "torch.Tensor"  # [max_blocks] int32
    num_post_pad: "torch.Tensor"     # [1] int32 (device)


def sort_from_ids(ids, E: int, block: int, *, out: Optional[SortOutput] = None, workspace=None,
                  stream=None, counters=None, rows_capacity: Optional[int] = None) -> SortOutput:
    """The two sort phases from caller-given expert ids ([M, k] int32 GPU
    tensor); ids outside [0, E) are dropped routes.

    counters: optional int32 [E] GPU tensor of initial per-expert counters
    (moe_sort_from_ids_counters): counters[e] rows at the head of expert e's
    segment belong to the caller and are not written; the counters advance by
    this call's routes.  rows_capacity (with counters): the sorted_ids entries
    the call may use; by default the length of out.sorted_ids, required when
    no out is given.  If a counter is negative or the rows do not fit,
    num_post_pad reads -1 and nothing else is written."""
    import torch
    if not (isinstance(ids, torch.Tensor) and ids.is_cuda and ids.dtype == torch.int32 and ids.dim() == 2
            and ids.is_contiguous()):
        raise ValueError("ids must be a contiguous int32 [M, k] GPU tensor")
    M, k = ids.shape
    dev = ids.device
    if counters is not None:
        _check_tensor(counters, dev, torch.int32, E, "counters")
        if out is None:
            if rows_capacity is None:
                raise ValueError("rows_capacity is required with counters when no out is given")
            rows, blocks = int(rows_capacity), int(rows_capacity) // block
        else:
            rows = int(out.sorted_ids.numel()) if rows_capacity is None else int(rows_capacity)
            blocks = rows // block
    else:
        rows = max_rows(M, E, k, block)
        blocks = max_blocks(M, E, k, block)
        if rows < 0:
            raise ValueError("invalid sizes or row capacity overflow")
    if out is None:
        out = SortOutput(torch.empty((max(rows, 1),), dtype=torch.int32, device=dev),
                         torch.empty((max(blocks, 1),), dtype=torch.int32, device=dev),
                         torch.empty((1,), dtype=torch.int32, device=dev))
    else:
        _check_metadata(out.sorted_ids, out.expert_of_block, out.num_post_pad, rows, blocks, dev)
    nbytes = workspace_bytes(M, E, k, block)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    if workspace is None:
        workspace = _workspace(dev, stream.cuda_stream, nbytes) if nbytes else None
    else:
        _check_tensor(workspace, dev, None, 0, "workspace")
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if counters is not None:
        rc = int(lib().moe_sort_from_ids_counters(ids.data_ptr() if M else None, M, E, k, block,
                                                  counters.data_ptr(), rows, out.sorted_ids.data_ptr(),
                                                  out.expert_of_block.data_ptr(), out.num_post_pad.data_ptr(),
                                                  ws_ptr, ws_len, stream.cuda_stream))
    else:
        rc = int(lib().moe_sort_from_ids(ids.data_ptr(), M, E, k, block, out.sorted_ids.data_ptr(),
                                         out.expert_of_block.data_ptr(), out.num_post_pad.data_ptr(), ws_ptr,
                                         ws_len, stream.cuda_stream))
    if rc != MRS_OK:
        raise RouteSortError(rc)
    return out


def grouped_gemm1(x, w, sorted_ids, expert_of_block, num_post_pad, k: int, block: int, *,
                  out=None, stream=None, events=None):
    """First grouped GEMM of the MoE over the route-sort metadata
    (include/moe_gemm1.h): y[r] = x[sorted_ids[r] // k] . W[expert_of_block[r // block]]^T
    for sorted rows below num_post_pad, zeros for padding rows.

    x: [M, K] bfloat16, w: [E, N, K] bfloat16, metadata as returned by
    route_sort / sort_from_ids.  Returns y, [max_rows, N] bfloat16 (rows at
    or past num_post_pad are left as they were).  `events` = (start, stop)
    torch.cuda.Event pair stamped by the kernel's own launch."""
    import torch
    if not (isinstance(x, torch.Tensor) and x.is_cuda and x.dtype == torch.bfloat16 and x.dim() == 2
            and x.is_contiguous()):
        raise ValueError("x must be a contiguous bfloat16 [M, K] GPU tensor")
    if not (isinstance(w, torch.Tensor) and w.device == x.device and w.dtype == torch.bfloat16 and w.dim() == 3
            and w.is_contiguous()):
        raise ValueError("w must be a contiguous bfloat16 [E, N, K] tensor on x's device")
    M, K = x.shape
    E, N, K2 = w.shape
    if K2 != K:
        raise ValueError("x and w disagree on K")
    rows = max_rows(M, E, k, block)
    blocks = max_blocks(M, E, k, block)
    if rows < 0:
        raise ValueError("invalid sizes or row capacity overflow")
    _check_metadata(sorted_ids, expert_of_block, num_post_pad, rows, blocks, x.device)
    if out is None:
        out = torch.empty((max(rows, 1), N), dtype=torch.bfloat16, device=x.device)
    elif not (out.device == x.device and out.dtype == torch.bfloat16 and out.is_contiguous()
              and out.dim() == 2 and out.shape[1] == N and out.shape[0] >= rows):
        raise ValueError("out must be a contiguous bfloat16 [max_rows, N] tensor on x's device")
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    args = (x.data_ptr(), w.data_ptr(), sorted_ids.data_ptr(), expert_of_block.data_ptr(),
            num_post_pad.data_ptr(), M, k, E, K, N, block, out.data_ptr(), stream.cuda_stream)
    if events is not None:
        ev0, ev1 = events
        for ev in (ev0, ev1):
            if not ev.cuda_event:
                ev.record(stream)  # torch creates the HIP event on its first record
        rc = int(lib().moe_grouped_gemm1_profiled(*args, ev0.cuda_event, ev1.cuda_event))
    else:
        rc = int(lib().moe_grouped_gemm1(*args))
    if rc != MRS_OK:
        raise RouteSortError(rc)
    return out


def gate_route_sort(hidden, w_gate, bias, k: int, n_group: int, topk_group: int, block: int, *,
                    out: Optional[RouteSortOutput] = None, logits=None, stream=None):
    """Router gate projection then the route-sort path (include/moe_gate.h).

    hidden: [M, H] bfloat16 (M <= 64), w_gate: [E, H] bfloat16, bias: [E]
    float32, all on one GPU.  Returns (logits [M, E] float32, RouteSortOutput)."""
    import torch
    if not (isinstance(hidden, torch.Tensor) and hidden.is_cuda and hidden.dtype == torch.bfloat16 and
            hidden.dim() == 2 and hidden.is_contiguous()):
        raise ValueError("hidden must be a contiguous bfloat16 [M, H] GPU tensor")
    if not (isinstance(w_gate, torch.Tensor) and w_gate.device == hidden.device and
            w_gate.dtype == torch.bfloat16 and w_gate.dim() == 2 and w_gate.is_contiguous()):
        raise ValueError("w_gate must be a contiguous bfloat16 [E, H] tensor on hidden's device")
    M, H = hidden.shape
    E = w_gate.shape[0]
    if w_gate.shape[1] != H:
        raise ValueError("hidden and w_gate disagree on H")
    if not (isinstance(bias, torch.Tensor) and bias.device == hidden.device and bias.dtype == torch.float32 and
            bias.shape == (E,) and bias.is_contiguous()):
        raise ValueError("bias must be a contiguous float32 [E] tensor on hidden's device")
    dev = hidden.device
    rows, blocks = max_rows(M, E, k, block), max_blocks(M, E, k, block)
    if rows < 0:
        raise ValueError("invalid sizes or row capacity overflow")
    if logits is None:
        logits = torch.empty((M, E), dtype=torch.float32, device=dev)
    elif not (logits.dtype == torch.float32 and tuple(logits.shape) == (M, E) and logits.is_contiguous() and
              logits.device == dev):
        raise ValueError("logits must be a contiguous float32 [M, E] tensor on hidden's device")
    if out is None:
        out = RouteSortOutput(torch.empty((M, k), dtype=torch.int32, device=dev),
                              torch.empty((M, k), dtype=torch.float32, device=dev),
                              torch.empty((max(rows, 1),), dtype=torch.int32, device=dev),
                              torch.empty((max(blocks, 1),), dtype=torch.int32, device=dev),
                              torch.empty((1,), dtype=torch.int32, device=dev))
    else:
        _check_route_output(out, M, k, rows, blocks, dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    rc = int(lib().moe_gate_route_sort(hidden.data_ptr(), w_gate.data_ptr(), bias.data_ptr(), M, E, H, k, n_group,
                                       topk_group, block, logits.data_ptr(), out.ids.data_ptr(),
                                       out.weights.data_ptr(), out.sorted_ids.data_ptr(),
                                       out.expert_of_block.data_ptr(), out.num_post_pad.data_ptr(),
                                       stream.cuda_stream))
    if rc != MRS_OK:
        raise RouteSortError(rc)
    return logits, out
