"""Python binding of the VSA C ABI in libvsa_amd.so (include/vsa.h).

Argument marshalling only: every step of the hot path runs in the library's
HIP kernels.  Functions carry the C names.  Tensor arguments may be torch
tensors (their device pointer is passed and their size and dtype are checked
against what the call will touch) or raw integer device addresses.  Streams
default to torch's current stream on the tensors' device.

The library must have been built (python -m block_sparse_video_tile_amd.build);
loading fails loudly otherwise -- there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import re

__all__ = [
    "VsaError", "Plan", "lib_path", "load_library", "exported_symbols",
    "VSA_OK", "VSA_ERR_INVALID_ARGUMENT", "VSA_ERR_UNSUPPORTED", "VSA_ERR_HIP",
    "VSA_DTYPE_BF16", "VSA_DTYPE_FP16", "VSA_ROLE_Q", "VSA_ROLE_K", "VSA_ROLE_V",
    "vsa_plan", "vsa_plan_destroy", "vsa_plan_get_info", "vsa_plan_describe",
    "vsa_plan_block_counts", "vsa_gather", "vsa_scatter", "vsa_score_topk",
    "vsa_block_sparse_attn_fwd", "vsa_block_sparse_attn_bwd_workspace_size",
    "vsa_block_sparse_attn_bwd", "vsa_compress_attn", "vsa_scatter_gated",
    "vsa_forward_workspace_size", "vsa_forward", "vsa_block_sparse_attn_fwd_raster",
    "vsa_forward_fused_workspace_size", "vsa_forward_fused", "vsa_attn_fwd_workspace_size",
    "vsa_block_sparse_attn_fwd_ws", "vsa_block_sparse_attn_fwd_raster_ws", "vsa_status_string",
    "vsa_last_error", "vsa_bench_mfma_peak", "vsa_bench_hbm_copy",
    "vsa_block_sparse_attn_fwd_noalloc",
]

VSA_OK, VSA_ERR_INVALID_ARGUMENT, VSA_ERR_UNSUPPORTED, VSA_ERR_HIP = 0, 1, 2, 3
VSA_DTYPE_BF16, VSA_DTYPE_FP16 = 0, 1
VSA_ROLE_Q, VSA_ROLE_K, VSA_ROLE_V = 0, 1, 2

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
_HEADER = os.path.join(os.path.dirname(_PKG_DIR), "include", "vsa.h")


def lib_path() -> str:
    """The library to load: libvsa_amd.so of this package, or the file named by
    VSA_LIBRARY (the host-sanitizer build of the host-only tests)."""
    return os.environ.get("VSA_LIBRARY") or os.path.join(_PKG_DIR, "libvsa_amd.so")


class VsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


class _PlanDesc(ctypes.Structure):
    _fields_ = [("seq_len", ctypes.c_int64), ("dit_seq_shape", ctypes.c_int32 * 3),
                ("block_size", ctypes.c_int32 * 3), ("batch", ctypes.c_int32),
                ("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class _PlanInfo(ctypes.Structure):
    _fields_ = [("block_grid", ctypes.c_int32 * 3), ("num_blocks", ctypes.c_int32),
                ("block_volume", ctypes.c_int32), ("padded_len", ctypes.c_int64),
                ("blocked_elems", ctypes.c_int64), ("pooled_elems", ctypes.c_int64),
                ("num_rows", ctypes.c_int64)]


_P = ctypes.c_void_p
_SIGS = {
    "vsa_plan": ([ctypes.POINTER(_PlanDesc), ctypes.POINTER(_P)], ctypes.c_int),
    "vsa_plan_destroy": ([_P], ctypes.c_int),
    "vsa_plan_get_info": ([_P, ctypes.POINTER(_PlanInfo)], ctypes.c_int),
    "vsa_plan_describe": ([_P, ctypes.c_char_p, ctypes.c_size_t], ctypes.c_int),
    "vsa_plan_block_counts": ([_P, ctypes.POINTER(ctypes.c_int32), ctypes.c_int64], ctypes.c_int),
    "vsa_gather": ([_P, ctypes.c_int32, _P, _P, _P, _P], ctypes.c_int),
    "vsa_scatter": ([_P, _P, _P, _P], ctypes.c_int),
    "vsa_score_topk": ([_P, _P, _P, ctypes.c_int32, _P, _P, _P], ctypes.c_int),
    "vsa_block_sparse_attn_fwd": ([_P, _P, _P, _P, _P, _P, ctypes.c_int32, ctypes.c_int64, _P,
                                   _P, _P], ctypes.c_int),
    "vsa_forward_workspace_size": ([_P, ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "vsa_block_sparse_attn_bwd_workspace_size": ([_P, ctypes.POINTER(ctypes.c_size_t)],
                                                 ctypes.c_int),
    "vsa_block_sparse_attn_bwd": ([_P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int32,
                                   ctypes.c_int64, _P, _P, _P, _P, ctypes.c_size_t, _P],
                                  ctypes.c_int),
    "vsa_compress_attn": ([_P, _P, _P, _P, _P, _P], ctypes.c_int),
    "vsa_scatter_gated": ([_P, _P, _P, _P, _P, _P], ctypes.c_int),
    "vsa_forward": ([_P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P, _P, _P], ctypes.c_int),
    "vsa_block_sparse_attn_fwd_raster": ([_P, _P, _P, _P, _P, _P, ctypes.c_int32, ctypes.c_int64,
                                          _P, _P, _P, _P, _P], ctypes.c_int),
    "vsa_forward_fused_workspace_size": ([_P, ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "vsa_forward_fused": ([_P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P, _P, _P],
                          ctypes.c_int),
    "vsa_attn_fwd_workspace_size": ([_P, ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "vsa_block_sparse_attn_fwd_ws": ([_P, _P, _P, _P, _P, _P, ctypes.c_int32, ctypes.c_int64, _P,
                                      _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "vsa_block_sparse_attn_fwd_raster_ws": ([_P, _P, _P, _P, _P, _P, ctypes.c_int32,
                                             ctypes.c_int64, _P, _P, _P, _P, _P, ctypes.c_size_t,
                                             _P], ctypes.c_int),
    "vsa_block_sparse_attn_fwd_noalloc": ([_P, _P, _P, _P, _P, _P, ctypes.c_int32, ctypes.c_int64,
                                           _P, _P, _P], ctypes.c_int),
    "vsa_bench_mfma_peak": ([ctypes.c_int32, ctypes.c_int32, _P, ctypes.POINTER(ctypes.c_int64),
                             _P], ctypes.c_int),
    "vsa_bench_hbm_copy": ([_P, _P, ctypes.c_int64, _P], ctypes.c_int),
    "vsa_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "vsa_last_error": ([], ctypes.c_char_p),
}

_LIB = None


def load_library():
    """Load libvsa_amd.so once; raise if it has not been built."""
    global _LIB
    if _LIB is None:
        path = lib_path()
        if not os.path.exists(path):
            raise VsaError(VSA_ERR_HIP, f"{path} is not built; run "
                           "`python -m block_sparse_video_tile_amd.build` first")
        lib = ctypes.CDLL(path)
        for name, (args, res) in _SIGS.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _LIB = lib
    return _LIB


def exported_symbols():
    """Function names declared in include/vsa.h."""
    with open(_HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:vsa_status|const char\*)\s+(vsa_\w+)\s*\(", text, re.M)))


def _status_name(st: int) -> str:
    return {0: "VSA_OK", 1: "VSA_ERR_INVALID_ARGUMENT", 2: "VSA_ERR_UNSUPPORTED",
            3: "VSA_ERR_HIP"}.get(st, f"status {st}")


def _check(st: int):
    if st != VSA_OK:
        raise VsaError(st, load_library().vsa_last_error().decode())


def vsa_status_string(status: int) -> str:
    return load_library().vsa_status_string(status).decode()


def vsa_last_error() -> str:
    return load_library().vsa_last_error().decode()


# ------------------------------------------------------------------ plans

class Plan:
    """Owning handle of a vsa_plan_t (destroyed with the object)."""

    def __init__(self, handle, desc: _PlanDesc):
        self.handle = handle
        self.desc = desc
        self.info = vsa_plan_get_info(self)

    def __del__(self):
        h, self.handle = getattr(self, "handle", None), None
        if h and _LIB is not None:
            _LIB.vsa_plan_destroy(h)

    # shapes of the buffers each call touches
    @property
    def batch(self):
        return self.desc.batch

    @property
    def heads(self):
        return self.desc.num_heads

    @property
    def head_dim(self):
        return self.desc.head_dim

    @property
    def seq_len(self):
        return self.desc.seq_len

    @property
    def topk(self):
        return self.desc.topk

    @property
    def num_blocks(self):
        return self.info["num_blocks"]

    @property
    def dtype(self):
        return self.desc.dtype

    def torch_dtype(self):
        """torch element type of the Q, K, V and O tensors of this plan."""
        import torch
        return torch.float16 if self.desc.dtype == VSA_DTYPE_FP16 else torch.bfloat16

    @property
    def padded_len(self):
        return self.info["padded_len"]

    def raster_shape(self):
        return (self.batch, self.seq_len, self.heads, self.head_dim)

    def blocked_shape(self):
        return (self.batch, self.heads, self.padded_len, self.head_dim)

    def blocked_vt_shape(self):
        return (self.batch, self.heads, self.padded_len // 64, self.head_dim, 64)

    def pooled_shape(self):
        return (self.batch, self.heads, self.num_blocks, self.head_dim)

    def num_rows(self):
        return self.info["num_rows"]


def vsa_plan(seq_len, dit_seq_shape, block_size, batch=1, num_heads=1, head_dim=128, topk=0,
             dtype=VSA_DTYPE_BF16) -> Plan:
    desc = _PlanDesc(int(seq_len), (ctypes.c_int32 * 3)(*[int(x) for x in dit_seq_shape]),
                     (ctypes.c_int32 * 3)(*[int(x) for x in block_size]), int(batch),
                     int(num_heads), int(head_dim), int(topk), int(dtype))
    h = _P()
    _check(load_library().vsa_plan(ctypes.byref(desc), ctypes.byref(h)))
    return Plan(h, desc)


def vsa_plan_destroy(plan: Plan):
    h, plan.handle = plan.handle, None
    _check(load_library().vsa_plan_destroy(h))


def vsa_plan_get_info(plan: Plan) -> dict:
    info = _PlanInfo()
    _check(load_library().vsa_plan_get_info(plan.handle, ctypes.byref(info)))
    return {"block_grid": tuple(info.block_grid), "num_blocks": info.num_blocks,
            "block_volume": info.block_volume, "padded_len": info.padded_len,
            "blocked_elems": info.blocked_elems, "pooled_elems": info.pooled_elems,
            "num_rows": info.num_rows}


def vsa_plan_describe(plan: Plan, buf_len: int = 512) -> str:
    buf = ctypes.create_string_buffer(buf_len)
    _check(load_library().vsa_plan_describe(plan.handle, buf, buf_len))
    return buf.value.decode()


def vsa_plan_block_counts(plan: Plan):
    n = plan.num_blocks
    arr = (ctypes.c_int32 * n)()
    _check(load_library().vsa_plan_block_counts(plan.handle, arr, n))
    return list(arr)


# ------------------------------------------------------------------ device calls

def _ptr(x, numel=None, dtype=None, name="tensor"):
    """Device address of a torch tensor (size/dtype checked) or a raw int; None -> NULL."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    import torch
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor, an int address or None")
    if x.device.type != "cuda":
        raise ValueError(f"{name}: must be a device tensor, got {x.device}")
    if not x.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype is not None and x.dtype != dtype:
        raise ValueError(f"{name}: dtype {x.dtype}, expected {dtype}")
    if numel is not None and x.numel() < numel:
        raise ValueError(f"{name}: {x.numel()} elements < {numel} required")
    return x.data_ptr()


def _stream(stream, *tensors):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    for t in tensors:
        if isinstance(t, torch.Tensor) and t.device.type == "cuda":
            return torch.cuda.current_stream(t.device).cuda_stream
    return None


def _f32():
    import torch
    return torch.float32


def _i32():
    import torch
    return torch.int32


def vsa_gather(plan: Plan, role: int, x_raster, x_blk, pooled=None, stream=None):
    n_raster = plan.batch * plan.seq_len * plan.heads * plan.head_dim
    et = plan.torch_dtype()
    _check(load_library().vsa_gather(
        plan.handle, int(role), _ptr(x_raster, n_raster, et, "x_raster"),
        _ptr(x_blk, plan.info["blocked_elems"], et, "x_blk"),
        _ptr(pooled, plan.info["pooled_elems"], _f32(), "pooled"),
        _stream(stream, x_raster, x_blk)))


def vsa_scatter(plan: Plan, o_blk, o_raster, stream=None):
    n_raster = plan.batch * plan.seq_len * plan.heads * plan.head_dim
    et = plan.torch_dtype()
    _check(load_library().vsa_scatter(
        plan.handle, _ptr(o_blk, plan.info["blocked_elems"], et, "o_blk"),
        _ptr(o_raster, n_raster, et, "o_raster"), _stream(stream, o_blk, o_raster)))


def vsa_score_topk(plan: Plan, q_pooled, k_pooled, topk: int, col_idx, scores=None, stream=None):
    rows = plan.num_rows()
    _check(load_library().vsa_score_topk(
        plan.handle, _ptr(q_pooled, plan.info["pooled_elems"], _f32(), "q_pooled"),
        _ptr(k_pooled, plan.info["pooled_elems"], _f32(), "k_pooled"), int(topk),
        _ptr(col_idx, rows * max(int(topk), 0), _i32(), "col_idx"),
        _ptr(scores, rows * plan.num_blocks, _f32(), "scores"),
        _stream(stream, q_pooled, col_idx)))


def vsa_block_sparse_attn_fwd(plan: Plan, q_blk, k_blk, v_blk, row_ptr, col_idx, uniform_k: int,
                              nnz: int, o_blk, lse=None, stream=None):
    be = plan.info["blocked_elems"]
    rows = plan.num_rows()
    et = plan.torch_dtype()
    _check(load_library().vsa_block_sparse_attn_fwd(
        plan.handle, _ptr(q_blk, be, et, "q_blk"), _ptr(k_blk, be, et, "k_blk"),
        _ptr(v_blk, be, et, "v_blk"), _ptr(row_ptr, rows + 1, _i32(), "row_ptr"),
        _ptr(col_idx, int(nnz), _i32(), "col_idx"), int(uniform_k), int(nnz),
        _ptr(o_blk, be, et, "o_blk"),
        _ptr(lse, plan.batch * plan.heads * plan.padded_len, _f32(), "lse"),
        _stream(stream, q_blk, o_blk)))


def vsa_block_sparse_attn_fwd_raster(plan: Plan, q, k, v, row_ptr, col_idx, uniform_k: int,
                                     nnz: int, o_raster, lse=None, stream=None, gate=None,
                                     o_coarse=None):
    """Block-sparse attention on raster [B,S,NH,D] tensors (no gather/scatter);
    with gate and o_coarse the rows are written as vsa_scatter_gated writes them."""
    n_raster = plan.batch * plan.seq_len * plan.heads * plan.head_dim
    rows = plan.num_rows()
    et = plan.torch_dtype()
    _check(load_library().vsa_block_sparse_attn_fwd_raster(
        plan.handle, _ptr(q, n_raster, et, "q"), _ptr(k, n_raster, et, "k"),
        _ptr(v, n_raster, et, "v"), _ptr(row_ptr, rows + 1, _i32(), "row_ptr"),
        _ptr(col_idx, int(nnz), _i32(), "col_idx"), int(uniform_k), int(nnz),
        _ptr(gate, n_raster, et, "gate"),
        _ptr(o_coarse, plan.info["pooled_elems"], _f32(), "o_coarse"),
        _ptr(o_raster, n_raster, et, "o_raster"),
        _ptr(lse, plan.batch * plan.heads * plan.padded_len, _f32(), "lse"),
        _stream(stream, q, o_raster)))


def vsa_attn_fwd_workspace_size(plan: Plan) -> int:
    n = ctypes.c_size_t()
    _check(load_library().vsa_attn_fwd_workspace_size(plan.handle, ctypes.byref(n)))
    return n.value


def _workspace(workspace, ws_bytes):
    """Device pointer and byte size of a workspace tensor (or a raw pointer)."""
    import torch
    if isinstance(workspace, torch.Tensor):
        if workspace.numel() * workspace.element_size() < ws_bytes:
            raise ValueError(f"workspace: fewer than {ws_bytes} bytes")
        return _ptr(workspace, name="workspace"), workspace.numel() * workspace.element_size()
    return int(workspace), ws_bytes


def vsa_block_sparse_attn_fwd_ws(plan: Plan, q_blk, k_blk, v_blk, row_ptr, col_idx,
                                 uniform_k: int, nnz: int, o_blk, workspace, lse=None,
                                 stream=None):
    """vsa_block_sparse_attn_fwd with rows claimed from per-XCD queues (balanced launch)."""
    be = plan.info["blocked_elems"]
    rows = plan.num_rows()
    et = plan.torch_dtype()
    ws_ptr, ws_len = _workspace(workspace, vsa_attn_fwd_workspace_size(plan))
    _check(load_library().vsa_block_sparse_attn_fwd_ws(
        plan.handle, _ptr(q_blk, be, et, "q_blk"), _ptr(k_blk, be, et, "k_blk"),
        _ptr(v_blk, be, et, "v_blk"), _ptr(row_ptr, rows + 1, _i32(), "row_ptr"),
        _ptr(col_idx, int(nnz), _i32(), "col_idx"), int(uniform_k), int(nnz),
        _ptr(o_blk, be, et, "o_blk"),
        _ptr(lse, plan.batch * plan.heads * plan.padded_len, _f32(), "lse"),
        ws_ptr, ws_len, _stream(stream, q_blk, o_blk)))


def vsa_block_sparse_attn_fwd_noalloc(plan: Plan, q_blk, k_blk, v_blk, row_ptr, col_idx,
                                      uniform_k: int, nnz: int, o_blk, lse=None, stream=None):
    """The balanced launch with its row queues in the library's static device
    scratch (no workspace, no allocation); calls on one GPU must not overlap."""
    be = plan.info["blocked_elems"]
    rows = plan.num_rows()
    et = plan.torch_dtype()
    _check(load_library().vsa_block_sparse_attn_fwd_noalloc(
        plan.handle, _ptr(q_blk, be, et, "q_blk"), _ptr(k_blk, be, et, "k_blk"),
        _ptr(v_blk, be, et, "v_blk"), _ptr(row_ptr, rows + 1, _i32(), "row_ptr"),
        _ptr(col_idx, int(nnz), _i32(), "col_idx"), int(uniform_k), int(nnz),
        _ptr(o_blk, be, et, "o_blk"),
        _ptr(lse, plan.batch * plan.heads * plan.padded_len, _f32(), "lse"),
        _stream(stream, q_blk, o_blk)))


def vsa_block_sparse_attn_fwd_raster_ws(plan: Plan, q, k, v, row_ptr, col_idx, uniform_k: int,
                                        nnz: int, o_raster, workspace, lse=None, stream=None,
                                        gate=None, o_coarse=None):
    """vsa_block_sparse_attn_fwd_raster with rows claimed from per-XCD queues (balanced launch)."""
    n_raster = plan.batch * plan.seq_len * plan.heads * plan.head_dim
    rows = plan.num_rows()
    et = plan.torch_dtype()
    ws_ptr, ws_len = _workspace(workspace, vsa_attn_fwd_workspace_size(plan))
    _check(load_library().vsa_block_sparse_attn_fwd_raster_ws(
        plan.handle, _ptr(q, n_raster, et, "q"), _ptr(k, n_raster, et, "k"),
        _ptr(v, n_raster, et, "v"), _ptr(row_ptr, rows + 1, _i32(), "row_ptr"),
        _ptr(col_idx, int(nnz), _i32(), "col_idx"), int(uniform_k), int(nnz),
        _ptr(gate, n_raster, et, "gate"),
        _ptr(o_coarse, plan.info["pooled_elems"], _f32(), "o_coarse"),
        _ptr(o_raster, n_raster, et, "o_raster"),
        _ptr(lse, plan.batch * plan.heads * plan.padded_len, _f32(), "lse"),
        ws_ptr, ws_len, _stream(stream, q, o_raster)))


def vsa_forward_fused_workspace_size(plan: Plan) -> int:
    n = ctypes.c_size_t()
    _check(load_library().vsa_forward_fused_workspace_size(plan.handle, ctypes.byref(n)))
    return n.value


def vsa_forward_fused(plan: Plan, q, k, v, out, workspace, col_idx_out=None, lse=None,
                      stream=None, gate=None):
    """vsa_forward_fused: the gather-free hot path (raster in, raster out)."""
    vsa_forward(plan, q, k, v, out, workspace, col_idx_out, lse, stream, gate, fused=True)


def vsa_forward_workspace_size(plan: Plan) -> int:
    n = ctypes.c_size_t()
    _check(load_library().vsa_forward_workspace_size(plan.handle, ctypes.byref(n)))
    return n.value


def vsa_block_sparse_attn_bwd_workspace_size(plan: Plan) -> int:
    n = ctypes.c_size_t()
    _check(load_library().vsa_block_sparse_attn_bwd_workspace_size(plan.handle, ctypes.byref(n)))
    return n.value


def vsa_block_sparse_attn_bwd(plan: Plan, q_blk, k_blk, v_blk, o_blk, do_blk, lse, row_ptr,
                              col_idx, uniform_k: int, nnz: int, dq_blk, dk_blk, dv_blk, workspace,
                              stream=None):
    """Gradients of the block-sparse forward; v_blk is token-major (gathered with role K)."""
    be = plan.info["blocked_elems"]
    rows = plan.num_rows()
    et = plan.torch_dtype()
    ws_bytes = vsa_block_sparse_attn_bwd_workspace_size(plan)
    if workspace.numel() * workspace.element_size() < ws_bytes:
        raise ValueError(f"workspace: fewer than {ws_bytes} bytes")
    _check(load_library().vsa_block_sparse_attn_bwd(
        plan.handle, _ptr(q_blk, be, et, "q_blk"), _ptr(k_blk, be, et, "k_blk"),
        _ptr(v_blk, be, et, "v_blk"), _ptr(o_blk, be, et, "o_blk"), _ptr(do_blk, be, et, "do_blk"),
        _ptr(lse, plan.batch * plan.heads * plan.padded_len, _f32(), "lse"),
        _ptr(row_ptr, rows + 1, _i32(), "row_ptr"), _ptr(col_idx, int(nnz), _i32(), "col_idx"),
        int(uniform_k), int(nnz), _ptr(dq_blk, be, et, "dq_blk"), _ptr(dk_blk, be, et, "dk_blk"),
        _ptr(dv_blk, be, et, "dv_blk"), _ptr(workspace, name="workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream, q_blk, dq_blk)))


def vsa_compress_attn(plan: Plan, q_pooled, k_pooled, v_pooled, o_coarse, stream=None):
    pe = plan.info["pooled_elems"]
    _check(load_library().vsa_compress_attn(
        plan.handle, _ptr(q_pooled, pe, _f32(), "q_pooled"), _ptr(k_pooled, pe, _f32(), "k_pooled"),
        _ptr(v_pooled, pe, _f32(), "v_pooled"), _ptr(o_coarse, pe, _f32(), "o_coarse"),
        _stream(stream, q_pooled, o_coarse)))


def vsa_scatter_gated(plan: Plan, o_blk, o_coarse, gate, o_raster, stream=None):
    n_raster = plan.batch * plan.seq_len * plan.heads * plan.head_dim
    et = plan.torch_dtype()
    _check(load_library().vsa_scatter_gated(
        plan.handle, _ptr(o_blk, plan.info["blocked_elems"], et, "o_blk"),
        _ptr(o_coarse, plan.info["pooled_elems"], _f32(), "o_coarse"),
        _ptr(gate, n_raster, et, "gate"), _ptr(o_raster, n_raster, et, "o_raster"),
        _stream(stream, o_blk, o_raster)))


def vsa_forward(plan: Plan, q, k, v, out, workspace, col_idx_out=None, lse=None, stream=None,
                gate=None, fused=False):
    """The whole hot path, raster in and out; fused=True calls vsa_forward_fused
    (no gather or scatter passes) with its own, smaller workspace."""
    n_raster = plan.batch * plan.seq_len * plan.heads * plan.head_dim
    ws_bytes = (vsa_forward_fused_workspace_size if fused else vsa_forward_workspace_size)(plan)
    ws_ptr, ws_len = _workspace(workspace, ws_bytes)
    et = plan.torch_dtype()
    lib = load_library()
    _check((lib.vsa_forward_fused if fused else lib.vsa_forward)(
        plan.handle, _ptr(q, n_raster, et, "q"), _ptr(k, n_raster, et, "k"),
        _ptr(v, n_raster, et, "v"), _ptr(gate, n_raster, et, "gate"),
        _ptr(out, n_raster, et, "out"), ws_ptr, ws_len,
        _ptr(col_idx_out, plan.num_rows() * max(plan.topk, 0), _i32(), "col_idx_out"),
        _ptr(lse, plan.batch * plan.heads * plan.padded_len, _f32(), "lse"),
        _stream(stream, q, out)))


# ------------------------------------------------------------------ measurement kernels

def vsa_bench_mfma_peak(num_workgroups: int, iters: int, timing, stream=None) -> int:
    """Launch the dense bf16 MFMA loop; fills `timing` (int64 device tensor of
    16 * num_workgroups entries) and returns the wall clock's rate in Hz."""
    import torch
    hz = ctypes.c_int64()
    _check(load_library().vsa_bench_mfma_peak(
        int(num_workgroups), int(iters), _ptr(timing, 16 * int(num_workgroups), torch.int64,
                                              "timing"),
        ctypes.byref(hz), _stream(stream, timing)))
    return hz.value


def vsa_bench_hbm_copy(src, dst, nbytes: int, stream=None):
    """dst[:nbytes] = src[:nbytes] on the device (uint8 tensors or raw addresses)."""
    _check(load_library().vsa_bench_hbm_copy(
        _ptr(src, int(nbytes), None, "src"), _ptr(dst, int(nbytes), None, "dst"), int(nbytes),
        _stream(stream, src, dst)))
