"""Python binding of libmoe.so, the gfx950 MoE FFN layer (see include/moe.h).

Argument marshalling only: every step of the layer runs in the HIP kernels
behind the C ABI.  torch supplies device memory and the stream; the functions
below take torch tensors (or raw device addresses as ints) and pass their
pointers through.  There is no fallback: if libmoe.so is missing or cannot be
loaded, importing the binding raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_NULL_ARG, MOE_ERR_BAD_SHAPE, MOE_ERR_UNSUPPORTED = 0, 1, 2, 3
MOE_ERR_ALIGNMENT, MOE_ERR_WORKSPACE, MOE_ERR_HIP, MOE_ERR_DEVICE = 4, 5, 6, 7
MOE_W_E4M3_B128, MOE_W_E2M1_UE8M0_G32, MOE_W_E2M1_E4M3_G16 = 0, 1, 2
MOE_PATH_AUTO, MOE_PATH_DECODE, MOE_PATH_GROUPED = 0, 1, 2
MOE_ACT_BF16, MOE_ACT_E4M3_G128 = 0, 1
MOE_OPT_DEC_KERNEL, MOE_OPT_DEC_MFMA_MIN_T, MOE_OPT_GROUPED_TILE = 0, 1, 2
MOE_OPT_Q8_TILE, MOE_OPT_SMALL_ROUTE_T = 3, 4
STAGES = ("router", "topk", "permute", "gateup", "down", "combine")
WFMT = {"e4m3": MOE_W_E4M3_B128, "e2m1": MOE_W_E2M1_UE8M0_G32, "nvfp4": MOE_W_E2M1_E4M3_G16}


class moe_desc(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("max_tokens", ctypes.c_int32), ("wfmt", ctypes.c_int32),
                ("renorm", ctypes.c_int32), ("path", ctypes.c_int32), ("act_fmt", ctypes.c_int32),
                ("shared_expert", ctypes.c_int32)]


class moe_mat(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("q_expert_stride", ctypes.c_int64), ("s_expert_stride", ctypes.c_int64)]


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str, info: str = ""):
        self.status = status
        super().__init__(f"{where}: {moe_status_str(status)}" + (f" ({info})" if info else ""))


def _load():
    # One HIP runtime per process: torch ships its own libamdhip64, and a
    # libmoe.so loaded before torch would bind the system copy, leaving two
    # runtimes that each claim the device.  Loading torch first makes
    # libmoe.so share torch's (same soname); without torch the system copy
    # serves alone.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                          "python -m mixture_experts_layer_f32_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.moe_plan.argtypes = [ctypes.POINTER(moe_desc), ctypes.POINTER(vp)]
    L.moe_plan.restype = ctypes.c_int
    L.moe_plan_set.argtypes = [vp, i32, i32]
    L.moe_plan_set.restype = ctypes.c_int
    L.moe_workspace_size.argtypes = [vp, i32]
    L.moe_workspace_size.restype = sz
    L.moe_forward.argtypes = [vp, i32, vp, vp, vp, ctypes.POINTER(moe_mat),
                              ctypes.POINTER(moe_mat), ctypes.POINTER(moe_mat), vp, vp, vp, vp,
                              vp, vp, vp, sz, vp]
    L.moe_forward.restype = ctypes.c_int
    L.moe_forward_block.argtypes = [vp, i32, vp, vp, vp, ctypes.POINTER(moe_mat),
                                    ctypes.POINTER(moe_mat), ctypes.POINTER(moe_mat),
                                    ctypes.POINTER(moe_mat), ctypes.POINTER(moe_mat),
                                    ctypes.POINTER(moe_mat), vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                    vp]
    L.moe_forward_block.restype = ctypes.c_int
    L.moe_forward_noalloc.argtypes = [vp, i32, vp, vp, vp, ctypes.POINTER(moe_mat),
                                      ctypes.POINTER(moe_mat), ctypes.POINTER(moe_mat), vp, vp,
                                      vp, vp, vp, vp, vp]
    L.moe_forward_noalloc.restype = ctypes.c_int
    L.moe_noalloc_scratch_bytes.argtypes = []
    L.moe_noalloc_scratch_bytes.restype = sz
    L.moe_workspace_h_offset.argtypes = [vp, i32]
    L.moe_workspace_h_offset.restype = i64
    L.moe_plan_path.argtypes = [vp, i32]
    L.moe_plan_path.restype = i32
    L.moe_timing_enable.argtypes = [vp, ctypes.c_uint32, i32]
    L.moe_timing_enable.restype = ctypes.c_int
    L.moe_timing_collect.argtypes = [vp, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(i32)]
    L.moe_timing_collect.restype = ctypes.c_int
    L.moe_timing_disable.argtypes = [vp]
    L.moe_timing_disable.restype = ctypes.c_int
    L.moe_rmsnorm.argtypes = [i32, i32, vp, vp, ctypes.c_float, vp, vp]
    L.moe_rmsnorm.restype = ctypes.c_int
    L.moe_residual_add.argtypes = [i32, i32, vp, vp, vp, vp, vp]
    L.moe_residual_add.restype = ctypes.c_int
    L.moe_act_quant.argtypes = [i32, i32, vp, vp, vp, vp]
    L.moe_act_quant.restype = ctypes.c_int
    L.moe_plan_free.argtypes = [vp]
    L.moe_plan_free.restype = None
    L.moe_status_str.argtypes = [ctypes.c_int]
    L.moe_status_str.restype = ctypes.c_char_p
    L.moe_plan_info.argtypes = [vp]
    L.moe_plan_info.restype = ctypes.c_char_p
    return L


lib = _load()


def moe_status_str(status: int) -> str:
    return lib.moe_status_str(int(status)).decode()


class Plan:
    """Owns a moe_plan_t; freed with the object."""

    def __init__(self, handle: int, desc: moe_desc):
        self.handle = handle
        self.desc = desc

    def __del__(self):
        if getattr(self, "handle", None):
            lib.moe_plan_free(self.handle)
            self.handle = None


def moe_plan(d_model: int, d_ff: int, n_experts: int, top_k: int, max_tokens: int,
             wfmt: int | str, renorm: bool, path: int = MOE_PATH_AUTO,
             act_fmt: int = MOE_ACT_BF16, shared_expert: bool = False) -> Plan:
    if isinstance(wfmt, str):
        wfmt = WFMT[wfmt]
    desc = moe_desc(d_model, d_ff, n_experts, top_k, max_tokens, int(wfmt), int(bool(renorm)),
                    int(path), int(act_fmt), int(bool(shared_expert)))
    h = ctypes.c_void_p()
    st = lib.moe_plan(ctypes.byref(desc), ctypes.byref(h))
    if st != MOE_OK:
        raise MoeError(st, "moe_plan")
    return Plan(h.value, desc)


def moe_plan_status(desc: moe_desc) -> int:
    """Raw status of moe_plan for a descriptor (the plan, if any, is freed)."""
    h = ctypes.c_void_p()
    st = lib.moe_plan(ctypes.byref(desc), ctypes.byref(h))
    if h.value:
        lib.moe_plan_free(h.value)
    return st


def moe_plan_set(plan: Plan, option: int, value: int) -> None:
    """Override one of the plan's shape-based kernel choices (MOE_OPT_*)."""
    st = lib.moe_plan_set(plan.handle, int(option), int(value))
    if st != MOE_OK:
        raise MoeError(st, "moe_plan_set")


def moe_workspace_size(plan: Plan, n_tokens: int) -> int:
    return int(lib.moe_workspace_size(plan.handle, int(n_tokens)))


def moe_workspace_h_offset(plan: Plan, n_tokens: int) -> int:
    return int(lib.moe_workspace_h_offset(plan.handle, int(n_tokens)))


def moe_plan_path(plan: Plan, n_tokens: int) -> int:
    return int(lib.moe_plan_path(plan.handle, int(n_tokens)))


def moe_plan_info(plan: Plan) -> str:
    return lib.moe_plan_info(plan.handle).decode()


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def mat(q, scale, q_expert_stride: Optional[int] = None,
        s_expert_stride: Optional[int] = None) -> moe_mat:
    """moe_mat from device tensors with a leading expert axis (strides in bytes
    default to one expert's contiguous size)."""
    if q_expert_stride is None:
        q_expert_stride = q.stride(0) * q.element_size()
    if s_expert_stride is None:
        s_expert_stride = scale.stride(0) * scale.element_size()
    return moe_mat(_ptr(q), _ptr(scale), int(q_expert_stride), int(s_expert_stride))


def moe_forward(plan: Plan, n_tokens: int, x, w_router, logit_bias, gate: moe_mat, up: moe_mat,
                down: moe_mat, out, topk_ids=None, topk_w=None, counts=None, offsets=None,
                perm=None, workspace=None, workspace_bytes: Optional[int] = None,
                stream=None) -> None:
    """Enqueue the forward on `stream` (a torch stream, a raw hipStream_t int,
    or None for torch's current stream).  Raises MoeError on a non-OK status."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    if workspace_bytes is None:
        workspace_bytes = (workspace.numel() * workspace.element_size()
                           if hasattr(workspace, "numel") else 0)
    st = lib.moe_forward(plan.handle, int(n_tokens), _ptr(x), _ptr(w_router), _ptr(logit_bias),
                         ctypes.byref(gate), ctypes.byref(up), ctypes.byref(down), _ptr(out),
                         _ptr(topk_ids), _ptr(topk_w), _ptr(counts), _ptr(offsets), _ptr(perm),
                         _ptr(workspace), int(workspace_bytes), stream or None)
    if st != MOE_OK:
        raise MoeError(st, "moe_forward", moe_plan_info(plan))


def moe_forward_block(plan: Plan, n_tokens: int, x, w_router, logit_bias, gate: moe_mat,
                      up: moe_mat, down: moe_mat, shared=None, residual=None, out_bf16=None,
                      out=None, topk_ids=None, topk_w=None, counts=None, offsets=None, perm=None,
                      workspace=None, workspace_bytes: Optional[int] = None, stream=None) -> None:
    """The layer inside a block: `shared` = (gate, up, down) moe_mats of the
    shared expert (plans made with shared_expert=True), and out_bf16 =
    bf16(residual + out) written by the combine.  Raises MoeError."""
    if workspace_bytes is None:
        workspace_bytes = (workspace.numel() * workspace.element_size()
                           if hasattr(workspace, "numel") else 0)
    sg, su, sd = (ctypes.byref(m) for m in shared) if shared is not None else (None, None, None)
    st = lib.moe_forward_block(plan.handle, int(n_tokens), _ptr(x), _ptr(w_router),
                               _ptr(logit_bias), ctypes.byref(gate), ctypes.byref(up),
                               ctypes.byref(down), sg, su, sd, _ptr(residual), _ptr(out_bf16),
                               _ptr(out), _ptr(topk_ids), _ptr(topk_w), _ptr(counts),
                               _ptr(offsets), _ptr(perm), _ptr(workspace), int(workspace_bytes),
                               _stream(stream))
    if st != MOE_OK:
        raise MoeError(st, "moe_forward_block", moe_plan_info(plan))


def moe_forward_noalloc(plan: Plan, n_tokens: int, x, w_router, logit_bias, gate: moe_mat,
                        up: moe_mat, down: moe_mat, out, topk_ids=None, topk_w=None, counts=None,
                        offsets=None, perm=None, stream=None) -> None:
    """moe_forward without a workspace: the library's per-device scratch array
    (moe_noalloc_scratch_bytes()) serves instead.  Raises MoeError."""
    st = lib.moe_forward_noalloc(plan.handle, int(n_tokens), _ptr(x), _ptr(w_router),
                                 _ptr(logit_bias), ctypes.byref(gate), ctypes.byref(up),
                                 ctypes.byref(down), _ptr(out), _ptr(topk_ids), _ptr(topk_w),
                                 _ptr(counts), _ptr(offsets), _ptr(perm), _stream(stream))
    if st != MOE_OK:
        raise MoeError(st, "moe_forward_noalloc", moe_plan_info(plan))


def moe_noalloc_scratch_bytes() -> int:
    return int(lib.moe_noalloc_scratch_bytes())


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream or None
    return stream if isinstance(stream, int) else stream.cuda_stream


def moe_rmsnorm(x, gamma, eps: float, xn, stream=None) -> None:
    """RMS normalisation of bf16 rows x [T, d] (bf16 bits) with gain gamma [d]
    into xn [T, d]; raises MoeError on a non-OK status."""
    T, d = x.shape
    st = lib.moe_rmsnorm(int(T), int(d), _ptr(x), _ptr(gamma), float(eps), _ptr(xn), _stream(stream))
    if st != MOE_OK:
        raise MoeError(st, "moe_rmsnorm")


def moe_residual_add(residual, a, b, out, stream=None) -> None:
    """out = bf16(residual + (a + b)) over [T, d] (b may be None); raises MoeError."""
    T, d = residual.shape
    st = lib.moe_residual_add(int(T), int(d), _ptr(residual), _ptr(a), _ptr(b), _ptr(out),
                              _stream(stream))
    if st != MOE_OK:
        raise MoeError(st, "moe_residual_add")


def moe_timing_enable(plan: Plan, stages=STAGES, max_forwards: int = 1024) -> None:
    mask = 0
    for st in stages:
        mask |= 1 << (STAGES.index(st) if isinstance(st, str) else int(st))
    st = lib.moe_timing_enable(plan.handle, mask, int(max_forwards))
    if st != MOE_OK:
        raise MoeError(st, "moe_timing_enable", moe_plan_info(plan))


def moe_timing_collect(plan: Plan):
    """-> (dict stage -> summed ms, number of recorded forwards)."""
    ms = (ctypes.c_float * len(STAGES))()
    n = ctypes.c_int32()
    st = lib.moe_timing_collect(plan.handle, ms, ctypes.byref(n))
    if st != MOE_OK:
        raise MoeError(st, "moe_timing_collect", moe_plan_info(plan))
    return {name: float(ms[i]) for i, name in enumerate(STAGES)}, int(n.value)


def moe_timing_disable(plan: Plan) -> None:
    lib.moe_timing_disable(plan.handle)


def moe_act_quant(x, q, scales, stream=None) -> None:
    """bf16 rows x [R, K] (bits) -> e4m3 codes q [R, K] and UE8M0 scale bytes
    [R, ceil(K / 128)]; raises MoeError on a non-OK status."""
    R, K = x.shape
    st = lib.moe_act_quant(int(R), int(K), _ptr(x), _ptr(q), _ptr(scales), _stream(stream))
    if st != MOE_OK:
        raise MoeError(st, "moe_act_quant")
