"""ctypes binding of libbdattn.so (argument marshalling only).

Every step of the attention runs in the library's HIP kernels; this module only
turns torch tensors into pointers and the metadata into the C descriptor. There
is no CPU fallback: if the library cannot be loaded, importing this module
raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch  # loaded first so the library binds to the HIP runtime torch already mapped

_HERE = os.path.dirname(os.path.abspath(__file__))
# BDATTN_LIBRARY selects another build of the same library (the host-sanitized
# copy that build.py --sanitize writes); by default the in-tree libbdattn.so
LIB_PATH = os.environ.get("BDATTN_LIBRARY") or os.path.join(_HERE, "libbdattn.so")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = range(5)
BF16, FP32 = 0, 1
FLAG_NO_SPLIT, FLAG_FORCE_SPLIT, FLAG_NO_XCD, FLAG_FWD_DIRECT, FLAG_FWD_VT = 1, 2, 4, 8, 16
FLAG_CLEAN_CAUSAL = 32
FLAG_CHECK_PLAN = 64
FLAG_DEBUG_CHECKS = 128
FLAG_DKDV_RUNS = 1 << 16


def flag_split_tiles(n: int) -> int:
    """Plan flag: n key tiles (of 64 keys) per split on the forward split path."""
    return (int(n) & 0xFF) << 8


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with block_diffusion_attention_amd/build.py")
_lib = ctypes.CDLL(LIB_PATH)

_i32p = ctypes.POINTER(ctypes.c_int32)


class Desc(ctypes.Structure):
    _fields_ = [
        ("num_segments", ctypes.c_int32),
        ("ctx_len", _i32p),
        ("ctx_q_begin", _i32p),
        ("canvas_offsets", _i32p),
        ("canvas_block_idx", _i32p),
        ("block_size", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("flags", ctypes.c_uint32),
        ("block_offset", _i32p),
    ]


_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_lib.bd_attn_plan.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(_vp)]
_lib.bd_attn_plan_sizes.argtypes = [_vp, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64),
                                    ctypes.POINTER(_sz), ctypes.POINTER(_sz), ctypes.POINTER(_sz),
                                    ctypes.POINTER(ctypes.c_int64)]
_lib.bd_attn_plan_serialize.argtypes = [_vp, _vp, _sz]
_lib.bd_attn_plan_check.argtypes = [_vp, _vp, _sz]
_lib.bd_attn_device_check_errors.argtypes = [ctypes.POINTER(ctypes.c_uint64), ctypes.c_int]


class PlanInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("split", "split_tiles", "split_grid", "fwd_vt", "dkdv_masked",
                                              "debug_checks")] + \
               [(n, ctypes.c_int64) for n in ("query_tiles", "key_tiles", "fwd_workgroups", "dq_workgroups",
                                              "dkdv_workgroups", "dkdv_split_tiles")]


_lib.bd_attn_plan_info.argtypes = [_vp, ctypes.POINTER(PlanInfo)]
_lib.bd_attn_plan_upload.argtypes = [_vp, _vp, _vp]
_lib.bd_attn_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.bd_attn_bwd.argtypes = [_vp] * 13
_lib.bd_attn_fwd_noalloc.argtypes = [_vp] * 8
_lib.bd_attn_fwd_timed.argtypes = [_vp] * 10 + [ctypes.c_int]
_lib.bd_attn_bwd_timed.argtypes = [_vp] * 14 + [ctypes.c_int]
_lib.bd_attn_plan_kernels.argtypes = [_vp, ctypes.c_int32]
_lib.bd_attn_plan_kernels.restype = ctypes.c_int32
_lib.bd_attn_plan_kernel_name.argtypes = [_vp, ctypes.c_int32, ctypes.c_int32]
_lib.bd_attn_plan_kernel_name.restype = ctypes.c_char_p
_lib.bd_attn_plan_destroy.argtypes = [_vp]
_lib.bd_attn_last_error.restype = ctypes.c_char_p
_lib.bd_attn_version.restype = ctypes.c_char_p
for _f in ("bd_attn_plan", "bd_attn_plan_sizes", "bd_attn_plan_serialize", "bd_attn_plan_upload",
           "bd_attn_fwd", "bd_attn_bwd", "bd_attn_fwd_timed", "bd_attn_bwd_timed", "bd_attn_plan_destroy",
           "bd_attn_fwd_noalloc", "bd_attn_plan_check", "bd_attn_device_check_errors", "bd_attn_plan_info"):
    getattr(_lib, _f).restype = ctypes.c_int


class PackDesc(ctypes.Structure):
    _fields_ = [
        ("num_responses", ctypes.c_int32),
        ("clean_len", _i32p),
        ("block_offset", _i32p),
        ("num_states", ctypes.c_int32),
        ("state_resp", _i32p),
        ("state_block", _i32p),
        ("state_step", _i32p),
        ("state_supervised", _i32p),
        ("state_pages", _i32p),
        ("block_size", ctypes.c_int32),
        ("num_groups", ctypes.c_int32),
        ("w_tokens", ctypes.c_int32),
        ("w_supervised", ctypes.c_int32),
        ("w_pages", ctypes.c_int32),
    ]


_i64p = ctypes.POINTER(ctypes.c_int64)


class PackOut(ctypes.Structure):
    _fields_ = [
        ("state_row", _i32p),
        ("row_resp", _i32p),
        ("row_step", _i32p),
        ("row_ctx_len", _i32p),
        ("row_group", _i32p),
        ("row_cost", _i64p),
        ("row_state_offsets", _i32p),
        ("row_states", _i32p),
        ("group_row_offsets", _i32p),
        ("group_rows", _i32p),
        ("group_cost", _i64p),
        ("n_rows", ctypes.c_int32),
    ]


_lib.bd_attn_pack.argtypes = [ctypes.POINTER(PackDesc), ctypes.POINTER(PackOut)]
_lib.bd_attn_pack.restype = ctypes.c_int

class AecDesc(ctypes.Structure):
    _fields_ = [
        ("num_rows", ctypes.c_int32),
        ("vocab", ctypes.c_int32),
        ("row_stride", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("num_states", ctypes.c_int32),
        ("num_pairs", ctypes.c_int32),
        ("rho", ctypes.c_float),
        ("gate_max", ctypes.c_float),
    ]


_lib.bd_aec_workspace.argtypes = [ctypes.POINTER(AecDesc), ctypes.POINTER(_sz)]
_lib.bd_aec_workspace.restype = ctypes.c_int
_lib.bd_aec_fwd.argtypes = [ctypes.POINTER(AecDesc)] + [_vp] * 12
_lib.bd_aec_fwd.restype = ctypes.c_int
_lib.bd_aec_fwd_timed.argtypes = [ctypes.POINTER(AecDesc)] + [_vp] * 13 + [ctypes.c_int]
_lib.bd_aec_fwd_timed.restype = ctypes.c_int
_lib.bd_aec_bwd.argtypes = [ctypes.POINTER(AecDesc)] + [_vp] * 13
_lib.bd_aec_bwd.restype = ctypes.c_int
_lib.bd_aec_bwd_timed.argtypes = [ctypes.POINTER(AecDesc)] + [_vp] * 14 + [ctypes.c_int]
_lib.bd_aec_bwd_timed.restype = ctypes.c_int
_lib.bd_aec_kernels.argtypes = [ctypes.POINTER(AecDesc)]
_lib.bd_aec_kernels.restype = ctypes.c_int32

EXPORTED = ("bd_attn_plan", "bd_attn_plan_sizes", "bd_attn_plan_serialize", "bd_attn_plan_upload",
            "bd_attn_fwd", "bd_attn_bwd", "bd_attn_fwd_timed", "bd_attn_bwd_timed", "bd_attn_plan_kernels",
            "bd_attn_plan_kernel_name", "bd_attn_plan_destroy", "bd_attn_last_error", "bd_attn_version",
            "bd_attn_pack", "bd_aec_workspace", "bd_aec_fwd", "bd_aec_fwd_timed", "bd_aec_kernels",
            "bd_aec_bwd", "bd_aec_bwd_timed", "bd_attn_fwd_noalloc", "bd_attn_plan_check",
            "bd_attn_device_check_errors", "bd_attn_plan_info")

# size of the fixed forward workspace of bd_attn_fwd_noalloc (BD_ATTN_NOALLOC_WS_BYTES)
NOALLOC_WS_BYTES = 32 << 20


class BdAttnError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"bd_attn status {status}: {msg}")
        self.status = status


def _check(st):
    if st != OK:
        raise BdAttnError(st, _lib.bd_attn_last_error().decode())


def version() -> str:
    return _lib.bd_attn_version().decode()


def device_check_errors(reset: bool = False) -> int:
    """Workgroups of plans made with FLAG_DEBUG_CHECKS that rejected a work
    record on the current device since the last reset (blocking)."""
    n = ctypes.c_uint64(0)
    _check(_lib.bd_attn_device_check_errors(ctypes.byref(n), 1 if reset else 0))
    return int(n.value)


def _arr(vals):
    a = (ctypes.c_int32 * max(1, len(vals)))(*[int(x) for x in vals])
    return a


def pack(clean_len, state_resp, state_block, state_step, block_size, num_groups, *, block_offset=None,
         state_supervised=None, state_pages=None, w_tokens=1, w_supervised=0, w_pages=0):
    """Replay rows and their largest-cost-first assignment to data-parallel groups
    (bd_attn_pack). Returns a dict of numpy arrays trimmed to the row count."""
    import numpy as np
    R, N, G = len(clean_len), len(state_resp), int(num_groups)
    d = PackDesc()
    d.num_responses, d.num_states, d.block_size, d.num_groups = R, N, int(block_size), G
    d.w_tokens, d.w_supervised, d.w_pages = int(w_tokens), int(w_supervised), int(w_pages)
    keep = {}
    for n, v in (("clean_len", clean_len), ("state_resp", state_resp), ("state_block", state_block),
                 ("state_step", state_step), ("block_offset", block_offset),
                 ("state_supervised", state_supervised), ("state_pages", state_pages)):
        if v is not None:
            keep[n] = np.ascontiguousarray(np.asarray(v, dtype=np.int64).astype(np.int32))
            setattr(d, n, keep[n].ctypes.data_as(_i32p))
    n1 = max(1, N)
    bufs = {n: np.zeros(n1, np.int32) for n in ("state_row", "row_resp", "row_step", "row_ctx_len", "row_group",
                                                "row_states", "group_rows")}
    bufs["row_cost"] = np.zeros(n1, np.int64)
    bufs["row_state_offsets"] = np.zeros(n1 + 1, np.int32)
    bufs["group_row_offsets"] = np.zeros(G + 1, np.int32)
    bufs["group_cost"] = np.zeros(max(1, G), np.int64)
    o = PackOut()
    for n, a in bufs.items():
        setattr(o, n, a.ctypes.data_as(_i64p if a.dtype == np.int64 else _i32p))
    _check(_lib.bd_attn_pack(ctypes.byref(d), ctypes.byref(o)))
    nr = o.n_rows
    res = {"n_rows": nr, "state_row": bufs["state_row"][:N], "row_states": bufs["row_states"][:N],
           "row_state_offsets": bufs["row_state_offsets"][:nr + 1], "group_rows": bufs["group_rows"][:nr],
           "group_row_offsets": bufs["group_row_offsets"], "group_cost": bufs["group_cost"][:G]}
    for n in ("row_resp", "row_step", "row_ctx_len", "row_group", "row_cost"):
        res[n] = bufs[n][:nr]
    return res


class Plan:
    """A validated plan (host work lists) plus, once uploaded, its device copy."""

    def __init__(self, meta, flags: int = 0):
        self.meta = meta
        offs = getattr(meta, "block_offset", None)
        self._keep = [_arr(meta.ctx_len), _arr(meta.ctx_q_begin), _arr(meta.canvas_offsets),
                      _arr(meta.flat_canvas_block_idx), None if offs is None else _arr(offs)]
        d = Desc()
        d.num_segments = len(meta.ctx_len)
        d.ctx_len = ctypes.cast(self._keep[0], _i32p)
        d.ctx_q_begin = ctypes.cast(self._keep[1], _i32p)
        d.canvas_offsets = ctypes.cast(self._keep[2], _i32p)
        d.canvas_block_idx = ctypes.cast(self._keep[3], _i32p)
        d.block_size = meta.block_size
        d.num_q_heads = meta.num_q_heads
        d.num_kv_heads = meta.num_kv_heads
        d.head_dim = meta.head_dim
        d.dtype = BF16 if meta.dtype == "bf16" else FP32
        d.softmax_scale = float(meta.softmax_scale)
        if getattr(meta, "clean_causal", False):
            flags |= FLAG_CLEAN_CAUSAL
        d.flags = flags
        if self._keep[4] is not None:
            d.block_offset = ctypes.cast(self._keep[4], _i32p)
        h = _vp()
        _check(_lib.bd_attn_plan(ctypes.byref(d), ctypes.byref(h)))
        self.handle = h
        tq, tk = ctypes.c_int64(), ctypes.c_int64()
        mb, wf, wb = _sz(), _sz(), _sz()
        pairs = ctypes.c_int64()
        _check(_lib.bd_attn_plan_sizes(h, ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(mb),
                                       ctypes.byref(wf), ctypes.byref(wb), ctypes.byref(pairs)))
        self.tq, self.tk = tq.value, tk.value
        self.meta_bytes, self.ws_fwd_bytes, self.ws_bwd_bytes = mb.value, wf.value, wb.value
        self.visible_pairs = pairs.value
        self.dtype = torch.bfloat16 if meta.dtype == "bf16" else torch.float32
        self.meta_dev: Optional[torch.Tensor] = None
        self.ws_fwd: Optional[torch.Tensor] = None
        self.ws_bwd: Optional[torch.Tensor] = None

    def kernels(self, backward: bool) -> int:
        return int(_lib.bd_attn_plan_kernels(self.handle, 1 if backward else 0))

    def kernel_names(self, backward: bool):
        bw = 1 if backward else 0
        return [_lib.bd_attn_plan_kernel_name(self.handle, bw, i).decode() for i in range(self.kernels(backward))]

    def info(self) -> dict:
        """The plan's scheduling choices and list sizes (bd_attn_plan_info)."""
        r = PlanInfo()
        _check(_lib.bd_attn_plan_info(self.handle, ctypes.byref(r)))
        return {n: getattr(r, n) for n, _ in PlanInfo._fields_}

    def host_blob(self):
        buf = (ctypes.c_int32 * (self.meta_bytes // 4))()
        _check(_lib.bd_attn_plan_serialize(self.handle, ctypes.cast(buf, _vp), self.meta_bytes))
        return list(buf)

    def check(self, blob=None):
        """Runs the work-list self-check on blob (a list of int32, by default the
        plan's own image); raises BdAttnError naming the first bad record."""
        vals = self.host_blob() if blob is None else list(blob)
        buf = (ctypes.c_int32 * len(vals))(*vals)
        _check(_lib.bd_attn_plan_check(self.handle, ctypes.cast(buf, _vp), ctypes.sizeof(buf)))

    def upload(self, device="cuda"):
        """Allocates (torch) and fills the device metadata buffer and workspaces."""
        dev = torch.device(device)
        self.meta_dev = torch.empty(max(16, self.meta_bytes), dtype=torch.uint8, device=dev)
        _check(_lib.bd_attn_plan_upload(self.handle, _vp(self.meta_dev.data_ptr()), _stream(dev)))
        # the copy reads the plan's host memory: finish it before anything can free the plan
        torch.cuda.current_stream(dev).synchronize()
        self.ws_fwd = torch.empty(max(16, self.ws_fwd_bytes), dtype=torch.uint8, device=dev) if self.ws_fwd_bytes else None
        self.ws_bwd = torch.empty(max(16, self.ws_bwd_bytes), dtype=torch.uint8, device=dev)
        return self

    def __del__(self, _destroy=_lib.bd_attn_plan_destroy):
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            _destroy(h)
            self.handle = None


def _stream(dev) -> _vp:
    return _vp(torch.cuda.current_stream(dev).cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> _vp:
    return _vp(0 if t is None else t.data_ptr())


def _expect(t, shape, dtype, name, device=None):
    """Every tensor handed to the library must match the plan's layout exactly:
    the kernels index raw pointers with the contiguous [rows, heads, D] strides."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if (tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous() or not t.is_cuda
            or (device is not None and t.device != device)):
        raise ValueError(f"{name}: expected contiguous cuda {dtype} {tuple(shape)}"
                         f"{'' if device is None else ' on ' + str(device)}, got {t.dtype} {tuple(t.shape)} "
                         f"contiguous={t.is_contiguous()} device={t.device}")
    if t.data_ptr() % 16:
        raise ValueError(f"{name}: data pointer is not 16-byte aligned")


def _shapes(plan):
    m = plan.meta
    return ((plan.tq, m.num_q_heads, m.head_dim), (plan.tk, m.num_kv_heads, m.head_dim),
            (plan.tq, m.num_q_heads))


def _out(t, shape, dtype, device, name):
    """A caller-supplied output is checked like an input; otherwise a fresh
    contiguous tensor of the plan's shape."""
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _expect(t, shape, dtype, name, device)
    return t


def _expect_meta(plan, device):
    if plan.meta_dev.device != device:
        raise ValueError(f"the plan was uploaded to {plan.meta_dev.device}, the tensors are on {device}")


def _events_arg(events):
    if events is None:
        return None, 0
    for e in events:
        if not e.cuda_event:          # torch creates the HIP event on first record
            e.record()
    arr = (_vp * len(events))(*[e.cuda_event for e in events])
    return arr, len(events)


def fwd(plan: Plan, q, k, v, o=None, lse=None, events=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Forward; ``events`` (optional list of torch.cuda.Event) time each kernel."""
    qshape, kshape, lshape = _shapes(plan)
    _expect(q, qshape, plan.dtype, "q")
    _expect(k, kshape, plan.dtype, "k", q.device)
    _expect(v, kshape, plan.dtype, "v", q.device)
    if plan.meta_dev is None:
        plan.upload(q.device)
    _expect_meta(plan, q.device)
    o = _out(o, qshape, plan.dtype, q.device, "o")
    lse = _out(lse, lshape, torch.float32, q.device, "lse")
    args = (plan.handle, _ptr(plan.meta_dev), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
            _ptr(plan.ws_fwd), _stream(q.device))
    if events is None:
        _check(_lib.bd_attn_fwd(*args))
    else:
        arr, n = _events_arg(events)
        _check(_lib.bd_attn_fwd_timed(*args, ctypes.cast(arr, _vp), n))
    return o, lse


def fwd_noalloc(plan: Plan, q, k, v, o, lse):
    """Forward through bd_attn_fwd_noalloc: the workspace is the library's fixed
    per-GPU array, and o / lse are the caller's (no allocation in the call)."""
    qshape, kshape, lshape = _shapes(plan)
    _expect(q, qshape, plan.dtype, "q")
    _expect(k, kshape, plan.dtype, "k", q.device)
    _expect(v, kshape, plan.dtype, "v", q.device)
    _expect(o, qshape, plan.dtype, "o", q.device)
    _expect(lse, lshape, torch.float32, "lse", q.device)
    if plan.meta_dev is None:
        raise ValueError("upload the plan before calling fwd_noalloc")
    _expect_meta(plan, q.device)
    _check(_lib.bd_attn_fwd_noalloc(plan.handle, _ptr(plan.meta_dev), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                    _ptr(lse), _stream(q.device)))
    return o, lse


def bwd(plan: Plan, q, k, v, o, lse, do, dq=None, dk=None, dv=None, events=None):
    """Backward; ``events`` (optional list of 4 torch.cuda.Event) time each kernel."""
    qshape, kshape, lshape = _shapes(plan)
    _expect(q, qshape, plan.dtype, "q")
    dev = q.device
    _expect(k, kshape, plan.dtype, "k", dev)
    _expect(v, kshape, plan.dtype, "v", dev)
    _expect(o, qshape, plan.dtype, "o", dev)
    _expect(lse, lshape, torch.float32, "lse", dev)
    _expect(do, qshape, plan.dtype, "do", dev)
    if plan.meta_dev is None:
        plan.upload(dev)
    _expect_meta(plan, dev)
    dq = _out(dq, qshape, plan.dtype, dev, "dq")
    dk = _out(dk, kshape, plan.dtype, dev, "dk")
    dv = _out(dv, kshape, plan.dtype, dev, "dv")
    args = (plan.handle, _ptr(plan.meta_dev), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
            _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(plan.ws_bwd), _stream(q.device))
    if events is None:
        _check(_lib.bd_attn_bwd(*args))
    else:
        arr, n = _events_arg(events)
        _check(_lib.bd_attn_bwd_timed(*args, ctypes.cast(arr, _vp), n))
    return dq, dk, dv


class BdAttnFunction(torch.autograd.Function):
    """Autograd wrapper: forward and backward both run in libbdattn."""

    @staticmethod
    def forward(ctx, q, k, v, plan):
        # the kernels read the contiguous layout: the same copies serve the backward
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        o, lse = fwd(plan, q, k, v)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.plan = plan
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = bwd(ctx.plan, q, k, v, o, lse, do.contiguous())
        return dq, dk, dv, None


def attention(q, k, v, plan: Plan):
    return BdAttnFunction.apply(q, k, v, plan)


# ------------------------------------------------ normalized entropy / AEC loss

def aec_desc(num_rows, vocab, row_stride, dtype, num_states, num_pairs, rho, gate_max) -> AecDesc:
    d = AecDesc()
    d.num_rows, d.vocab, d.row_stride = int(num_rows), int(vocab), int(row_stride)
    d.dtype = BF16 if dtype in ("bf16", torch.bfloat16, BF16) else FP32
    d.num_states, d.num_pairs = int(num_states), int(num_pairs)
    d.rho, d.gate_max = float(rho), float(gate_max)
    return d


def aec_kernels(d: AecDesc) -> int:
    return int(_lib.bd_aec_kernels(ctypes.byref(d)))


def aec_workspace_bytes(d: AecDesc) -> int:
    n = _sz()
    _check(_lib.bd_aec_workspace(ctypes.byref(d), ctypes.byref(n)))
    return n.value


def aec_fwd(logits, vocab, unresolved, state_rows, pair_next, pair_h_source, pair_weight, rho, gate_max,
            events=None, ws=None):
    """Per-row log-normalizer and normalized entropy, per-state means over the
    unresolved rows and the AEC loss (bd_aec_fwd). logits: [N, row_stride] bf16 or
    fp32 device tensor whose first ``vocab`` columns are the vocabulary; the other
    arguments are device tensors (uint8, int32, int32, float32, float32).
    Returns (lse [N], hbar [N], h_state [S], loss [1]), all float32."""
    if logits.dim() != 2 or not logits.is_contiguous():
        raise ValueError("logits must be a contiguous [N, row_stride] tensor")
    N, stride = logits.shape
    S = state_rows.numel() - 1 if state_rows is not None else 0
    P = pair_next.numel() if pair_next is not None else 0
    d = aec_desc(N, vocab, stride, logits.dtype, S, P, rho, gate_max)
    dev = logits.device
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    hbar = torch.empty(N, dtype=torch.float32, device=dev)
    h_state = torch.empty(max(S, 1), dtype=torch.float32, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    nbytes = aec_workspace_bytes(d)
    if nbytes and ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    args = [ctypes.byref(d), _ptr(logits), _ptr(unresolved), _ptr(state_rows), _ptr(pair_next), _ptr(pair_h_source),
            _ptr(pair_weight), _ptr(lse), _ptr(hbar), _ptr(h_state), _ptr(loss), _ptr(ws), _stream(dev)]
    if events is None:
        _check(_lib.bd_aec_fwd(*args))
    else:
        ev, n = _events_arg(events)
        _check(_lib.bd_aec_fwd_timed(*args, ev, n))
    return lse, hbar, h_state[:S], loss


def aec_bwd(logits, vocab, unresolved, state_rows, pair_next, pair_h_source, pair_weight, rho, gate_max,
            lse, hbar, h_state, grad_loss, events=None, ws=None):
    """Gradient of grad_loss * loss with respect to the logits (bd_aec_bwd); lse,
    hbar and h_state are aec_fwd's outputs, grad_loss a one-element float32 device
    tensor. Returns dlogits shaped like logits (columns past ``vocab`` are zero)."""
    N, stride = logits.shape
    S = state_rows.numel() - 1 if state_rows is not None else 0
    P = pair_next.numel() if pair_next is not None else 0
    d = aec_desc(N, vocab, stride, logits.dtype, S, P, rho, gate_max)
    dev = logits.device
    dlogits = torch.zeros_like(logits) if stride != vocab else torch.empty_like(logits)
    if ws is None:
        ws = torch.empty(max(16, aec_workspace_bytes(d)), dtype=torch.uint8, device=dev)
    args = [ctypes.byref(d), _ptr(logits), _ptr(unresolved), _ptr(state_rows), _ptr(pair_next), _ptr(pair_h_source),
            _ptr(pair_weight), _ptr(lse), _ptr(hbar), _ptr(h_state if S else None), _ptr(grad_loss), _ptr(dlogits),
            _ptr(ws), _stream(dev)]
    if events is None:
        _check(_lib.bd_aec_bwd(*args))
    else:
        ev, n = _events_arg(events)
        _check(_lib.bd_aec_bwd_timed(*args, ev, n))
    return dlogits
