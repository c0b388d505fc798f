"""ctypes binding of libgsz (include/gsz.h): argument marshalling only.

Every function here converts PyTorch tensors to device pointers, takes the
current HIP stream, and calls the C entry point of the same name; all
arithmetic runs in the library's HIP kernels.  There is no fallback: if the
library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgsz.so")

LAYOUT_BUCKET_FLAT = 0
LAYOUT_SHARD_COMPACT = 1
MAX_RANKS = 256

_STATUS = {0: "GSZ_OK", -1: "GSZ_ERR_INVALID_ARG", -2: "GSZ_ERR_MISALIGNED", -3: "GSZ_ERR_SIZE",
           -4: "GSZ_ERR_BAD_RANK", -5: "GSZ_ERR_PLAN_MISMATCH", -6: "GSZ_ERR_NOT_UPLOADED",
           -7: "GSZ_ERR_DEVICE", -8: "GSZ_ERR_HIP", -9: "GSZ_ERR_NO_MEMORY"}


class GszError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status
        self.name = _STATUS.get(status, str(status))


class PlanInfo(ctypes.Structure):
    _fields_ = [("n_tensors", ctypes.c_int32), ("n_buckets", ctypes.c_int32),
                ("world_size", ctypes.c_int32), ("align", ctypes.c_int32),
                ("bucket_cap_bytes", ctypes.c_int64), ("flat_len", ctypes.c_int64),
                ("shard_len", ctypes.c_int64), ("n_params", ctypes.c_int64),
                ("hash", ctypes.c_uint64)]


class BucketInfo(ctypes.Structure):
    _fields_ = [("first_tensor", ctypes.c_int32), ("n_tensors", ctypes.c_int32),
                ("base", ctypes.c_int64), ("n_elems", ctypes.c_int64),
                ("padded", ctypes.c_int64), ("chunk", ctypes.c_int64),
                ("shard_off", ctypes.c_int64)]


class AdamWHP(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double),
                ("step", ctypes.c_int64)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SIGS = {
    "gsz_plan_create": [_P, _I32, _I64, _I32, _I32, ctypes.POINTER(_P)],
    "gsz_plan_destroy": [_P],
    "gsz_plan_get_info": [_P, ctypes.POINTER(PlanInfo)],
    "gsz_plan_bucket": [_P, _I32, ctypes.POINTER(BucketInfo)],
    "gsz_plan_tensor": [_P, _I32, ctypes.POINTER(_I64), ctypes.POINTER(_I32)],
    "gsz_plan_check": [_P, ctypes.c_uint64],
    "gsz_plan_upload": [_P],
    "gsz_ledger_bytes_per_param": [_I32, _I32, ctypes.POINTER(ctypes.c_double)],
    "gsz_workspace_bytes": [ctypes.c_int64, ctypes.POINTER(ctypes.c_size_t)],
    "gsz_set_grid_limit": [ctypes.c_int64],
    "gsz_bucket_pack": [_P, _P, _P, _P],
    "gsz_shard_reduce_mean": [_P, _I32, _P, _I32, _P, _P, _P, ctypes.c_size_t, _P],
    "gsz_shard_grad_sqnorm": [_P, _I64, _P, _P, ctypes.c_size_t, _P],
    "gsz_clip_coef": [_P, _I32, ctypes.c_float, _P, _P, _P, _P],
    "gsz_shard_adamw_step": [_P, _I32, _P, _P, _P, _P, _P, ctypes.POINTER(AdamWHP), _P, _P, _P],
    "gsz_allgather_layout_write": [_P, _I32, _P, _P, _P],
    "gsz_bucket_unpack": [_P, _P, _P, _P],
    "gsz_bucket_accumulate": [_P, _P, _P, _P],
    "gsz_bucket_pack_f32": [_P, _P, _P, _P],
    "gsz_bucket_accumulate_f32": [_P, _P, _P, _P],
    "gsz_shard_reduce_mean_f32": [_P, _I32, _P, _I32, _P, _P, _P, ctypes.c_size_t, _P],
    "gsz_shard_reduce_mean_bf16_wire": [_P, _I32, _P, _I32, _P, _P, _P, ctypes.c_size_t, _P],
    "gsz_allreduce_mean": [_P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "gsz_adamw_step": [_P, _P, _P, _P, _I64, _P, ctypes.POINTER(AdamWHP), _P, _P],
}

_lib = None


def load():
    """Loads libgsz.so (raises if it is not built).

    torch is imported first, on purpose: torch ships its own HIP runtime with
    the same soname (libamdhip64.so.7) but asks for it as libamdhip64.so, so if
    libgsz pulled in /opt/rocm's copy first, the process would hold two HIP
    runtimes and torch's would find no GPU.  With torch loaded first, libgsz's
    dependency resolves to the runtime torch already loaded."""
    global _lib
    if _lib is None:
        import torch  # noqa: F401  (load order; see above)
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: the HIP library is not built "
                              "(run __graft_entry__.build()); there is no fallback")
        lib = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        lib.gsz_last_error.argtypes = []
        lib.gsz_last_error.restype = ctypes.c_char_p
        lib.gsz_status_string.argtypes = [ctypes.c_int]
        lib.gsz_status_string.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def _check(rc: int):
    if rc != 0:
        raise GszError(rc, load().gsz_last_error().decode())


def _stream(stream):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _ptr(t, name, dtypes, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _bf16_types():
    import torch
    return (torch.bfloat16, torch.uint16, torch.int16)


def _f32():
    import torch
    return (torch.float32,)


def _f64():
    import torch
    return (torch.float64,)


class Plan:
    """Owns a gsz_plan (host tables; device tables after upload())."""

    def __init__(self, numel, bucket_cap_bytes, world_size, align=64):
        lib = load()
        n = len(numel)
        arr = (_I64 * max(n, 1))(*[int(x) for x in numel])
        h = _P()
        _check(lib.gsz_plan_create(arr, n, int(bucket_cap_bytes), int(world_size), int(align),
                                   ctypes.byref(h)))
        self._h = h
        info = PlanInfo()
        _check(lib.gsz_plan_get_info(h, ctypes.byref(info)))
        self.n_tensors = info.n_tensors
        self.n_buckets = info.n_buckets
        self.world_size = info.world_size
        self.align = info.align
        self.bucket_cap_bytes = info.bucket_cap_bytes
        self.flat_len = info.flat_len
        self.shard_len = info.shard_len
        self.n_params = info.n_params
        self.hash = info.hash

    @property
    def handle(self):
        return self._h

    def bucket(self, b):
        out = BucketInfo()
        _check(load().gsz_plan_bucket(self._h, b, ctypes.byref(out)))
        return {f: getattr(out, f) for f, _ in BucketInfo._fields_}

    def buckets(self):
        return [self.bucket(b) for b in range(self.n_buckets)]

    def tensor(self, t):
        off, b = _I64(), _I32()
        _check(load().gsz_plan_tensor(self._h, t, ctypes.byref(off), ctypes.byref(b)))
        return off.value, b.value

    def check(self, peer_hash):
        _check(load().gsz_plan_check(self._h, ctypes.c_uint64(peer_hash)))

    def upload(self):
        _check(load().gsz_plan_upload(self._h))
        return self

    def close(self):
        if getattr(self, "_h", None):
            load().gsz_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def ledger_bytes_per_param(world_size, zero_stage):
    out = ctypes.c_double()
    _check(load().gsz_ledger_bytes_per_param(world_size, zero_stage, ctypes.byref(out)))
    return out.value


def workspace_bytes(n):
    """Device scratch bytes for a shard reduce over n elements (the plan's
    shard_len) or a squared norm of n values."""
    out = ctypes.c_size_t()
    _check(load().gsz_workspace_bytes(int(n), ctypes.byref(out)))
    return out.value


def set_grid_limit(max_blocks):
    """Caps the blocks of every later data-sized launch, process-wide (0 restores
    the built-in caps); blocks then stride over several tiles."""
    _check(load().gsz_set_grid_limit(int(max_blocks)))


def bucket_pack(plan, grads, flat, stream=None):
    bt = _bf16_types()
    if len(grads) != plan.n_tensors:
        raise ValueError("need one gradient per plan tensor")
    ptrs = (_P * max(len(grads), 1))(*[_ptr(t, f"grads[{i}]", bt) if t.numel() else None
                                       for i, t in enumerate(grads)])
    _check(load().gsz_bucket_pack(plan.handle, ptrs, _ptr(flat, "flat", bt), _stream(stream)))


def bucket_accumulate(plan, grads, flat, stream=None):
    bt = _bf16_types()
    if len(grads) != plan.n_tensors:
        raise ValueError("need one gradient per plan tensor")
    ptrs = (_P * max(len(grads), 1))(*[_ptr(t, f"grads[{i}]", bt) if t.numel() else None
                                       for i, t in enumerate(grads)])
    _check(load().gsz_bucket_accumulate(plan.handle, ptrs, _ptr(flat, "flat", bt),
                                        _stream(stream)))


def _grad_ptrs(plan, grads):
    bt = _bf16_types()
    if len(grads) != plan.n_tensors:
        raise ValueError("need one gradient per plan tensor")
    return (_P * max(len(grads), 1))(*[_ptr(t, f"grads[{i}]", bt) if t.numel() else None
                                       for i, t in enumerate(grads)])


def bucket_pack_f32(plan, grads, flat32, stream=None):
    """First micro-batch of an fp32 accumulation window: flat32 = f32(grads), pads 0."""
    _check(load().gsz_bucket_pack_f32(plan.handle, _grad_ptrs(plan, grads),
                                      _ptr(flat32, "flat32", _f32()), _stream(stream)))


def bucket_accumulate_f32(plan, grads, flat32, stream=None):
    """Later micro-batches: flat32 += f32(grads) (fp32 adds)."""
    _check(load().gsz_bucket_accumulate_f32(plan.handle, _grad_ptrs(plan, grads),
                                            _ptr(flat32, "flat32", _f32()), _stream(stream)))


def shard_reduce_mean_f32(plan, owner, contribs, layout, g, partial_out=None, ws=None, stream=None):
    """gsz_shard_reduce_mean_f32: the ring-order mean of P fp32 contributions."""
    if len(contribs) != plan.world_size:
        raise ValueError("need one contribution per rank")
    ptrs = (_P * len(contribs))(*[_ptr(t, f"contribs[{i}]", _f32()) for i, t in enumerate(contribs)])
    wsp = _ptr(ws, "ws", (ws.dtype,) if ws is not None else (), allow_none=True)
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(load().gsz_shard_reduce_mean_f32(plan.handle, owner, ptrs, layout, _ptr(g, "g", _f32()),
                                            _ptr(partial_out, "partial_out", _f64(), allow_none=True),
                                            wsp, nbytes, _stream(stream)))


def shard_reduce_mean(plan, owner, contribs, layout, g, partial_out=None, ws=None, stream=None,
                      bf16_wire=False):
    """gsz_shard_reduce_mean (or gsz_shard_reduce_mean_bf16_wire when bf16_wire)."""
    bt = _bf16_types()
    if len(contribs) != plan.world_size:
        raise ValueError("need one contribution per rank")
    ptrs = (_P * len(contribs))(*[_ptr(t, f"contribs[{i}]", bt) for i, t in enumerate(contribs)])
    wsp = _ptr(ws, "ws", (ws.dtype,) if ws is not None else (), allow_none=True)
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    fn = load().gsz_shard_reduce_mean_bf16_wire if bf16_wire else load().gsz_shard_reduce_mean
    _check(fn(plan.handle, owner, ptrs, layout, _ptr(g, "g", _f32()),
                                        _ptr(partial_out, "partial_out", _f64(), allow_none=True),
                                        wsp, nbytes, _stream(stream)))


def shard_grad_sqnorm(g, partial_out, ws, n=None, stream=None):
    n = g.numel() if n is None else n
    _check(load().gsz_shard_grad_sqnorm(_ptr(g, "g", _f32()), n,
                                        _ptr(partial_out, "partial_out", _f64()),
                                        _ptr(ws, "ws", (ws.dtype,)), ws.numel() * ws.element_size(),
                                        _stream(stream)))


def clip_coef(partials, max_norm, coef_out, norm_out=None, total_out=None, stream=None):
    _check(load().gsz_clip_coef(_ptr(partials, "partials", _f64()), partials.numel(),
                                float(max_norm), _ptr(coef_out, "coef_out", _f32()),
                                _ptr(norm_out, "norm_out", _f32(), allow_none=True),
                                _ptr(total_out, "total_out", _f64(), allow_none=True),
                                _stream(stream)))


def make_hp(lr, beta1, beta2, eps, weight_decay, step):
    return AdamWHP(lr, beta1, beta2, eps, weight_decay, step)


def shard_adamw_step(plan, owner, master, m, v, g, coef, hp, gathered=None, shard_bf16=None,
                     stream=None):
    bt = _bf16_types()
    if not isinstance(hp, AdamWHP):
        hp = AdamWHP(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, hp.step)
    _check(load().gsz_shard_adamw_step(plan.handle, owner, _ptr(master, "master", _f32()),
                                       _ptr(m, "m", _f32()), _ptr(v, "v", _f32()),
                                       _ptr(g, "g", _f32()), _ptr(coef, "coef", _f32()),
                                       ctypes.byref(hp),
                                       _ptr(gathered, "gathered", bt, allow_none=True),
                                       _ptr(shard_bf16, "shard_bf16", bt, allow_none=True),
                                       _stream(stream)))


def allgather_layout_write(plan, owner, shard_bf16, gathered, stream=None):
    bt = _bf16_types()
    _check(load().gsz_allgather_layout_write(plan.handle, owner, _ptr(shard_bf16, "shard_bf16", bt),
                                             _ptr(gathered, "gathered", bt), _stream(stream)))


def bucket_unpack(plan, flat, params, stream=None):
    bt = _bf16_types()
    if len(params) != plan.n_tensors:
        raise ValueError("need one parameter tensor per plan tensor")
    ptrs = (_P * max(len(params), 1))(*[_ptr(t, f"params[{i}]", bt) if t.numel() else None
                                        for i, t in enumerate(params)])
    _check(load().gsz_bucket_unpack(plan.handle, _ptr(flat, "flat", bt), ptrs, _stream(stream)))


def allreduce_mean(plan, contribs, g_flat, partials=None, ws=None, stream=None):
    """gsz_allreduce_mean; with partials (P doubles) and ws, the per-chunk-owner
    squared-norm partials are written in the same pass."""
    bt = _bf16_types()
    if len(contribs) != plan.world_size:
        raise ValueError("need one contribution per rank")
    ptrs = (_P * len(contribs))(*[_ptr(t, f"contribs[{i}]", bt) for i, t in enumerate(contribs)])
    wsp = _ptr(ws, "ws", (ws.dtype,) if ws is not None else (), allow_none=True)
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(load().gsz_allreduce_mean(plan.handle, ptrs, _ptr(g_flat, "g_flat", _f32()),
                                     _ptr(partials, "partials", _f64(), allow_none=True),
                                     wsp, nbytes, _stream(stream)))


def adamw_step(master, m, v, g, coef, hp, out_bf16, stream=None):
    bt = _bf16_types()
    if not isinstance(hp, AdamWHP):
        hp = AdamWHP(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, hp.step)
    _check(load().gsz_adamw_step(_ptr(master, "master", _f32()), _ptr(m, "m", _f32()),
                                 _ptr(v, "v", _f32()), _ptr(g, "g", _f32()), g.numel(),
                                 _ptr(coef, "coef", _f32()), ctypes.byref(hp),
                                 _ptr(out_bf16, "out_bf16", bt), _stream(stream)))
