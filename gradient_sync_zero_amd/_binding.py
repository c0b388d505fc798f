"""ctypes binding of libgsz (include/gsz.h): argument marshalling only.

Every function here converts PyTorch tensors to device pointers, takes the
current HIP stream, and calls the C entry point of the same name; all
arithmetic runs in the library's HIP kernels.  There is no fallback: if the
library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgsz.so")
# The same sources built with the test hooks (include/gsz_test.h): used only
# inside test_hooks().
TEST_LIB_PATH = os.path.join(_HERE, "libgsz_test.so")

LAYOUT_BUCKET_FLAT = 0
LAYOUT_SHARD_COMPACT = 1
LAYOUT_RANK_INTERLEAVED = 2
INTERLEAVE_PIECE = 512
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
    "gsz_plan_device_bytes": [_P, ctypes.POINTER(ctypes.c_size_t)],
    "gsz_plan_upload": [_P, _P, ctypes.c_size_t, _P],
    "gsz_ledger_bytes_per_param": [_I32, _I32, ctypes.POINTER(ctypes.c_double)],
    "gsz_workspace_bytes": [ctypes.c_int64, ctypes.POINTER(ctypes.c_size_t)],
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
    "gsz_shard_reduce_mean_noalloc": [_P, _I32, _P, _I32, _P, _P, _P],
    "gsz_allreduce_mean": [_P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "gsz_adamw_step": [_P, _P, _P, _P, _I64, _P, ctypes.POINTER(AdamWHP), _P, _P],
}

_TEST_SIGS = {"gsz_test_set_grid_limit": [ctypes.c_int64],
              "gsz_test_set_reduce_path": [_I32],
              "gsz_test_set_burst_window": [ctypes.c_uint32, ctypes.c_uint32],
              "gsz_test_set_flat_wide": [_I32],
              "gsz_test_max_tile_span": [_P, _I32, _I64, ctypes.POINTER(ctypes.c_int64)]}

_libs = {}
_active = threading.local()


def load(path=None):
    """Loads a build of libgsz (default: the one calls go to in this thread,
    libgsz.so outside test_hooks()); raises if it is not built.

    torch is imported first, on purpose: torch ships its own HIP runtime with
    the same soname (libamdhip64.so.7) but asks for it as libamdhip64.so, so if
    libgsz pulled in /opt/rocm's copy first, the process would hold two HIP
    runtimes and torch's would find no GPU.  With torch loaded first, libgsz's
    dependency resolves to the runtime torch already loaded."""
    if path is None:
        path = getattr(_active, "path", LIB_PATH)
    lib = _libs.get(path)
    if lib is None:
        import torch  # noqa: F401  (load order; see above)
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: the HIP library is not built "
                              "(run __graft_entry__.build()); there is no fallback")
        lib = ctypes.CDLL(path)
        sigs = dict(_SIGS, **(_TEST_SIGS if path == TEST_LIB_PATH else {}))
        for name, args in sigs.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        lib.gsz_last_error.argtypes = []
        lib.gsz_last_error.restype = ctypes.c_char_p
        lib.gsz_status_string.argtypes = [ctypes.c_int]
        lib.gsz_status_string.restype = ctypes.c_char_p
        _libs[path] = lib
    return lib


@contextlib.contextmanager
def test_hooks():
    """Within the block, calls made by this thread go to libgsz_test.so, the
    same sources built with the test hooks (set_grid_limit, set_reduce_path,
    set_burst_window, set_flat_wide).  Plans keep the library they were created with, so
    create them inside the block."""
    load(TEST_LIB_PATH)
    prev = getattr(_active, "path", LIB_PATH)
    _active.path = TEST_LIB_PATH
    try:
        yield
    finally:
        _active.path = prev


def _check(rc: int, lib=None):
    if rc != 0:
        lib = lib or load()
        raise GszError(rc, lib.gsz_last_error().decode())


def _lib_for(plan):
    """The library a plan was created with; it must be the one calls go to."""
    lib = load()
    if plan._lib is not lib:
        raise ValueError("this plan was created with another build of libgsz "
                         "(inside or outside test_hooks())")
    return lib


def _stream(stream):
    """A raw hipStream_t (int), a torch.cuda.Stream, or None for torch's
    current stream."""
    if stream is not None:
        return getattr(stream, "cuda_stream", stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


def _ptr(t, name, dtypes, allow_none=False, min_numel=None, numel=None):
    """Device address of tensor t after checking it.  The library receives
    bare pointers and cannot see how long a buffer is, so the lengths the plan
    implies are checked here: min_numel for buffers the call reads or writes
    a known range of, numel for tensors whose size the plan fixes exactly.  A
    short buffer would otherwise be read or written past its end on the GPU."""
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, the plan needs exactly {numel}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} has {t.numel()} elements, the call needs at least {min_numel}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def interleaved_len(plan):
    """Elements of the one receive buffer of the rank-interleaved layout: P
    pieces of INTERLEAVE_PIECE per started tile of the shard."""
    tiles = -(-plan.shard_len // INTERLEAVE_PIECE)
    return plan.world_size * tiles * INTERLEAVE_PIECE


def _contrib_len(plan, layout):
    """Elements each contribution must hold: the whole bucket-flat buffer, the
    owner's shard in shard-compact layout, or the interleaved receive buffer
    (unknown layouts are left to the library, which rejects them)."""
    if layout == LAYOUT_BUCKET_FLAT:
        return plan.flat_len
    if layout == LAYOUT_SHARD_COMPACT:
        return plan.shard_len
    if layout == LAYOUT_RANK_INTERLEAVED:
        return interleaved_len(plan)
    return None


def _contrib_ptrs(plan, contribs, layout, dtypes):
    """Host array of contribution pointers: one per rank, or the single
    receive buffer of the rank-interleaved layout."""
    n = 1 if layout == LAYOUT_RANK_INTERLEAVED else plan.world_size
    if len(contribs) != n:
        raise ValueError(f"need {n} contribution buffer(s) for layout {layout}, got {len(contribs)}")
    clen = _contrib_len(plan, layout)
    return (_P * n)(*[_ptr(t, f"contribs[{i}]", dtypes, min_numel=clen)
                      for i, t in enumerate(contribs)])


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
        self._lib = lib
        self._tables = None
        n = len(numel)
        self.numel = [int(x) for x in numel]
        arr = (_I64 * max(n, 1))(*self.numel)
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
        _check(self._lib.gsz_plan_bucket(self._h, b, ctypes.byref(out)), self._lib)
        return {f: getattr(out, f) for f, _ in BucketInfo._fields_}

    def buckets(self):
        return [self.bucket(b) for b in range(self.n_buckets)]

    def tensor(self, t):
        off, b = _I64(), _I32()
        _check(self._lib.gsz_plan_tensor(self._h, t, ctypes.byref(off), ctypes.byref(b)), self._lib)
        return off.value, b.value

    def check(self, peer_hash):
        _check(self._lib.gsz_plan_check(self._h, ctypes.c_uint64(peer_hash)), self._lib)

    def device_bytes(self):
        out = ctypes.c_size_t()
        _check(self._lib.gsz_plan_device_bytes(self._h, ctypes.byref(out)), self._lib)
        return out.value

    def upload(self, stream=None):
        """Copies the device tables into a device buffer this object owns (a
        torch allocation on the current device), on the current stream."""
        import torch
        nbytes = self.device_bytes()
        tables = torch.empty((nbytes + 15) // 16 * 2, dtype=torch.int64, device="cuda")
        _check(self._lib.gsz_plan_upload(self._h, tables.data_ptr(), tables.numel() * 8,
                                         _stream(stream)), self._lib)
        self._tables = tables
        return self

    def close(self):
        if getattr(self, "_h", None):
            self._lib.gsz_plan_destroy(self._h)
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


def _test_lib(what):
    lib = load()
    if lib is not _libs.get(TEST_LIB_PATH):
        raise RuntimeError(f"{what} exists only in the test build; call it inside test_hooks()")
    return lib


def set_grid_limit(max_blocks):
    """Test build only (inside test_hooks()): caps the blocks of every later
    data-sized launch, process-wide (0 restores the built-in caps); blocks then
    stride over several tiles."""
    lib = _test_lib("set_grid_limit")
    _check(lib.gsz_test_set_grid_limit(int(max_blocks)), lib)


REDUCE_PATH_BY_SIZE, REDUCE_PATH_BURST, REDUCE_PATH_TILE = 0, 1, 2


def set_reduce_path(path):
    """Test build only (inside test_hooks()): the kernel of every later bf16
    reduce at P > 16, process-wide: REDUCE_PATH_BY_SIZE (the product's rule),
    REDUCE_PATH_BURST or REDUCE_PATH_TILE."""
    lib = _test_lib("set_reduce_path")
    _check(lib.gsz_test_set_reduce_path(int(path)), lib)


def set_burst_window(period, window):
    """Test build only (inside test_hooks()): how the burst reduce writes g in
    every later launch, process-wide.  period 0 restores the product's choice;
    else period (100 MHz clock ticks) is a power of two and window 0 means
    chunk writes, window > 0 per-wave rings written while (clock mod period) <
    window or when full."""
    lib = _test_lib("set_burst_window")
    _check(lib.gsz_test_set_burst_window(int(period), int(window)), lib)


def set_flat_wide(on):
    """Test build only (inside test_hooks()): while on, every later
    bucket-flat reduce on the lane-contiguous kernel (bf16 at P <= 16, fp32 at
    any P) reads its contributions, and every shard AdamW writes its
    all-gather output, through 64-bit addresses: the paths of plans whose
    buckets exceed 2^29 elements; process-wide."""
    lib = _test_lib("set_flat_wide")
    _check(lib.gsz_test_set_flat_wide(1 if on else 0), lib)


def max_tile_span(plan, owner, tile):
    """Test build only (inside test_hooks(), host only): the largest span of
    positions in the bucket-flat layout that `tile` consecutive shard
    elements of `owner` take."""
    lib = _test_lib("max_tile_span")
    out = ctypes.c_int64(0)
    _check(lib.gsz_test_max_tile_span(plan.handle, int(owner), int(tile), ctypes.byref(out)), lib)
    return out.value


def bucket_pack(plan, grads, flat, stream=None):
    bt = _bf16_types()
    ptrs = _tensor_ptrs(plan, grads, "grads")
    _check(_lib_for(plan).gsz_bucket_pack(plan.handle, ptrs,
                                  _ptr(flat, "flat", bt, min_numel=plan.flat_len), _stream(stream)))


def bucket_accumulate(plan, grads, flat, stream=None):
    bt = _bf16_types()
    ptrs = _tensor_ptrs(plan, grads, "grads")
    _check(_lib_for(plan).gsz_bucket_accumulate(plan.handle, ptrs,
                                        _ptr(flat, "flat", bt, min_numel=plan.flat_len),
                                        _stream(stream)))


def _tensor_ptrs(plan, tensors, name):
    """Host array of the per-tensor device pointers, forward order; each tensor
    must hold exactly the plan's size for it (NULL for empty tensors)."""
    bt = _bf16_types()
    if len(tensors) != plan.n_tensors:
        raise ValueError(f"need one {name} tensor per plan tensor ({plan.n_tensors}), "
                         f"got {len(tensors)}")
    return (_P * max(len(tensors), 1))(*[
        _ptr(t, f"{name}[{i}]", bt, numel=plan.numel[i]) if plan.numel[i] else None
        for i, t in enumerate(tensors)])


def _grad_ptrs(plan, grads):
    return _tensor_ptrs(plan, grads, "grads")


def bucket_pack_f32(plan, grads, flat32, stream=None):
    """First micro-batch of an fp32 accumulation window: flat32 = f32(grads), pads 0."""
    _check(_lib_for(plan).gsz_bucket_pack_f32(plan.handle, _grad_ptrs(plan, grads),
                                      _ptr(flat32, "flat32", _f32(), min_numel=plan.flat_len),
                                      _stream(stream)))


def bucket_accumulate_f32(plan, grads, flat32, stream=None):
    """Later micro-batches: flat32 += f32(grads) (fp32 adds)."""
    _check(_lib_for(plan).gsz_bucket_accumulate_f32(plan.handle, _grad_ptrs(plan, grads),
                                            _ptr(flat32, "flat32", _f32(), min_numel=plan.flat_len),
                                            _stream(stream)))


def shard_reduce_mean_f32(plan, owner, contribs, layout, g, partial_out=None, ws=None, stream=None):
    """gsz_shard_reduce_mean_f32: the ring-order mean of P fp32 contributions."""
    ptrs = _contrib_ptrs(plan, contribs, layout, _f32())
    wsp = _ptr(ws, "ws", (ws.dtype,) if ws is not None else (), allow_none=True)
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(_lib_for(plan).gsz_shard_reduce_mean_f32(plan.handle, owner, ptrs, layout,
                                            _ptr(g, "g", _f32(), min_numel=plan.shard_len),
                                            _ptr(partial_out, "partial_out", _f64(),
                                                 allow_none=True,
                                                 min_numel=1),
                                            wsp, nbytes, _stream(stream)))


def shard_reduce_mean(plan, owner, contribs, layout, g, partial_out=None, ws=None, stream=None,
                      bf16_wire=False):
    """gsz_shard_reduce_mean (or gsz_shard_reduce_mean_bf16_wire when bf16_wire)."""
    ptrs = _contrib_ptrs(plan, contribs, layout, _bf16_types())
    wsp = _ptr(ws, "ws", (ws.dtype,) if ws is not None else (), allow_none=True)
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    lib = _lib_for(plan)
    fn = lib.gsz_shard_reduce_mean_bf16_wire if bf16_wire else lib.gsz_shard_reduce_mean
    _check(fn(plan.handle, owner, ptrs, layout, _ptr(g, "g", _f32(), min_numel=plan.shard_len),
              _ptr(partial_out, "partial_out", _f64(), allow_none=True, min_numel=1),
              wsp, nbytes, _stream(stream)))


def shard_reduce_mean_noalloc(plan, owner, contribs, layout, g, partial_out=None, stream=None):
    """gsz_shard_reduce_mean_noalloc: the same reduce with the library's own
    fixed scratch in place of a workspace (shards of up to 2^31 elements; calls
    that overlap on one device race)."""
    ptrs = _contrib_ptrs(plan, contribs, layout, _bf16_types())
    _check(_lib_for(plan).gsz_shard_reduce_mean_noalloc(
        plan.handle, owner, ptrs, layout, _ptr(g, "g", _f32(), min_numel=plan.shard_len),
        _ptr(partial_out, "partial_out", _f64(), allow_none=True, min_numel=1),
        _stream(stream)))


def shard_grad_sqnorm(g, partial_out, ws, n=None, stream=None):
    n = g.numel() if n is None else int(n)
    _check(load().gsz_shard_grad_sqnorm(_ptr(g, "g", _f32(), min_numel=n), n,
                                        _ptr(partial_out, "partial_out", _f64(), min_numel=1),
                                        _ptr(ws, "ws", (ws.dtype,)), ws.numel() * ws.element_size(),
                                        _stream(stream)))


def clip_coef(partials, max_norm, coef_out, norm_out=None, total_out=None, stream=None):
    _check(load().gsz_clip_coef(_ptr(partials, "partials", _f64()), partials.numel(),
                                float(max_norm), _ptr(coef_out, "coef_out", _f32(), min_numel=1),
                                _ptr(norm_out, "norm_out", _f32(), allow_none=True, min_numel=1),
                                _ptr(total_out, "total_out", _f64(), allow_none=True, min_numel=1),
                                _stream(stream)))


def make_hp(lr, beta1, beta2, eps, weight_decay, step):
    return AdamWHP(lr, beta1, beta2, eps, weight_decay, step)


def shard_adamw_step(plan, owner, master, m, v, g, coef, hp, gathered=None, shard_bf16=None,
                     stream=None):
    bt = _bf16_types()
    if not isinstance(hp, AdamWHP):
        hp = AdamWHP(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, hp.step)
    S = plan.shard_len
    _check(_lib_for(plan).gsz_shard_adamw_step(plan.handle, owner,
                                       _ptr(master, "master", _f32(), min_numel=S),
                                       _ptr(m, "m", _f32(), min_numel=S),
                                       _ptr(v, "v", _f32(), min_numel=S),
                                       _ptr(g, "g", _f32(), min_numel=S),
                                       _ptr(coef, "coef", _f32(), min_numel=1),
                                       ctypes.byref(hp),
                                       _ptr(gathered, "gathered", bt, allow_none=True,
                                            min_numel=plan.flat_len),
                                       _ptr(shard_bf16, "shard_bf16", bt, allow_none=True,
                                            min_numel=S),
                                       _stream(stream)))


def allgather_layout_write(plan, owner, shard_bf16, gathered, stream=None):
    bt = _bf16_types()
    _check(_lib_for(plan).gsz_allgather_layout_write(plan.handle, owner,
                                             _ptr(shard_bf16, "shard_bf16", bt,
                                                  min_numel=plan.shard_len),
                                             _ptr(gathered, "gathered", bt,
                                                  min_numel=plan.flat_len),
                                             _stream(stream)))


def bucket_unpack(plan, flat, params, stream=None):
    bt = _bf16_types()
    ptrs = _tensor_ptrs(plan, params, "params")
    _check(_lib_for(plan).gsz_bucket_unpack(plan.handle, _ptr(flat, "flat", bt, min_numel=plan.flat_len),
                                    ptrs, _stream(stream)))


def allreduce_mean(plan, contribs, g_flat, partials=None, ws=None, stream=None):
    """gsz_allreduce_mean; with partials (P doubles) and ws, the per-chunk-owner
    squared-norm partials are written in the same pass."""
    bt = _bf16_types()
    if len(contribs) != plan.world_size:
        raise ValueError("need one contribution per rank")
    ptrs = (_P * len(contribs))(*[_ptr(t, f"contribs[{i}]", bt, min_numel=plan.flat_len)
                                  for i, t in enumerate(contribs)])
    wsp = _ptr(ws, "ws", (ws.dtype,) if ws is not None else (), allow_none=True)
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(_lib_for(plan).gsz_allreduce_mean(plan.handle, ptrs,
                                     _ptr(g_flat, "g_flat", _f32(), min_numel=plan.flat_len),
                                     _ptr(partials, "partials", _f64(), allow_none=True,
                                          min_numel=plan.world_size),
                                     wsp, nbytes, _stream(stream)))


def adamw_step(master, m, v, g, coef, hp, out_bf16, stream=None):
    bt = _bf16_types()
    if not isinstance(hp, AdamWHP):
        hp = AdamWHP(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, hp.step)
    n = g.numel()
    _check(load().gsz_adamw_step(_ptr(master, "master", _f32(), min_numel=n),
                                 _ptr(m, "m", _f32(), min_numel=n),
                                 _ptr(v, "v", _f32(), min_numel=n), _ptr(g, "g", _f32()), n,
                                 _ptr(coef, "coef", _f32(), min_numel=1), ctypes.byref(hp),
                                 _ptr(out_bf16, "out_bf16", bt, min_numel=n), _stream(stream)))
