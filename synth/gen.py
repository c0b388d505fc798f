"""ctypes wrappers around the two implementations of the input generator.

host_fill / host_fill_idx run the C implementation (OpenMP) into NumPy arrays;
dev_fill runs the HIP implementation into device memory on a stream.  Both
produce the same bits for the same (workload id, kind, rank, element index).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libsynth_host.so")
DEV_LIB = os.path.join(_HERE, "libsynth_dev.so")

MODE_F32 = 0
MODE_ABS = 1
MODE_BF16 = 2

_host = None
_dev = None


def key1(cfg_id: int, kind: int, rank: int) -> int:
    if not (0 <= cfg_id < 256 and 0 <= kind < 256 and 0 <= rank < 65536):
        raise ValueError("generator key field out of range")
    return (cfg_id << 24) | (kind << 16) | rank


def scale_for(std: float) -> np.float32:
    """fp32 multiplier of the standard normal value: the standard deviation."""
    return np.float32(std)


def _load_host():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            raise RuntimeError(f"{HOST_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(HOST_LIB)
        lib.synth_fill_host.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint64,
                                        ctypes.c_int64, ctypes.c_float, ctypes.c_int,
                                        ctypes.c_void_p]
        lib.synth_fill_host.restype = ctypes.c_int
        lib.synth_fill_host_idx.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p,
                                            ctypes.c_int64, ctypes.c_float, ctypes.c_int,
                                            ctypes.c_void_p]
        lib.synth_fill_host_idx.restype = ctypes.c_int
        lib.synth_philox4x32_10.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.synth_philox4x32_10.restype = None
        lib.synth_normal_quantile_host.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        lib.synth_normal_quantile_host.restype = None
        _host = lib
    return _host


def _load_dev():
    global _dev
    if _dev is None:
        import torch  # noqa: F401  (torch's HIP runtime must be the one loaded first)
        if not os.path.exists(DEV_LIB):
            raise RuntimeError(f"{DEV_LIB} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(DEV_LIB)
        lib.synth_fill_dev.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint64,
                                       ctypes.c_int64, ctypes.c_float, ctypes.c_int,
                                       ctypes.c_void_p, ctypes.c_void_p]
        lib.synth_fill_dev.restype = ctypes.c_int
        lib.synth_fill_dev_pieces.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p,
                                              ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                                              ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_void_p]
        lib.synth_fill_dev_pieces.restype = ctypes.c_int
        lib.synth_copy_dev.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                       ctypes.c_int, ctypes.c_void_p]
        lib.synth_copy_dev.restype = ctypes.c_int
        lib.synth_read_dev.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                       ctypes.c_int, ctypes.c_void_p]
        lib.synth_read_dev.restype = ctypes.c_int
        lib.synth_write_dev.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                        ctypes.c_void_p]
        lib.synth_write_dev.restype = ctypes.c_int
        lib.synth_read_streams_dev.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                               ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
        lib.synth_read_streams_dev.restype = ctypes.c_int
        lib.synth_probe_out_words.argtypes = [ctypes.c_int64]
        lib.synth_probe_out_words.restype = ctypes.c_int64
        _dev = lib
    return _dev


def philox4x32_10(ctr, key):
    """One Philox4x32-10 block (for the known-answer test)."""
    lib = _load_host()
    c = (ctypes.c_uint32 * 4)(*ctr)
    k = (ctypes.c_uint32 * 2)(*key)
    o = (ctypes.c_uint32 * 4)()
    lib.synth_philox4x32_10(c, k, o)
    return list(o)


def normal_quantile(p):
    """The generator's standard normal quantile at each p in (0, 1), fp64."""
    p = np.ascontiguousarray(p, dtype=np.float64)
    out = np.empty_like(p)
    _load_host().synth_normal_quantile_host(p.ctypes.data, p.size, out.ctypes.data)
    return out


def _dtype(mode):
    return np.uint16 if mode == MODE_BF16 else np.float32


def host_fill(cfg_id, kind, rank, start, n, std, mode, seed=None, out=None):
    from .workloads import SEED
    seed = SEED if seed is None else seed
    if out is None:
        out = np.empty(n, dtype=_dtype(mode))
    assert out.dtype == _dtype(mode) and out.flags.c_contiguous and out.size == n
    rc = _load_host().synth_fill_host(seed, key1(cfg_id, kind, rank), start, n,
                                      scale_for(std), mode, out.ctypes.data)
    if rc != 0:
        raise RuntimeError("synth_fill_host failed")
    return out


def host_fill_idx(cfg_id, kind, rank, idx, std, mode, seed=None):
    from .workloads import SEED
    seed = SEED if seed is None else seed
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    out = np.empty(idx.size, dtype=_dtype(mode))
    rc = _load_host().synth_fill_host_idx(seed, key1(cfg_id, kind, rank), idx.ctypes.data,
                                          idx.size, scale_for(std), mode, out.ctypes.data)
    if rc != 0:
        raise RuntimeError("synth_fill_host_idx failed")
    return out


# Device fill launches issued by this process (dev_fill and dev_fill_pieces).
# Benchmarks and profiled commands keep this small: they place every buffer
# with one piece-table launch.
fill_launches = 0


def dev_fill(out, cfg_id, kind, rank, start, std, mode, seed=None, stream=None):
    """Fill the contiguous device tensor `out` with value(start + i)."""
    global fill_launches
    import torch
    from .workloads import SEED
    seed = SEED if seed is None else seed
    want = torch.uint16 if mode == MODE_BF16 else torch.float32
    if out.dtype != want or not out.is_contiguous() or not out.is_cuda:
        raise ValueError("dev_fill needs a contiguous device tensor of the mode's dtype")
    s = torch.cuda.current_stream().cuda_stream if stream is None else stream
    rc = _load_dev().synth_fill_dev(seed, key1(cfg_id, kind, rank), start, out.numel(),
                                    scale_for(std), mode, out.data_ptr(), s)
    if rc != 0:
        raise RuntimeError(f"synth_fill_dev failed ({rc})")
    fill_launches += 1
    return out


def interleaved_place(d, P, q):
    """Index of rank q's value for shard element d in a rank-interleaved
    receive buffer of P ranks (pieces of 512 elements)."""
    return ((d >> 9) * P + q) * 512 + (d & 511)


def dev_fill_pieces(out, pieces, cfg_id, kind, rank, std, mode, seed=None, interleave=None):
    """out[dst + j] = value(param + j), j < n, for every (dst, param, n) in pieces,
    in one launch on the current stream; elements no piece covers are left as
    they are.  With interleave = (P, q) the values go to
    out[interleaved_place(dst + j, P, q)] instead.  The piece table is a device
    tensor on the same stream, so the caching allocator reuses its memory only
    after the launch."""
    global fill_launches
    import torch
    from .workloads import SEED
    seed = SEED if seed is None else seed
    want = torch.uint16 if mode == MODE_BF16 else torch.float32
    if out.dtype != want or not out.is_contiguous() or not out.is_cuda:
        raise ValueError("dev_fill_pieces needs a contiguous device tensor of the mode's dtype")
    ilv_P, ilv_q = interleave if interleave is not None else (0, 0)
    if interleave is not None and not 0 <= ilv_q < ilv_P:
        raise ValueError(f"interleave rank {ilv_q} outside [0, {ilv_P})")
    rows, cum = [], 0
    for dst, param, n in pieces:
        last = dst + n - 1
        end = (interleaved_place(last, ilv_P, ilv_q) if ilv_P else last) + 1
        if n < 0 or dst < 0 or param < 0 or (n > 0 and end > out.numel()):
            raise ValueError(f"piece ({dst}, {param}, {n}) does not fit a tensor of {out.numel()}")
        rows += [cum, dst, param]
        cum += n
    if cum == 0:
        return out
    rows += [cum, 0, 0]
    tab = torch.tensor(rows, dtype=torch.int64).to(out.device)
    rc = _load_dev().synth_fill_dev_pieces(seed, key1(cfg_id, kind, rank), tab.data_ptr(),
                                           len(pieces), cum, scale_for(std), mode,
                                           out.data_ptr(), ilv_P, ilv_q,
                                           torch.cuda.current_stream().cuda_stream)
    if rc != 0:
        raise RuntimeError(f"synth_fill_dev_pieces failed ({rc})")
    fill_launches += 1
    return out


def dev_copy(src, dst, nbytes, grid=0, stream=None):
    import torch
    s = torch.cuda.current_stream().cuda_stream if stream is None else stream
    rc = _load_dev().synth_copy_dev(src.data_ptr(), dst.data_ptr(), nbytes, grid, s)
    if rc != 0:
        raise RuntimeError(f"synth_copy_dev failed ({rc})")


def probe_out_words(nbytes, grid=0):
    """uint32 words a read probe over nbytes (per buffer) writes: 4 per block."""
    return 4 * grid if grid > 0 else int(_load_dev().synth_probe_out_words(nbytes))


def _check_sink(out, nbytes, grid):
    need = probe_out_words(nbytes, grid)
    if out.element_size() != 4 or out.numel() < need:
        raise ValueError(f"probe sink needs {need} 32-bit words, got {out.numel()}")


def dev_read(src, out, nbytes, grid=0, stream=None):
    """Read-only bandwidth probe; out must hold probe_out_words(nbytes, grid) uint32."""
    import torch
    _check_sink(out, nbytes, grid)
    s = torch.cuda.current_stream().cuda_stream if stream is None else stream
    rc = _load_dev().synth_read_dev(src.data_ptr(), out.data_ptr(), nbytes, grid, s)
    if rc != 0:
        raise RuntimeError(f"synth_read_dev failed ({rc})")


def dev_write(dst, nbytes, grid=0, stream=None):
    import torch
    s = torch.cuda.current_stream().cuda_stream if stream is None else stream
    rc = _load_dev().synth_write_dev(dst.data_ptr(), nbytes, grid, s)
    if rc != 0:
        raise RuntimeError(f"synth_write_dev failed ({rc})")


def dev_read_streams(srcs, nbytes, out, grid=0, stream=None):
    """Reads nbytes from each device tensor in srcs at the same offsets; out must
    hold probe_out_words(nbytes, grid) uint32."""
    import torch
    _check_sink(out, nbytes, grid)
    s = torch.cuda.current_stream().cuda_stream if stream is None else stream
    arr = (ctypes.c_void_p * len(srcs))(*[t.data_ptr() for t in srcs])
    rc = _load_dev().synth_read_streams_dev(arr, len(srcs), nbytes, out.data_ptr(), grid, s)
    if rc != 0:
        raise RuntimeError(f"synth_read_streams_dev failed ({rc})")
