"""Python binding of libkvtc (KV-cache transform coding on MI355X / gfx950).

Thin ctypes marshalling over the C ABI in include/kvtc.h; every function has
the C name. Device buffers and streams are passed as integers or as objects
with ``data_ptr()`` (torch tensors); torch is used by callers for device
memory and streams only. All codec arithmetic runs inside libkvtc.so.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvtc.so")

KVTC_OK = 0
KVTC_E_INVALID, KVTC_E_CAPACITY, KVTC_E_CORRUPT = -1, -2, -3
KVTC_E_MISMATCH, KVTC_E_NOT_CALIBRATED, KVTC_E_HIP, KVTC_E_UNSUPPORTED = -4, -5, -6, -7
KVTC_F32, KVTC_BF16 = 0, 1
KVTC_K, KVTC_V = 0, 1
KVTC_MAX_REFF = 256
KVTC_MAX_JOBS = 4096
KVTC_CAL_SHARED_BASIS, KVTC_CAL_GLOBAL_BUDGET, KVTC_CAL_COMPONENT_WIDTHS = 1, 2, 4


class kvtc_params(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("sink", C.c_int32), ("window", C.c_int32), ("group", C.c_int32),
                ("max_bits", C.c_int32), ("bits_per_value", C.c_float), ("dtype", C.c_int32)]


class kvtc_calib_input(C.Structure):
    _fields_ = [("layer", C.c_int32), ("kind", C.c_int32), ("host_kv", C.c_void_p),
                ("n_tokens", C.c_int64)]


class kvtc_job(C.Structure):
    _fields_ = [("layer", C.c_int32), ("kind", C.c_int32), ("n_tokens", C.c_int64),
                ("src", C.c_void_p), ("src_capacity", C.c_size_t), ("dst", C.c_void_p),
                ("dst_capacity", C.c_size_t),
                ("block_table", C.c_void_p), ("block_size", C.c_int32), ("n_blocks", C.c_int32)]


class kvtc_slot_info(C.Structure):
    _fields_ = [("calibrated", C.c_int32), ("n_act", C.c_int32), ("r_eff", C.c_int32),
                ("record_bytes", C.c_int32), ("slot_id", C.c_uint64),
                ("widths", C.c_uint8 * 512), ("per_component", C.c_int32), ("folded_mean", C.c_int32)]


class KvtcError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"kvtc status {status}: {msg}")
        self.status = status


_lib = None


def lib():
    """Load libkvtc.so; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with kv_cache_transform_amd.build.build()")
    L = C.CDLL(LIB_PATH)
    vp, st, i32, i64, sz = C.c_void_p, C.c_int, C.c_int32, C.c_int64, C.c_size_t
    sig = {
        "kvtc_version": (C.c_char_p, []),
        "kvtc_last_error": (C.c_char_p, []),
        "kvtc_create": (st, [C.POINTER(kvtc_params), C.POINTER(vp)]),
        "kvtc_destroy": (None, [vp]),
        "kvtc_calibrate": (st, [vp, i32, i32, vp, i64, i32]),
        "kvtc_calibrate_set": (st, [vp, C.POINTER(kvtc_calib_input), i32, C.c_uint32, i32]),
        "kvtc_slot_info_get": (st, [vp, i32, i32, C.POINTER(kvtc_slot_info)]),
        "kvtc_save": (st, [vp, vp, sz, C.POINTER(sz)]),
        "kvtc_load": (st, [vp, sz, C.POINTER(vp)]),
        "kvtc_device_state_bytes": (sz, [vp]),
        "kvtc_upload": (st, [vp, vp, sz, vp]),
        "kvtc_encoded_bytes": (sz, [vp, i32, i32, i64]),
        "kvtc_workspace_bytes": (sz, [i32]),
        "kvtc_encode": (st, [vp, C.POINTER(kvtc_job), i32, vp, vp]),
        "kvtc_decode": (st, [vp, C.POINTER(kvtc_job), i32, i32, vp, sz, vp]),
        "kvtc_decode_workspace_bytes": (sz, [vp, C.POINTER(kvtc_job), i32]),
        "kvtc_decode_noalloc": (st, [vp, C.POINTER(kvtc_job), i32, i32, vp, vp]),
        "kvtc_unpack": (st, [vp, C.POINTER(kvtc_job), vp, vp, vp, vp]),
        "kvtc_staging_bytes": (sz, [vp, C.POINTER(kvtc_job), i32]),
        "kvtc_decode_unpack": (st, [vp, C.POINTER(kvtc_job), i32, i32, vp, sz, vp, vp]),
        "kvtc_decode_restore": (st, [vp, C.POINTER(kvtc_job), i32, i32, vp, sz, vp, vp]),
        "kvtc_pack": (st, [vp, C.POINTER(kvtc_job), vp, vp, vp, vp]),
        "kvtc_read_device_status": (st, [vp, i32, C.POINTER(i32), vp]),
        "kvtc_deflate": (st, [vp, sz, vp, sz, C.POINTER(sz), i32]),
        "kvtc_lossless_bound": (sz, [vp, i32, i32, i64]),
        "kvtc_lossless_workspace_bytes": (sz, [vp, vp, i32, i32]),
        "kvtc_lossless_encode": (st, [vp, vp, i32, vp, sz, vp]),
        "kvtc_lossless_decode": (st, [vp, vp, i32, vp, sz, vp]),
        "kvtc_lossless_sizes": (st, [vp, i32, C.POINTER(C.c_uint64), vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _check(status: int):
    if status != KVTC_OK:
        raise KvtcError(status, lib().kvtc_last_error().decode())


def _ptr(x) -> int:
    if x is None:
        return 0
    if hasattr(x, "data_ptr"):
        return int(x.data_ptr())
    return int(x)


def _stream(s) -> int:
    if s is None:
        return 0
    if hasattr(s, "cuda_stream"):
        return int(s.cuda_stream)
    return int(s)


def _jobs(jobs):
    arr = (kvtc_job * len(jobs))()
    for i, j in enumerate(jobs):
        arr[i] = j
    return arr


def make_job(layer, kind, n_tokens, src, dst, dst_capacity, block_table=None, block_size=0,
             n_blocks=0, src_capacity=None) -> kvtc_job:
    """src_capacity defaults to the byte size of src when src is a tensor; a
    raw pointer needs it given."""
    if src_capacity is None:
        if not hasattr(src, "numel"):
            raise ValueError("make_job: src_capacity is required when src is a raw pointer")
        src_capacity = src.numel() * src.element_size()
    return kvtc_job(int(layer), int(kind), int(n_tokens), _ptr(src), int(src_capacity), _ptr(dst),
                    int(dst_capacity), _ptr(block_table), int(block_size), int(n_blocks))


# ------------------------------------------------------------ C entry points ---

def kvtc_version() -> str:
    return lib().kvtc_version().decode()


def kvtc_last_error() -> str:
    return lib().kvtc_last_error().decode()


def kvtc_create(params: kvtc_params) -> int:
    h = C.c_void_p()
    _check(lib().kvtc_create(C.byref(params), C.byref(h)))
    return h.value


def kvtc_destroy(codec: int) -> None:
    lib().kvtc_destroy(codec)


def kvtc_calibrate(codec: int, layer: int, kind: int, host_kv: np.ndarray, threads: int = 0) -> None:
    a = np.ascontiguousarray(host_kv)
    _check(lib().kvtc_calibrate(codec, layer, kind, a.ctypes.data, a.shape[0], threads))


def kvtc_calibrate_set(codec: int, inputs, flags: int = 0, threads: int = 0) -> None:
    """inputs: (layer, kind, host_kv [n, F]) triples."""
    arrs = [np.ascontiguousarray(x) for _, _, x in inputs]
    arr = (kvtc_calib_input * max(1, len(arrs)))()
    for i, ((layer, kind, _), a) in enumerate(zip(inputs, arrs)):
        arr[i] = kvtc_calib_input(layer, kind, a.ctypes.data, a.shape[0])
    _check(lib().kvtc_calibrate_set(codec, arr, len(arrs), flags, threads))


def kvtc_slot_info_get(codec: int, layer: int, kind: int) -> kvtc_slot_info:
    info = kvtc_slot_info()
    _check(lib().kvtc_slot_info_get(codec, layer, kind, C.byref(info)))
    return info


def kvtc_save(codec: int) -> bytes:
    n = C.c_size_t()
    _check(lib().kvtc_save(codec, None, 0, C.byref(n)))
    buf = C.create_string_buffer(n.value)
    _check(lib().kvtc_save(codec, buf, n.value, C.byref(n)))
    return buf.raw[: n.value]


def kvtc_load(data: bytes) -> int:
    h = C.c_void_p()
    buf = C.create_string_buffer(bytes(data), len(data))
    _check(lib().kvtc_load(buf, len(data), C.byref(h)))
    return h.value


def kvtc_device_state_bytes(codec: int) -> int:
    return lib().kvtc_device_state_bytes(codec)


def kvtc_upload(codec: int, d_state, nbytes: int, stream=None) -> None:
    _check(lib().kvtc_upload(codec, _ptr(d_state), nbytes, _stream(stream)))


def kvtc_encoded_bytes(codec: int, layer: int, kind: int, n_tokens: int) -> int:
    return lib().kvtc_encoded_bytes(codec, layer, kind, n_tokens)


def kvtc_workspace_bytes(max_jobs: int) -> int:
    return lib().kvtc_workspace_bytes(max_jobs)


def kvtc_encode(codec: int, jobs, d_ws, stream=None) -> None:
    _check(lib().kvtc_encode(codec, _jobs(jobs), len(jobs), _ptr(d_ws), _stream(stream)))


def kvtc_decode(codec: int, jobs, out_dtype: int, d_ws, ws_bytes: int, stream=None) -> None:
    _check(lib().kvtc_decode(codec, _jobs(jobs), len(jobs), out_dtype, _ptr(d_ws), ws_bytes,
                             _stream(stream)))


def kvtc_decode_workspace_bytes(codec: int, jobs) -> int:
    return lib().kvtc_decode_workspace_bytes(codec, _jobs(jobs), len(jobs))


def kvtc_decode_noalloc(codec: int, jobs, out_dtype: int, d_status=None, stream=None) -> None:
    _check(lib().kvtc_decode_noalloc(codec, _jobs(jobs), len(jobs), out_dtype, _ptr(d_status),
                                     _stream(stream)))


def kvtc_staging_bytes(codec: int, jobs) -> int:
    return lib().kvtc_staging_bytes(codec, _jobs(jobs), len(jobs))


def kvtc_decode_unpack(codec: int, jobs, out_dtype: int, d_staging, staging_bytes: int, d_ws,
                       stream=None) -> None:
    _check(lib().kvtc_decode_unpack(codec, _jobs(jobs), len(jobs), out_dtype, _ptr(d_staging),
                                    staging_bytes, _ptr(d_ws), _stream(stream)))


def kvtc_decode_restore(codec: int, jobs, out_dtype: int, d_staging, staging_bytes: int, d_ws,
                        stream=None) -> None:
    _check(lib().kvtc_decode_restore(codec, _jobs(jobs), len(jobs), out_dtype, _ptr(d_staging),
                                     staging_bytes, _ptr(d_ws), _stream(stream)))


def kvtc_pack(codec: int, job: kvtc_job, d_codes, d_shift_scale, d_ws, stream=None) -> None:
    _check(lib().kvtc_pack(codec, C.byref(job), _ptr(d_codes), _ptr(d_shift_scale), _ptr(d_ws),
                           _stream(stream)))


def kvtc_unpack(codec: int, job: kvtc_job, d_codes, d_shift_scale, d_ws, stream=None) -> None:
    _check(lib().kvtc_unpack(codec, C.byref(job), _ptr(d_codes), _ptr(d_shift_scale), _ptr(d_ws),
                             _stream(stream)))


def kvtc_read_device_status(d_ws, n_jobs: int, stream=None) -> np.ndarray:
    out = np.zeros(n_jobs, np.int32)
    _check(lib().kvtc_read_device_status(_ptr(d_ws), n_jobs,
                                         out.ctypes.data_as(C.POINTER(C.c_int32)), _stream(stream)))
    return out


def kvtc_lossless_bound(codec: int, layer: int, kind: int, n_tokens: int) -> int:
    return lib().kvtc_lossless_bound(codec, layer, kind, n_tokens)


def kvtc_lossless_workspace_bytes(codec: int, jobs, encode: bool) -> int:
    return lib().kvtc_lossless_workspace_bytes(codec, _jobs(jobs), len(jobs), int(bool(encode)))


def kvtc_lossless_encode(codec: int, jobs, d_ws, ws_bytes: int, stream=None) -> None:
    _check(lib().kvtc_lossless_encode(codec, _jobs(jobs), len(jobs), _ptr(d_ws), ws_bytes, _stream(stream)))


def kvtc_lossless_decode(codec: int, jobs, d_ws, ws_bytes: int, stream=None) -> None:
    _check(lib().kvtc_lossless_decode(codec, _jobs(jobs), len(jobs), _ptr(d_ws), ws_bytes, _stream(stream)))


def kvtc_lossless_sizes(d_ws, n_jobs: int, stream=None) -> np.ndarray:
    out = np.zeros(n_jobs, np.uint64)
    _check(lib().kvtc_lossless_sizes(_ptr(d_ws), n_jobs, out.ctypes.data_as(C.POINTER(C.c_uint64)),
                                     _stream(stream)))
    return out


def kvtc_deflate(data: bytes, level: int = 6) -> bytes:
    n = C.c_size_t()
    _check(lib().kvtc_deflate(data, len(data), None, 0, C.byref(n), level))
    out = C.create_string_buffer(n.value)
    _check(lib().kvtc_deflate(data, len(data), out, n.value, C.byref(n), level))
    return out.raw[: n.value]


# --------------------------------------------------------------- convenience ---

class Codec:
    """Owns a codec handle; methods forward to the C entry points."""

    def __init__(self, params: kvtc_params | None = None, handle: int | None = None):
        self.h = handle if handle is not None else kvtc_create(params)

    @classmethod
    def load(cls, data: bytes) -> "Codec":
        return cls(handle=kvtc_load(data))

    def close(self):
        if getattr(self, "h", None):
            kvtc_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 - interpreter shutdown
            pass

    def calibrate(self, layer, kind, host_kv, threads=0):
        kvtc_calibrate(self.h, layer, kind, host_kv, threads)

    def calibrate_set(self, inputs, flags=0, threads=0):
        kvtc_calibrate_set(self.h, inputs, flags, threads)

    def slot(self, layer, kind) -> kvtc_slot_info:
        return kvtc_slot_info_get(self.h, layer, kind)

    def save(self) -> bytes:
        return kvtc_save(self.h)

    def state_bytes(self) -> int:
        return kvtc_device_state_bytes(self.h)

    def upload(self, d_state, nbytes, stream=None):
        kvtc_upload(self.h, d_state, nbytes, stream)

    def encoded_bytes(self, layer, kind, n_tokens) -> int:
        return kvtc_encoded_bytes(self.h, layer, kind, n_tokens)

    def encode(self, jobs, d_ws, stream=None):
        kvtc_encode(self.h, jobs, d_ws, stream)

    def decode(self, jobs, out_dtype, d_ws, ws_bytes, stream=None):
        kvtc_decode(self.h, jobs, out_dtype, d_ws, ws_bytes, stream)

    def decode_noalloc(self, jobs, out_dtype, d_status=None, stream=None):
        kvtc_decode_noalloc(self.h, jobs, out_dtype, d_status, stream)

    def lossless_bound(self, layer, kind, n_tokens) -> int:
        return kvtc_lossless_bound(self.h, layer, kind, n_tokens)

    def lossless_workspace_bytes(self, jobs, encode) -> int:
        return kvtc_lossless_workspace_bytes(self.h, jobs, encode)

    def lossless_encode(self, jobs, d_ws, ws_bytes, stream=None):
        kvtc_lossless_encode(self.h, jobs, d_ws, ws_bytes, stream)

    def lossless_decode(self, jobs, d_ws, ws_bytes, stream=None):
        kvtc_lossless_decode(self.h, jobs, d_ws, ws_bytes, stream)

    def decode_workspace_bytes(self, jobs) -> int:
        return kvtc_decode_workspace_bytes(self.h, jobs)

    def staging_bytes(self, jobs) -> int:
        return kvtc_staging_bytes(self.h, jobs)

    def decode_unpack(self, jobs, out_dtype, d_staging, staging_bytes, d_ws, stream=None):
        kvtc_decode_unpack(self.h, jobs, out_dtype, d_staging, staging_bytes, d_ws, stream)

    def decode_restore(self, jobs, out_dtype, d_staging, staging_bytes, d_ws, stream=None):
        kvtc_decode_restore(self.h, jobs, out_dtype, d_staging, staging_bytes, d_ws, stream)

    def pack(self, job, d_codes, d_shift_scale, d_ws, stream=None):
        kvtc_pack(self.h, job, d_codes, d_shift_scale, d_ws, stream)

    def unpack(self, job, d_codes, d_shift_scale, d_ws, stream=None):
        kvtc_unpack(self.h, job, d_codes, d_shift_scale, d_ws, stream)


def params(n_layers, kv_heads, head_dim, sink, window, group, max_bits, bits_per_value,
           dtype) -> kvtc_params:
    return kvtc_params(n_layers, kv_heads, head_dim, sink, window, group, max_bits,
                       bits_per_value, dtype)
