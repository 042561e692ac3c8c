"""ctypes binding of libkvtc.so: the same entry points as ``include/kvtc.h``.

Argument marshalling only.  Host buffers are numpy arrays, device buffers are
torch CUDA (HIP) tensors; every step of the method runs inside the library.
There is no fallback: if the library is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvtc.so")

OK, E_CONFIG, E_SHAPE, E_DTYPE, E_CAPACITY, E_STATE, E_BUFSIZE, E_DEVICE, E_ARG = 0, -1, -2, -3, -4, -5, -6, -7, -8
F32, F16 = 0, 1
MODE_DP, MODE_MIXED = 0, 1
MAX_CHOICES = 8
MAGIC = 0x4354564B


class KVTCError(RuntimeError):
    def __init__(self, status: int, what: str):
        msg = f"{what}: {status_string(status)} ({status})"
        if status == E_DEVICE and _lib is not None:
            msg += ": " + _lib.kvtc_device_error_string().decode()
        super().__init__(msg)
        self.status = status


class Config(C.Structure):
    _fields_ = [("mode", C.c_int32), ("head_dim", C.c_int32), ("heads_per_unit", C.c_int32),
                ("rank", C.c_int32), ("energy_threshold", C.c_double), ("bit_budget", C.c_int32),
                ("n_choices", C.c_int32), ("choices", C.c_int32 * MAX_CHOICES), ("beta", C.c_double),
                ("hi_bits", C.c_int32), ("lo_bits", C.c_int32), ("group_size", C.c_int32),
                ("hi_fraction", C.c_double)]


class UnitInfo(C.Structure):
    _fields_ = [("rank", C.c_int32), ("n_slots", C.c_int32), ("row_bits", C.c_int32),
                ("reserved", C.c_int32)]


class StateHeader(C.Structure):
    _fields_ = [("magic", C.c_uint32), ("version", C.c_uint32), ("mode", C.c_int32),
                ("head_dim", C.c_int32), ("heads_per_unit", C.c_int32), ("dg", C.c_int32),
                ("batch", C.c_int64), ("heads", C.c_int64), ("units", C.c_int64),
                ("rmax", C.c_int32), ("kslots", C.c_int32), ("row_stride", C.c_int32),
                ("n_qgroups", C.c_int32), ("group_size", C.c_int32), ("hi_bits", C.c_int32),
                ("lo_bits", C.c_int32), ("n_hi", C.c_int32), ("bit_budget", C.c_int32),
                ("n_choices", C.c_int32), ("choices", C.c_int32 * MAX_CHOICES), ("beta", C.c_double),
                ("energy_threshold", C.c_double), ("rank_cfg", C.c_int32), ("kfetch", C.c_int32),
                ("s_prefill", C.c_int64), ("off_unit", C.c_uint64), ("off_lambda", C.c_uint64),
                ("off_bits", C.c_uint64), ("off_qmin", C.c_uint64), ("off_qscale", C.c_uint64),
                ("off_mu", C.c_uint64), ("off_slot_comp", C.c_uint64), ("off_slot_bits", C.c_uint64),
                ("off_basis", C.c_uint64), ("off_qlo", C.c_uint64), ("off_qinv", C.c_uint64),
                ("off_w16", C.c_uint64), ("off_bias", C.c_uint64), ("total_bytes", C.c_uint64),
                ("off_kdesc", C.c_uint64), ("off_fslot", C.c_uint64), ("off_vdig", C.c_uint64),
                ("off_mv", C.c_uint64)]


class BytesReport(C.Structure):
    _fields_ = [(n, C.c_uint64) for n in ("fixed_payload", "entropy_payload", "entropy_table",
                                          "stored_payload", "basis", "quant_params", "total",
                                          "pre_entropy", "fp16_equiv", "device_store")] + \
               [("n_survived", C.c_int64), ("units_entropy_coded", C.c_int64)]

    def as_dict(self):
        return {f[0]: int(getattr(self, f[0])) for f in self._fields_}


class EntropyHeader(C.Structure):
    _fields_ = [("magic", C.c_uint32), ("version", C.c_uint32), ("S", C.c_int64), ("units", C.c_int64),
                ("kslots", C.c_int32), ("chunk_rows", C.c_int32), ("nchunks", C.c_int32), ("nsym", C.c_int32),
                ("archive_bytes", C.c_uint64), ("payload_bytes", C.c_uint64), ("table_bytes", C.c_uint64),
                ("units_coded", C.c_int64), ("off_unit", C.c_uint64), ("off_dec", C.c_uint64),
                ("off_syms", C.c_uint64), ("off_chunk", C.c_uint64), ("total_bytes", C.c_uint64)]


class EntropyUnit(C.Structure):
    _fields_ = [("offset", C.c_uint64), ("bytes", C.c_uint64), ("coded", C.c_uint32), ("table_bytes", C.c_uint32)]


class TensorRef(C.Structure):
    """One tensor's operands of a paired call (kvtc_tensor_ref)."""
    _fields_ = [("state_host", C.c_void_p), ("state_dev", C.c_void_p), ("codes_dev", C.c_void_p),
                ("params_dev", C.c_void_p), ("capacity", C.c_int64), ("rows_dev", C.c_void_p),
                ("dtype", C.c_int32), ("reserved", C.c_int32), ("strides", C.c_int64 * 4)]


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run python -m kv_cache_compression_kvtc_amd.build")
_lib = C.CDLL(LIB_PATH)

_vp, _i32, _i64, _sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
_P64 = C.POINTER(C.c_int64)
_sig = {
    "kvtc_config_default": (None, [C.POINTER(Config), _i32, _i32]),
    "kvtc_status_string": (C.c_char_p, [_i32]),
    "kvtc_build_id": (C.c_char_p, []),
    "kvtc_device_error_string": (C.c_char_p, []),
    "kvtc_fit_host": (_i32, [C.POINTER(Config), _vp, _i32, _i64, _i64, _i64, _vp, C.POINTER(_sz)]),
    "kvtc_fit_bytes_bound": (_i32, [C.POINTER(Config), _i64, _i64, C.POINTER(_sz)]),
    "kvtc_fit_workspace": (_i32, [C.POINTER(Config), _i64, _i64, _i64, C.POINTER(_sz)]),
    "kvtc_fit_device": (_i32, [C.POINTER(Config), _vp, _i32, _P64, _i64, _i64, _i64, _vp, _sz, _vp, C.POINTER(_sz),
                               _vp]),
    "kvtc_state_build": (_i32, [C.POINTER(Config), _i64, _i64, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                _vp, _i64, _vp, C.POINTER(_sz)]),
    "kvtc_allocate_bits": (_i32, [_vp, _i32, _i32, _vp, _i32, C.c_double, _vp]),
    "kvtc_store_bytes": (_i32, [_vp, _i64, C.POINTER(_sz), C.POINTER(_sz)]),
    "kvtc_append": (_i32, [_vp, _vp, _vp, _i32, _P64, _i64, _i64, _i64, _i64, _vp, _vp, _i64, _vp]),
    "kvtc_fetch": (_i32, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _P64, _vp]),
    "kvtc_bytes": (_i32, [_vp, _vp, _vp, _i64, _i64, C.POINTER(BytesReport)]),
    "kvtc_append_kv": (_i32, [C.POINTER(TensorRef), C.POINTER(TensorRef), _i64, _i64, _i64, _i64, _vp]),
    "kvtc_fetch_kv": (_i32, [C.POINTER(TensorRef), C.POINTER(TensorRef), _i64, _i64, _vp]),
    "kvtc_fetch_kv_probe": (_i32, [C.POINTER(TensorRef), C.POINTER(TensorRef), _i64, _i64, _vp]),
    "kvtc_refit_bytes": (_i32, [_vp, _i64, C.POINTER(_sz), C.POINTER(_sz)]),
    "kvtc_entropy_bytes": (_i32, [_vp, _i64, C.POINTER(_sz), C.POINTER(_sz), C.POINTER(_sz)]),
    "kvtc_entropy_encode": (_i32, [_vp, _vp, _vp, _i64, _i64, _vp, _sz, _vp, _sz, _vp, _sz, _vp]),
    "kvtc_entropy_decode": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp]),
    "kvtc_append_refit": (_i32, [_vp, _vp, _vp, _i32, _P64, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _i64, _vp]),
    "kvtc_fetch_refit": (_i32, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _P64, _vp]),
    "kvtc_attend_workspace": (_i32, [_vp, _vp, _i64, C.POINTER(_sz)]),
    "kvtc_attend": (_i32, [C.POINTER(TensorRef), C.POINTER(TensorRef), _vp, _i32, _P64, _i64, _vp, _P64, _vp,
                           _sz, _vp]),
    "kvtc_attend_noalloc": (_i32, [C.POINTER(TensorRef), C.POINTER(TensorRef), _vp, _i32, _P64, _i64, _vp, _P64,
                                   _vp]),
    "kvtc_attend_gqa_workspace": (_i32, [_vp, _vp, _i64, _i64, C.POINTER(_sz)]),
    "kvtc_attend_gqa": (_i32, [C.POINTER(TensorRef), C.POINTER(TensorRef), _i64, _vp, _i32, _P64, _i64, _vp, _P64,
                               _vp, _sz, _vp]),
}
for _name, (_res, _args) in _sig.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_sig)


def build_id() -> str:
    """Hash of the sources the loaded library was built from."""
    return _lib.kvtc_build_id().decode()


def status_string(status: int) -> str:
    return _lib.kvtc_status_string(status).decode()


def _check(status: int, what: str):
    if status != OK:
        raise KVTCError(status, what)


def _host_ptr(a):
    return None if a is None else a.ctypes.data


def _dev_ptr(t):
    return None if t is None else t.data_ptr()


def _strides4(t):
    return (C.c_int64 * 4)(*[int(s) for s in t.stride()])


def _stream_ptr(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


# ---------------------------------------------------------------- config
def config_default(mode: int = MODE_DP, head_dim: int = 128) -> Config:
    cfg = Config()
    _lib.kvtc_config_default(C.byref(cfg), mode, head_dim)
    return cfg


def make_config(mode="dp", head_dim=128, heads_per_unit=None, rank=0, energy=0.90, budget=None,
                choices=(0, 1, 2, 3, 4, 8), beta=1.0, hi_bits=4, lo_bits=2, group_size=32,
                hi_fraction=0.25) -> Config:
    m = MODE_DP if mode == "dp" else MODE_MIXED
    cfg = config_default(m, head_dim)
    cfg.heads_per_unit = heads_per_unit if heads_per_unit is not None else (1 if m == MODE_DP else 8)
    cfg.rank = rank
    cfg.energy_threshold = energy
    cfg.bit_budget = 4 * head_dim if budget is None else budget
    cfg.n_choices = len(choices)
    for i, b in enumerate(choices):
        cfg.choices[i] = b
    cfg.beta = beta
    cfg.hi_bits, cfg.lo_bits, cfg.group_size, cfg.hi_fraction = hi_bits, lo_bits, group_size, hi_fraction
    return cfg


# ---------------------------------------------------------------- host calls
def kvtc_fit_host(cfg: Config, rows: np.ndarray) -> np.ndarray:
    """Fit one tensor's frozen state on contiguous host rows [B, H, S, D]; returns the blob."""
    rows = np.ascontiguousarray(rows)
    dtype = {np.dtype(np.float32): F32, np.dtype(np.float16): F16}.get(rows.dtype)
    if dtype is None:
        raise KVTCError(E_DTYPE, "kvtc_fit_host")
    B, H, S, D = rows.shape
    buf, size = _fit_buffer(cfg, B, H)
    _check(_lib.kvtc_fit_host(C.byref(cfg), _host_ptr(rows), dtype, B, H, S, _host_ptr(buf), C.byref(size)),
           "kvtc_fit_host")
    return buf[: size.value].copy()


def _fit_buffer(cfg: Config, B: int, H: int):
    """A host buffer large enough for any fit of this configuration and shape,
    so that one fit call suffices (np.empty: pages are only touched as written)."""
    bound = C.c_size_t(0)
    _check(_lib.kvtc_fit_bytes_bound(C.byref(cfg), B, H, C.byref(bound)), "kvtc_fit_bytes_bound")
    return np.empty(bound.value, dtype=np.uint8), C.c_size_t(bound.value)


def kvtc_fit_device(cfg: Config, rows, stream=None) -> np.ndarray:
    """Fit one tensor's frozen state on device rows [B, H, S, D] (fp16/fp32 tensor,
    any strides with a unit innermost one); returns the host blob.  The device
    workspace is allocated here (torch) for the duration of the call."""
    import torch
    dtype = {torch.float16: F16, torch.float32: F32}.get(rows.dtype)
    if dtype is None:
        raise KVTCError(E_DTYPE, "kvtc_fit_device")
    if rows.dim() != 4 or not rows.is_cuda:
        raise KVTCError(E_SHAPE, "kvtc_fit_device: rows must be a device tensor [B, H, S, D]")
    B, H, S, D = rows.shape
    need = C.c_size_t(0)
    _check(_lib.kvtc_fit_workspace(C.byref(cfg), B, H, S, C.byref(need)), "kvtc_fit_workspace")
    work = torch.empty(need.value + 256, dtype=torch.uint8, device=rows.device)
    off = (-work.data_ptr()) % 256
    buf, size = _fit_buffer(cfg, B, H)
    _check(_lib.kvtc_fit_device(C.byref(cfg), _dev_ptr(rows), dtype, _strides4(rows), B, H, S, work.data_ptr() + off,
                                need.value, _host_ptr(buf), C.byref(size), _stream_ptr(stream)), "kvtc_fit_device")
    return buf[: size.value].copy()


def kvtc_state_build(cfg: Config, B: int, H: int, ranks, mu, basis, lam=None, bits=None, qmin=None,
                     qscale=None, s_prefill: int = 0) -> np.ndarray:
    """Blob from frozen parts: ranks [U], mu [U,dg] f32, basis [U,rmax,dg] f32 (row = component),
    lam [U,dg] f64 or None, bits [U,rmax] u8, qmin/qscale [U,rmax] f32 (DP)."""
    ranks = np.ascontiguousarray(ranks, dtype=np.int32)
    mu = np.ascontiguousarray(mu, dtype=np.float32)
    basis = np.ascontiguousarray(basis, dtype=np.float32)
    rmax = basis.shape[1]
    conv = lambda a, dt: None if a is None else np.ascontiguousarray(a, dtype=dt)
    lam, bits = conv(lam, np.float64), conv(bits, np.uint8)
    qmin, qscale = conv(qmin, np.float32), conv(qscale, np.float32)
    if cfg.heads_per_unit < 1 or H % cfg.heads_per_unit:
        raise KVTCError(E_SHAPE, "kvtc_state_build")
    U, dg = B * (H // cfg.heads_per_unit), cfg.head_dim * cfg.heads_per_unit
    want = {"ranks": (ranks, (U,)), "mu": (mu, (U, dg)), "basis": (basis, (U, rmax, dg)),
            "lam": (lam, (U, dg)), "bits": (bits, (U, rmax)), "qmin": (qmin, (U, rmax)),
            "qscale": (qscale, (U, rmax))}
    for name, (arr, shape) in want.items():
        if arr is not None and arr.shape != shape:
            raise KVTCError(E_SHAPE, f"kvtc_state_build: {name} must be {shape}, got {arr.shape}")
    args = [C.byref(cfg), B, H, rmax, _host_ptr(ranks), _host_ptr(mu), _host_ptr(basis),
            _host_ptr(lam), _host_ptr(bits), _host_ptr(qmin), _host_ptr(qscale), s_prefill]
    size = C.c_size_t(0)
    _check(_lib.kvtc_state_build(*args, None, C.byref(size)), "kvtc_state_build(size)")
    blob = np.zeros(size.value, dtype=np.uint8)
    _check(_lib.kvtc_state_build(*args, _host_ptr(blob), C.byref(size)), "kvtc_state_build")
    return blob


def kvtc_allocate_bits(lam, budget: int, choices, beta: float = 1.0) -> np.ndarray:
    lam = np.ascontiguousarray(lam, dtype=np.float64)
    ch = np.ascontiguousarray(choices, dtype=np.int32)
    out = np.zeros(len(lam), dtype=np.uint8)
    _check(_lib.kvtc_allocate_bits(_host_ptr(lam), len(lam), budget, _host_ptr(ch), len(ch), beta,
                                   _host_ptr(out)), "kvtc_allocate_bits")
    return out


def kvtc_store_bytes(blob: np.ndarray, capacity: int):
    _check_blob(blob, "kvtc_store_bytes")
    cb, pb = C.c_size_t(0), C.c_size_t(0)
    _check(_lib.kvtc_store_bytes(_host_ptr(blob), capacity, C.byref(cb), C.byref(pb)), "kvtc_store_bytes")
    return cb.value, pb.value


def kvtc_bytes(blob: np.ndarray, codes: np.ndarray, params, capacity: int, S: int) -> dict:
    h = _check_blob(blob, "kvtc_bytes")
    if np.asarray(codes).nbytes < h.units * capacity * h.row_stride:
        raise KVTCError(E_ARG, "kvtc_bytes: code store smaller than units*capacity*row_stride")
    rep = BytesReport()
    _check(_lib.kvtc_bytes(_host_ptr(blob), _host_ptr(np.ascontiguousarray(codes)), _host_ptr(params),
                           capacity, S, C.byref(rep)), "kvtc_bytes")
    return rep.as_dict()


# ---------------------------------------------------------------- device calls
def _check_blob(blob, what):
    """The C ABI takes no blob length: a host blob must hold the header and the
    total_bytes it declares before its pointer is passed."""
    if not isinstance(blob, np.ndarray) or blob.dtype != np.uint8 or not blob.flags.c_contiguous:
        raise KVTCError(E_ARG, what + ": state blob must be a contiguous uint8 array")
    if blob.nbytes < C.sizeof(StateHeader):
        raise KVTCError(E_STATE, what + ": state blob shorter than its header")
    h = header(blob)
    if h.magic != MAGIC or blob.nbytes < h.total_bytes:
        raise KVTCError(E_STATE, what + ": state blob shorter than its total_bytes or not a state")
    return h


def _check_buffers(blob, blob_dev, codes, params, capacity, what):
    h = _check_blob(blob, what)
    if blob_dev is None or not blob_dev.is_cuda or blob_dev.numel() * blob_dev.element_size() < h.total_bytes:
        raise KVTCError(E_ARG, what + ": device state copy")
    cb, pb = kvtc_store_bytes(blob, capacity)
    if cb and (codes is None or not codes.is_cuda or codes.numel() * codes.element_size() < cb):
        raise KVTCError(E_ARG, what + ": code store smaller than units*capacity*row_stride")
    if pb and (params is None or not params.is_cuda or params.numel() * params.element_size() < pb):
        raise KVTCError(E_ARG, what + ": parameter store too small")
    return h


def kvtc_append(blob: np.ndarray, blob_dev, x, s0: int, codes, params, capacity: int, stream=None):
    """Append rows x [B, H, n, D] (fp16/fp32 device tensor) at store rows [s0, s0+n)."""
    import torch
    dtype = {torch.float16: F16, torch.float32: F32}.get(x.dtype)
    if dtype is None:
        raise KVTCError(E_DTYPE, "kvtc_append")
    h = _check_buffers(blob, blob_dev, codes, params, capacity, "kvtc_append")
    if x.dim() != 4 or not x.is_cuda or x.shape[3] != h.head_dim:
        raise KVTCError(E_SHAPE, "kvtc_append: x must be a device tensor [B, H, n, D]")
    B, H, n, D = x.shape
    _check(_lib.kvtc_append(_host_ptr(blob), _dev_ptr(blob_dev), _dev_ptr(x), dtype, _strides4(x), B, H, n,
                            s0, _dev_ptr(codes), _dev_ptr(params), capacity, _stream_ptr(stream)),
           "kvtc_append")


def kvtc_fetch(blob: np.ndarray, blob_dev, codes, params, capacity: int, s_begin: int, s_end: int, out,
               stream=None):
    """Reconstruct store rows [s_begin, s_end) into the fp16 device tensor out [B, H, s_end-s_begin, D]."""
    import torch
    if out.dtype != torch.float16:
        raise KVTCError(E_DTYPE, "kvtc_fetch")
    h = _check_buffers(blob, blob_dev, codes, params, capacity, "kvtc_fetch")
    if not out.is_cuda or tuple(out.shape) != (h.batch, h.heads, s_end - s_begin, h.head_dim):
        raise KVTCError(E_SHAPE, "kvtc_fetch: out must be a device tensor [B, H, s_end - s_begin, D]")
    _check(_lib.kvtc_fetch(_host_ptr(blob), _dev_ptr(blob_dev), _dev_ptr(codes), _dev_ptr(params), capacity,
                           s_begin, s_end, _dev_ptr(out), _strides4(out), _stream_ptr(stream)), "kvtc_fetch")


def _tensor_ref(blob, blob_dev, codes, params, capacity, rows, dtype) -> TensorRef:
    ref = TensorRef()
    ref.state_host, ref.state_dev = _host_ptr(blob), _dev_ptr(blob_dev)
    ref.codes_dev, ref.params_dev = _dev_ptr(codes), _dev_ptr(params)
    ref.capacity = capacity
    ref.rows_dev = _dev_ptr(rows)
    ref.dtype = dtype
    for i, st in enumerate(rows.stride()):
        ref.strides[i] = int(st)
    return ref


def kvtc_append_kv(k, v, s0: int, capacity: int, stream=None):
    """Append rows to the key and the value tensor in one call.  ``k`` and ``v`` are
    (blob, blob_dev, x, codes, params) with x a device tensor [B, H, n, D]; both x
    must have the same shape.  Same results as kvtc_append on each."""
    import torch
    refs = []
    for (blob, blob_dev, x, codes, params) in (k, v):
        dtype = {torch.float16: F16, torch.float32: F32}.get(x.dtype)
        if dtype is None:
            raise KVTCError(E_DTYPE, "kvtc_append_kv")
        h = _check_buffers(blob, blob_dev, codes, params, capacity, "kvtc_append_kv")
        if x.dim() != 4 or not x.is_cuda or x.shape[3] != h.head_dim:
            raise KVTCError(E_SHAPE, "kvtc_append_kv: x must be a device tensor [B, H, n, D]")
        refs.append(_tensor_ref(blob, blob_dev, codes, params, capacity, x, dtype))
    if tuple(k[2].shape) != tuple(v[2].shape):
        raise KVTCError(E_SHAPE, "kvtc_append_kv: key and value rows differ in shape")
    B, H, n, _ = k[2].shape
    _check(_lib.kvtc_append_kv(C.byref(refs[0]), C.byref(refs[1]), B, H, n, s0, _stream_ptr(stream)),
           "kvtc_append_kv")


def kvtc_fetch_kv(k, v, capacity: int, s_begin: int, s_end: int, stream=None):
    """Reconstruct rows [s_begin, s_end) of the key and the value tensor in one call.
    ``k`` and ``v`` are (blob, blob_dev, codes, params, out) with out an fp16 device
    tensor [B, H, s_end - s_begin, D].  Same results as kvtc_fetch on each."""
    import torch
    refs = []
    for (blob, blob_dev, codes, params, out) in (k, v):
        if out.dtype != torch.float16:
            raise KVTCError(E_DTYPE, "kvtc_fetch_kv")
        h = _check_buffers(blob, blob_dev, codes, params, capacity, "kvtc_fetch_kv")
        if not out.is_cuda or tuple(out.shape) != (h.batch, h.heads, s_end - s_begin, h.head_dim):
            raise KVTCError(E_SHAPE, "kvtc_fetch_kv: out must be a device tensor [B, H, s_end - s_begin, D]")
        refs.append(_tensor_ref(blob, blob_dev, codes, params, capacity, out, F16))
    _check(_lib.kvtc_fetch_kv(C.byref(refs[0]), C.byref(refs[1]), s_begin, s_end, _stream_ptr(stream)),
           "kvtc_fetch_kv")


# ---------------------------------------------------------------- refit mode
def kvtc_refit_bytes(blob: np.ndarray, capacity: int):
    """(latent store bytes, refit buffer bytes) of a refit-mode DP tensor."""
    _check_blob(blob, "kvtc_refit_bytes")
    lb, rb = C.c_size_t(0), C.c_size_t(0)
    _check(_lib.kvtc_refit_bytes(_host_ptr(blob), capacity, C.byref(lb), C.byref(rb)), "kvtc_refit_bytes")
    return lb.value, rb.value


def refit_sections(blob: np.ndarray, capacity: int) -> dict:
    """Byte offsets of the refit buffer's sections (the layout kvtc.h documents)."""
    h = header(blob)
    U, ks = h.units, h.kslots
    chunks = min(max((capacity + 255) // 256, 1), 256)
    out, o = {}, 0
    for name, nbytes in (("qmin32", U * ks * 4), ("qscale32", U * ks * 4), ("qlo", U * ks * 8),
                         ("qinv", U * ks * 8), ("w16", U * h.dg * h.kfetch * 2), ("bias", U * h.dg * 4),
                         ("part", U * chunks * ks * 16)):
        out[name] = (o, nbytes)
        o = (o + max(nbytes, 1) + 255) // 256 * 256
    return out


class RefitStore:
    """Device buffers of one refit-mode tensor for ``capacity`` rows: the fp64
    latent store, the code store and the refit buffer (torch allocations)."""

    def __init__(self, blob, blob_dev, capacity, device="cuda:0"):
        import torch
        _check_blob(blob, "RefitStore")
        lb, rb = kvtc_refit_bytes(blob, capacity)
        cb, _ = kvtc_store_bytes(blob, capacity)
        self.blob, self.blob_dev, self.capacity = blob, blob_dev, capacity
        self.latents = torch.zeros(max(lb // 8, 1), dtype=torch.float64, device=device)
        self.codes = torch.zeros(max(cb, 4), dtype=torch.uint8, device=device)
        self._refit = torch.zeros(rb + 256, dtype=torch.uint8, device=device)
        self._off = (-self._refit.data_ptr()) % 256
        self.refit = self._refit[self._off: self._off + rb]
        _check_buffers(blob, blob_dev, self.codes, None, capacity, "RefitStore")

    def append(self, x, s0: int, stream=None):
        """kvtc_append_refit of rows x [B, H, n, D] at store rows [s0, s0 + n)."""
        import torch
        dtype = {torch.float16: F16, torch.float32: F32}.get(x.dtype)
        if dtype is None:
            raise KVTCError(E_DTYPE, "kvtc_append_refit")
        h = header(self.blob)
        if x.dim() != 4 or not x.is_cuda or x.shape[3] != h.head_dim:
            raise KVTCError(E_SHAPE, "kvtc_append_refit: x must be a device tensor [B, H, n, D]")
        B, H, n, _ = x.shape
        _check(_lib.kvtc_append_refit(_host_ptr(self.blob), _dev_ptr(self.blob_dev), _dev_ptr(x), dtype, _strides4(x),
                                      B, H, n, s0, _dev_ptr(self.latents), _dev_ptr(self.codes),
                                      self.refit.data_ptr(), self.capacity, _stream_ptr(stream)), "kvtc_append_refit")

    def fetch(self, s_begin: int, s_end: int, out, stream=None):
        """kvtc_fetch_refit of store rows [s_begin, s_end) into fp16 out [B, H, s_end - s_begin, D]."""
        import torch
        h = header(self.blob)
        if out.dtype != torch.float16 or not out.is_cuda or \
                tuple(out.shape) != (h.batch, h.heads, s_end - s_begin, h.head_dim):
            raise KVTCError(E_SHAPE, "kvtc_fetch_refit: out must be fp16 [B, H, s_end - s_begin, D]")
        _check(_lib.kvtc_fetch_refit(_host_ptr(self.blob), _dev_ptr(self.blob_dev), _dev_ptr(self.codes),
                                     self.refit.data_ptr(), self.capacity, s_begin, s_end, _dev_ptr(out),
                                     _strides4(out), _stream_ptr(stream)), "kvtc_fetch_refit")

    def ranges(self):
        """The refitted (qmin32, qscale32) per slot, as host arrays [units, kslots]."""
        h = header(self.blob)
        sec = refit_sections(self.blob, self.capacity)
        raw = self.refit.cpu().numpy()
        get = lambda name: raw[sec[name][0]: sec[name][0] + sec[name][1]].view(np.float32).reshape(h.units, h.kslots)
        return get("qmin32").copy(), get("qscale32").copy()


# ---------------------------------------------------------------- entropy-coded storage
def kvtc_entropy_bytes(blob: np.ndarray, S: int):
    """(device workspace, archive bound, index) bytes of entropy coding S rows."""
    _check_blob(blob, "kvtc_entropy_bytes")
    w, a, i = C.c_size_t(0), C.c_size_t(0), C.c_size_t(0)
    _check(_lib.kvtc_entropy_bytes(_host_ptr(blob), S, C.byref(w), C.byref(a), C.byref(i)), "kvtc_entropy_bytes")
    return w.value, a.value, i.value


class EntropyArchive:
    """The entropy-coded storage of rows [0, S) of a DP tensor's device code
    store (kvtc_entropy_encode): ``archive`` (a device uint8 tensor holding
    ``header.archive_bytes`` bytes) and ``index`` (host uint8 array) with its
    device copy.  ``decode(codes)`` restores the rows into a code store."""

    def __init__(self, blob, blob_dev, codes, capacity: int, S: int, stream=None):
        import torch
        _check_buffers(blob, blob_dev, codes, None, capacity, "EntropyArchive")
        wb, ab, ib = kvtc_entropy_bytes(blob, S)
        dev = blob_dev.device
        work = torch.empty(wb + 256, dtype=torch.uint8, device=dev)
        woff = (-work.data_ptr()) % 256
        self.archive = torch.empty(ab, dtype=torch.uint8, device=dev)
        self.index = np.zeros(ib, dtype=np.uint8)
        self.blob, self.blob_dev, self.S = blob, blob_dev, S
        _check(_lib.kvtc_entropy_encode(_host_ptr(blob), _dev_ptr(blob_dev), _dev_ptr(codes), capacity, S,
                                        work.data_ptr() + woff, wb, _dev_ptr(self.archive), ab, _host_ptr(self.index),
                                        ib, _stream_ptr(stream)), "kvtc_entropy_encode")
        self.header = EntropyHeader.from_buffer_copy(self.index[: C.sizeof(EntropyHeader)].tobytes())
        self.index_dev = torch.from_numpy(self.index).to(dev)

    def units(self):
        h = self.header
        return [EntropyUnit.from_buffer_copy(self.index[h.off_unit + C.sizeof(EntropyUnit) * u:
                                                        h.off_unit + C.sizeof(EntropyUnit) * (u + 1)].tobytes())
                for u in range(h.units)]

    def bytes(self) -> np.ndarray:
        """The archive's stored bytes, on the host."""
        return self.archive[: self.header.archive_bytes].cpu().numpy()

    def decode(self, codes, capacity: int, stream=None):
        """kvtc_entropy_decode into the code store ``codes`` (rows [0, S))."""
        _check_buffers(self.blob, self.blob_dev, codes, None, capacity, "kvtc_entropy_decode")
        _check(_lib.kvtc_entropy_decode(_host_ptr(self.blob), _dev_ptr(self.blob_dev), _host_ptr(self.index),
                                        _dev_ptr(self.index_dev), _dev_ptr(self.archive), _dev_ptr(codes), capacity,
                                        _stream_ptr(stream)), "kvtc_entropy_decode")


def kvtc_attend_workspace(blob_k: np.ndarray, blob_v: np.ndarray, s_end: int) -> int:
    _check_blob(blob_k, "kvtc_attend_workspace")
    _check_blob(blob_v, "kvtc_attend_workspace")
    n = C.c_size_t(0)
    _check(_lib.kvtc_attend_workspace(_host_ptr(blob_k), _host_ptr(blob_v), s_end, C.byref(n)),
           "kvtc_attend_workspace")
    return n.value


def kvtc_attend_gqa_workspace(blob_k: np.ndarray, blob_v: np.ndarray, q_heads: int, s_end: int) -> int:
    _check_blob(blob_k, "kvtc_attend_gqa_workspace")
    _check_blob(blob_v, "kvtc_attend_gqa_workspace")
    n = C.c_size_t(0)
    _check(_lib.kvtc_attend_gqa_workspace(_host_ptr(blob_k), _host_ptr(blob_v), q_heads, s_end, C.byref(n)),
           "kvtc_attend_gqa_workspace")
    return n.value


class Attend:
    """kvtc_attend with its buffers checked once: decode attention of queries
    [B, H, D] over store rows [0, s_end) of a key and a value tensor.  ``k`` and
    ``v`` are (blob, blob_dev, codes, params); the device workspace is allocated
    here (torch) for ``capacity`` rows and reused by every call.  With
    ``q_heads`` set, queries are [B, q_heads, D] and the call is kvtc_attend_gqa
    (q_heads a multiple of H; query head hq attends KV head hq // (q_heads / H))."""

    def __init__(self, k, v, capacity: int, stream=None, q_heads=None):
        import torch
        self._keep = (k, v)
        self._refs = []
        for (blob, blob_dev, codes, params) in (k, v):
            _check_buffers(blob, blob_dev, codes, params, capacity, "Attend")
            ref = TensorRef()
            ref.state_host, ref.state_dev = _host_ptr(blob), _dev_ptr(blob_dev)
            ref.codes_dev, ref.params_dev = _dev_ptr(codes), _dev_ptr(params)
            ref.capacity = capacity
            self._refs.append(ref)
        self.h = header(k[0])
        self.capacity = capacity
        self.q_heads = q_heads
        nbytes = (kvtc_attend_workspace(k[0], v[0], capacity) if q_heads is None else
                  kvtc_attend_gqa_workspace(k[0], v[0], q_heads, capacity))
        self.work = torch.empty(max(nbytes, 256) + 256, dtype=torch.uint8, device=k[1].device)
        off = (-self.work.data_ptr()) % 256
        self._work, self._work_bytes = self.work.data_ptr() + off, self.work.numel() - off
        self._stream = _stream_ptr(stream)

    def __call__(self, q, s_end: int, out=None):
        """Queries q: device tensor [B, H, D] (fp16 or fp32); returns fp16 [B, H, D]."""
        import torch
        h = self.h
        dtype = {torch.float16: F16, torch.float32: F32}.get(q.dtype)
        if dtype is None:
            raise KVTCError(E_DTYPE, "kvtc_attend")
        hq = h.heads if self.q_heads is None else self.q_heads
        if not q.is_cuda or tuple(q.shape) != (h.batch, hq, h.head_dim):
            raise KVTCError(E_SHAPE, "kvtc_attend: q must be a device tensor [B, Hq, D]")
        if out is None:
            out = torch.empty((h.batch, hq, h.head_dim), dtype=torch.float16, device=q.device)
        if out.dtype != torch.float16 or tuple(out.shape) != tuple(q.shape):
            raise KVTCError(E_SHAPE, "kvtc_attend: out must be fp16 [B, Hq, D]")
        qs = (C.c_int64 * 3)(*[int(x) for x in q.stride()])
        os_ = (C.c_int64 * 3)(*[int(x) for x in out.stride()])
        if self.q_heads is None:
            _check(_lib.kvtc_attend(C.byref(self._refs[0]), C.byref(self._refs[1]), q.data_ptr(), dtype, qs, s_end,
                                    out.data_ptr(), os_, self._work, self._work_bytes, self._stream), "kvtc_attend")
        else:
            _check(_lib.kvtc_attend_gqa(C.byref(self._refs[0]), C.byref(self._refs[1]), self.q_heads, q.data_ptr(),
                                        dtype, qs, s_end, out.data_ptr(), os_, self._work, self._work_bytes,
                                        self._stream), "kvtc_attend_gqa")
        return out

    def noalloc(self, q, s_end: int, out):
        """The same attention through kvtc_attend_noalloc (the library's fixed
        scratch instead of this object's workspace); out: fp16 [B, H, D]."""
        import torch
        dtype = {torch.float16: F16, torch.float32: F32}.get(q.dtype)
        if dtype is None:
            raise KVTCError(E_DTYPE, "kvtc_attend_noalloc")
        qs = (C.c_int64 * 3)(*[int(x) for x in q.stride()])
        os_ = (C.c_int64 * 3)(*[int(x) for x in out.stride()])
        _check(_lib.kvtc_attend_noalloc(C.byref(self._refs[0]), C.byref(self._refs[1]), q.data_ptr(), dtype, qs,
                                        s_end, out.data_ptr(), os_, self._stream), "kvtc_attend_noalloc")
        return out


# ---------------------------------------------------------------- blob introspection
def header(blob: np.ndarray) -> StateHeader:
    return StateHeader.from_buffer_copy(blob[: C.sizeof(StateHeader)].tobytes())


def state_view(blob: np.ndarray) -> dict:
    """Numpy views of the blob's sections (layout of include/kvtc.h)."""
    h = header(blob)
    if h.magic != MAGIC:
        raise KVTCError(E_STATE, "state_view")
    U, dg, rmax, ks, kf = h.units, h.dg, h.rmax, h.kslots, h.kfetch

    def sec(off, dt, shape):
        n = int(np.prod(shape))
        return np.frombuffer(blob, dtype=dt, count=n, offset=off).reshape(shape)

    unit = sec(h.off_unit, np.int32, (U, 4))
    return {
        "header": h,
        "rank": unit[:, 0], "n_slots": unit[:, 1], "row_bits": unit[:, 2],
        "lambda": sec(h.off_lambda, np.float64, (U, dg)),
        "bits": sec(h.off_bits, np.uint8, (U, rmax)),
        "qmin": sec(h.off_qmin, np.float32, (U, rmax)),
        "qscale": sec(h.off_qscale, np.float32, (U, rmax)),
        "mu": sec(h.off_mu, np.float32, (U, dg)),
        "slot_comp": sec(h.off_slot_comp, np.int32, (U, ks)),
        "slot_bits": sec(h.off_slot_bits, np.uint32, (U, ks)),
        "basis": sec(h.off_basis, np.float32, (U, ks, dg)),
        "qlo": sec(h.off_qlo, np.float64, (U, ks)),
        "qinv": sec(h.off_qinv, np.float64, (U, ks)),
        "w16": sec(h.off_w16, np.float16, (U, dg, kf)),
        "kdesc": sec(h.off_kdesc, np.uint32, (U, kf // 16)),
        "fslot": sec(h.off_fslot, np.int32, (U, kf)),
        "bias": sec(h.off_bias, np.float32, (U, dg)),
        "vdig": sec(h.off_vdig, np.int8, (U, 5, ks, dg)) if h.off_vdig else None,
        "mv": sec(h.off_mv, np.float64, (U, ks)) if h.off_mv else None,
    }


# ---------------------------------------------------------------- prepared calls
class PreparedAppend:
    """kvtc_append with every buffer checked once; each call passes only the rows.

    ``x_full`` is a device tensor [B, H, N, D] of rows to append; ``call(s0, s1)``
    appends its rows [s0, s1) at store rows [s0, s1) (the same index in both).
    """

    def __init__(self, blob, blob_dev, x_full, codes, params, capacity, stream=None):
        import torch
        self.dtype = {torch.float16: F16, torch.float32: F32}.get(x_full.dtype)
        if self.dtype is None:
            raise KVTCError(E_DTYPE, "PreparedAppend")
        h = _check_buffers(blob, blob_dev, codes, params, capacity, "PreparedAppend")
        if x_full.dim() != 4 or not x_full.is_cuda or x_full.shape[3] != h.head_dim:
            raise KVTCError(E_SHAPE, "PreparedAppend: x must be a device tensor [B, H, N, D]")
        self.B, self.H, self.N = int(x_full.shape[0]), int(x_full.shape[1]), int(x_full.shape[2])
        self.capacity = capacity
        self._keep = (blob, blob_dev, x_full, codes, params)
        self._args = (_host_ptr(blob), _dev_ptr(blob_dev))
        self._x = x_full.data_ptr()
        self._xs = int(x_full.stride(2)) * x_full.element_size()
        self._strides = _strides4(x_full)
        self._codes, self._params = _dev_ptr(codes), _dev_ptr(params)
        self._stream = _stream_ptr(stream)
        self._fn = _lib.kvtc_append

    def __call__(self, s0: int, s1: int):
        if not (0 <= s0 <= s1 <= self.N):
            raise KVTCError(E_ARG, "PreparedAppend: rows outside x")
        _check(self._fn(self._args[0], self._args[1], self._x + s0 * self._xs, self.dtype, self._strides,
                        self.B, self.H, s1 - s0, s0, self._codes, self._params, self.capacity, self._stream),
               "kvtc_append")


class PreparedFetch:
    """kvtc_fetch with every buffer checked once; ``call(s0, s1)`` reconstructs
    store rows [s0, s1) into rows [s0, s1) of ``out_full`` [B, H, capacity, D]."""

    def __init__(self, blob, blob_dev, codes, params, capacity, out_full, stream=None):
        import torch
        if out_full.dtype != torch.float16:
            raise KVTCError(E_DTYPE, "PreparedFetch")
        h = _check_buffers(blob, blob_dev, codes, params, capacity, "PreparedFetch")
        if not out_full.is_cuda or out_full.dim() != 4 or tuple(out_full.shape[:2]) != (h.batch, h.heads) \
                or out_full.shape[2] < capacity or out_full.shape[3] != h.head_dim:
            raise KVTCError(E_SHAPE, "PreparedFetch: out must be a device tensor [B, H, >=capacity, D]")
        self.capacity = capacity
        self._keep = (blob, blob_dev, codes, params, out_full)
        self._args = (_host_ptr(blob), _dev_ptr(blob_dev), _dev_ptr(codes), _dev_ptr(params))
        self._out = out_full.data_ptr()
        self._os = int(out_full.stride(2)) * out_full.element_size()
        self._strides = _strides4(out_full)
        self._stream = _stream_ptr(stream)
        self._fn = _lib.kvtc_fetch

    def __call__(self, s0: int, s1: int):
        a = self._args
        _check(self._fn(a[0], a[1], a[2], a[3], self.capacity, s0, s1, self._out + s0 * self._os,
                        self._strides, self._stream), "kvtc_fetch")


class PreparedAppendKV:
    """kvtc_append_kv with every buffer checked once: ``k`` and ``v`` are
    (blob, blob_dev, x_full, codes, params) with x_full [B, H, N, D] device rows of
    the same shape; ``call(s0, s1)`` appends rows [s0, s1) of both at store rows [s0, s1)."""

    def __init__(self, k, v, capacity, stream=None):
        import torch
        self._keep = (k, v)
        self._refs = []
        for (blob, blob_dev, x, codes, params) in (k, v):
            dtype = {torch.float16: F16, torch.float32: F32}.get(x.dtype)
            if dtype is None:
                raise KVTCError(E_DTYPE, "PreparedAppendKV")
            h = _check_buffers(blob, blob_dev, codes, params, capacity, "PreparedAppendKV")
            if x.dim() != 4 or not x.is_cuda or x.shape[3] != h.head_dim:
                raise KVTCError(E_SHAPE, "PreparedAppendKV: x must be a device tensor [B, H, N, D]")
            self._refs.append(_tensor_ref(blob, blob_dev, codes, params, capacity, x, dtype))
        if tuple(k[2].shape) != tuple(v[2].shape):
            raise KVTCError(E_SHAPE, "PreparedAppendKV: key and value rows differ in shape")
        self.B, self.H, self.N = int(k[2].shape[0]), int(k[2].shape[1]), int(k[2].shape[2])
        self._x = [k[2].data_ptr(), v[2].data_ptr()]
        self._xs = [int(t[2].stride(2)) * t[2].element_size() for t in (k, v)]
        self._stream = _stream_ptr(stream)
        self._fn = _lib.kvtc_append_kv

    def __call__(self, s0: int, s1: int):
        if not (0 <= s0 <= s1 <= self.N):
            raise KVTCError(E_ARG, "PreparedAppendKV: rows outside x")
        for i in range(2):
            self._refs[i].rows_dev = self._x[i] + s0 * self._xs[i]
        _check(self._fn(C.byref(self._refs[0]), C.byref(self._refs[1]), self.B, self.H, s1 - s0, s0,
                        self._stream), "kvtc_append_kv")


class PreparedFetchKV:
    """kvtc_fetch_kv with every buffer checked once: ``k`` and ``v`` are
    (blob, blob_dev, codes, params, out_full) with out_full fp16 [B, H, >=capacity, D];
    ``call(s0, s1)`` reconstructs store rows [s0, s1) of both into rows [s0, s1) of out_full."""

    def __init__(self, k, v, capacity, stream=None):
        import torch
        self._keep = (k, v)
        self._refs = []
        self.capacity = capacity
        for (blob, blob_dev, codes, params, out) in (k, v):
            if out.dtype != torch.float16:
                raise KVTCError(E_DTYPE, "PreparedFetchKV")
            h = _check_buffers(blob, blob_dev, codes, params, capacity, "PreparedFetchKV")
            if not out.is_cuda or out.dim() != 4 or tuple(out.shape[:2]) != (h.batch, h.heads) \
                    or out.shape[2] < capacity or out.shape[3] != h.head_dim:
                raise KVTCError(E_SHAPE, "PreparedFetchKV: out must be a device tensor [B, H, >=capacity, D]")
            self._refs.append(_tensor_ref(blob, blob_dev, codes, params, capacity, out, F16))
        self._out = [k[4].data_ptr(), v[4].data_ptr()]
        self._os = [int(t[4].stride(2)) * t[4].element_size() for t in (k, v)]
        self._stream = _stream_ptr(stream)
        self._fn = _lib.kvtc_fetch_kv

    def __call__(self, s0: int, s1: int):
        for i in range(2):
            self._refs[i].rows_dev = self._out[i] + s0 * self._os[i]
        _check(self._fn(C.byref(self._refs[0]), C.byref(self._refs[1]), s0, s1, self._stream), "kvtc_fetch_kv")

    def probe(self, s0: int, s1: int):
        """kvtc_fetch_kv_probe with the same buffers: the fetch's traffic alone
        (overwrites the output rows with placeholder values)."""
        for i in range(2):
            self._refs[i].rows_dev = self._out[i] + s0 * self._os[i]
        _check(_lib.kvtc_fetch_kv_probe(C.byref(self._refs[0]), C.byref(self._refs[1]), s0, s1, self._stream),
               "kvtc_fetch_kv_probe")
