"""ctypes binding of the C ABI in ``include/ddpb.h``.

Argument marshalling only: every function forwards to the entry point of the
same name (without the ``ddpb_`` prefix) and raises ``DdpbError`` on a non-zero
status. No step of the reduction runs in Python.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import List, Optional, Sequence, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
HIP_LIB = os.path.join(_HERE, "lib", "libddpb.so")
HOSTONLY_LIB = os.path.join(_HERE, "lib", "libddpb_hostonly.so")

F32, BF16 = 0, 1
MODE_FUSED, MODE_STAGED = 0, 1
BIND_DEVICE_TIMESTAMPS, BIND_TIME_LAUNCHES, BIND_ROCTX, BIND_OVERLAP = 1, 2, 4, 8

STATIC_SCRATCH_BYTES = 32 << 20      # DDPB_STATIC_SCRATCH_BYTES

OK, E_ARG, E_INDEX, E_DOUBLE_READY, E_INCOMPLETE, E_STATE, E_HIP, E_NOMEM = 0, -1, -2, -3, -4, -5, -6, -7
_NAMES = {E_ARG: "E_ARG", E_INDEX: "E_INDEX", E_DOUBLE_READY: "E_DOUBLE_READY",
          E_INCOMPLETE: "E_INCOMPLETE", E_STATE: "E_STATE", E_HIP: "E_HIP", E_NOMEM: "E_NOMEM"}

# every entry point declared in include/ddpb.h
SYMBOLS = [
    "ddpb_reducer_create", "ddpb_destroy", "ddpb_num_buckets", "ddpb_get_locator", "ddpb_get_bucket",
    "ddpb_num_segments", "ddpb_get_bucket_segments", "ddpb_get_segment", "ddpb_workspace_bytes",
    "ddpb_bind", "ddpb_ensure_prior_reduction_finished", "ddpb_mark_ready", "ddpb_mark_ready_many",
    "ddpb_finalize", "ddpb_set_sync", "ddpb_no_sync_accumulate", "ddpb_reset", "ddpb_get_launch_log",
    "ddpb_get_launch_times", "ddpb_device_clock_hz", "ddpb_last_error", "ddpb_set_launch_blocks",
    "ddpb_set_workgroups_per_cu", "ddpb_set_sync_step",
    "ddpb_view_storage_elems", "ddpb_get_view_offset", "ddpb_bind_bucket_views",
    "ddpb_rebuild_buckets", "ddpb_get_ready_order", "ddpb_set_local_used", "ddpb_bind_static",
]


class DdpbError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_NAMES.get(code, code)}: {msg}")
        self.code = code


i32, i64, vp = C.c_int32, C.c_int64, C.c_void_p
P32, P64 = C.POINTER(C.c_int32), C.POINTER(C.c_int64)


def ptr_array(ptrs: Sequence[int]):
    """A void* array of the given addresses (0 = NULL), at least one element long."""
    return (vp * max(len(ptrs), 1))(*ptrs)


def _sig(lib):
    S = {
        "ddpb_reducer_create": [P64, P32, i32, i32, i64, i32, C.POINTER(vp)],
        "ddpb_destroy": [vp],
        "ddpb_num_buckets": [vp, P32],
        "ddpb_get_locator": [vp, i32, P32, P32, P64, P64],
        "ddpb_get_bucket": [vp, i32, P32, P64, P32],
        "ddpb_num_segments": [vp, P32, P64],
        "ddpb_get_bucket_segments": [vp, i32, P32, P32],
        "ddpb_get_segment": [vp, i32, P32, P32, P64, P64, P64],
        "ddpb_workspace_bytes": [vp, i32, P64],
        "ddpb_bind": [vp, C.POINTER(vp), vp, i64, vp, C.POINTER(vp), i32, i32, i32],
        "ddpb_bind_static": [vp, C.POINTER(vp), vp, i32],
        "ddpb_ensure_prior_reduction_finished": [vp],
        "ddpb_mark_ready": [vp, i32],
        "ddpb_mark_ready_many": [vp, P32, i32],
        "ddpb_finalize": [vp],
        "ddpb_set_sync": [vp, i32],
        "ddpb_no_sync_accumulate": [vp, C.POINTER(vp), i32, i32],
        "ddpb_set_sync_step": [vp, C.POINTER(vp), i32, i32],
        "ddpb_reset": [vp],
        "ddpb_get_launch_log": [vp, P32, P32, P64, P64, i32, P32],
        "ddpb_get_launch_times": [vp, i32, C.POINTER(C.c_float), C.POINTER(C.c_float), i32, P32],
        "ddpb_device_clock_hz": [vp, P64],
        "ddpb_set_launch_blocks": [vp, i32],
        "ddpb_set_workgroups_per_cu": [vp, i32],
        "ddpb_set_local_used": [vp, C.POINTER(C.c_uint8)],
        "ddpb_rebuild_buckets": [vp, i64],
        "ddpb_get_ready_order": [vp, P32, i32, P32],
        "ddpb_view_storage_elems": [vp, P64],
        "ddpb_get_view_offset": [vp, i32, P64],
        "ddpb_bind_bucket_views": [vp, C.POINTER(vp), i64, vp, C.POINTER(vp), i32, i32],
        "ddpb_last_error": [],
    }
    for name, args in S.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = None if name == "ddpb_destroy" else (C.c_char_p if name == "ddpb_last_error" else C.c_int)


class Lib:
    """One loaded copy of the library (the HIP product, or the host-only test
    build when a test names it)."""

    def __init__(self, path: str = HIP_LIB):
        if not os.path.exists(path):
            raise ImportError(
                f"{path} is missing: build it with `python -m ddp_bucketed_gradient_amd.build` "
                "(there is no fallback implementation)")
        self.path = path
        self.dll = C.CDLL(path)
        _sig(self.dll)

    def _check(self, rc: int):
        if rc != OK:
            raise DdpbError(rc, self.last_error())

    def last_error(self) -> str:
        return self.dll.ddpb_last_error().decode("utf-8", "replace")

    # -- construction and plan ------------------------------------------------
    def reducer_create(self, shapes: Sequence[Sequence[int]], dtype: int, bucket_cap_bytes: int, R: int):
        flat = [int(d) for s in shapes for d in s]
        nd = [len(s) for s in shapes]
        h = vp()
        self._check(self.dll.ddpb_reducer_create((C.c_int64 * max(len(flat), 1))(*flat),
                                                 (C.c_int32 * max(len(nd), 1))(*nd), len(nd), dtype,
                                                 int(bucket_cap_bytes), int(R), C.byref(h)))
        return h

    def destroy(self, h):
        self.dll.ddpb_destroy(h)

    def num_buckets(self, h) -> int:
        b = i32()
        self._check(self.dll.ddpb_num_buckets(h, C.byref(b)))
        return b.value

    def get_locator(self, h, v: int) -> Tuple[int, int, int, int]:
        b, i, o, n = i32(), i32(), i64(), i64()
        self._check(self.dll.ddpb_get_locator(h, v, C.byref(b), C.byref(i), C.byref(o), C.byref(n)))
        return b.value, i.value, o.value, n.value

    def get_bucket(self, h, b: int) -> Tuple[List[int], int]:
        nv, nb = i32(), i64()
        self._check(self.dll.ddpb_get_bucket(h, b, C.byref(nv), C.byref(nb), None))
        arr = (C.c_int32 * max(nv.value, 1))()
        self._check(self.dll.ddpb_get_bucket(h, b, C.byref(nv), C.byref(nb), arr))
        return list(arr[:nv.value]), nb.value

    def num_segments(self, h) -> Tuple[int, int]:
        n, e = i32(), i64()
        self._check(self.dll.ddpb_num_segments(h, C.byref(n), C.byref(e)))
        return n.value, e.value

    def get_bucket_segments(self, h, b: int) -> Tuple[int, int]:
        f, c = i32(), i32()
        self._check(self.dll.ddpb_get_bucket_segments(h, b, C.byref(f), C.byref(c)))
        return f.value, c.value

    def get_segment(self, h, s: int) -> Tuple[int, int, int, int, int]:
        v, b, st, ln, bo = i32(), i32(), i64(), i64(), i64()
        self._check(self.dll.ddpb_get_segment(h, s, C.byref(v), C.byref(b), C.byref(st), C.byref(ln), C.byref(bo)))
        return v.value, b.value, st.value, ln.value, bo.value

    # -- binding ------------------------------------------------------------------
    def workspace_bytes(self, h, mode: int) -> int:
        n = i64()
        self._check(self.dll.ddpb_workspace_bytes(h, mode, C.byref(n)))
        return n.value

    def bind(self, h, grad_ptrs: Sequence[int], workspace: int, ws_bytes: int, compute_stream: int,
             side_streams: Sequence[int], mode: int, flags: int = 0):
        gp = (vp * max(len(grad_ptrs), 1))(*[vp(int(p)) for p in grad_ptrs])
        ss = (vp * len(side_streams))(*[vp(int(s)) for s in side_streams])
        self._check(self.dll.ddpb_bind(h, gp, vp(int(workspace)) if workspace else None, int(ws_bytes),
                                       vp(int(compute_stream)) if compute_stream else None, ss,
                                       len(side_streams), mode, flags))

    def bind_static(self, h, grad_ptrs: Sequence[int], compute_stream: int, mode: int):
        gp = (vp * max(len(grad_ptrs), 1))(*[vp(int(p)) for p in grad_ptrs])
        self._check(self.dll.ddpb_bind_static(h, gp, vp(int(compute_stream)) if compute_stream else None, mode))

    # -- iteration ------------------------------------------------------------------
    def ensure_prior_reduction_finished(self, h):
        self._check(self.dll.ddpb_ensure_prior_reduction_finished(h))

    def mark_ready(self, h, v: int):
        rc = self.dll.ddpb_mark_ready(h, v)
        if rc != OK:
            raise DdpbError(rc, self.last_error())

    def mark_ready_many(self, h, vs: Sequence[int]):
        arr = (C.c_int32 * max(len(vs), 1))(*vs)
        self._check(self.dll.ddpb_mark_ready_many(h, arr, len(vs)))

    def finalize(self, h):
        self._check(self.dll.ddpb_finalize(h))

    def set_sync(self, h, enabled: bool):
        self._check(self.dll.ddpb_set_sync(h, 1 if enabled else 0))

    def no_sync_accumulate(self, h, step_ptrs, step_dtype: int, first_step: bool):
        """step_ptrs: R * P device addresses (0 = no step), or an array made by ptr_array."""
        sp = step_ptrs if isinstance(step_ptrs, C.Array) else ptr_array(step_ptrs)
        self._check(self.dll.ddpb_no_sync_accumulate(h, sp, step_dtype, 1 if first_step else 0))

    def set_sync_step(self, h, step_ptrs, step_dtype: int, first_step: bool):
        """step_ptrs as for no_sync_accumulate."""
        sp = step_ptrs if isinstance(step_ptrs, C.Array) else ptr_array(step_ptrs)
        self._check(self.dll.ddpb_set_sync_step(h, sp, step_dtype, 1 if first_step else 0))

    def reset(self, h):
        self._check(self.dll.ddpb_reset(h))

    # -- diagnostics ------------------------------------------------------------------
    def get_launch_log(self, h, with_stamps: bool = False):
        n = i32()
        self._check(self.dll.ddpb_get_launch_log(h, None, None, None, None, 0, C.byref(n)))
        m = n.value
        b, t = (C.c_int32 * max(m, 1))(), (C.c_int32 * max(m, 1))()
        t0, t1 = (C.c_int64 * max(m, 1))(), (C.c_int64 * max(m, 1))()
        self._check(self.dll.ddpb_get_launch_log(h, b, t, t0 if with_stamps else None,
                                                 t1 if with_stamps else None, m, C.byref(n)))
        rows = [(b[i], t[i]) for i in range(m)]
        if with_stamps:
            return rows, [t0[i] for i in range(m)], [t1[i] for i in range(m)]
        return rows

    def get_launch_times(self, h, iterations_ago: int = 0, with_starts: bool = False):
        """Durations (ms) of each launch of a finalized iteration; with
        ``with_starts`` also their starts relative to its first launch."""
        n = i32()
        self._check(self.dll.ddpb_get_launch_times(h, iterations_ago, None, None, 0, C.byref(n)))
        arr = (C.c_float * max(n.value, 1))()
        st = (C.c_float * max(n.value, 1))()
        self._check(self.dll.ddpb_get_launch_times(h, iterations_ago, st, arr, n.value, C.byref(n)))
        if with_starts:
            return list(st[:n.value]), list(arr[:n.value])
        return list(arr[:n.value])

    def rebuild_buckets(self, h, bucket_cap_bytes: int):
        self._check(self.dll.ddpb_rebuild_buckets(h, int(bucket_cap_bytes)))

    def get_ready_order(self, h) -> List[int]:
        n = i32()
        self._check(self.dll.ddpb_get_ready_order(h, None, 0, C.byref(n)))
        arr = (C.c_int32 * max(n.value, 1))()
        self._check(self.dll.ddpb_get_ready_order(h, arr, n.value, C.byref(n)))
        return list(arr[:n.value])

    def view_storage_elems(self, h) -> int:
        n = i64()
        self._check(self.dll.ddpb_view_storage_elems(h, C.byref(n)))
        return n.value

    def get_view_offset(self, h, v: int) -> int:
        n = i64()
        self._check(self.dll.ddpb_get_view_offset(h, v, C.byref(n)))
        return n.value

    def bind_bucket_views(self, h, storages: Sequence[int], storage_elems: int, compute_stream: int,
                          side_streams: Sequence[int], flags: int = 0):
        st = (vp * max(len(storages), 1))(*[vp(int(p)) for p in storages])
        ss = (vp * len(side_streams))(*[vp(int(s)) for s in side_streams])
        self._check(self.dll.ddpb_bind_bucket_views(h, st, int(storage_elems),
                                                    vp(int(compute_stream)) if compute_stream else None, ss,
                                                    len(side_streams), flags))

    def set_launch_blocks(self, h, max_blocks: int):
        self._check(self.dll.ddpb_set_launch_blocks(h, int(max_blocks)))

    def set_workgroups_per_cu(self, h, n: int):
        self._check(self.dll.ddpb_set_workgroups_per_cu(h, int(n)))

    def set_local_used(self, h, used):
        """used: R*P flags, replica-major (a sequence, or a contiguous uint8
        NumPy array passed without copying), or None for all used."""
        if used is None:
            self._check(self.dll.ddpb_set_local_used(h, None))
            return
        if hasattr(used, "ctypes") and getattr(used, "dtype", None) is not None and str(used.dtype) == "uint8" \
                and used.flags["C_CONTIGUOUS"]:
            self._check(self.dll.ddpb_set_local_used(h, used.ctypes.data_as(C.POINTER(C.c_uint8))))
            return
        buf = (C.c_uint8 * max(len(used), 1))(*[1 if u else 0 for u in used])
        self._check(self.dll.ddpb_set_local_used(h, buf))

    def device_clock_hz(self, h) -> int:
        hz = i64()
        self._check(self.dll.ddpb_device_clock_hz(h, C.byref(hz)))
        return hz.value


_DEFAULT: Optional[Lib] = None


def lib() -> Lib:
    """The HIP product library (raises ImportError if it has not been built)."""
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Lib(HIP_LIB)
    return _DEFAULT
