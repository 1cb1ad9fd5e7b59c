"""Bucketed gradient synchronisation for MI355X (gfx950).

The data-parallel reducer's hot path: parameters are assigned to buckets in
reverse definition order under a byte cap; each gradient hook marks its
variable ready; complete buckets are launched strictly in bucket-index order on
a side HIP stream, where hand-written CDNA4 kernels average the R replicas'
gradients in HBM and write the mean back to every replica; ``no_sync``
accumulates local steps before one synchronisation.

The native library (``lib/libddpb.so``, C ABI in ``include/ddpb.h``) does all
of the work; this package only marshals arguments. Importing the package does
not load the library; the first use does, and fails loudly if it was not built.
"""
from ._abi import (DdpbError, Lib, lib, F32, BF16, MODE_FUSED, MODE_STAGED, STATIC_SCRATCH_BYTES,  # noqa: F401
                   BIND_DEVICE_TIMESTAMPS, BIND_TIME_LAUNCHES, BIND_ROCTX, BIND_OVERLAP, HIP_LIB, HOSTONLY_LIB, SYMBOLS,
                   OK, E_ARG, E_INDEX, E_DOUBLE_READY, E_INCOMPLETE, E_STATE, E_HIP, E_NOMEM)
from .reducer import Reducer, StepTable  # noqa: F401


def _fwd(name):
    def f(*args, **kw):
        return getattr(lib(), name)(*args, **kw)
    f.__name__ = name
    f.__doc__ = f"Forwards to ddpb_{name} of the HIP library."
    return f


# Module-level functions with the C ABI's names (without the ddpb_ prefix).
for _n in ["reducer_create", "destroy", "num_buckets", "get_locator", "get_bucket", "num_segments",
           "get_bucket_segments", "get_segment", "workspace_bytes", "bind", "ensure_prior_reduction_finished",
           "mark_ready", "mark_ready_many", "finalize", "set_sync", "no_sync_accumulate", "reset",
           "get_launch_log", "get_launch_times", "device_clock_hz", "last_error", "set_launch_blocks",
           "set_workgroups_per_cu",
           "view_storage_elems", "get_view_offset", "bind_bucket_views", "rebuild_buckets", "get_ready_order",
           "set_local_used", "set_sync_step", "bind_static"]:
    globals()[_n] = _fwd(_n)
del _n
