"""ctypes declarations of libgclip's C ABI (include/gclip.h).

Marshalling only: every step of the clipping path runs in the HIP kernels of
libgclip.so.  Importing this module fails loudly when the library has not
been built -- there is no fallback.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# GCLIP_LIBRARY may name another build of the same library to load instead:
# the phase-timeline build of include/gclip_stamps.h, _stamps/libgclip.so.
LIB_PATH = os.environ.get("GCLIP_LIBRARY") or os.path.join(HERE, "libgclip.so")

GCLIP_F32, GCLIP_F16, GCLIP_BF16 = 0, 1, 2
GCLIP_OK, GCLIP_EINVAL, GCLIP_EDTYPE, GCLIP_ENOMEM, GCLIP_EHIP, GCLIP_ENONFINITE, GCLIP_EDEVICE, GCLIP_ERANGE = range(8)
GCLIP_NOALLOC_SCRATCH_BYTES = 4 << 20
GCLIP_PATH_AUTO, GCLIP_PATH_FUSED, GCLIP_PATH_SPLIT = 0, 1, 2

STATUS_NAMES = {GCLIP_OK: "GCLIP_OK", GCLIP_EINVAL: "GCLIP_EINVAL", GCLIP_EDTYPE: "GCLIP_EDTYPE",
                GCLIP_ENOMEM: "GCLIP_ENOMEM", GCLIP_EHIP: "GCLIP_EHIP", GCLIP_ENONFINITE: "GCLIP_ENONFINITE",
                GCLIP_EDEVICE: "GCLIP_EDEVICE", GCLIP_ERANGE: "GCLIP_ERANGE"}


class GclipResult(ctypes.Structure):
    _fields_ = [("sumsq", ctypes.c_double), ("norm", ctypes.c_double), ("scale", ctypes.c_double),
                ("max_norm", ctypes.c_double), ("nonfinite", ctypes.c_int32), ("clipped", ctypes.c_int32),
                ("skipped", ctypes.c_int32), ("decided", ctypes.c_int32), ("status", ctypes.c_int32),
                ("handed_back", ctypes.c_int32), ("reserved", ctypes.c_int32 * 2)]

    def as_dict(self):
        return {"sumsq": self.sumsq, "norm": self.norm, "scale": self.scale, "max_norm": self.max_norm,
                "nonfinite": bool(self.nonfinite), "clipped": bool(self.clipped), "skipped": bool(self.skipped),
                "decided": bool(self.decided), "status": int(self.status),
                "handed_back": int(self.handed_back)}


class GclipListInfo(ctypes.Structure):
    _fields_ = [("n_tensors", ctypes.c_int64), ("n_elements", ctypes.c_int64), ("n_bytes", ctypes.c_int64),
                ("n_segments", ctypes.c_int64), ("n_vectors", ctypes.c_int64), ("n_scalars", ctypes.c_int64),
                ("n_workers", ctypes.c_int32), ("worker_threads", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("path", ctypes.c_int32), ("resident_vectors", ctypes.c_int64)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


class GclipPlanEntry(ctypes.Structure):
    _fields_ = [("worker", ctypes.c_int32), ("tensor", ctypes.c_int32), ("elem_begin", ctypes.c_int64),
                ("elem_count", ctypes.c_int64), ("kind", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class GclipAdamwHparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double), ("step", ctypes.c_int64)]


class GclipAmpState(ctypes.Structure):
    _fields_ = [("scale", ctypes.c_float), ("growth_tracker", ctypes.c_int32), ("found_inf", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class GclipAmpParams(ctypes.Structure):
    _fields_ = [("growth_factor", ctypes.c_double), ("backoff_factor", ctypes.c_double),
                ("growth_interval", ctypes.c_int32), ("reserved", ctypes.c_int32)]


assert ctypes.sizeof(GclipResult) == 64
assert ctypes.sizeof(GclipAmpState) == 16


def _declare(lib):
    vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    sig = {
        "gclip_list_create": ([ctypes.POINTER(vp), ctypes.POINTER(i64), i32, i32, ctypes.POINTER(vp)], i32),
        "gclip_list_destroy": ([vp], i32),
        "gclip_list_info": ([vp, ctypes.POINTER(GclipListInfo)], i32),
        "gclip_list_set_path": ([vp, i32], i32),
        "gclip_list_set_wait": ([vp, ctypes.c_int64], i32),
        "gclip_norm": ([vp, dbl, vp, vp], i32),
        "gclip_scale": ([vp, dbl, dbl, i32, vp, vp], i32),
        "gclip_clip_": ([vp, dbl, dbl, i32, vp, vp], i32),
        "gclip_result_read": ([vp, vp, ctypes.POINTER(GclipResult), i32], i32),
        "gclip_plan_query": ([ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(i64), i32, i32, i32, i32,
                              ctypes.POINTER(GclipPlanEntry), i64, ctypes.POINTER(i64)], i32),
        "gclip_plan_trace": ([ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(i64), i32, i32, i32, i32,
                              ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(i32), i64, ctypes.POINTER(i64)], i32),
        "gclip_adamw_create": ([ctypes.POINTER(vp)] * 4 + [ctypes.POINTER(i64), i32, i32, ctypes.POINTER(vp)], i32),
        "gclip_adamw_destroy": ([vp], i32),
        "gclip_adamw_step": ([vp, ctypes.POINTER(GclipAdamwHparams), dbl, dbl, i32, vp, vp], i32),
        "gclip_tensor_norms": ([vp, dbl, vp, vp, vp], i32),
        "gclip_contrib_create": ([vp, ctypes.POINTER(vp), ctypes.POINTER(vp)], i32),
        "gclip_contrib_destroy": ([vp], i32),
        "gclip_accumulate_norm": ([vp, vp, dbl, vp, vp, vp], i32),
        "gclip_accumulate_clip_": ([vp, vp, dbl, dbl, i32, vp, vp], i32),
        "gclip_clip_per_tensor_": ([vp, dbl, dbl, i32, vp, vp, vp], i32),
        "gclip_set_gather_wait": ([i64], i32),
        "gclip_norm_amp": ([vp, dbl, vp, vp, vp], i32),
        "gclip_clip_amp_": ([vp, dbl, dbl, vp, ctypes.POINTER(GclipAmpParams), vp, vp], i32),
        "gclip_adamw_step_amp": ([vp, ctypes.POINTER(GclipAdamwHparams), dbl, dbl, vp,
                                  ctypes.POINTER(GclipAmpParams), vp, vp], i32),
        "gclip_clip_noalloc_": ([ctypes.POINTER(vp), ctypes.POINTER(i64), i32, i32, dbl, dbl, i32, vp, vp], i32),
        "gclip_ref_read": ([vp, i64, vp, vp], i32),
        "gclip_ref_copy": ([vp, vp, i64, vp], i32),
        "gclip_status_string": ([i32], ctypes.c_char_p),
        "gclip_last_hip_error": ([], i32),
        "gclip_version": ([], i32),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    return lib


def load():
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m global_l2_norm_amd.build` "
                           "(hipcc --offload-arch=gfx950); there is no fallback path")
    # PyTorch-ROCm wheels carry their own HIP runtime.  Loading torch first
    # lets libgclip bind to that same runtime, so the process holds one HIP
    # runtime and the device memory and streams torch hands over are valid
    # for our kernels; loaded the other way round, two runtimes end up in the
    # process and the second one finds no device.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    return _declare(ctypes.CDLL(LIB_PATH))


lib = load()

# The C ABI's declared entry points (include/gclip.h, include/gclip_ref.h), for the export check.
EXPORTS = ("gclip_list_create", "gclip_list_destroy", "gclip_list_info", "gclip_list_set_path",
           "gclip_list_set_wait", "gclip_norm",
           "gclip_scale", "gclip_clip_", "gclip_result_read", "gclip_plan_query", "gclip_plan_trace", "gclip_status_string",
           "gclip_last_hip_error", "gclip_version", "gclip_adamw_create", "gclip_adamw_destroy", "gclip_adamw_step",
           "gclip_norm_amp", "gclip_clip_amp_", "gclip_adamw_step_amp", "gclip_tensor_norms",
           "gclip_clip_per_tensor_", "gclip_contrib_create", "gclip_contrib_destroy", "gclip_accumulate_norm",
           "gclip_accumulate_clip_", "gclip_set_gather_wait", "gclip_clip_noalloc_", "gclip_ref_read",
           "gclip_ref_copy")
