"""global_l2_norm_amd -- global L2-norm gradient clipping on MI355X.

A thin Python face of libgclip (include/gclip.h).  The functions named like
the C ABI take raw device addresses; ``GradList`` wraps a list of torch
tensors (torch is used here only for device memory and streams).

The path (grad clip lesson, unhomeschool.com ru, section "Math"): the norm is
the square root of the sum of g^2 over every element of every tensor; only
if it exceeds max_norm is every element multiplied by max_norm / norm.  The
averaging factor a (backprop lesson, unhomeschool.com vi, "Accumulation
across microbatches") multiplies g before its norm is taken, and the
error-if-nonfinite switch (glossary page, paweldubiel.com, "Mechanism and
details") stops the update when a NaN or Inf is present.
"""
import ctypes

from . import _lib
from ._lib import (GCLIP_BF16, GCLIP_F16, GCLIP_F32, GCLIP_PATH_AUTO, GCLIP_PATH_FUSED, GCLIP_PATH_SPLIT,
                   GclipAdamwHparams, GclipAmpParams, GclipListInfo, GclipPlanEntry, GclipResult)

__all__ = ["GclipError", "GclipResult", "GradList", "clip_grad_norm_", "gclip_list_create", "gclip_list_destroy",
           "gclip_list_info", "gclip_list_set_path", "gclip_list_set_wait", "gclip_norm", "gclip_scale", "gclip_clip_",
           "gclip_result_read", "gclip_plan_query", "gclip_plan_trace", "gclip_status_string", "gclip_version",
           "gclip_adamw_create", "gclip_adamw_destroy", "gclip_adamw_step", "AdamWList",
           "gclip_norm_amp", "gclip_clip_amp_", "gclip_adamw_step_amp", "AmpState",
           "gclip_tensor_norms", "gclip_clip_per_tensor_", "gclip_set_gather_wait", "TENSOR_RESULT_DTYPE",
           "GCLIP_DEVICE_WAIT_TIMEOUT", "gclip_contrib_create",
           "gclip_contrib_destroy", "gclip_accumulate_norm", "gclip_accumulate_clip_", "Contribution",
           "GCLIP_F32", "GCLIP_F16", "GCLIP_BF16", "GCLIP_PATH_AUTO", "GCLIP_PATH_FUSED", "GCLIP_PATH_SPLIT"]

DTYPE_CODES = {"f32": GCLIP_F32, "f16": GCLIP_F16, "bf16": GCLIP_BF16}

# gclip_result.status: the per-tensor clip's gathering workgroup gave up waiting
GCLIP_DEVICE_WAIT_TIMEOUT = 1

# gclip_tensor_result, 32 bytes per tensor
TENSOR_RESULT_DTYPE = [("sumsq", "<f8"), ("norm", "<f8"), ("scale", "<f8"), ("nonfinite", "<i4"),
                       ("clipped", "<i4")]


class GclipError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = f"{where}: {_lib.STATUS_NAMES.get(status, status)} ({_lib.lib.gclip_status_string(status).decode()})"
        if status == _lib.GCLIP_EHIP:
            msg += f", hipError {_lib.lib.gclip_last_hip_error()}"
        super().__init__(msg)


def _check(status, where):
    if status != _lib.GCLIP_OK:
        raise GclipError(status, where)


# ---------------------------------------------------------------- C ABI names
def gclip_list_create(d_ptrs, numels, dtype):
    """Handle (int) of a new list; d_ptrs are device addresses, numels sizes."""
    n = len(d_ptrs)
    ptrs = (ctypes.c_void_p * max(n, 1))(*d_ptrs)
    sizes = (ctypes.c_int64 * max(n, 1))(*numels)
    out = ctypes.c_void_p()
    _check(_lib.lib.gclip_list_create(ptrs, sizes, n, int(dtype), ctypes.byref(out)), "gclip_list_create")
    return out.value


def gclip_list_destroy(handle):
    _check(_lib.lib.gclip_list_destroy(handle), "gclip_list_destroy")


def gclip_list_info(handle):
    info = GclipListInfo()
    _check(_lib.lib.gclip_list_info(handle, ctypes.byref(info)), "gclip_list_info")
    return info.as_dict()


def gclip_list_set_path(handle, path):
    _check(_lib.lib.gclip_list_set_path(handle, int(path)), "gclip_list_set_path")


def gclip_list_set_wait(handle, microseconds):
    _check(_lib.lib.gclip_list_set_wait(handle, int(microseconds)), "gclip_list_set_wait")


def gclip_norm(handle, avg_factor, d_result, stream):
    _check(_lib.lib.gclip_norm(handle, float(avg_factor), d_result, stream), "gclip_norm")


def gclip_scale(handle, max_norm, avg_factor, error_if_nonfinite, d_result, stream):
    _check(_lib.lib.gclip_scale(handle, float(max_norm), float(avg_factor), int(bool(error_if_nonfinite)),
                                d_result, stream), "gclip_scale")


def gclip_clip_(handle, max_norm, avg_factor, error_if_nonfinite, d_result, stream):
    _check(_lib.lib.gclip_clip_(handle, float(max_norm), float(avg_factor), int(bool(error_if_nonfinite)),
                                d_result, stream), "gclip_clip_")


def gclip_result_read(d_result, stream, error_if_nonfinite=False):
    """(status, dict) after the stream's queued work has finished."""
    r = GclipResult()
    st = _lib.lib.gclip_result_read(d_result, stream, ctypes.byref(r), int(bool(error_if_nonfinite)))
    if st not in (_lib.GCLIP_OK, _lib.GCLIP_ENONFINITE, _lib.GCLIP_EDEVICE):
        raise GclipError(st, "gclip_result_read")
    return st, r.as_dict()


def gclip_plan_query(addrs, numels, dtype, n_workers, worker_threads):
    """List of (worker, tensor, elem_begin, elem_count, kind) runs; no GPU involved."""
    n = len(addrs)
    a = (ctypes.c_uint64 * max(n, 1))(*addrs)
    s = (ctypes.c_int64 * max(n, 1))(*numels)
    need = ctypes.c_int64()
    st = _lib.lib.gclip_plan_query(a, s, n, int(dtype), int(n_workers), int(worker_threads), None, 0,
                                   ctypes.byref(need))
    if st not in (_lib.GCLIP_OK, _lib.GCLIP_ERANGE):
        raise GclipError(st, "gclip_plan_query")
    cap = need.value
    buf = (GclipPlanEntry * max(cap, 1))()
    _check(_lib.lib.gclip_plan_query(a, s, n, int(dtype), int(n_workers), int(worker_threads), buf, cap,
                                     ctypes.byref(need)), "gclip_plan_query")
    return [(e.worker, e.tensor, e.elem_begin, e.elem_count, e.kind) for e in buf[:need.value]]


def gclip_plan_trace(addrs, numels, dtype, n_workers, mode):
    """(addresses, workers) numpy arrays of every lane access a kernel would
    make (mode 0 norm, 1 scale, 2/3 fused first/second pass, 4 per-tensor pieces, 5/6 contribution reads of
    the fused kernel with the +=, first pass / a block handed back); no GPU involved."""
    import numpy as np
    n = len(addrs)
    a = (ctypes.c_uint64 * max(n, 1))(*addrs)
    s = (ctypes.c_int64 * max(n, 1))(*numels)
    need = ctypes.c_int64()
    st = _lib.lib.gclip_plan_trace(a, s, n, int(dtype), int(n_workers), int(mode), None, None, 0, ctypes.byref(need))
    if st not in (_lib.GCLIP_OK, _lib.GCLIP_ERANGE):
        raise GclipError(st, "gclip_plan_trace")
    cap = need.value
    out_a = np.zeros(max(cap, 1), dtype=np.uint64)
    out_w = np.zeros(max(cap, 1), dtype=np.int32)
    _check(_lib.lib.gclip_plan_trace(a, s, n, int(dtype), int(n_workers), int(mode),
                                     out_a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)),
                                     out_w.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), cap, ctypes.byref(need)),
           "gclip_plan_trace")
    return out_a[:cap], out_w[:cap]


def gclip_status_string(status):
    return _lib.lib.gclip_status_string(int(status)).decode()


def gclip_version():
    return _lib.lib.gclip_version()


def gclip_adamw_create(d_params, d_grads, d_exp_avg, d_exp_avg_sq, numels, grad_dtype):
    n = len(numels)
    arrs = [(ctypes.c_void_p * max(n, 1))(*[ctypes.c_void_p(int(a)) for a in x])
            for x in (d_params, d_grads, d_exp_avg, d_exp_avg_sq)]
    ne = (ctypes.c_int64 * max(n, 1))(*[int(x) for x in numels])
    out = ctypes.c_void_p()
    _check(_lib.lib.gclip_adamw_create(*arrs, ne, n, int(grad_dtype), ctypes.byref(out)), "gclip_adamw_create")
    return out


def gclip_adamw_destroy(handle):
    _check(_lib.lib.gclip_adamw_destroy(handle), "gclip_adamw_destroy")


def gclip_adamw_step(handle, lr, beta1, beta2, eps, weight_decay, step, max_norm, avg_factor, error_if_nonfinite,
                     d_result, stream):
    hp = GclipAdamwHparams(float(lr), float(beta1), float(beta2), float(eps), float(weight_decay), int(step))
    _check(_lib.lib.gclip_adamw_step(handle, ctypes.byref(hp), float(max_norm), float(avg_factor),
                                     int(bool(error_if_nonfinite)), ctypes.c_void_p(int(d_result)),
                                     ctypes.c_void_p(int(stream))), "gclip_adamw_step")


def gclip_tensor_norms(handle, avg_factor, d_tensors, d_result, stream):
    _check(_lib.lib.gclip_tensor_norms(handle, float(avg_factor), ctypes.c_void_p(int(d_tensors)),
                                       ctypes.c_void_p(int(d_result)), ctypes.c_void_p(int(stream))),
           "gclip_tensor_norms")


def gclip_clip_per_tensor_(handle, max_norm, avg_factor, error_if_nonfinite, d_tensors, d_result, stream):
    _check(_lib.lib.gclip_clip_per_tensor_(handle, float(max_norm), float(avg_factor), int(bool(error_if_nonfinite)),
                                           ctypes.c_void_p(int(d_tensors)), ctypes.c_void_p(int(d_result)),
                                           ctypes.c_void_p(int(stream))), "gclip_clip_per_tensor_")


def gclip_set_gather_wait(microseconds):
    """Process-wide wait of the per-tensor clip's gathering workgroup
    (negative: the default, 10 s); for tests of GCLIP_DEVICE_WAIT_TIMEOUT."""
    _check(_lib.lib.gclip_set_gather_wait(int(microseconds)), "gclip_set_gather_wait")


def gclip_contrib_create(handle, d_contrib):
    n = len(d_contrib)
    arr = (ctypes.c_void_p * max(n, 1))(*[ctypes.c_void_p(int(a)) for a in d_contrib])
    out = ctypes.c_void_p()
    _check(_lib.lib.gclip_contrib_create(handle, arr, ctypes.byref(out)), "gclip_contrib_create")
    return out


def gclip_contrib_destroy(handle):
    _check(_lib.lib.gclip_contrib_destroy(handle), "gclip_contrib_destroy")


def gclip_accumulate_norm(handle, contrib, avg_factor, d_tensors, d_result, stream):
    _check(_lib.lib.gclip_accumulate_norm(handle, contrib, float(avg_factor), ctypes.c_void_p(int(d_tensors or 0)),
                                          ctypes.c_void_p(int(d_result)), ctypes.c_void_p(int(stream))),
           "gclip_accumulate_norm")


def gclip_accumulate_clip_(handle, contrib, max_norm, avg_factor, error_if_nonfinite, d_result, stream):
    _check(_lib.lib.gclip_accumulate_clip_(handle, contrib, float(max_norm), float(avg_factor),
                                           int(bool(error_if_nonfinite)), ctypes.c_void_p(int(d_result)),
                                           ctypes.c_void_p(int(stream))), "gclip_accumulate_clip_")


def _amp_params(growth_factor, backoff_factor, growth_interval):
    return GclipAmpParams(float(growth_factor), float(backoff_factor), int(growth_interval), 0)


def gclip_norm_amp(handle, n_microbatches, d_amp, d_result, stream):
    _check(_lib.lib.gclip_norm_amp(handle, float(n_microbatches), ctypes.c_void_p(int(d_amp)),
                                   ctypes.c_void_p(int(d_result)), ctypes.c_void_p(int(stream))), "gclip_norm_amp")


def gclip_clip_amp_(handle, max_norm, n_microbatches, d_amp, growth_factor, backoff_factor, growth_interval,
                    d_result, stream):
    prm = _amp_params(growth_factor, backoff_factor, growth_interval)
    _check(_lib.lib.gclip_clip_amp_(handle, float(max_norm), float(n_microbatches), ctypes.c_void_p(int(d_amp)),
                                    ctypes.byref(prm), ctypes.c_void_p(int(d_result)), ctypes.c_void_p(int(stream))),
           "gclip_clip_amp_")


def gclip_adamw_step_amp(handle, lr, beta1, beta2, eps, weight_decay, step, max_norm, n_microbatches, d_amp,
                         growth_factor, backoff_factor, growth_interval, d_result, stream):
    hp = GclipAdamwHparams(float(lr), float(beta1), float(beta2), float(eps), float(weight_decay), int(step))
    prm = _amp_params(growth_factor, backoff_factor, growth_interval)
    _check(_lib.lib.gclip_adamw_step_amp(handle, ctypes.byref(hp), float(max_norm), float(n_microbatches),
                                         ctypes.c_void_p(int(d_amp)), ctypes.byref(prm),
                                         ctypes.c_void_p(int(d_result)), ctypes.c_void_p(int(stream))),
           "gclip_adamw_step_amp")


# ---------------------------------------------------------------- torch-facing wrapper
def _torch_dtype_code(t):
    import torch
    m = {torch.float32: GCLIP_F32, torch.float16: GCLIP_F16, torch.bfloat16: GCLIP_BF16}
    if t.dtype not in m:
        raise TypeError(f"unsupported gradient dtype {t.dtype}")
    return m[t.dtype]


class GradList:
    """A fixed list of same-dtype, contiguous gradient tensors on one GPU.

    The descriptor table and a 64-byte device result block are allocated once
    here; norm / scale / clip_ only enqueue kernels on the given (default:
    current) stream and allocate nothing.  The tensors are referenced so that
    their storage cannot be freed while the list exists.
    """

    def __init__(self, tensors):
        import torch
        tensors = list(tensors)
        if not torch.cuda.is_available():
            raise RuntimeError("GradList needs a GPU")
        codes = {_torch_dtype_code(t) for t in tensors}
        if len(codes) > 1:
            raise TypeError("all tensors of a list must share one dtype")
        for t in tensors:
            if not t.is_cuda or not t.is_contiguous():
                raise ValueError("tensors must be contiguous device tensors")
        self.tensors = tensors
        self.dtype = codes.pop() if codes else GCLIP_F32
        self.device = tensors[0].device if tensors else torch.device("cuda", torch.cuda.current_device())
        with torch.cuda.device(self.device):
            self.result = torch.zeros(64, dtype=torch.uint8, device=self.device)
            self.tensor_results = torch.zeros(32 * max(len(tensors), 1), dtype=torch.uint8, device=self.device)
            self.handle = gclip_list_create([t.data_ptr() for t in tensors], [t.numel() for t in tensors],
                                            self.dtype)

    @staticmethod
    def _stream(stream):
        import torch
        s = torch.cuda.current_stream() if stream is None else stream
        return s.cuda_stream

    @property
    def d_result(self):
        return self.result.data_ptr()

    def info(self):
        return gclip_list_info(self.handle)

    def set_path(self, path):
        gclip_list_set_path(self.handle, path)

    def set_wait(self, microseconds):
        gclip_list_set_wait(self.handle, microseconds)

    def norm(self, avg_factor=1.0, stream=None):
        gclip_norm(self.handle, avg_factor, self.d_result, self._stream(stream))

    def scale(self, max_norm, avg_factor=1.0, error_if_nonfinite=False, stream=None):
        gclip_scale(self.handle, max_norm, avg_factor, error_if_nonfinite, self.d_result, self._stream(stream))

    def clip_(self, max_norm, avg_factor=1.0, error_if_nonfinite=False, stream=None):
        gclip_clip_(self.handle, max_norm, avg_factor, error_if_nonfinite, self.d_result, self._stream(stream))

    def tensor_norms(self, avg_factor=1.0, stream=None):
        """Every tensor's norm (and the list's, into the result block)."""
        gclip_tensor_norms(self.handle, avg_factor, self.tensor_results.data_ptr(), self.d_result,
                           self._stream(stream))

    def clip_per_tensor_(self, max_norm, avg_factor=1.0, error_if_nonfinite=False, stream=None):
        """Every tensor clipped by its own norm, in place."""
        gclip_clip_per_tensor_(self.handle, max_norm, avg_factor, error_if_nonfinite, self.tensor_results.data_ptr(),
                               self.d_result, self._stream(stream))

    def read_tensors(self, stream=None):
        """Wait for the stream; the per-tensor figures as a numpy record array."""
        import numpy as np
        self._wait(stream)
        raw = self.tensor_results.cpu().numpy()[:32 * len(self.tensors)]
        return raw.view(np.dtype(TENSOR_RESULT_DTYPE))

    def _wait(self, stream=None):
        import torch
        (torch.cuda.current_stream() if stream is None else stream).synchronize()

    def accumulate_norm(self, contrib, avg_factor=1.0, per_tensor=False, stream=None):
        """The last += (grads += contrib) fused with the norm pass; the
        per-tensor figures too when per_tensor is set (read_tensors)."""
        gclip_accumulate_norm(self.handle, contrib.handle, avg_factor,
                              self.tensor_results.data_ptr() if per_tensor else 0, self.d_result,
                              self._stream(stream))

    def accumulate_clip_(self, contrib, max_norm, avg_factor=1.0, error_if_nonfinite=False, stream=None):
        """The last += and the global clip of the sum."""
        gclip_accumulate_clip_(self.handle, contrib.handle, max_norm, avg_factor, error_if_nonfinite, self.d_result,
                               self._stream(stream))

    def norm_amp(self, n_microbatches, amp, stream=None):
        """Norm of the unscaled, averaged gradient: a = 1 / (n * S), S read
        from ``amp`` on the device."""
        gclip_norm_amp(self.handle, n_microbatches, amp.d_state, self.d_result, self._stream(stream))

    def clip_amp_(self, max_norm, n_microbatches, amp, stream=None):
        """Unscale, clip (nothing written on found-inf) and update ``amp``."""
        gclip_clip_amp_(self.handle, max_norm, n_microbatches, amp.d_state, amp.growth_factor, amp.backoff_factor,
                        amp.growth_interval, self.d_result, self._stream(stream))

    def read(self, error_if_nonfinite=False, stream=None):
        """Wait for the stream and return (status, result dict)."""
        return gclip_result_read(self.d_result, self._stream(stream), error_if_nonfinite)

    def close(self):
        if getattr(self, "handle", None):
            gclip_list_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Contribution:
    """One microbatch's gradient buffers registered for a GradList (same
    shapes and dtype, each at the same address modulo 16 bytes as the list's
    tensor): ``grads.accumulate_norm(contrib)`` is the last += fused with the
    norm pass."""

    def __init__(self, grad_list, tensors):
        tensors = list(tensors)
        if len(tensors) != len(grad_list.tensors):
            raise ValueError("one contribution tensor per gradient tensor")
        for c, t in zip(tensors, grad_list.tensors):
            if c.dtype != t.dtype or c.numel() != t.numel() or not c.is_contiguous() or c.device != t.device:
                raise ValueError("contribution tensors must match the gradients in dtype, size and device")
        self.tensors = tensors
        self.grad_list = grad_list
        self.handle = gclip_contrib_create(grad_list.handle, [c.data_ptr() for c in tensors])

    def close(self):
        if getattr(self, "handle", None):
            gclip_contrib_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class AmpState:
    """The loss-scale state of loss-scaled steps: 16 bytes in device memory
    (binary32 scale, int32 count of clean steps, int32 found-inf flag of the
    last step) and the update's parameters (dynamic loss scaling)."""

    def __init__(self, device, init_scale=65536.0, growth_factor=2.0, backoff_factor=0.5, growth_interval=2000):
        import torch
        self.buf = torch.zeros(4, dtype=torch.int32, device=device)
        self.growth_factor = float(growth_factor)
        self.backoff_factor = float(backoff_factor)
        self.growth_interval = int(growth_interval)
        self.set(init_scale, 0)

    @property
    def d_state(self):
        return self.buf.data_ptr()

    def set(self, scale, growth_tracker=0, found_inf=0):
        import torch
        self.buf[0:1].view(torch.float32).fill_(float(scale))
        self.buf[1] = int(growth_tracker)
        self.buf[2] = int(found_inf)

    def read(self):
        """(scale, growth_tracker, found_inf) after the work queued so far."""
        import torch
        h = self.buf.cpu()
        return float(h[0:1].view(torch.float32).item()), int(h[1]), bool(h[2])


class AdamWList:
    """AdamW over a fixed list of binary32 weights, their gradients (any list
    dtype) and binary32 moments, driven by the clip decision of a GradList
    over the same gradients: ``grads.norm(a)`` then ``opt.step(grads, ...)``
    is the clip followed by the optimizer step with the clipped gradient,
    without writing the clipped gradient back."""

    def __init__(self, params, grads, exp_avg, exp_avg_sq):
        import torch
        params, grads, exp_avg, exp_avg_sq = (list(x) for x in (params, grads, exp_avg, exp_avg_sq))
        if not (len(params) == len(grads) == len(exp_avg) == len(exp_avg_sq)):
            raise ValueError("the four lists must have the same length")
        for x in params + exp_avg + exp_avg_sq:
            if x.dtype != torch.float32:
                raise TypeError("weights and moments must be float32")
        codes = {_torch_dtype_code(g) for g in grads}
        if len(codes) > 1:
            raise TypeError("all gradients must share one dtype")
        for group in (params, grads, exp_avg, exp_avg_sq):
            for x in group:
                if not x.is_cuda or not x.is_contiguous():
                    raise ValueError("tensors must be contiguous device tensors")
        for a, b, c, d in zip(params, grads, exp_avg, exp_avg_sq):
            if not (a.numel() == b.numel() == c.numel() == d.numel()):
                raise ValueError("weight, gradient and moments of one tensor must have the same size")
        self.tensors = (params, grads, exp_avg, exp_avg_sq)
        self.dtype = codes.pop() if codes else GCLIP_F32
        self.device = params[0].device if params else torch.device("cuda", torch.cuda.current_device())
        with torch.cuda.device(self.device):
            self.handle = gclip_adamw_create([p.data_ptr() for p in params], [g.data_ptr() for g in grads],
                                             [m.data_ptr() for m in exp_avg], [v.data_ptr() for v in exp_avg_sq],
                                             [p.numel() for p in params], self.dtype)

    def step(self, grad_list, *, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step, max_norm,
             avg_factor=1.0, error_if_nonfinite=False, stream=None):
        """One optimizer step; grad_list.norm(avg_factor) must have run first
        on the same stream.  The decision lands in grad_list's result block."""
        gclip_adamw_step(self.handle, lr, beta1, beta2, eps, weight_decay, step, max_norm, avg_factor,
                         error_if_nonfinite, grad_list.d_result, GradList._stream(stream))

    def step_amp(self, grad_list, amp, *, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step, max_norm,
                 n_microbatches=1.0, stream=None):
        """A loss-scaled step: grad_list.norm_amp(n, amp) must have run first
        on the same stream; skipped on found-inf; then ``amp`` is updated."""
        gclip_adamw_step_amp(self.handle, lr, beta1, beta2, eps, weight_decay, step, max_norm, n_microbatches,
                             amp.d_state, amp.growth_factor, amp.backoff_factor, amp.growth_interval,
                             grad_list.d_result, GradList._stream(stream))

    def close(self):
        if getattr(self, "handle", None):
            gclip_adamw_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def clip_grad_norm_(tensors, max_norm, avg_factor=1.0, error_if_nonfinite=False, grad_list=None):
    """Clip a list of gradient tensors in place by their global L2 norm and
    return the pre-clip norm (of avg_factor * g).  Raises GclipError when
    error_if_nonfinite is set and a NaN/Inf element was found (nothing is
    written then).  Pass a persistent ``grad_list`` to avoid rebuilding the
    descriptor table on every call."""
    gl = grad_list if grad_list is not None else GradList(tensors)
    gl.clip_(max_norm, avg_factor, error_if_nonfinite)
    st, r = gl.read(error_if_nonfinite)
    if grad_list is None:
        gl.close()
    if st != _lib.GCLIP_OK:
        raise GclipError(st, "clip_grad_norm_")
    return r["norm"]
