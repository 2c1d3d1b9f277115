"""ctypes front end of the C oracle in gclip_oracle.c (test infrastructure only).

Each function works on host numpy arrays holding the raw storage of one
gradient tensor: float32 arrays for "f32", uint16 bit patterns for "f16" and
"bf16".  The arithmetic all happens in the C file, in binary64:

- ``sumsq``/``clip_`` follow the "Math" section of the grad-clip lesson page
  (unhomeschool.com, ru): the norm is the square root of the sum of squares of
  every element of every tensor, and a clip multiplies every element by
  max_norm / norm;
- ``decide`` follows the case split of the glossary page (paweldubiel.com,
  "Mechanism and details"): unchanged when the norm is at most c, otherwise
  scaled by c / norm; the averaging factor 1/n_microbatches of the backprop
  page (unhomeschool.com, vi, "Accumulation across microbatches") multiplies
  the gradient before its norm is taken and is folded into the written factor.
"""
import ctypes
import os

import numpy as np

from . import build as _build

F32, F16, BF16 = "f32", "f16", "bf16"
DTYPES = (F32, F16, BF16)
_CODE = {F32: 0, F16: 1, BF16: 2}
_NP = {F32: np.float32, F16: np.uint16, BF16: np.uint16}

class Oracle:
    """Handle on one build of the C oracle (the default build, or another
    build of the same source that a test asks for)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        vp = ctypes.c_void_p
        i64p = ctypes.POINTER(ctypes.c_int64)
        dp = ctypes.POINTER(ctypes.c_double)
        i32p = ctypes.POINTER(ctypes.c_int32)
        lib.oracle_decode_bits.argtypes = [ctypes.c_uint32, ctypes.c_int32]
        lib.oracle_decode_bits.restype = ctypes.c_double
        lib.oracle_encode.argtypes = [ctypes.c_double, ctypes.c_int32]
        lib.oracle_encode.restype = ctypes.c_uint32
        lib.oracle_sumsq.argtypes = [ctypes.POINTER(vp), i64p, ctypes.c_int32, ctypes.c_int32, ctypes.c_double,
                                     dp, i32p]
        lib.oracle_sumsq.restype = ctypes.c_int
        lib.oracle_tensor_sumsq.argtypes = [ctypes.POINTER(vp), i64p, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_double, dp]
        lib.oracle_tensor_sumsq.restype = ctypes.c_int
        lib.oracle_decide.argtypes = [ctypes.c_double, ctypes.c_int32, ctypes.c_double, ctypes.c_double,
                                      ctypes.c_int32, dp, i32p, i32p]
        lib.oracle_decide.restype = ctypes.c_int
        lib.oracle_scale.argtypes = [ctypes.POINTER(vp), i64p, ctypes.c_int32, ctypes.c_int32, ctypes.c_double]
        lib.oracle_scale.restype = ctypes.c_int
        lib.oracle_clip.argtypes = [ctypes.POINTER(vp), i64p, ctypes.c_int32, ctypes.c_int32, ctypes.c_double,
                                    ctypes.c_double, ctypes.c_int32, dp, i32p]
        lib.oracle_clip.restype = ctypes.c_int
        lib.oracle_accumulate.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), i64p, ctypes.c_int32,
                                          ctypes.c_int32]
        lib.oracle_accumulate.restype = ctypes.c_int
        lib.oracle_clip_per_tensor.argtypes = [ctypes.POINTER(vp), i64p, ctypes.c_int32, ctypes.c_int32,
                                               ctypes.c_double, ctypes.c_double, ctypes.c_int32, dp, i32p, dp, i32p]
        lib.oracle_clip_per_tensor.restype = ctypes.c_int
        f32p = ctypes.POINTER(ctypes.c_float)
        lib.oracle_adamw.argtypes = [f32p, vp, f32p, f32p, ctypes.c_int64, ctypes.c_int32, ctypes.c_double,
                                     ctypes.c_double, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                     ctypes.c_double, ctypes.c_int64, dp, dp, dp]
        lib.oracle_adamw.restype = ctypes.c_int
        lib.oracle_amp_avg.argtypes = [ctypes.c_double, ctypes.c_float]
        lib.oracle_amp_avg.restype = ctypes.c_double
        lib.oracle_amp_update.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int32),
                                          ctypes.c_int32, ctypes.c_double, ctypes.c_double, ctypes.c_int32]
        lib.oracle_amp_update.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def decode_bits(self, bits: int, dtype: str) -> float:
        """Value of one stored bit pattern, as a Python float (binary64)."""
        return self.lib.oracle_decode_bits(int(bits), _CODE[dtype])

    def encode(self, x: float, dtype: str) -> int:
        """Bit pattern of x rounded once to nearest-even in the storage format."""
        return int(self.lib.oracle_encode(float(x), _CODE[dtype]))

    def sumsq(self, arrays, dtype: str, avg_factor: float = 1.0):
        """(sum over all elements of (a*g)^2, any element NaN/Inf) in binary64."""
        ptrs, numels, n = _marshal(arrays, dtype)
        s = ctypes.c_double()
        nf = ctypes.c_int32()
        rc = self.lib.oracle_sumsq(ptrs, numels, n, _CODE[dtype], float(avg_factor), ctypes.byref(s),
                                   ctypes.byref(nf))
        if rc != 0:
            raise ValueError("oracle_sumsq rejected its arguments")
        return s.value, bool(nf.value)

    def tensor_sumsq(self, arrays, dtype: str, avg_factor: float = 1.0) -> np.ndarray:
        """Per-tensor sums of (a*g)^2 in binary64."""
        ptrs, numels, n = _marshal(arrays, dtype)
        out = np.zeros(max(n, 1), dtype=np.float64)
        rc = self.lib.oracle_tensor_sumsq(ptrs, numels, n, _CODE[dtype], float(avg_factor),
                                          out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
        if rc != 0:
            raise ValueError("oracle_tensor_sumsq rejected its arguments")
        return out[:n]

    def decide(self, norm: float, nonfinite: bool, max_norm: float, avg_factor: float = 1.0,
               error_if_nonfinite: bool = False):
        """(factor a*coef, clipped, skipped) for a given norm."""
        s = ctypes.c_double()
        c = ctypes.c_int32()
        k = ctypes.c_int32()
        self.lib.oracle_decide(float(norm), int(bool(nonfinite)), float(max_norm), float(avg_factor),
                               int(bool(error_if_nonfinite)), ctypes.byref(s), ctypes.byref(c), ctypes.byref(k))
        return s.value, bool(c.value), bool(k.value)

    def scale_(self, arrays, dtype: str, s: float) -> None:
        """In place: every element becomes round(g*s); nothing is written when s == 1."""
        ptrs, numels, n = _marshal(arrays, dtype)
        if self.lib.oracle_scale(ptrs, numels, n, _CODE[dtype], float(s)) != 0:
            raise ValueError("oracle_scale rejected its arguments")

    def clip_(self, arrays, dtype: str, max_norm: float, avg_factor: float = 1.0,
              error_if_nonfinite: bool = False) -> dict:
        """The whole path, in place.  Returns sumsq, norm (pre-clip), scale, flags."""
        ptrs, numels, n = _marshal(arrays, dtype)
        out = (ctypes.c_double * 3)()
        flags = (ctypes.c_int32 * 3)()
        rc = self.lib.oracle_clip(ptrs, numels, n, _CODE[dtype], float(max_norm), float(avg_factor),
                                  int(bool(error_if_nonfinite)), out, flags)
        if rc != 0:
            raise ValueError("oracle_clip rejected its arguments")
        return {"sumsq": out[0], "norm": out[1], "scale": out[2], "nonfinite": bool(flags[0]),
                "clipped": bool(flags[1]), "skipped": bool(flags[2])}


    def adamw(self, p, grad, m, v, dtype: str, s: float, lr: float, beta1: float, beta2: float, eps: float,
              weight_decay: float, step: int):
        """One AdamW step on one tensor with the clipped gradient s * grad.
        p, m, v: float32 arrays (left as they are); grad: raw storage of dtype.
        Returns binary64 arrays (p', m', v')."""
        p = np.ascontiguousarray(p, dtype=np.float32)
        m = np.ascontiguousarray(m, dtype=np.float32)
        v = np.ascontiguousarray(v, dtype=np.float32)
        grad = np.ascontiguousarray(grad, dtype=_NP[dtype])
        n = p.size
        if not (grad.size == m.size == v.size == n):
            raise ValueError("p, grad, m and v must have the same size")
        outs = [np.empty(n, dtype=np.float64) for _ in range(3)]
        f32p = ctypes.POINTER(ctypes.c_float)
        dp = ctypes.POINTER(ctypes.c_double)
        rc = self.lib.oracle_adamw(p.ctypes.data_as(f32p), ctypes.c_void_p(grad.ctypes.data),
                                   m.ctypes.data_as(f32p), v.ctypes.data_as(f32p), n, _CODE[dtype], float(s),
                                   float(lr), float(beta1), float(beta2), float(eps), float(weight_decay), int(step),
                                   *[o.ctypes.data_as(dp) for o in outs])
        if rc != 0:
            raise ValueError("oracle_adamw rejected its arguments")
        return tuple(outs)

    def clip_adamw(self, params, grads, m, v, dtype: str, max_norm: float, avg_factor: float = 1.0,
                   error_if_nonfinite: bool = False, *, lr: float, beta1: float, beta2: float, eps: float,
                   weight_decay: float, step: int):
        """The clip of the gradient list followed by one AdamW step on every
        tensor with the clipped gradient (nothing changes when the stop switch
        fires).  The gradients themselves are not written.  Returns the
        decision (as clip_ does) and lists of binary64 p', m', v'."""
        ptrs, numels, n = _marshal(grads, dtype)
        sumsq = ctypes.c_double()
        nonfinite = ctypes.c_int32()
        if self.lib.oracle_sumsq(ptrs, numels, n, _CODE[dtype], float(avg_factor), ctypes.byref(sumsq),
                                 ctypes.byref(nonfinite)) != 0:
            raise ValueError("oracle_sumsq rejected its arguments")
        norm = float(np.sqrt(sumsq.value))
        scale, clipped, skip = self.decide(norm, bool(nonfinite.value), max_norm, avg_factor, error_if_nonfinite)
        res = {"sumsq": sumsq.value, "norm": norm, "scale": 1.0 if skip else scale,
               "nonfinite": bool(nonfinite.value), "clipped": clipped, "skipped": skip}
        if skip:
            return res, ([np.asarray(x, np.float64) for x in params], [np.asarray(x, np.float64) for x in m],
                         [np.asarray(x, np.float64) for x in v])
        outs = [self.adamw(pp, g, mm, vv, dtype, scale, lr, beta1, beta2, eps, weight_decay, step)
                for pp, g, mm, vv in zip(params, grads, m, v)]
        return res, ([o[0] for o in outs], [o[1] for o in outs], [o[2] for o in outs])

    def accumulate_(self, acc, contrib, dtype: str) -> None:
        """acc[t] += contrib[t] in place, every element rounded once to the
        storage format (backprop lesson, "Accumulation across microbatches")."""
        if len(acc) != len(contrib) or any(a.shape != g.shape for a, g in zip(acc, contrib)):
            raise ValueError("accumulate: the two lists must have the same shapes")
        pa, numels, n = _marshal(acc, dtype)
        pg, _, _ = _marshal(contrib, dtype)
        if self.lib.oracle_accumulate(pa, pg, numels, n, _CODE[dtype]) != 0:
            raise ValueError("oracle_accumulate rejected its arguments")

    def accumulate_clip_(self, acc, contrib, dtype: str, max_norm: float, avg_factor: float = 1.0,
                         error_if_nonfinite: bool = False) -> dict:
        """The last microbatch's += followed by the clip of the sum: the norm
        is that of a times the accumulated buffer (glossary page, "Order
        changes the result": clip after the whole effective batch is in)."""
        self.accumulate_(acc, contrib, dtype)
        return self.clip_(acc, dtype, max_norm, avg_factor, error_if_nonfinite)

    def clip_per_tensor_(self, arrays, dtype: str, max_norm: float, avg_factor: float = 1.0,
                         error_if_nonfinite: bool = False) -> dict:
        """Per-tensor clipping in place: every tensor by its own norm (grad
        clip lesson, "Two variants: Per-Tensor or Global").  Returns the
        list's sumsq, norm and flags, and under "tensors" one dict per tensor
        (sumsq, norm, scale written, nonfinite, clipped)."""
        ptrs, numels, n = _marshal(arrays, dtype)
        tout = np.zeros(3 * max(n, 1), dtype=np.float64)
        tfl = np.zeros(2 * max(n, 1), dtype=np.int32)
        out = (ctypes.c_double * 2)()
        flags = (ctypes.c_int32 * 3)()
        rc = self.lib.oracle_clip_per_tensor(ptrs, numels, n, _CODE[dtype], float(max_norm), float(avg_factor),
                                             int(bool(error_if_nonfinite)),
                                             tout.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                             tfl.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), out, flags)
        if rc != 0:
            raise ValueError("oracle_clip_per_tensor rejected its arguments")
        tensors = [{"sumsq": tout[3 * t], "norm": tout[3 * t + 1], "scale": tout[3 * t + 2],
                    "nonfinite": bool(tfl[2 * t]), "clipped": bool(tfl[2 * t + 1])} for t in range(n)]
        return {"sumsq": out[0], "norm": out[1], "nonfinite": bool(flags[0]), "clipped": bool(flags[1]),
                "skipped": bool(flags[2]), "tensors": tensors}

    def amp_avg(self, n_microbatches: float, scale: float) -> float:
        """The averaging factor 1 / (n * S) of a loss-scaled step (S binary32)."""
        return self.lib.oracle_amp_avg(float(n_microbatches), float(np.float32(scale)))

    def amp_update(self, scale: float, tracker: int, found_inf: bool, growth: float = 2.0, backoff: float = 0.5,
                   interval: int = 2000):
        """(scale', tracker') after one step (dynamic loss scaling)."""
        sc = ctypes.c_float(float(np.float32(scale)))
        tr = ctypes.c_int32(int(tracker))
        if self.lib.oracle_amp_update(ctypes.byref(sc), ctypes.byref(tr), int(bool(found_inf)), float(growth),
                                      float(backoff), int(interval)) != 0:
            raise ValueError("oracle_amp_update rejected its arguments")
        return float(np.float32(sc.value)), int(tr.value)

    def clip_amp_(self, arrays, dtype: str, max_norm: float, n_microbatches: float, scale: float,
                  tracker: int = 0, growth: float = 2.0, backoff: float = 0.5, interval: int = 2000):
        """Unscale by 1 / (n * S), clip in place -- nothing written when an
        element is NaN or Inf (found-inf) -- and update the loss scale.
        Returns the clip result dict plus found_inf, scale' and tracker'."""
        r = self.clip_(arrays, dtype, max_norm, self.amp_avg(n_microbatches, scale), True)
        sc, tr = self.amp_update(scale, tracker, r["nonfinite"], growth, backoff, interval)
        r.update({"found_inf": r["nonfinite"], "loss_scale": sc, "growth_tracker": tr})
        return r


_default = None


def default() -> Oracle:
    """The oracle built from gclip_oracle.c (built on first use if absent)."""
    global _default
    if _default is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _default = Oracle(_build.LIB)
    return _default


def lib_path() -> str:
    return _build.LIB


def shards(arrays, parts: int):
    """The list cut into `parts` runs of consecutive elements, as equal in
    size as whole elements allow, each a list of contiguous views (a tensor
    may be split between two runs)."""
    total = sum(a.size for a in arrays)
    bounds = [total * k // parts for k in range(parts + 1)]
    out, t, off = [], 0, 0
    for k in range(parts):
        want, run = bounds[k + 1] - bounds[k], []
        while want > 0:
            a = arrays[t]
            take = min(want, a.size - off)
            run.append(a[off:off + take])
            want -= take
            off += take
            if off == a.size:
                t, off = t + 1, 0
        out.append(run)
    return out


def clip_sharded_(arrays, dtype: str, max_norm: float, avg_factor: float = 1.0, error_if_nonfinite: bool = False,
                  threads: int = 1) -> dict:
    """The clip of clip_ with its two passes spread over `threads` host
    threads, for timing the oracle on every core of a machine: the list is
    cut into as many runs of consecutive elements (shards); each thread sums
    one run with the oracle's own sum of squares, the runs' sums are added in
    run order, the decision is the oracle's, and each thread scales one run
    with the oracle's scale.  The C calls release the interpreter lock.  The
    elements come out as clip_ writes them for the same factor; the sum
    differs from clip_'s only by the order of its binary64 additions."""
    import math
    from concurrent.futures import ThreadPoolExecutor
    o = default()
    runs = shards(arrays, max(1, threads))
    with ThreadPoolExecutor(max_workers=max(1, threads)) as pool:
        parts = list(pool.map(lambda r: o.sumsq(r, dtype, avg_factor), runs))
        S = 0.0
        for p, _ in parts:
            S += p
        nonfinite = any(nf for _, nf in parts)
        norm = math.sqrt(S)
        s, clipped, skipped = o.decide(norm, nonfinite, max_norm, avg_factor, error_if_nonfinite)
        if not skipped and s != 1.0:
            list(pool.map(lambda r: o.scale_(r, dtype, s), runs))
    return {"sumsq": S, "norm": norm, "scale": s if not skipped else 1.0, "nonfinite": nonfinite,
            "clipped": clipped, "skipped": skipped}


def _marshal(arrays, dtype):
    if dtype not in _CODE:
        raise ValueError(f"unknown dtype {dtype!r}")
    for a in arrays:
        if a.dtype != _NP[dtype] or not a.flags.c_contiguous:
            raise TypeError(f"oracle expects contiguous {np.dtype(_NP[dtype]).name} storage for {dtype}")
    n = len(arrays)
    ptrs = (ctypes.c_void_p * max(n, 1))(*[a.ctypes.data for a in arrays])
    numels = (ctypes.c_int64 * max(n, 1))(*[a.size for a in arrays])
    return ptrs, numels, n


def decode_bits(bits, dtype):
    return default().decode_bits(bits, dtype)


def encode(x, dtype):
    return default().encode(x, dtype)


def sumsq(arrays, dtype, avg_factor=1.0):
    return default().sumsq(arrays, dtype, avg_factor)


def tensor_sumsq(arrays, dtype, avg_factor=1.0):
    return default().tensor_sumsq(arrays, dtype, avg_factor)


def decide(norm, nonfinite, max_norm, avg_factor=1.0, error_if_nonfinite=False):
    return default().decide(norm, nonfinite, max_norm, avg_factor, error_if_nonfinite)


def scale_(arrays, dtype, s):
    return default().scale_(arrays, dtype, s)


def clip_(arrays, dtype, max_norm, avg_factor=1.0, error_if_nonfinite=False):
    return default().clip_(arrays, dtype, max_norm, avg_factor, error_if_nonfinite)


def adamw(p, grad, m, v, dtype, s, lr, beta1, beta2, eps, weight_decay, step):
    return default().adamw(p, grad, m, v, dtype, s, lr, beta1, beta2, eps, weight_decay, step)


def accumulate_(acc, contrib, dtype):
    return default().accumulate_(acc, contrib, dtype)


def accumulate_clip_(acc, contrib, dtype, max_norm, avg_factor=1.0, error_if_nonfinite=False):
    return default().accumulate_clip_(acc, contrib, dtype, max_norm, avg_factor, error_if_nonfinite)


def clip_per_tensor_(arrays, dtype, max_norm, avg_factor=1.0, error_if_nonfinite=False):
    return default().clip_per_tensor_(arrays, dtype, max_norm, avg_factor, error_if_nonfinite)


def amp_avg(n_microbatches, scale):
    return default().amp_avg(n_microbatches, scale)


def amp_update(scale, tracker, found_inf, growth=2.0, backoff=0.5, interval=2000):
    return default().amp_update(scale, tracker, found_inf, growth, backoff, interval)


def clip_amp_(arrays, dtype, max_norm, n_microbatches, scale, tracker=0, growth=2.0, backoff=0.5, interval=2000):
    return default().clip_amp_(arrays, dtype, max_norm, n_microbatches, scale, tracker, growth, backoff, interval)


def clip_adamw(params, grads, m, v, dtype, max_norm, avg_factor=1.0, error_if_nonfinite=False, **hp):
    return default().clip_adamw(params, grads, m, v, dtype, max_norm, avg_factor, error_if_nonfinite, **hp)
