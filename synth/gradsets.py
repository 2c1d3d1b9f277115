"""Synthetic gradient lists with the shapes of the models on the pages.

Shapes:
- ANDREA-120M (backprop lesson page, unhomeschool.com vi, section "One
  gradient tensor per weight tensor"): token embedding [8449, 768] (the size
  also quoted in the grad-clip lesson's "heterogeneous tensors" paragraph),
  position embedding [1024, 768], and per block W_Q, W_K, W_V, W_O [768, 768],
  W_1 [768, 3072], W_2 [3072, 768], LN1/LN2 gamma and beta [768], twelve
  blocks, then the final layer norm gamma and beta [768].  124 tensors,
  92,248,320 elements.
- A ~1.3B GPT-shaped list in bf16 (embedding [50304, 2048], 24 blocks of fused
  QKV [2048, 6144], O [2048, 2048], W_1 [2048, 8192], W_2 [8192, 2048] and four
  [2048] norms, then 4096 one-element tensors): 4,289 tensors, 1,311,182,848
  elements.
- A tiny list [2], [64, 64], [128], [33, 17], [1].

Values: each tensor t draws from numpy's default generator seeded with
SeedSequence([seed, t]) (or [seed, k, t] for microbatch k), standard normal in
binary64, times sigma, rounded to nearest-even into float32 and then, for the
16-bit sets, into float16 (numpy) or bfloat16 (torch).  Arrays hold the raw
storage: float32 for "f32", uint16 bit patterns for "f16" and "bf16".
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field

import numpy as np

F32, F16, BF16 = "f32", "f16", "bf16"


def storage_dtype(dtype: str):
    return np.float32 if dtype == F32 else np.uint16


def shapes_tiny():
    return [("t0", (2,)), ("t1", (64, 64)), ("t2", (128,)), ("t3", (33, 17)), ("t4", (1,))]


def shapes_andrea120m():
    d, v, ctx, ff, layers = 768, 8449, 1024, 3072, 12
    out = [("tok_embed", (v, d)), ("pos_embed", (ctx, d))]
    for l in range(layers):
        out += [(f"h{l}.W_Q", (d, d)), (f"h{l}.W_K", (d, d)), (f"h{l}.W_V", (d, d)), (f"h{l}.W_O", (d, d)),
                (f"h{l}.W_1", (d, ff)), (f"h{l}.W_2", (ff, d)),
                (f"h{l}.LN1.gamma", (d,)), (f"h{l}.LN1.beta", (d,)),
                (f"h{l}.LN2.gamma", (d,)), (f"h{l}.LN2.beta", (d,))]
    out += [("lnf.gamma", (d,)), ("lnf.beta", (d,))]
    return out


def shapes_gpt1p3b():
    d, v, layers = 2048, 50304, 24
    out = [("embed", (v, d))]
    for l in range(layers):
        out += [(f"h{l}.QKV", (d, 3 * d)), (f"h{l}.O", (d, d)), (f"h{l}.W_1", (d, 4 * d)), (f"h{l}.W_2", (4 * d, d)),
                (f"h{l}.LN1.gamma", (d,)), (f"h{l}.LN1.beta", (d,)),
                (f"h{l}.LN2.gamma", (d,)), (f"h{l}.LN2.beta", (d,))]
    out += [(f"scalar{i}", (1,)) for i in range(4096)]
    return out


def to_storage(x64: np.ndarray, dtype: str) -> np.ndarray:
    """Round binary64 draws to float32, then to the 16-bit format if asked."""
    f = np.ascontiguousarray(x64, dtype=np.float64).astype(np.float32)
    if dtype == F32:
        return f
    if dtype == F16:
        return f.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        import torch
        return torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(dtype)


def _draw(seed_words, n: int, sigma: float) -> np.ndarray:
    rng = np.random.default_rng(np.random.SeedSequence(list(seed_words)))
    return rng.standard_normal(n) * sigma


@dataclass
class GradSet:
    name: str
    dtype: str
    names: list
    shapes: list
    arrays: list
    max_norm: float = 1.0
    avg_factor: float = 1.0
    error_if_nonfinite: bool = False
    notes: dict = field(default_factory=dict)

    @property
    def numel(self) -> int:
        return int(sum(a.size for a in self.arrays))

    @property
    def nbytes(self) -> int:
        return int(sum(a.nbytes for a in self.arrays))

    def copy(self) -> "GradSet":
        return GradSet(self.name, self.dtype, list(self.names), list(self.shapes), [a.copy() for a in self.arrays],
                       self.max_norm, self.avg_factor, self.error_if_nonfinite, dict(self.notes))


def _pool_map(fn, items, threads):
    if threads <= 1 or len(items) < 2:
        return [fn(i) for i in items]
    with _cf.ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(fn, items))


def _default_threads():
    return max(1, min(16, os.cpu_count() or 1))


def _gen(name, shapes, dtype, seed, sigma_of, threads=None):
    threads = threads or _default_threads()
    idx = list(range(len(shapes)))

    def one(t):
        n = int(np.prod(shapes[t][1]))
        return to_storage(_draw([seed, t], n, sigma_of(t)), dtype)

    arrays = _pool_map(one, idx, threads)
    return GradSet(name, dtype, [s[0] for s in shapes], [tuple(s[1]) for s in shapes], arrays)


def tiny_f32(seed: int = 0):
    """Tiny fp32 list, N(0,1), max_norm 1.0."""
    g = _gen("tiny_f32", shapes_tiny(), F32, seed, lambda t: 1.0)
    g.max_norm = 1.0
    return g


def worked_6_8(dtype: str = F32):
    """The glossary page's worked example: [6, 8] with threshold 5."""
    a = to_storage(np.array([6.0, 8.0]), dtype)
    return GradSet("worked_6_8", dtype, ["g"], [(2,)], [a], max_norm=5.0)


def andrea120m_f32(seed: int = 1, threads=None):
    """ANDREA-120M-shaped fp32 grads, N(0, 1e-3^2), max_norm 1.0 (norm ~9.6)."""
    g = _gen("andrea120m_f32", shapes_andrea120m(), F32, seed, lambda t: 1e-3, threads)
    return g


SPIKED = ("tok_embed", "h0.W_1")


def andrea120m_f16_spike(seed: int = 2, threads=None):
    """fp16 storage; tok_embed and layer-0 W_1 drawn 100x larger (a data-source
    switch shock), max_norm 1.0 (norm ~297.6)."""
    shapes = shapes_andrea120m()
    spiked = {i for i, (n, _) in enumerate(shapes) if n in SPIKED}
    g = _gen("andrea120m_f16_spike", shapes, F16, seed, lambda t: 1e-1 if t in spiked else 1e-3, threads)
    g.notes["spiked"] = sorted(spiked)
    return g


def andrea120m_f16_small(seed: int = 3, threads=None):
    """fp16 storage, N(0, 1e-5^2), no spikes: norm ~0.096 < max_norm 1.0 (no writes)."""
    return _gen("andrea120m_f16_small", shapes_andrea120m(), F16, seed, lambda t: 1e-5, threads)


def andrea120m_f32_accum4(seed: int = 4, threads=None):
    """Four fp32 microbatch contributions per tensor, each N(0, 1e-3^2), added
    into one buffer in order ((c0 + c1) + c2) + c3 in float32 (the += of the
    backward kernels); the clip then averages by 1/4 (norm of the average ~4.8)."""
    shapes = shapes_andrea120m()
    threads = threads or _default_threads()

    def one(t):
        n = int(np.prod(shapes[t][1]))
        acc = to_storage(_draw([seed, 0, t], n, 1e-3), F32)
        for k in range(1, 4):
            acc = acc + to_storage(_draw([seed, k, t], n, 1e-3), F32)  # float32 add, round to nearest
        return acc

    arrays = _pool_map(one, list(range(len(shapes))), threads)
    g = GradSet("andrea120m_f32_accum4", F32, [s[0] for s in shapes], [tuple(s[1]) for s in shapes], arrays)
    g.avg_factor = 0.25
    g.notes["microbatches"] = 4
    return g


def andrea120m_f32_accum4_parts(seed: int = 4, threads=None):
    """The same four microbatch draws as andrea120m_f32_accum4, split before
    the last +=: the buffer after three contributions ((c0 + c1) + c2, float32
    adds in order) and the fourth contribution c3.  (buffer, contribution)."""
    shapes = shapes_andrea120m()
    threads = threads or _default_threads()

    def one(t):
        n = int(np.prod(shapes[t][1]))
        acc = to_storage(_draw([seed, 0, t], n, 1e-3), F32)
        for k in range(1, 3):
            acc = acc + to_storage(_draw([seed, k, t], n, 1e-3), F32)
        return acc, to_storage(_draw([seed, 3, t], n, 1e-3), F32)

    pairs = _pool_map(one, list(range(len(shapes))), threads)
    names, dims = [s[0] for s in shapes], [tuple(s[1]) for s in shapes]
    buf = GradSet("andrea120m_f32_accum4_buffer", F32, names, dims, [p[0] for p in pairs])
    buf.avg_factor = 0.25
    buf.notes["microbatches"] = 4
    return buf, GradSet("andrea120m_f32_accum4_last", F32, names, dims, [p[1] for p in pairs])


def flat_f32(seed: int = 6, threads=None):
    """The ANDREA-120M element count as one fp32 tensor (the same bytes with
    no tensor boundaries), N(0, 1e-3^2), max_norm 1.0."""
    n = sum(int(np.prod(s)) for _, s in shapes_andrea120m())
    chunks = 16
    sizes = [n // chunks + (1 if i < n % chunks else 0) for i in range(chunks)]
    parts = _pool_map(lambda i: to_storage(_draw([seed, i], sizes[i], 1e-3), F32), list(range(chunks)),
                      threads or _default_threads())
    return GradSet("flat_f32", F32, ["flat"], [(n,)], [np.concatenate(parts)])


NAN_TENSOR = "h23.W_2"
NAN_INDEX = 1_234_567


def gpt1p3b_bf16(seed: int = 5, threads=None):
    """~1.3B GPT-shaped bf16 grads, N(0, 1e-4^2), max_norm 1.0 (norm ~3.6)."""
    return _gen("gpt1p3b_bf16", shapes_gpt1p3b(), BF16, seed, lambda t: 1e-4, threads)


def inject_nan(g: GradSet, tensor: str = NAN_TENSOR, index: int = NAN_INDEX) -> GradSet:
    """Put one quiet NaN at a flat index of a named tensor (in place)."""
    t = g.names.index(tensor)
    a = g.arrays[t]
    if g.dtype == F32:
        a[index] = np.float32("nan")
    elif g.dtype == F16:
        a[index] = 0x7E00
    else:
        a[index] = 0x7FC0
    g.notes.setdefault("nonfinite_at", []).append((tensor, index))
    return g


def inject_value(g: GradSet, tensor: str, index: int, value: float) -> GradSet:
    """Store one value (e.g. +-inf) at a flat index of a named tensor."""
    t = g.names.index(tensor)
    g.arrays[t][index] = to_storage(np.array([value]), g.dtype)[0]
    g.notes.setdefault("injected", []).append((tensor, index, value))
    return g


def bf16_bits(n: int, seed: int, exp_lo: int = 116, chunk: int = 1 << 27) -> np.ndarray:
    """n bfloat16 bit patterns with a random sign, a random mantissa and a
    biased exponent in exp_lo .. exp_lo + 3 (116: magnitudes in [2^-11,
    2^-7)), drawn in chunks from one seeded generator (cheap for billions of
    elements: no binary64 temporaries)."""
    rng = np.random.default_rng([seed, 0xbf16])
    out = np.empty(n, dtype=np.uint16)
    for b in range(0, n, chunk):
        r = rng.integers(0, 1 << 16, size=min(chunk, n - b), dtype=np.uint16)
        out[b:b + r.size] = (r & np.uint16(0x807F)) | ((((r >> np.uint16(7)) & np.uint16(3)) + np.uint16(exp_lo))
                                                       << np.uint16(7))
    return out


def f16_bits(n: int, seed: int, exp_lo: int = 7, chunk: int = 1 << 27) -> np.ndarray:
    """n IEEE binary16 bit patterns with a random sign, a random mantissa and
    a biased exponent in exp_lo .. exp_lo + 3 (7: magnitudes in [2^-8,
    2^-4)), drawn in chunks like bf16_bits."""
    rng = np.random.default_rng([seed, 0xf16])
    out = np.empty(n, dtype=np.uint16)
    for b in range(0, n, chunk):
        r = rng.integers(0, 1 << 16, size=min(chunk, n - b), dtype=np.uint16)
        out[b:b + r.size] = (r & np.uint16(0x83FF)) | ((((r >> np.uint16(10)) & np.uint16(3)) + np.uint16(exp_lo))
                                                       << np.uint16(10))
    return out


CONFIGS = {
    "tiny_f32": tiny_f32,
    "andrea120m_f32": andrea120m_f32,
    "andrea120m_f16_spike": andrea120m_f16_spike,
    "andrea120m_f16_small": andrea120m_f16_small,
    "andrea120m_f32_accum4": andrea120m_f32_accum4,
    "gpt1p3b_bf16": gpt1p3b_bf16,
    "flat_f32": flat_f32,
}


def make(name: str, **kw) -> GradSet:
    return CONFIGS[name](**kw)


def random_list(rng: np.random.Generator, dtype: str, max_tensors: int = 6, max_numel: int = 50,
                sigma: float = 1.0) -> GradSet:
    """A small random list for brute-force checks: sizes 0..max_numel."""
    n = int(rng.integers(0, max_tensors + 1))
    arrays = []
    for _ in range(n):
        k = int(rng.integers(0, max_numel + 1))
        arrays.append(to_storage(rng.standard_normal(k) * sigma, dtype))
    return GradSet("random", dtype, [f"r{i}" for i in range(n)], [(a.size,) for a in arrays], arrays)
