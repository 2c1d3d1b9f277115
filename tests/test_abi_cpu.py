"""The C ABI on the CPU: the library loads and exports every function that
include/gclip.h declares; argument errors come back before any GPU work; the
descriptor table covers every element exactly once, in balanced shares; and
the kernels' own address walk, replayed on the host, stays inside the
tensors and visits every byte once per pass."""
import glob
import os
import re
import subprocess

import numpy as np
import pytest

import global_l2_norm_amd as g
from global_l2_norm_amd import _lib
from synth import gradsets as gs
from tests.abi_util import ESIZE, TAG, check_walk, fake_layout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# the diagnostic header's call is exported by the phase-stamps build only
STAMPS_HEADER = os.path.join(ROOT, "include", "gclip_stamps.h")
STAMPS_LIB = os.path.join(ROOT, "global_l2_norm_amd", "_stamps", "libgclip.so")
HEADERS = sorted(h for h in glob.glob(os.path.join(ROOT, "include", "*.h")) if h != STAMPS_HEADER)


def declared_functions(headers=HEADERS):
    names = set()
    for h in headers:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(gclip_[a-z_]+)\s*\(", text))
    return sorted(names)


def exported_functions(lib_path):
    out = subprocess.run(["nm", "-D", "--defined-only", lib_path], capture_output=True, text=True,
                         check=True).stdout
    return {line.split()[-1] for line in out.splitlines() if line.strip()}


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("gclip_norm", "gclip_scale", "gclip_clip_", "gclip_list_create", "gclip_list_destroy",
                     "gclip_result_read"):
        assert required in names


def test_library_exports_every_declared_function():
    exported = exported_functions(_lib.LIB_PATH)
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    assert set(_lib.EXPORTS) == set(declared_functions())
    for n in declared_functions():
        assert hasattr(_lib.lib, n)


def test_phase_stamps_only_in_the_diagnostic_build():
    """The library records no phase timeline and does not export its reader;
    the --phase-stamps build exports it besides every other call."""
    stamps_calls = declared_functions([STAMPS_HEADER])
    assert stamps_calls == ["gclip_phase_stamps"]
    assert not set(stamps_calls) & exported_functions(_lib.LIB_PATH)
    if not os.path.exists(STAMPS_LIB):
        pytest.skip("the --phase-stamps build is not there (python -m global_l2_norm_amd.build --phase-stamps)")
    exported = exported_functions(STAMPS_LIB)
    missing = [n for n in declared_functions() + stamps_calls if n not in exported]
    assert not missing, missing


def test_version_and_status_strings():
    assert g.gclip_version() == 3
    for code in range(8):
        assert g.gclip_status_string(code) not in ("", "unknown status")
    assert g.gclip_status_string(99) == "unknown status"


def test_reference_kernels_reject_bad_spans_before_any_gpu_work():
    """gclip_ref_read / gclip_ref_copy check their spans on the host: an
    empty span is a no-op, a misaligned or ragged one or an overlapping copy
    is GCLIP_EINVAL, and neither touches a GPU."""
    L = _lib.lib
    sink = 0x1000
    assert L.gclip_ref_read(None, 0, sink, None) == _lib.GCLIP_OK
    assert L.gclip_ref_copy(None, None, 0, None) == _lib.GCLIP_OK
    assert L.gclip_ref_read(0x1008, 64, sink, None) == _lib.GCLIP_EINVAL   # misaligned
    assert L.gclip_ref_read(0x1000, 24, sink, None) == _lib.GCLIP_EINVAL   # not whole vectors
    assert L.gclip_ref_read(0x1000, -16, sink, None) == _lib.GCLIP_EINVAL
    assert L.gclip_ref_read(0x1000, 64, None, None) == _lib.GCLIP_EINVAL
    assert L.gclip_ref_copy(0x2000, 0x1000, 8192, None) == _lib.GCLIP_EINVAL  # overlapping ranges
    assert L.gclip_ref_copy(0x1000, 0x2000, 8192, None) == _lib.GCLIP_EINVAL
    assert L.gclip_ref_copy(0x3000, 0x1001, 64, None) == _lib.GCLIP_EINVAL


def test_gather_wait_setter_bounds():
    """The process-wide bound of the per-tensor gathering wait: above 60 s is
    rejected, a negative value restores the default (no GPU involved)."""
    assert _lib.lib.gclip_set_gather_wait(61 * 1000 * 1000) == _lib.GCLIP_EINVAL
    assert _lib.lib.gclip_set_gather_wait(60 * 1000 * 1000) == _lib.GCLIP_OK
    assert _lib.lib.gclip_set_gather_wait(0) == _lib.GCLIP_OK
    assert _lib.lib.gclip_set_gather_wait(-1) == _lib.GCLIP_OK


@pytest.mark.parametrize("args,code", [
    (([0x1000], [-1], 0), _lib.GCLIP_EINVAL),               # negative size
    (([0x1002], [10], 0), _lib.GCLIP_EINVAL),               # fp32 tensor not 4-byte aligned
    (([0x1001], [10], 1), _lib.GCLIP_EINVAL),               # fp16 tensor at an odd address
    (([0x1000, 0x1010], [10, 10], 0), _lib.GCLIP_EINVAL),   # overlap
    (([0x1000, 0x1000], [4, 4], 2), _lib.GCLIP_EINVAL),     # the same tensor twice
    (([0], [10], 0), _lib.GCLIP_EINVAL),                    # NULL with elements
    (([0x1000], [10], 3), _lib.GCLIP_EDTYPE),               # unknown dtype
])
def test_list_create_rejects_bad_lists(args, code):
    with pytest.raises(g.GclipError) as e:
        g.gclip_list_create(*args)
    assert e.value.status == code


def test_hot_calls_reject_bad_arguments_before_any_gpu_work():
    L = _lib.lib
    assert L.gclip_norm(None, 1.0, None, None) == _lib.GCLIP_EINVAL
    assert L.gclip_scale(None, 1.0, 1.0, 0, None, None) == _lib.GCLIP_EINVAL
    assert L.gclip_clip_(None, float("nan"), 1.0, 0, None, None) == _lib.GCLIP_EINVAL
    assert L.gclip_list_destroy(None) == _lib.GCLIP_OK
    assert L.gclip_result_read(None, None, None, 0) == _lib.GCLIP_EINVAL


def _random_numels(rng):
    sizes = [0, 1, 2, 3, 5, 7, 63, 64 * 4 - 1, 64 * 4, 64 * 4 + 1, 1000, 4099, 40000, 123457]
    return [int(rng.choice(sizes)) for _ in range(int(rng.integers(1, 30)))]


@pytest.mark.parametrize("dtype", [0, 1, 2])
@pytest.mark.parametrize("seed", range(6))
def test_plan_covers_every_element_once(dtype, seed):
    rng = np.random.default_rng(100 + seed)
    numels = _random_numels(rng)
    es = ESIZE[dtype]
    addrs = fake_layout(rng, numels, es, misalign=bool(seed % 2))
    nw = int(rng.choice([1, 3, 7, 256]))
    entries = g.gclip_plan_query(addrs, numels, dtype, nw, 512)
    # the summing passes read blocks, single elements and the sum chunks of
    # the streamed region; the split scale pass the scale chunks over the
    # whole list and the same single elements; the fused scale pass blocks,
    # single elements and the scale chunks of the streamed region
    sum_cover = [np.zeros(n, dtype=np.int32) for n in numels]
    scale_cover = [np.zeros(n, dtype=np.int32) for n in numels]
    fused_cover = [np.zeros(n, dtype=np.int32) for n in numels]
    blk_vectors = np.zeros(nw, dtype=np.int64)
    sc_per_worker = np.zeros(nw, dtype=np.int64)
    streamed = 0
    for w, t, b, c, kind in entries:
        assert c > 0 and kind in (0, 1, 2, 3, 4)
        assert (w == -1) == (kind in (2, 3, 4)) and -1 <= w < nw
        if kind in (0, 1, 3):
            sum_cover[t][b:b + c] += 1
        if kind in (1, 2):
            scale_cover[t][b:b + c] += 1
        if kind in (0, 1, 4):
            fused_cover[t][b:b + c] += 1
        if kind != 1:
            assert (addrs[t] + b * es) % 16 == 0 and (c * es) % 16 == 0
        if kind == 0:
            blk_vectors[w] += c * es // 16
        elif kind == 3:
            streamed += c * es // 16
        elif kind == 1:
            sc_per_worker[w] += c
    for cv in sum_cover + scale_cover + fused_cover:
        assert np.all(cv == 1)
    # blocks: equal, except that the last non-empty one may be cut short;
    # a streamed region only once every block is full
    full = blk_vectors[blk_vectors > 0]
    if len(full) > 1:
        assert np.all(full[:-1] == full[0]) and full[-1] <= full[0]
    if streamed > 0:
        assert np.all(blk_vectors == blk_vectors[0])
    assert sc_per_worker.max() - sc_per_worker.min() <= 1


def _runs_cover_once(entries, numels, kinds):
    runs = [[] for _ in numels]
    for w, t, b, c, kind in entries:
        if kind in kinds:
            runs[t].append((b, c))
    for t, n in enumerate(numels):
        at = 0
        for b, c in sorted(runs[t]):
            assert b == at, f"tensor {t}: gap or overlap at element {at}"
            at = b + c
        assert at == n, f"tensor {t}: {at} of {n} elements covered"


def test_plan_over_1gib_covers_every_element_once():
    """A list of 1 GiB or more (the 1.3B bf16 shapes, 2.6 GB) has sum chunks
    of two sizes in turn; the summing passes (blocks, single elements, sum
    chunks) and both scale passes still take every element exactly once.
    Counted by runs, without a per-element array."""
    numels = [int(np.prod(s)) for _, s in gs.shapes_gpt1p3b()]
    assert sum(numels) * 2 >= 1 << 30
    addrs = fake_layout(np.random.default_rng(9), numels, 2, misalign=True)
    entries = g.gclip_plan_query(addrs, numels, 2, 256, 512)
    _runs_cover_once(entries, numels, (0, 1, 3))
    _runs_cover_once(entries, numels, (1, 2))
    _runs_cover_once(entries, numels, (0, 1, 4))
    # inside the largest tensor the sum-chunk runs are whole chunks, larger
    # and smaller in turn (even- and odd-numbered workers), 1.07 : 0.93 to
    # within a group; a list under 1 GiB keeps one size
    big = int(np.argmax(numels))
    lens = [c for _, c in sorted((b, c) for w, t, b, c, k in entries if k == 3 and t == big)][1:-1]
    assert len(lens) >= 4 and len(set(lens)) == 2
    assert all(lens[i] != lens[i + 1] for i in range(len(lens) - 1))
    hi, lo = max(lens), min(lens)
    group = 8 * 512 * 8  # elements of a group of bf16 vectors
    assert abs(hi * 0.93 - lo * 1.07) <= 2 * group
    numels = [int(np.prod(s)) for _, s in gs.shapes_andrea120m()]
    addrs = fake_layout(np.random.default_rng(9), numels, 4, misalign=False)
    entries = g.gclip_plan_query(addrs, numels, 0, 256, 512)
    big = int(np.argmax(numels))
    lens = [c for _, c in sorted((b, c) for w, t, b, c, k in entries if k == 3 and t == big)][1:-1]
    assert len(set(lens)) == 1


@pytest.mark.parametrize("mode", [0, 1, 2, 3])
@pytest.mark.parametrize("dtype", [0, 1, 2])
@pytest.mark.parametrize("seed", range(4))
def test_kernel_walk_stays_inside_and_covers_once(mode, dtype, seed):
    rng = np.random.default_rng(200 + seed)
    es = ESIZE[dtype]
    numels = _random_numels(rng)
    if seed >= 2:  # big enough that the fused kernel also streams part of each share
        numels += [3_000_001, 777_777]
    addrs = fake_layout(rng, numels, es, misalign=bool(seed % 2))
    nw = [1, 3, 4, 8][seed]
    ta, tw = g.gclip_plan_trace(addrs, numels, dtype, nw, mode)
    check_walk(ta, addrs, numels, es)
    assert tw.min() >= -1 and tw.max() < nw


@pytest.mark.parametrize("mode", [0, 2, 3])
def test_kernel_walk_on_andrea120m_shapes(mode):
    shapes = gs.shapes_andrea120m()
    numels = [int(np.prod(s)) for _, s in shapes]
    rng = np.random.default_rng(7)
    addrs = fake_layout(rng, numels, 4, misalign=False)
    ta, _ = g.gclip_plan_trace(addrs, numels, 0, 256, mode)
    check_walk(ta, addrs, numels, 4)


def test_kernel_walk_on_shrunk_gpt_shapes_with_4096_scalars():
    shapes = [("embed", (503, 2048))]
    for l in range(2):
        shapes += [(f"h{l}.QKV", (2048, 6144)), (f"h{l}.LN1.gamma", (2048,)), (f"h{l}.O", (2048, 2048))]
    shapes += [(f"s{i}", (1,)) for i in range(4096)]
    numels = [int(np.prod(s)) for _, s in shapes]
    rng = np.random.default_rng(8)
    addrs = fake_layout(rng, numels, 2, misalign=True)
    for mode in (0, 1, 2, 3):
        ta, _ = g.gclip_plan_trace(addrs, numels, 2, 256, mode)
        check_walk(ta, addrs, numels, 2)


# ---------------------------------------------------------------- per-tensor pieces
def _check_tensor_attribution(ta, tw, addrs, numels, es):
    """Every access of the per-tensor kernels is credited to the tensor that
    holds it (out_worker is the piece's tensor in mode 4)."""
    start = (ta & ~TAG).astype(np.uint64)
    for t, (a, n) in enumerate(zip(addrs, numels)):
        mine = start[tw == t]
        assert np.all(mine >= a) and np.all(mine < a + n * es), f"tensor {t}: access outside it"
        tagged = (ta[tw == t] & TAG) != 0
        covered = int(np.where(tagged, es, 16).sum())
        assert covered == n * es, f"tensor {t}: {covered} bytes credited, {n * es} held"


@pytest.mark.parametrize("dtype", [0, 1, 2])
@pytest.mark.parametrize("seed", range(4))
def test_tensor_pieces_cover_once_and_credit_their_tensor(dtype, seed):
    rng = np.random.default_rng(400 + seed)
    es = ESIZE[dtype]
    numels = _random_numels(rng)
    if seed >= 2:  # several pieces per tensor, and a ragged last piece
        numels += [3_000_001, 0, 777_777, 5]
    addrs = fake_layout(rng, numels, es, misalign=bool(seed % 2))
    ta, tw = g.gclip_plan_trace(addrs, numels, dtype, 4, 4)
    check_walk(ta, addrs, numels, es)
    _check_tensor_attribution(ta, tw, addrs, numels, es)


def test_tensor_pieces_on_andrea120m_shapes():
    shapes = gs.shapes_andrea120m()
    numels = [int(np.prod(s)) for _, s in shapes]
    addrs = fake_layout(np.random.default_rng(9), numels, 4, misalign=False)
    ta, tw = g.gclip_plan_trace(addrs, numels, 0, 256, 4)
    check_walk(ta, addrs, numels, 4)
    _check_tensor_attribution(ta, tw, addrs, numels, 4)


# ---------------------------------------------------------------- the += in the fused kernel
def _contrib_addrs(addrs):
    return [a + (1 << 44) + (t << 34) for t, a in enumerate(addrs)]


@pytest.mark.parametrize("dtype", [0, 1, 2])
@pytest.mark.parametrize("seed", range(4))
def test_fused_accumulate_reads_every_contribution_byte_once(dtype, seed):
    """The contribution reads of the fused kernel with the += (first pass):
    inside the contribution tensors, no overlap, every byte once -- so the
    per-segment offsets and the per-lane segment of crossing groups are
    right."""
    rng = np.random.default_rng(500 + seed)
    es = ESIZE[dtype]
    numels = _random_numels(rng)
    if seed >= 2:
        numels += [3_000_001, 777_777]
    addrs = fake_layout(rng, numels, es, misalign=bool(seed % 2))
    nw = [1, 3, 4, 8][seed]
    ta, tw = g.gclip_plan_trace(addrs, numels, dtype, nw, 5)
    check_walk(ta, _contrib_addrs(addrs), numels, es)


@pytest.mark.parametrize("seed", range(3))
def test_handed_back_block_reads_its_contribution(seed):
    """A block handed back is read with its contribution in one walk: the
    same vectors as the first pass read for the blocks."""
    rng = np.random.default_rng(600 + seed)
    numels = _random_numels(rng) + [2_000_003]
    addrs = fake_layout(rng, numels, 4, misalign=bool(seed % 2))
    ta6, tw6 = g.gclip_plan_trace(addrs, numels, 0, 4, 6)
    ta5, tw5 = g.gclip_plan_trace(addrs, numels, 0, 4, 5)
    blocks5 = np.sort(ta5[(tw5 >= 0) & ((ta5 & TAG) == 0)])
    assert np.array_equal(np.sort(ta6), blocks5)


def test_fused_accumulate_on_andrea120m_shapes():
    shapes = gs.shapes_andrea120m()
    numels = [int(np.prod(s)) for _, s in shapes]
    addrs = fake_layout(np.random.default_rng(10), numels, 4, misalign=False)
    ta, _ = g.gclip_plan_trace(addrs, numels, 0, 256, 5)
    check_walk(ta, _contrib_addrs(addrs), numels, 4)
