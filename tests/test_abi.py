"""The C ABI on the CPU: the library loads, exports every declared symbol, and
rejects bad arguments before anything is queued (no kernel runs here)."""
import ctypes
import os
import re

import pytest
import torch

import oasis_score_summaries_amd as oa
from oasis_score_summaries_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "oasis.h")

INVALID_ARG, UNSUPPORTED, WORKSPACE = 1, 2, 3
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first

# Calls with fake pointers run only where no GPU exists: should a check ever let
# one through, the launch then fails in the runtime instead of touching memory.
cpu_only = pytest.mark.skipif(torch.cuda.is_available(),
                              reason="fake-pointer validation tests run on CPU-only hosts")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(oasis_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return oa.load()


def _dims(**kw):
    base = dict(batch=2, num_kv_heads=2, group=4, max_blocks=64, num_queries=5, top_k=16,
                window_tokens=64, fetch_ratio=0.05)
    base.update(kw)
    head_dim = base.pop("head_dim", 128)
    block = base.pop("block_size", 16)
    return oa.make_dims(**base, head_dim=head_dim, block_size=block)


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert len(names) == 30
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.exported_symbols())


def test_version_and_status_strings(lib):
    text = open(HEADER).read()
    assert lib.oasis_abi_version() == int(re.search(r"#define OASIS_ABI_VERSION (\d+)", text).group(1))
    for code in range(5):
        assert lib.oasis_status_string(code)
    assert lib.oasis_status_string(99) == b"unknown status"


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 64, UNSUPPORTED), ("block_size", 24, UNSUPPORTED), ("block_size", 4, UNSUPPORTED),
    ("block_size", 128, UNSUPPORTED), ("block_size", 0, UNSUPPORTED), ("batch", 0, INVALID_ARG),
    ("num_kv_heads", 0, INVALID_ARG), ("group", 0, INVALID_ARG), ("num_queries", 0, INVALID_ARG),
    ("max_blocks", 0, INVALID_ARG), ("top_k", 0, INVALID_ARG), ("top_k", 65, INVALID_ARG),
    ("window_tokens", -1, INVALID_ARG), ("fetch_ratio", -0.1, INVALID_ARG),
    ("fetch_ratio", 1.5, INVALID_ARG), ("fetch_ratio", float("nan"), INVALID_ARG),
    ("max_blocks", 40000, UNSUPPORTED), ("group", 17, UNSUPPORTED), ("num_queries", 40, UNSUPPORTED),
])
@cpu_only
def test_dims_validation(lib, field, value, status):
    d = _dims(**{field: value})
    assert lib.oasis_fetch_cap(ctypes.byref(d)) == -1
    assert lib.oasis_table_stride(ctypes.byref(d)) == -1
    assert lib.oasis_decode_step_redoes_touched_splits(ctypes.byref(d)) == -1
    assert lib.oasis_workspace_bytes(ctypes.byref(d)) == 0
    st = lib.oasis_score_summaries(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None)
    assert st == status
    assert lib.oasis_last_error()
    st = lib.oasis_decode_step(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                               FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == status


@pytest.mark.parametrize("block,W,stride", [(8, 64, 16 + 8 + 1), (16, 64, 16 + 4 + 1),
                                             (32, 64, 16 + 2 + 1), (64, 64, 16 + 1 + 1),
                                             (32, 40, 16 + 2 + 1), (64, 0, 16 + 0 + 1)])
@cpu_only
def test_block_sizes_accepted(lib, block, W, stride):
    """8-, 16-, 32- and 64-token blocks: the table holds K slots plus the most window
    blocks a length has (ceil(W / block) + 1), the ring as many slots."""
    d = _dims(block_size=block, window_tokens=W)
    assert lib.oasis_table_stride(ctypes.byref(d)) == stride
    assert lib.oasis_window_ring_slots(ctypes.byref(d)) == stride - 16
    assert lib.oasis_workspace_bytes(ctypes.byref(d)) > 0
    assert lib.oasis_fetch_cap(ctypes.byref(d)) == 0


@cpu_only
def test_null_pointers_rejected(lib):
    d = _dims()
    args = [FAKE] * 4
    for i in range(4):
        a = list(args)
        a[i] = None
        assert lib.oasis_score_summaries(ctypes.byref(d), *a, None) == INVALID_ARG
        assert b"NULL" in lib.oasis_last_error()
    assert lib.oasis_score_summaries(None, FAKE, FAKE, FAKE, FAKE, None) == INVALID_ARG
    assert lib.oasis_build_summaries(ctypes.byref(d), None, FAKE, FAKE, None) == INVALID_ARG
    assert lib.oasis_topk_blocks(ctypes.byref(d), FAKE, FAKE, None, None) == INVALID_ARG
    d4 = _dims(fetch_ratio=0.25)                                # cap 4: the plan is required
    assert lib.oasis_fetch_cap(ctypes.byref(d4)) == 4
    assert lib.oasis_build_plan(ctypes.byref(d4), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE,
                                None) == INVALID_ARG
    d0 = _dims(fetch_ratio=0.01)                                # cap 0: plan may be NULL
    assert lib.oasis_fetch_cap(ctypes.byref(d0)) == 0
    assert lib.oasis_build_plan(ctypes.byref(d0), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE,
                                None) == INVALID_ARG          # plan_count is still required


@cpu_only
def test_noalloc_step_rejects_dims_beyond_its_array(lib):
    """The step on the library's own scratch array refuses dims whose workspace exceeds
    the array (16 MiB), before any HIP call, and names the reason."""
    big = _dims(batch=256, num_kv_heads=8, max_blocks=2048, top_k=128)
    assert lib.oasis_workspace_bytes(ctypes.byref(big)) > 16 << 20
    st = lib.oasis_decode_step_overlapped_noalloc(ctypes.byref(big), *([FAKE] * 13), 0.1, FAKE, FAKE, None)
    assert st == WORKSPACE
    assert b"scratch array" in lib.oasis_last_error()
    bad = _dims(group=0)
    assert lib.oasis_decode_step_overlapped_noalloc(ctypes.byref(bad), *([FAKE] * 13), 0.1, FAKE, FAKE,
                                                    None) == INVALID_ARG


@cpu_only
def test_workspace_and_table_stride_checks(lib):
    d = _dims()
    step_need = lib.oasis_workspace_bytes(ctypes.byref(d))
    assert step_need > 0 and step_need % 256 == 0
    T = lib.oasis_table_stride(ctypes.byref(d))
    assert T == 16 + 4 + 1
    need = lib.oasis_attn_workspace_bytes(ctypes.byref(d), T)
    assert need > 0 and need % 256 == 0
    # the step workspace: the split records, then the hand-off region (flags, status
    # word, a score mailbox of B*H*NB words)
    assert step_need >= need + 2 * 2 * 64 * 4
    assert lib.oasis_overlapped_selects_in_launch1(ctypes.byref(d)) == 1
    # every row count launch 1 fuses (up to 96 query rows per KV head), none beyond
    assert lib.oasis_overlapped_selects_in_launch1(ctypes.byref(_dims(group=8))) == 1
    assert lib.oasis_overlapped_selects_in_launch1(ctypes.byref(_dims(group=16, num_queries=6))) == 1
    assert lib.oasis_overlapped_selects_in_launch1(ctypes.byref(_dims(group=16, num_queries=7))) == 0
    assert lib.oasis_overlapped_selects_in_launch1(ctypes.byref(_dims(max_blocks=4096, top_k=16))) == 0
    # the serial step redoes the touched splits where the selection fits launch 1 and
    # a plan touches at most 16 splits and half of them (cap 6 of 35 here), else four
    # kernels: more new blocks per step, or Qwen3-235B's shape (5 splits of 8 rounds)
    assert lib.oasis_decode_step_redoes_touched_splits(ctypes.byref(_dims(max_blocks=2048, top_k=128))) == 1
    assert lib.oasis_decode_step_redoes_touched_splits(ctypes.byref(_dims(max_blocks=2048, top_k=128,
                                                                          fetch_ratio=0.25))) == 0
    assert lib.oasis_decode_step_redoes_touched_splits(ctypes.byref(_dims(batch=32, num_kv_heads=4, group=16,
                                                                          max_blocks=2048, top_k=128))) == 0
    assert lib.oasis_decode_step_redoes_touched_splits(ctypes.byref(_dims(group=16, num_queries=7))) == 0
    assert lib.oasis_overlapped_selects_in_launch1(ctypes.byref(_dims(batch=32, num_kv_heads=8))) == 1
    assert lib.oasis_overlapped_selects_in_launch1(ctypes.byref(_dims(batch=64, num_kv_heads=8))) == 0
    assert lib.oasis_overlapped_selects_in_launch1(ctypes.byref(_dims(group=0))) == -1
    off = lib.oasis_workspace_status_offset(ctypes.byref(d))
    assert need <= off < step_need and off % 4 == 0
    assert lib.oasis_attn_workspace_bytes(ctypes.byref(d), 0) == 0
    st = lib.oasis_sparse_decode_attn(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, T, FAKE, 0.1,
                                      FAKE, None, FAKE, need - 1, None)
    assert st == WORKSPACE
    st = lib.oasis_sparse_decode_attn(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 5000, FAKE, 0.1,
                                      FAKE, None, FAKE, need, None)
    assert st == INVALID_ARG
    st = lib.oasis_sparse_decode_attn(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, T, FAKE,
                                      float("inf"), FAKE, None, FAKE, need, None)
    assert st == INVALID_ARG
    st = lib.oasis_decode_step(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                               FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, None, None, step_need, None)
    assert st == WORKSPACE
    st = lib.oasis_decode_step(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                               FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, None, FAKE, step_need - 1, None)
    assert st == WORKSPACE
    assert lib.oasis_workspace_clear(ctypes.byref(d), None, step_need, None) == WORKSPACE
    assert lib.oasis_workspace_clear(ctypes.byref(d), FAKE, step_need - 1, None) == WORKSPACE
    # overlapping double-buffered slot tables are rejected
    res = ctypes.c_void_p(0x10000)
    st = lib.oasis_decode_step(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, res,
                               ctypes.c_void_p(0x10000 + 64), FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, None,
                               FAKE, step_need, None)
    assert st == INVALID_ARG and b"overlap" in lib.oasis_last_error()


def test_fetch_cap_rounding(lib):
    assert lib.oasis_fetch_cap(ctypes.byref(_dims(max_blocks=2048, top_k=128))) == 6
    assert lib.oasis_fetch_cap(ctypes.byref(_dims(max_blocks=2048, top_k=100, fetch_ratio=0.29))) == 29
    assert lib.oasis_fetch_cap(ctypes.byref(_dims(max_blocks=2048, top_k=128, fetch_ratio=1.0))) == 128


def test_binding_rejects_bad_tensors_before_the_library():
    d = _dims()
    with pytest.raises(ValueError):   # CPU tensors never reach the library
        oa.topk_blocks(d, torch.zeros((2, 2, 64)), torch.zeros(2, dtype=torch.int32))


def test_overlapped_step_argument_checks(lib):
    """The overlapped step needs its own resident_next buffer; checked before anything
    is queued."""
    d = _dims()
    need = lib.oasis_workspace_bytes(ctypes.byref(d))
    res = ctypes.c_void_p(0x10000)

    def call(res_next, ws_bytes=need):
        return lib.oasis_decode_step_overlapped(
            ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, res, res_next, FAKE, FAKE,
            FAKE, FAKE, 0.1, FAKE, None, FAKE, ws_bytes, None)

    assert call(None) == INVALID_ARG
    assert call(res) == INVALID_ARG
    assert b"own buffer" in lib.oasis_last_error()
    assert call(ctypes.c_void_p(0x10000 + 64)) == INVALID_ARG   # overlaps
    assert b"overlap" in lib.oasis_last_error()
    assert call(ctypes.c_void_p(0x20000), need - 1) == WORKSPACE
    st = lib.oasis_sparse_decode_attn_resident(ctypes.byref(d), FAKE, FAKE, FAKE, None, FAKE, 0.1,
                                               FAKE, None, FAKE, need, None)
    assert st == INVALID_ARG
    # the attention over slot tables needs the split records only
    attn_need = lib.oasis_attn_workspace_bytes(ctypes.byref(d), lib.oasis_table_stride(ctypes.byref(d)))
    assert attn_need < need
    st = lib.oasis_sparse_decode_attn_resident(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 0.1,
                                               FAKE, None, FAKE, attn_need - 1, None)
    assert st == WORKSPACE


@cpu_only
def test_working_set_argument_checks(lib):
    """NULL and overlapping working-set buffers are rejected before any launch."""
    d = _dims()
    assert lib.oasis_window_ring_slots(ctypes.byref(d)) == lib.oasis_table_stride(ctypes.byref(d)) - 16
    assert lib.oasis_window_ring_slots(ctypes.byref(_dims(window_tokens=0))) == 1
    assert lib.oasis_window_ring_slots(ctypes.byref(_dims(batch=0))) == -1
    blk = 16 * 128 * 2
    full = 2 * 2 * 64 * blk
    k, v = 0x100000, 0x100000 + full
    pk, pv = 0x10000000, 0x10000000 + 2 * 2 * 16 * blk
    rk, rv = 0x20000000, 0x20000000 + 2 * 2 * 5 * blk
    P = ctypes.c_void_p

    def fill(*ptrs):
        return lib.oasis_fill_working_set(ctypes.byref(d), FAKE, FAKE, *[P(x) if x else None for x in ptrs], None)

    assert fill(k, v, pk, pv, rk, None) == INVALID_ARG and b"NULL" in lib.oasis_last_error()
    assert fill(k, k + 64, pk, pv, rk, rv) == INVALID_ARG and b"overlap" in lib.oasis_last_error()
    assert fill(k, v, pk, pk + blk, rk, rv) == INVALID_ARG                       # pool_k / pool_v
    assert fill(k, v, pk, pv, pv + 64, rv) == INVALID_ARG                        # pool_v / ring_k
    d4 = _dims(fetch_ratio=0.25)
    assert lib.oasis_execute_plan(ctypes.byref(d4), None, FAKE, P(k), P(v), P(pk), P(pv), None) \
        == INVALID_ARG                                                           # cap 4: plan needed
    d0 = _dims(fetch_ratio=0.01)
    assert lib.oasis_execute_plan(ctypes.byref(d0), None, None, P(k), P(v), P(pk), P(pv), None) \
        == INVALID_ARG                                                           # plan_count needed
    assert lib.oasis_append_token(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, P(k), None, P(rk), P(rv),
                                  None) == INVALID_ARG                            # k without v
    need = lib.oasis_workspace_bytes(ctypes.byref(d))
    attn_need = lib.oasis_attn_workspace_bytes(ctypes.byref(d), lib.oasis_table_stride(ctypes.byref(d)))
    assert lib.oasis_sparse_decode_attn_pool(ctypes.byref(d), FAKE, P(pk), P(pv), P(rk), P(rv), FAKE,
                                             FAKE, 0.1, FAKE, None, FAKE, attn_need - 1, None) == WORKSPACE
    st = lib.oasis_decode_step_pool(ctypes.byref(d), FAKE, FAKE, P(k), P(v), P(pk), P(pv), P(rk),
                                    P(rv), FAKE, FAKE, FAKE, P(0x30000000), P(0x30000000), FAKE, FAKE,
                                    FAKE, FAKE, 0.1, FAKE, None, FAKE, need, None)
    assert st == INVALID_ARG and b"own buffer" in lib.oasis_last_error()


@cpu_only
def test_layer_pipelined_argument_checks(lib):
    """Both layers NULL, a shared scores buffer, an overlapping next slot table or a
    small workspace are rejected before anything is queued."""
    from oasis_score_summaries_amd import LayerIO
    d = _dims()
    need = lib.oasis_workspace_bytes(ctypes.byref(d))

    def io(base, ws_bytes=need):
        x = LayerIO(*[base + 0x100000 * i for i in range(16)], ws_bytes)
        return x

    a, b = io(0x10000000), io(0x30000000)
    call = lambda l, p: lib.oasis_decode_layer_pipelined(ctypes.byref(d), l, p, 0.1, None)
    assert call(None, None) == INVALID_ARG
    assert call(ctypes.byref(io(0x10000000, need - 1)), None) == WORKSPACE
    shared = io(0x30000000)
    shared.scores = a.scores
    assert call(ctypes.byref(a), ctypes.byref(shared)) == INVALID_ARG
    assert b"share scores" in lib.oasis_last_error()
    bad = io(0x30000000)
    bad.resident_next = bad.resident + 16
    assert call(ctypes.byref(a), ctypes.byref(bad)) == INVALID_ARG
    clash = io(0x30000000)
    clash.resident_next = a.resident
    assert call(ctypes.byref(a), ctypes.byref(clash)) == INVALID_ARG
    assert b"overlaps" in lib.oasis_last_error()
