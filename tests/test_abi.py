"""The C ABI without a GPU: the library loads, exports what include/qsa.h declares,
and every validation error returns before anything touches a device."""
import ctypes
import subprocess

import numpy as np
import pytest

import long_context_block_qsa_amd as qsa

FAKE = 0x100000  # never dereferenced: every call below fails validation first


def _seqs(cu_q, cu_k, batch=None, dev=True):
    cq = np.ascontiguousarray(np.asarray(cu_q, dtype=np.int32))
    ck = np.ascontiguousarray(np.asarray(cu_k, dtype=np.int32))
    s = qsa.qsa_seqs(len(ck) - 1 if batch is None else batch, cq.ctypes.data, ck.ctypes.data,
                     FAKE if dev else None, FAKE if dev else None)
    s._keep = (cq, ck)
    return s


def _ws(dims, seqs):
    n = ctypes.c_size_t(0)
    st = qsa.lib().qsa_workspace_size(ctypes.byref(dims), ctypes.byref(seqs), ctypes.byref(n))
    return st, n.value


def test_exports_every_declared_symbol():
    names = qsa.header_functions()
    assert set(names) == {"qsa_abi_version", "qsa_status_string", "qsa_workspace_size",
                          "qsa_compress", "qsa_select", "qsa_score", "qsa_attend",
                          "qsa_forward", "qsa_forward_noalloc",
                          "qsa_quantize_kv", "qsa_attend_fp8", "qsa_forward_fp8",
                          "qsa_backward_workspace_size", "qsa_attend_backward",
                          "qsa_trace_begin", "qsa_trace_end", "qsa_kernel_name"}
    out = subprocess.run(["nm", "-D", "--defined-only", qsa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(names) <= exported
    for n in names:
        assert hasattr(qsa.lib(), n)


def test_version_and_status_strings():
    assert qsa.lib().qsa_abi_version() == 1
    for s in range(6):
        assert qsa.status_string(s).startswith(("QSA_OK", "QSA_ERR"))
    assert "unknown" in qsa.status_string(99)


@pytest.mark.parametrize("field,value,expect", [
    ("n_q_heads", 32, qsa.QSA_ERR_UNSUPPORTED), ("n_kv_heads", 4, qsa.QSA_ERR_UNSUPPORTED),
    ("head_dim", 64, qsa.QSA_ERR_UNSUPPORTED), ("n_idx_heads", 8, qsa.QSA_ERR_UNSUPPORTED),
    ("idx_dim", 128, qsa.QSA_ERR_UNSUPPORTED), ("block_size", 8, qsa.QSA_ERR_UNSUPPORTED),
    ("topk_blocks", 0, qsa.QSA_ERR_SHAPE), ("topk_blocks", 513, qsa.QSA_ERR_SHAPE),
    ("softmax_scale", float("nan"), qsa.QSA_ERR_SHAPE),
])
def test_dims_rejected(field, value, expect):
    d = qsa.make_dims()
    setattr(d, field, value)
    s = _seqs([0, 1], [0, 10])
    assert _ws(d, s)[0] == expect


@pytest.mark.parametrize("cu_q,cu_k,expect", [
    ([1, 2], [0, 10], qsa.QSA_ERR_SHAPE),            # cu_q not starting at 0
    ([0, 1], [2, 10], qsa.QSA_ERR_SHAPE),            # cu_k not starting at 0
    ([0, 11], [0, 10], qsa.QSA_ERR_SHAPE),           # more queries than tokens
    ([0, 1, 0], [0, 5, 9], qsa.QSA_ERR_SHAPE),       # decreasing cu_q
    ([0, 1, 2], [0, 5, 4], qsa.QSA_ERR_SHAPE),       # decreasing cu_k
])
def test_bad_offsets_rejected(cu_q, cu_k, expect):
    assert _ws(qsa.make_dims(), _seqs(cu_q, cu_k))[0] == expect


def test_null_pointers_rejected():
    d = qsa.make_dims()
    n = ctypes.c_size_t(0)
    L = qsa.lib()
    assert L.qsa_workspace_size(None, ctypes.byref(_seqs([0, 1], [0, 4])), ctypes.byref(n)) == 1
    assert L.qsa_workspace_size(ctypes.byref(d), None, ctypes.byref(n)) == 1
    assert L.qsa_workspace_size(ctypes.byref(d), ctypes.byref(_seqs([0, 1], [0, 4])), None) == 1
    no_dev = _seqs([0, 1], [0, 4], dev=False)
    assert L.qsa_workspace_size(ctypes.byref(d), ctypes.byref(no_dev), ctypes.byref(n)) == 1
    s = _seqs([0, 1], [0, 40])
    st, nbytes = _ws(d, s)
    assert st == 0
    f = ctypes.c_void_p(FAKE)
    # forward: missing q / out / workspace
    assert L.qsa_forward(ctypes.byref(d), ctypes.byref(s), None, f, f, f, f, f, f, f, f, f, f,
                         nbytes, None) == qsa.QSA_ERR_NULL
    assert L.qsa_forward(ctypes.byref(d), ctypes.byref(s), f, f, f, f, f, f, f, f, None, f, f,
                         nbytes, None) == qsa.QSA_ERR_NULL
    assert L.qsa_forward(ctypes.byref(d), ctypes.byref(s), f, f, f, f, f, f, f, f, f, f, None,
                         nbytes, None) == qsa.QSA_ERR_NULL
    assert L.qsa_attend(ctypes.byref(d), ctypes.byref(s), f, f, f, None, f, f, f, nbytes,
                        None) == qsa.QSA_ERR_NULL
    assert L.qsa_select(ctypes.byref(d), ctypes.byref(s), f, f, f, None, f, nbytes,
                        None) == qsa.QSA_ERR_NULL
    assert L.qsa_compress(ctypes.byref(d), ctypes.byref(s), None, f, None) == qsa.QSA_ERR_NULL


def test_fp8_entry_points_validate_first():
    """FP8 entry points reject missing or misaligned operands before any device call."""
    d = qsa.make_dims()
    L = qsa.lib()
    s = _seqs([0, 1], [0, 40])
    st, nbytes = _ws(d, s)
    assert st == 0
    f = ctypes.c_void_p(FAKE)
    odd = ctypes.c_void_p(FAKE + 4)
    assert L.qsa_quantize_kv(ctypes.byref(d), ctypes.byref(s), f, f, None, f, f, f,
                             None) == qsa.QSA_ERR_NULL
    assert L.qsa_quantize_kv(ctypes.byref(d), ctypes.byref(s), f, f, f, f, odd, f,
                             None) == qsa.QSA_ERR_SHAPE
    assert L.qsa_attend_fp8(ctypes.byref(d), ctypes.byref(s), f, f, f, None, f, f, f, f, f,
                            nbytes, None) == qsa.QSA_ERR_NULL
    assert L.qsa_attend_fp8(ctypes.byref(d), ctypes.byref(s), f, odd, f, f, f, f, f, f, f,
                            nbytes, None) == qsa.QSA_ERR_SHAPE
    assert L.qsa_forward_fp8(ctypes.byref(d), ctypes.byref(s), f, f, None, f, f, f, f, f, f,
                             f, f, f, f, nbytes, None) == qsa.QSA_ERR_NULL
    assert L.qsa_forward_fp8(ctypes.byref(d), ctypes.byref(s), f, f, f, f, f, f, f, f, f,
                             f, f, f, f, nbytes - 1, None) == qsa.QSA_ERR_WORKSPACE


def _bws(dims, seqs):
    n = ctypes.c_size_t(0)
    st = qsa.lib().qsa_backward_workspace_size(ctypes.byref(dims), ctypes.byref(seqs),
                                               ctypes.byref(n))
    return st, n.value


def test_backward_entry_point_validates_first():
    """qsa_attend_backward rejects missing, misaligned or undersized operands before any
    device call; its workspace covers the block -> rows lists."""
    d = qsa.make_dims()
    L = qsa.lib()
    s = _seqs([0, 40], [0, 40])
    st, nbytes = _bws(d, s)
    assert st == 0
    assert nbytes >= 4 * 40 * (512 + 1)
    f = ctypes.c_void_p(FAKE)
    odd = ctypes.c_void_p(FAKE + 4)
    args = [f] * 10   # q k v sel out lse dout dq dk dv
    def call(a, ws=f, n=nbytes):
        return L.qsa_attend_backward(ctypes.byref(d), ctypes.byref(s), *a, ws, n, None)
    for i in range(10):
        a = list(args)
        a[i] = None
        assert call(a) == qsa.QSA_ERR_NULL, i
        a[i] = odd
        assert call(a) == qsa.QSA_ERR_SHAPE, i
    assert call(args, ws=None) == qsa.QSA_ERR_NULL
    assert call(args, n=nbytes - 1) == qsa.QSA_ERR_WORKSPACE
    assert call(args, ws=ctypes.c_void_p(FAKE + 16)) == qsa.QSA_ERR_WORKSPACE
    # totals beyond int32 list positions are refused
    big = _seqs([0, 2**22 + 8], [0, 2**22 + 8])
    assert _bws(d, big)[0] == qsa.QSA_ERR_UNSUPPORTED
    # dims are validated as in the forward
    d2 = qsa.make_dims()
    d2.head_dim = 64
    assert _bws(d2, s)[0] == qsa.QSA_ERR_UNSUPPORTED


def test_backward_workspace_grows_with_rows_and_budget():
    d = qsa.make_dims(topk=512)
    a = _bws(d, _seqs([0, 1000], [0, 1000]))[1]
    b = _bws(d, _seqs([0, 4000], [0, 4000]))[1]
    c = _bws(qsa.make_dims(topk=16), _seqs([0, 4000], [0, 4000]))[1]
    assert b > a and b > c


def test_workspace_checks():
    d = qsa.make_dims()
    s = _seqs([0, 40000], [0, 40000])
    L = qsa.lib()
    st, nbytes = _ws(d, s)
    assert st == 0 and nbytes > 0
    f = ctypes.c_void_p(FAKE)
    assert L.qsa_select(ctypes.byref(d), ctypes.byref(s), f, f, f, f, f, nbytes - 1,
                        None) == qsa.QSA_ERR_WORKSPACE
    assert L.qsa_select(ctypes.byref(d), ctypes.byref(s), f, f, f, f,
                        ctypes.c_void_p(FAKE + 16), nbytes, None) == qsa.QSA_ERR_WORKSPACE
    assert L.qsa_attend(ctypes.byref(d), ctypes.byref(s), f, f, f, f, f, f, None, nbytes,
                        None) == qsa.QSA_ERR_NULL


def test_misaligned_tensor_rejected():
    d = qsa.make_dims()
    s = _seqs([0, 1], [0, 40])
    st, nbytes = _ws(d, s)
    f, g = ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE + 2)
    assert qsa.lib().qsa_attend(ctypes.byref(d), ctypes.byref(s), g, f, f, f, f, f, f, nbytes,
                                None) == qsa.QSA_ERR_SHAPE


def test_empty_work_is_a_no_op():
    """batch 0, or sequences with no query rows: success, nothing enqueued."""
    d = qsa.make_dims()
    L = qsa.lib()
    for cu_q, cu_k in (([0], [0]), ([0, 0, 0], [0, 0, 7])):
        s = _seqs(cu_q, cu_k)
        st, nbytes = _ws(d, s)
        assert st == 0
        assert L.qsa_forward(ctypes.byref(d), ctypes.byref(s), None, None, None, None, None,
                             None, None, None, None, None, None, 0, None) == 0


def test_workspace_size_grows_with_scored_rows():
    """Rows within the budget need no score slots; longer prefills need more."""
    d = qsa.make_dims(topk=512)
    small = _ws(d, _seqs([0, 2051], [0, 2051]))[1]
    large = _ws(d, _seqs([0, 4096], [0, 4096]))[1]
    assert large > small
    # scores of a 4096-token prefill: positions 2051..4095, F(4096) - F(2051) slots
    F = lambda t: 2 * (t // 4) * (t // 4 - 1) + (t // 4) * (t % 4 + 1)
    assert large >= 4 * (F(4096) - F(2051))


def test_trace_end_without_begin_and_names():
    L = qsa.lib()
    assert L.qsa_trace_end(0, None, None) == -1
    assert qsa.lib().qsa_kernel_name(2) == b"score"
    assert qsa.lib().qsa_kernel_name(12) == b"bwd_dq"
    assert qsa.lib().qsa_kernel_name(13) == b"bwd_dkv"
    assert qsa.lib().qsa_kernel_name(14) == b"score_select"
    assert qsa.lib().qsa_kernel_name(42) == b"unknown"
    assert L.qsa_trace_begin(0) == qsa.QSA_ERR_SHAPE


def test_prefill_workspace_bounded_by_key_budget():
    """Prefill scores are kept one pass of score tiles at a time (at most 2^26 keys of
    4 bytes, in two alternating buffers), so the workspace of a 262,144-token or a
    1,048,576-token prefill is the selection (4 * 512 bytes per query row, linear in the
    length) plus at most 512 MiB of keys, while the sum of its score slots
    (F(L) - F(2051)) would be 34 GB and 550 GB."""
    d = qsa.make_dims(topk=512)
    F = lambda t: 2 * (t // 4) * (t // 4 - 1) + (t // 4) * (t % 4 + 1)
    for L in (65535, 262144, 1 << 20):
        st, n = _ws(d, _seqs([0, L], [0, L]))
        assert st == 0
        assert n <= 4 * 512 * L + 8 * 2**26 + 2**20, (L, n)
        if L >= 262144:
            assert 4 * (F(L) - F(2051)) > 30 * n
    # a call whose keys fit one pass keeps all of them (as before)
    st, n = _ws(d, _seqs([0, 4096], [0, 4096]))
    assert n >= 4 * (F(4096) - F(2051))


def test_score_entry_point_validates_first():
    """qsa_score: ld below the longest sequence's block count, no query rows, null or
    misaligned operands are refused before any device call."""
    d = qsa.make_dims()
    L = qsa.lib()
    s = _seqs([0, 3], [0, 4001])            # 1000 complete blocks
    f, odd = ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE + 2)
    call = lambda qi, w, kb, rows, n, sc, ld: L.qsa_score(ctypes.byref(d), ctypes.byref(s), qi,
                                                           w, kb, rows, n, sc, ld, None)
    assert call(f, f, f, f, 3, f, 999) == qsa.QSA_ERR_SHAPE
    assert call(f, f, f, f, -1, f, 1000) == qsa.QSA_ERR_SHAPE
    assert call(f, f, f, None, 3, f, 1000) == qsa.QSA_ERR_NULL
    assert call(f, f, f, f, 3, None, 1000) == qsa.QSA_ERR_NULL
    assert call(f, None, f, f, 3, f, 1000) == qsa.QSA_ERR_NULL
    assert call(odd, f, f, f, 3, f, 1000) == qsa.QSA_ERR_SHAPE
    assert call(None, None, None, None, 0, None, 0) == qsa.QSA_OK
    empty = _seqs([0, 0], [0, 50])
    assert L.qsa_score(ctypes.byref(d), ctypes.byref(empty), f, f, f, f, 1, f, 100,
                       None) == qsa.QSA_ERR_SHAPE


def test_noalloc_entry_point_validates_first():
    """qsa_forward_noalloc refuses, before any device call, a call whose workspace would
    exceed its scratch (QSA_ERR_WORKSPACE) and invalid arguments as qsa_forward does."""
    d = qsa.make_dims()
    L = qsa.lib()
    f = ctypes.c_void_p(FAKE)
    big = _seqs([0, 65535], [0, 65535])
    assert _ws(d, big)[1] > qsa.NOALLOC_SCRATCH_BYTES
    assert L.qsa_forward_noalloc(ctypes.byref(d), ctypes.byref(big), f, f, f, f, f, f, f, f, f,
                                 f, None) == qsa.QSA_ERR_WORKSPACE
    small = _seqs([0, 1], [0, 40])
    assert L.qsa_forward_noalloc(ctypes.byref(d), ctypes.byref(small), None, f, f, f, f, f, f,
                                 f, f, f, None) == qsa.QSA_ERR_NULL
    bad = qsa.make_dims()
    bad.head_dim = 64
    assert L.qsa_forward_noalloc(ctypes.byref(bad), ctypes.byref(small), f, f, f, f, f, f, f,
                                 f, f, f, None) == qsa.QSA_ERR_UNSUPPORTED


def test_attention_length_limit():
    """Attention calls address a sequence's K and V with 32-bit byte offsets: sequences over
    4,194,304 tokens are refused (QSA_ERR_UNSUPPORTED) before any device call; scoring and
    compression are not limited."""
    d = qsa.make_dims()
    L = qsa.lib()
    f = ctypes.c_void_p(FAKE)
    n = 4194304
    ok = _seqs([0, 1], [0, n])
    big = _seqs([0, 1], [0, n + 1])
    st, nbytes = _ws(d, big)
    assert st == 0
    for s, expect in ((big, qsa.QSA_ERR_UNSUPPORTED), (ok, qsa.QSA_ERR_WORKSPACE)):
        assert L.qsa_attend(ctypes.byref(d), ctypes.byref(s), f, f, f, f, f, f, f, 0,
                            None) == expect
        assert L.qsa_forward(ctypes.byref(d), ctypes.byref(s), f, f, f, f, f, f, f, f, f, f, f,
                             0, None) == expect
    assert L.qsa_forward_noalloc(ctypes.byref(d), ctypes.byref(big), f, f, f, f, f, f, f, f, f,
                                 f, None) == qsa.QSA_ERR_UNSUPPORTED
