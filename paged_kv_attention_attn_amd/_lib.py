"""ctypes binding of libpkv.so: the C ABI of include/pkv.h under the same
names. Argument marshalling only -- every step of the computation runs in the
library's HIP kernels. torch supplies device memory and the stream.

The library is loaded after torch so that it binds to the HIP runtime torch
already loaded. There is no fallback: if the library is missing, importing
the binding raises.
"""

import ctypes
import os

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpkv.so")

PKV_PAGE_SIZE = 256
PKV_MAX_Q_LEN = 16
PKV_MAX_ROWS = 64
PKV_OK, PKV_ERR_NULL, PKV_ERR_SHAPE, PKV_ERR_WORKSPACE, PKV_ERR_HIP = 0, -1, -2, -3, -4
PKV_ERR_SPACE, PKV_ERR_STATE, PKV_ERR_SCRATCH = -5, -6, -7
PKV_ACCEPT_SCRATCH_BYTES = 1 << 20
PKV_EFLAG_PAGE, PKV_EFLAG_QLEN, PKV_EFLAG_ROWS, PKV_EFLAG_SPACE = 1, 2, 4, 8

EXPORTS = ("pkv_attn_workspace_bytes", "pkv_attn_workspace_init", "pkv_attn_fwd",
           "pkv_attn_check_errors", "pkv_accept_workspace_bytes", "pkv_accept", "pkv_accept_noalloc",
           "pkv_window_next", "pkv_status_string", "pkv_version", "pkv_kv_workspace_bytes",
           "pkv_kv_append", "pkv_kv_rollback", "pkv_kv_check_errors", "pkv_pool_create",
           "pkv_pool_destroy", "pkv_pool_stats", "pkv_pool_admit", "pkv_pool_alloc", "pkv_pool_retain",
           "pkv_pool_release", "pkv_pool_defrag", "pkv_pool_copy_pages", "pkv_table_remap",
           "pkv_attn_shared_workspace_bytes", "pkv_attn_fwd_shared", "pkv_attn_plan", "pkv_shared_prefix_pages",
           "pkv_q8_encode", "pkv_attn_fwd_q8", "pkv_q4_encode", "pkv_attn_fwd_q4", "pkv_kv_append_q8",
           "pkv_kv_append_q4", "pkv_pool_copy_page_bytes")


class pkv_attn_shape(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32), ("total_q", ctypes.c_int32),
                ("max_q_len", ctypes.c_int32), ("scale", ctypes.c_float),
                ("total_pages", ctypes.c_int32), ("pages_per_split", ctypes.c_int32)]


class pkv_accept_shape(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("total_rows", ctypes.c_int32), ("max_draft", ctypes.c_int32)]


class pkv_kv_shape(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
                ("total_q", ctypes.c_int32)]


class PkvError(RuntimeError):
    pass


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python paged_kv_attention_attn_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32p = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p
    lib.pkv_attn_workspace_bytes.argtypes = [ctypes.POINTER(pkv_attn_shape)]
    lib.pkv_attn_workspace_bytes.restype = sz
    lib.pkv_shared_prefix_pages.argtypes = [vp, vp, vp, ctypes.POINTER(pkv_attn_shape)]
    lib.pkv_shared_prefix_pages.restype = ctypes.c_int32
    lib.pkv_attn_plan.argtypes = [ctypes.POINTER(pkv_attn_shape), vp]
    lib.pkv_attn_plan.restype = ctypes.c_int
    lib.pkv_attn_workspace_init.argtypes = [vp, sz, vp]
    lib.pkv_attn_workspace_init.restype = ctypes.c_int
    lib.pkv_attn_fwd.argtypes = [vp, vp, vp, i32p, i32p, i32p, vp, ctypes.POINTER(pkv_attn_shape),
                                 vp, sz, vp]
    lib.pkv_attn_fwd.restype = ctypes.c_int
    lib.pkv_attn_fwd_q8.argtypes = [vp] * 9 + [ctypes.POINTER(pkv_attn_shape), vp, sz, vp]
    lib.pkv_attn_fwd_q8.restype = ctypes.c_int
    lib.pkv_q8_encode.argtypes = [vp, vp, vp, ctypes.c_int64, ctypes.c_int32, vp]
    lib.pkv_q8_encode.restype = ctypes.c_int
    for name in ("pkv_kv_append_q8", "pkv_kv_append_q4"):
        getattr(lib, name).argtypes = [vp] * 11 + [ctypes.POINTER(pkv_kv_shape), vp, sz, vp]
        getattr(lib, name).restype = ctypes.c_int
    lib.pkv_attn_fwd_q4.argtypes = [vp] * 9 + [ctypes.POINTER(pkv_attn_shape), vp, sz, vp]
    lib.pkv_attn_fwd_q4.restype = ctypes.c_int
    lib.pkv_q4_encode.argtypes = [vp, vp, vp, ctypes.c_int64, ctypes.c_int32, vp]
    lib.pkv_q4_encode.restype = ctypes.c_int
    lib.pkv_attn_shared_workspace_bytes.argtypes = [ctypes.POINTER(pkv_attn_shape), ctypes.c_int32]
    lib.pkv_attn_shared_workspace_bytes.restype = sz
    lib.pkv_attn_fwd_shared.argtypes = [vp, vp, vp, i32p, i32p, i32p, vp, ctypes.POINTER(pkv_attn_shape),
                                        ctypes.c_int32, vp, sz, vp]
    lib.pkv_attn_fwd_shared.restype = ctypes.c_int
    lib.pkv_attn_check_errors.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_uint32)]
    lib.pkv_attn_check_errors.restype = ctypes.c_int
    lib.pkv_accept_workspace_bytes.argtypes = [ctypes.POINTER(pkv_accept_shape)]
    lib.pkv_accept_workspace_bytes.restype = sz
    lib.pkv_accept.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.POINTER(pkv_accept_shape), vp, sz, vp]
    lib.pkv_accept.restype = ctypes.c_int
    lib.pkv_accept_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.POINTER(pkv_accept_shape), vp]
    lib.pkv_accept_noalloc.restype = ctypes.c_int
    lib.pkv_window_next.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
    lib.pkv_window_next.restype = ctypes.c_int32
    lib.pkv_status_string.argtypes = [ctypes.c_int]
    lib.pkv_status_string.restype = ctypes.c_char_p
    lib.pkv_version.argtypes = []
    lib.pkv_version.restype = ctypes.c_int
    lib.pkv_kv_workspace_bytes.argtypes = [ctypes.POINTER(pkv_kv_shape)]
    lib.pkv_kv_workspace_bytes.restype = sz
    lib.pkv_kv_append.argtypes = [vp] * 9 + [ctypes.POINTER(pkv_kv_shape), vp, sz, vp]
    lib.pkv_kv_append.restype = ctypes.c_int
    lib.pkv_kv_rollback.argtypes = [vp] * 6 + [ctypes.POINTER(pkv_kv_shape), vp, sz, vp]
    lib.pkv_kv_rollback.restype = ctypes.c_int
    lib.pkv_kv_check_errors.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_uint32)]
    lib.pkv_kv_check_errors.restype = ctypes.c_int
    i32 = ctypes.c_int32
    lib.pkv_pool_create.argtypes = [i32]
    lib.pkv_pool_create.restype = vp
    lib.pkv_pool_destroy.argtypes = [vp]
    lib.pkv_pool_destroy.restype = None
    lib.pkv_pool_stats.argtypes = [vp, vp]
    lib.pkv_pool_admit.argtypes = [vp, vp, i32, vp, i32, vp, vp]
    lib.pkv_pool_alloc.argtypes = [vp, i32, vp]
    lib.pkv_pool_retain.argtypes = [vp, vp, i32]
    lib.pkv_pool_release.argtypes = [vp, vp, i32]
    lib.pkv_pool_defrag.argtypes = [vp, i32, vp, vp, vp, vp]
    lib.pkv_pool_copy_pages.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, vp, vp]
    lib.pkv_table_remap.argtypes = [vp, i32, i32, vp, i32, vp, vp]
    lib.pkv_pool_copy_page_bytes.argtypes = [vp, vp, vp, vp, i32, i32, ctypes.c_int64, vp, vp]
    lib.pkv_pool_copy_page_bytes.restype = ctypes.c_int
    for name in ("pkv_pool_stats", "pkv_pool_admit", "pkv_pool_alloc", "pkv_pool_retain", "pkv_pool_release",
                 "pkv_pool_defrag", "pkv_pool_copy_pages", "pkv_table_remap"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


LIB = _load()


def _ptr(t):
    # a plain int: ctypes converts it for a c_void_p argument
    return None if t is None else t.data_ptr()


# the current device's current stream as a raw handle, without building a
# torch Stream object on every call (these run once per launch)
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_get_device = getattr(torch._C, "_cuda_getDevice", None)


def _stream(stream):
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None and _get_device is not None:
        return _raw_stream(_get_device())
    return torch.cuda.current_stream().cuda_stream


def _check(rc, what):
    if rc != PKV_OK:
        raise PkvError(f"{what}: {LIB.pkv_status_string(rc).decode()} ({rc})")


def _extents(name_call, *checks):
    """Each check is (tensor, element count the shape implies, name): the
    kernels index the buffers by the shape, so a tensor of another size is
    refused here, before any launch."""
    for t, n, name in checks:
        if t is not None and t.numel() != n:
            raise ValueError(f"{name_call}: {name} has {t.numel()} elements, the shape implies {n}")


def _attn_extents(call, shape, q, k_pool, v_pool, block_table, seq_lens, q_lens, out):
    s = shape
    qn = s.total_q * s.num_q_heads * s.head_dim
    pool = s.num_pages * s.num_kv_heads * s.page_size * s.head_dim
    _extents(call, (q, qn, "q"), (out, qn, "out"), (k_pool, pool, "k_pool"), (v_pool, pool, "v_pool"),
             (block_table, s.num_seqs * s.max_pages_per_seq, "block_table"), (seq_lens, s.num_seqs, "seq_lens"),
             (q_lens, s.num_seqs, "q_lens"))


def _need(t, dtype, name):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")


def attn_shape(q, k_pool, block_table, max_q_len, scale, total_pages=0):
    """pkv_attn_shape from tensor extents (q [total_q, Hq, D], pool [P, Hkv, 256, D],
    block_table [B, W]); total_pages is the host's count of referenced pages
    (sum of ceil(seq_len / 256)), a planning hint, 0 if unknown."""
    total_q, Hq, D = q.shape
    P, Hkv, page, D2 = k_pool.shape
    B, W = block_table.shape
    if D2 != D and not (k_pool.dtype == torch.uint8 and 2 * D2 == D):   # Q4 pools hold D / 2 bytes
        raise ValueError("q and pool head_dim differ")
    return pkv_attn_shape(B, Hq, Hkv, D, page, P, W, total_q, int(max_q_len), float(scale), int(total_pages), 0)


def pkv_attn_plan(shape, seq_lens_host):
    """Set shape.total_pages and shape.pages_per_split from host-side lengths
    (any int sequence or numpy array); returns the shape."""
    lens = np.ascontiguousarray(seq_lens_host, dtype=np.int32)
    if lens.size != shape.num_seqs:
        raise ValueError(f"pkv_attn_plan: {lens.size} lengths for {shape.num_seqs} sequences")
    _check(LIB.pkv_attn_plan(ctypes.byref(shape), lens.ctypes.data_as(ctypes.c_void_p)), "pkv_attn_plan")
    return shape


def pkv_attn_workspace_bytes(shape):
    return int(LIB.pkv_attn_workspace_bytes(ctypes.byref(shape)))


def pkv_attn_workspace_init(workspace, stream=None):
    _check(LIB.pkv_attn_workspace_init(_ptr(workspace), workspace.numel(), _stream(stream)),
           "pkv_attn_workspace_init")


def new_attn_workspace(shape, device="cuda"):
    n = pkv_attn_workspace_bytes(shape)
    if n == 0:
        raise PkvError("pkv_attn_workspace_bytes: shape rejected")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def pkv_attn_fwd(q, k_pool, v_pool, block_table, seq_lens, q_lens, out, shape, workspace, stream=None):
    """q, k_pool, v_pool: bf16; block_table, seq_lens, q_lens: int32; out: fp32."""
    _attn_extents("pkv_attn_fwd", shape, q, k_pool, v_pool, block_table, seq_lens, q_lens, out)
    for t, dt, n in ((q, torch.bfloat16, "q"), (k_pool, torch.bfloat16, "k_pool"),
                     (v_pool, torch.bfloat16, "v_pool"), (block_table, torch.int32, "block_table"),
                     (seq_lens, torch.int32, "seq_lens"), (q_lens, torch.int32, "q_lens"),
                     (out, torch.float32, "out"), (workspace, torch.uint8, "workspace")):
        _need(t, dt, n)
    rc = LIB.pkv_attn_fwd(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(seq_lens),
                          _ptr(q_lens), _ptr(out), ctypes.byref(shape), _ptr(workspace),
                          workspace.numel(), _stream(stream))
    _check(rc, "pkv_attn_fwd")


def pkv_q8_encode(src, codes, scales, stream=None):
    """bf16 vectors src [..., D] -> int8 codes [..., D] and fp32 scales [...] (the Q8 cache format)."""
    for t, dt, n in ((src, torch.bfloat16, "src"), (codes, torch.int8, "codes"), (scales, torch.float32, "scales")):
        _need(t, dt, n)
    D = src.shape[-1] if src.dim() else 0
    rows = src.numel() // D if D else 0
    _extents("pkv_q8_encode", (codes, rows * D, "codes"), (scales, rows, "scales"))
    rc = LIB.pkv_q8_encode(_ptr(src), _ptr(codes), _ptr(scales), rows, D, _stream(stream))
    _check(rc, "pkv_q8_encode")


def pkv_attn_fwd_q8(q, k_codes, k_scales, v_codes, v_scales, block_table, seq_lens, q_lens, out, shape, workspace,
                    stream=None):
    """pkv_attn_fwd over a Q8 cache: codes int8 [P, Hkv, 256, D], scales fp32 [P, Hkv, 256]."""
    s = shape
    _attn_extents("pkv_attn_fwd_q8", shape, q, k_codes, v_codes, block_table, seq_lens, q_lens, out)
    ns = s.num_pages * s.num_kv_heads * s.page_size
    _extents("pkv_attn_fwd_q8", (k_scales, ns, "k_scales"), (v_scales, ns, "v_scales"))
    for t, dt, n in ((q, torch.bfloat16, "q"), (k_codes, torch.int8, "k_codes"), (k_scales, torch.float32, "k_scales"),
                     (v_codes, torch.int8, "v_codes"), (v_scales, torch.float32, "v_scales"),
                     (block_table, torch.int32, "block_table"), (seq_lens, torch.int32, "seq_lens"),
                     (q_lens, torch.int32, "q_lens"), (out, torch.float32, "out"),
                     (workspace, torch.uint8, "workspace")):
        _need(t, dt, n)
    rc = LIB.pkv_attn_fwd_q8(_ptr(q), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes), _ptr(v_scales),
                             _ptr(block_table), _ptr(seq_lens), _ptr(q_lens), _ptr(out), ctypes.byref(shape),
                             _ptr(workspace), workspace.numel(), _stream(stream))
    _check(rc, "pkv_attn_fwd_q8")


def pkv_q4_encode(src, codes, scales, stream=None):
    """bf16 vectors src [..., D] -> packed uint8 codes [..., D / 2] and fp32 scales [...] (the Q4 format)."""
    for t, dt, n in ((src, torch.bfloat16, "src"), (codes, torch.uint8, "codes"), (scales, torch.float32, "scales")):
        _need(t, dt, n)
    D = src.shape[-1] if src.dim() else 0
    rows = src.numel() // D if D else 0
    _extents("pkv_q4_encode", (codes, rows * D // 2, "codes"), (scales, rows, "scales"))
    rc = LIB.pkv_q4_encode(_ptr(src), _ptr(codes), _ptr(scales), rows, D, _stream(stream))
    _check(rc, "pkv_q4_encode")


def pkv_attn_fwd_q4(q, k_codes, k_scales, v_codes, v_scales, block_table, seq_lens, q_lens, out, shape, workspace,
                    stream=None):
    """pkv_attn_fwd over a Q4 cache: codes uint8 [P, Hkv, 256, D / 2], scales fp32 [P, Hkv, 256]."""
    s = shape
    qn = s.total_q * s.num_q_heads * s.head_dim
    ns = s.num_pages * s.num_kv_heads * s.page_size
    _extents("pkv_attn_fwd_q4", (q, qn, "q"), (out, qn, "out"), (k_codes, ns * s.head_dim // 2, "k_codes"),
             (v_codes, ns * s.head_dim // 2, "v_codes"), (k_scales, ns, "k_scales"), (v_scales, ns, "v_scales"),
             (block_table, s.num_seqs * s.max_pages_per_seq, "block_table"), (seq_lens, s.num_seqs, "seq_lens"),
             (q_lens, s.num_seqs, "q_lens"))
    for t, dt, n in ((q, torch.bfloat16, "q"), (k_codes, torch.uint8, "k_codes"), (k_scales, torch.float32, "k_scales"),
                     (v_codes, torch.uint8, "v_codes"), (v_scales, torch.float32, "v_scales"),
                     (block_table, torch.int32, "block_table"), (seq_lens, torch.int32, "seq_lens"),
                     (q_lens, torch.int32, "q_lens"), (out, torch.float32, "out"),
                     (workspace, torch.uint8, "workspace")):
        _need(t, dt, n)
    rc = LIB.pkv_attn_fwd_q4(_ptr(q), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes), _ptr(v_scales),
                             _ptr(block_table), _ptr(seq_lens), _ptr(q_lens), _ptr(out), ctypes.byref(shape),
                             _ptr(workspace), workspace.numel(), _stream(stream))
    _check(rc, "pkv_attn_fwd_q4")


def pkv_attn_shared_workspace_bytes(shape, shared_pages):
    return int(LIB.pkv_attn_shared_workspace_bytes(ctypes.byref(shape), int(shared_pages)))


def new_attn_shared_workspace(shape, shared_pages, device="cuda"):
    n = pkv_attn_shared_workspace_bytes(shape, shared_pages)
    if n == 0:
        raise PkvError("pkv_attn_shared_workspace_bytes: shape rejected")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def pkv_attn_fwd_shared(q, k_pool, v_pool, block_table, seq_lens, q_lens, out, shape, shared_pages, workspace,
                        stream=None):
    """pkv_attn_fwd over a batch whose tables all begin with the same shared_pages pages."""
    _attn_extents("pkv_attn_fwd_shared", shape, q, k_pool, v_pool, block_table, seq_lens, q_lens, out)
    for t, dt, n in ((q, torch.bfloat16, "q"), (k_pool, torch.bfloat16, "k_pool"),
                     (v_pool, torch.bfloat16, "v_pool"), (block_table, torch.int32, "block_table"),
                     (seq_lens, torch.int32, "seq_lens"), (q_lens, torch.int32, "q_lens"),
                     (out, torch.float32, "out"), (workspace, torch.uint8, "workspace")):
        _need(t, dt, n)
    rc = LIB.pkv_attn_fwd_shared(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(seq_lens),
                                 _ptr(q_lens), _ptr(out), ctypes.byref(shape), int(shared_pages), _ptr(workspace),
                                 workspace.numel(), _stream(stream))
    _check(rc, "pkv_attn_fwd_shared")


def pkv_shared_prefix_pages(block_table_host, seq_lens_host, q_lens_host, shape):
    """The largest shared_pages pkv_attn_fwd_shared accepts for this batch,
    from host arrays (numpy or sequences) of the table, lengths and windows."""
    t = np.ascontiguousarray(block_table_host, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens_host, dtype=np.int32)
    ql = np.ascontiguousarray(q_lens_host, dtype=np.int32)
    if t.size != shape.num_seqs * shape.max_pages_per_seq or sl.size != shape.num_seqs or ql.size != shape.num_seqs:
        raise ValueError("pkv_shared_prefix_pages: host arrays do not match the shape")
    vp = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    n = int(LIB.pkv_shared_prefix_pages(vp(t), vp(sl), vp(ql), ctypes.byref(shape)))
    if n < 0:
        _check(n, "pkv_shared_prefix_pages")
    return n


def pkv_attn_check_errors(workspace, stream=None):
    flags = ctypes.c_uint32(0)
    _check(LIB.pkv_attn_check_errors(_ptr(workspace), _stream(stream), ctypes.byref(flags)),
           "pkv_attn_check_errors")
    return int(flags.value)


def accept_shape(logits, n_draft, max_draft):
    rows, V = logits.shape
    return pkv_accept_shape(int(n_draft.shape[0]), int(V), int(rows), int(max_draft))


def pkv_accept_workspace_bytes(shape):
    return int(LIB.pkv_accept_workspace_bytes(ctypes.byref(shape)))


def new_accept_workspace(shape, device="cuda"):
    n = pkv_accept_workspace_bytes(shape)
    if n == 0:
        raise PkvError("pkv_accept_workspace_bytes: shape rejected")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def _accept_args(what, logits, draft_ids, n_draft, out_accept, out_next, window, shape):
    B = shape.num_seqs
    _extents(what, (logits, shape.total_rows * shape.vocab, "logits"), (n_draft, B, "n_draft"),
             (out_accept, B, "out_accept"), (out_next, B, "out_next"), (window, B, "window"))
    if draft_ids is not None and draft_ids.numel() and draft_ids.numel() < shape.total_rows - B:
        raise ValueError(f"{what}: draft_ids has {draft_ids.numel()} elements, fewer than the "
                         f"{shape.total_rows - B} drafts the rows imply")
    for t, dt, n in ((logits, torch.float32, "logits"), (n_draft, torch.int32, "n_draft"),
                     (out_accept, torch.int32, "out_accept"), (out_next, torch.int32, "out_next")):
        _need(t, dt, n)
    if draft_ids is not None and draft_ids.numel():
        _need(draft_ids, torch.int32, "draft_ids")
    if window is not None:
        _need(window, torch.int32, "window")
    return draft_ids if (draft_ids is not None and draft_ids.numel()) else None


def pkv_accept(logits, draft_ids, n_draft, out_accept, out_next, window, shape, workspace, stream=None):
    """logits fp32; draft_ids, n_draft, out_accept, out_next, window (or None): int32."""
    drafts = _accept_args("pkv_accept", logits, draft_ids, n_draft, out_accept, out_next, window, shape)
    _need(workspace, torch.uint8, "workspace")
    rc = LIB.pkv_accept(_ptr(logits), _ptr(drafts), _ptr(n_draft), _ptr(out_accept), _ptr(out_next),
                        _ptr(window), ctypes.byref(shape), _ptr(workspace), workspace.numel(),
                        _stream(stream))
    _check(rc, "pkv_accept")


def pkv_accept_noalloc(logits, draft_ids, n_draft, out_accept, out_next, window, shape, stream=None):
    """pkv_accept on the library's fixed per-GPU scratch (no workspace, no allocation)."""
    drafts = _accept_args("pkv_accept_noalloc", logits, draft_ids, n_draft, out_accept, out_next, window, shape)
    rc = LIB.pkv_accept_noalloc(_ptr(logits), _ptr(drafts), _ptr(n_draft), _ptr(out_accept), _ptr(out_next),
                                _ptr(window), ctypes.byref(shape), _stream(stream))
    _check(rc, "pkv_accept_noalloc")


def pkv_window_next(window, n_draft, accepted):
    return int(LIB.pkv_window_next(int(window), int(n_draft), int(accepted)))


def pkv_status_string(status):
    return LIB.pkv_status_string(int(status)).decode()


def pkv_version():
    return int(LIB.pkv_version())


def kv_shape(k_pool, block_table, total_q, head_dim=None):
    """pkv_kv_shape from tensor extents (pool [P, Hkv, 256, D], block_table [B, W]);
    head_dim for packed Q4 code pools, whose last extent is D / 2."""
    P, Hkv, page, D = k_pool.shape
    D = int(head_dim) if head_dim is not None else D
    B, W = block_table.shape
    return pkv_kv_shape(B, Hkv, D, page, P, W, int(total_q))


def pkv_kv_workspace_bytes(shape):
    return int(LIB.pkv_kv_workspace_bytes(ctypes.byref(shape)))


def new_kv_workspace(shape, device="cuda"):
    n = pkv_kv_workspace_bytes(shape)
    if n == 0:
        raise PkvError("pkv_kv_workspace_bytes: shape rejected")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def _kv_append_quant(qbits, k_new, v_new, k_codes, k_scales, v_codes, v_scales, block_table, seq_lens, q_lens,
                     free_pages, free_count, shape, workspace, stream):
    call = f"pkv_kv_append_q{qbits}"
    s = shape
    vecs = s.num_pages * s.num_kv_heads * s.page_size
    code_dt = torch.int8 if qbits == 8 else torch.uint8
    win = s.total_q * s.num_kv_heads * s.head_dim
    _extents(call, (k_codes, vecs * s.head_dim * qbits // 8, "k_codes"),
             (v_codes, vecs * s.head_dim * qbits // 8, "v_codes"), (k_scales, vecs, "k_scales"),
             (v_scales, vecs, "v_scales"), (k_new if win else None, win, "k_new"),
             (v_new if win else None, win, "v_new"), (block_table, s.num_seqs * s.max_pages_per_seq, "block_table"),
             (seq_lens, s.num_seqs, "seq_lens"), (q_lens, s.num_seqs, "q_lens"),
             (free_pages, s.num_pages, "free_pages"), (free_count, 1, "free_count"))
    for t, dt, n in ((k_codes, code_dt, "k_codes"), (v_codes, code_dt, "v_codes"),
                     (k_scales, torch.float32, "k_scales"), (v_scales, torch.float32, "v_scales"),
                     (block_table, torch.int32, "block_table"), (seq_lens, torch.int32, "seq_lens"),
                     (q_lens, torch.int32, "q_lens"), (free_pages, torch.int32, "free_pages"),
                     (free_count, torch.int32, "free_count"), (workspace, torch.uint8, "workspace")):
        _need(t, dt, n)
    if k_new.numel():
        _need(k_new, torch.bfloat16, "k_new")
        _need(v_new, torch.bfloat16, "v_new")
    kn = k_new if k_new.numel() else None
    vn = v_new if v_new.numel() else None
    rc = getattr(LIB, call)(_ptr(kn), _ptr(vn), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes), _ptr(v_scales),
                            _ptr(block_table), _ptr(seq_lens), _ptr(q_lens), _ptr(free_pages), _ptr(free_count),
                            ctypes.byref(shape), _ptr(workspace), workspace.numel(), _stream(stream))
    _check(rc, call)


def pkv_kv_append_q8(k_new, v_new, k_codes, k_scales, v_codes, v_scales, block_table, seq_lens, q_lens,
                     free_pages, free_count, shape, workspace, stream=None):
    """pkv_kv_append into Q8 pools (codes int8 [P, Hkv, 256, D], scales fp32 [P, Hkv, 256])."""
    _kv_append_quant(8, k_new, v_new, k_codes, k_scales, v_codes, v_scales, block_table, seq_lens, q_lens,
                     free_pages, free_count, shape, workspace, stream)


def pkv_kv_append_q4(k_new, v_new, k_codes, k_scales, v_codes, v_scales, block_table, seq_lens, q_lens,
                     free_pages, free_count, shape, workspace, stream=None):
    """pkv_kv_append into Q4 pools (codes uint8 [P, Hkv, 256, D / 2], scales fp32 [P, Hkv, 256])."""
    _kv_append_quant(4, k_new, v_new, k_codes, k_scales, v_codes, v_scales, block_table, seq_lens, q_lens,
                     free_pages, free_count, shape, workspace, stream)


def pkv_kv_append(k_new, v_new, k_pool, v_pool, block_table, seq_lens, q_lens, free_pages, free_count,
                  shape, workspace, stream=None):
    """k_new, v_new, pools: bf16; block_table, seq_lens, q_lens, free_pages, free_count: int32."""
    s = shape
    pool = s.num_pages * s.num_kv_heads * s.page_size * s.head_dim
    win = s.total_q * s.num_kv_heads * s.head_dim
    _extents("pkv_kv_append", (k_pool, pool, "k_pool"), (v_pool, pool, "v_pool"),
             (k_new if win else None, win, "k_new"), (v_new if win else None, win, "v_new"),
             (block_table, s.num_seqs * s.max_pages_per_seq, "block_table"), (seq_lens, s.num_seqs, "seq_lens"),
             (q_lens, s.num_seqs, "q_lens"), (free_pages, s.num_pages, "free_pages"), (free_count, 1, "free_count"))
    for t, dt, n in ((k_pool, torch.bfloat16, "k_pool"), (v_pool, torch.bfloat16, "v_pool"),
                     (block_table, torch.int32, "block_table"), (seq_lens, torch.int32, "seq_lens"),
                     (q_lens, torch.int32, "q_lens"), (free_pages, torch.int32, "free_pages"),
                     (free_count, torch.int32, "free_count"), (workspace, torch.uint8, "workspace")):
        _need(t, dt, n)
    if k_new.numel():
        _need(k_new, torch.bfloat16, "k_new")
        _need(v_new, torch.bfloat16, "v_new")
    kn = k_new if k_new.numel() else None
    vn = v_new if v_new.numel() else None
    rc = LIB.pkv_kv_append(_ptr(kn), _ptr(vn), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(seq_lens),
                           _ptr(q_lens), _ptr(free_pages), _ptr(free_count), ctypes.byref(shape),
                           _ptr(workspace), workspace.numel(), _stream(stream))
    _check(rc, "pkv_kv_append")


def pkv_kv_rollback(block_table, seq_lens, q_lens, accepted, free_pages, free_count, shape, workspace,
                    stream=None):
    """All int32 device tensors; accepted is pkv_accept's out_accept."""
    s = shape
    _extents("pkv_kv_rollback", (block_table, s.num_seqs * s.max_pages_per_seq, "block_table"),
             (seq_lens, s.num_seqs, "seq_lens"), (q_lens, s.num_seqs, "q_lens"), (accepted, s.num_seqs, "accepted"),
             (free_pages, s.num_pages, "free_pages"), (free_count, 1, "free_count"))
    for t, n in ((block_table, "block_table"), (seq_lens, "seq_lens"), (q_lens, "q_lens"),
                 (accepted, "accepted"), (free_pages, "free_pages"), (free_count, "free_count")):
        _need(t, torch.int32, n)
    _need(workspace, torch.uint8, "workspace")
    rc = LIB.pkv_kv_rollback(_ptr(block_table), _ptr(seq_lens), _ptr(q_lens), _ptr(accepted),
                             _ptr(free_pages), _ptr(free_count), ctypes.byref(shape), _ptr(workspace),
                             workspace.numel(), _stream(stream))
    _check(rc, "pkv_kv_rollback")


def pkv_kv_check_errors(workspace, stream=None):
    flags = ctypes.c_uint32(0)
    _check(LIB.pkv_kv_check_errors(_ptr(workspace), _stream(stream), ctypes.byref(flags)),
           "pkv_kv_check_errors")
    return int(flags.value)


# ------------------------------------------------------------ page allocator
# Host object; these calls never touch the GPU. Page lists are Python ints.

def _i32_array(values):
    arr = (ctypes.c_int32 * max(1, len(values)))(*values)
    return arr


def pkv_pool_create(num_pages):
    h = LIB.pkv_pool_create(int(num_pages))
    if not h:
        raise PkvError("pkv_pool_create: bad size or out of host memory")
    return ctypes.c_void_p(h)


def pkv_pool_destroy(pool):
    LIB.pkv_pool_destroy(pool)


def pkv_pool_stats(pool):
    out = (ctypes.c_int32 * 3)()
    _check(LIB.pkv_pool_stats(pool, out), "pkv_pool_stats")
    return tuple(out)


def pkv_pool_admit(pool, tokens, max_pages=None):
    """(pages in table order, cached tokens) for a prompt (token ids: any
    int sequence or array)."""
    toks = np.ascontiguousarray(tokens, dtype=np.int32)
    cap = max_pages if max_pages is not None else -(-toks.size // PKV_PAGE_SIZE)
    pages = (ctypes.c_int32 * max(1, cap))()
    n, cached = ctypes.c_int32(0), ctypes.c_int32(0)
    rc = LIB.pkv_pool_admit(pool, toks.ctypes.data_as(ctypes.c_void_p), toks.size, pages, cap, ctypes.byref(n),
                            ctypes.byref(cached))
    _check(rc, "pkv_pool_admit")
    return list(pages[:n.value]), cached.value


def pkv_pool_alloc(pool, n):
    pages = (ctypes.c_int32 * max(1, n))()
    _check(LIB.pkv_pool_alloc(pool, int(n), pages), "pkv_pool_alloc")
    return list(pages[:n])


def pkv_pool_retain(pool, pages):
    _check(LIB.pkv_pool_retain(pool, _i32_array(pages), len(pages)), "pkv_pool_retain")


def pkv_pool_release(pool, pages):
    _check(LIB.pkv_pool_release(pool, _i32_array(pages), len(pages)), "pkv_pool_release")


def pkv_pool_defrag(pool, num_pages, move_referenced=False):
    """(remap list of num_pages entries, [(src, dst), ...])."""
    remap = (ctypes.c_int32 * num_pages)()
    src = (ctypes.c_int32 * num_pages)()
    dst = (ctypes.c_int32 * num_pages)()
    n = ctypes.c_int32(0)
    _check(LIB.pkv_pool_defrag(pool, int(bool(move_referenced)), remap, src, dst, ctypes.byref(n)),
           "pkv_pool_defrag")
    return list(remap), list(zip(src[:n.value], dst[:n.value]))


def pkv_pool_copy_pages(k_pool, v_pool, src, dst, err=None, stream=None):
    """k_pool, v_pool: bf16 [P, Hkv, 256, D]; src, dst: int32 device tensors."""
    _extents("pkv_pool_copy_pages", (v_pool, k_pool.numel(), "v_pool"), (dst, src.numel(), "dst"))
    if err is not None and err.numel() < 1:
        raise ValueError("pkv_pool_copy_pages: err needs one int32")
    for t, dt, n in ((k_pool, torch.bfloat16, "k_pool"), (v_pool, torch.bfloat16, "v_pool"),
                     (src, torch.int32, "src"), (dst, torch.int32, "dst")):
        _need(t, dt, n)
    P, Hkv, page, D = k_pool.shape
    rc = LIB.pkv_pool_copy_pages(_ptr(k_pool), _ptr(v_pool), _ptr(src), _ptr(dst), src.numel(), P, Hkv, D,
                                 _ptr(err), _stream(stream))
    _check(rc, "pkv_pool_copy_pages")


def pkv_pool_copy_page_bytes(pool_a, pool_b, src, dst, err=None, stream=None):
    """Page moves on two pools of any element type whose first extent is the
    page (e.g. Q8 / Q4 code pools, or their scale pools); src, dst: int32."""
    _extents("pkv_pool_copy_page_bytes", (pool_b, pool_a.numel(), "pool_b"), (dst, src.numel(), "dst"))
    if pool_a.dtype != pool_b.dtype:
        raise TypeError("pkv_pool_copy_page_bytes: the two pools differ in type")
    if err is not None and err.numel() < 1:
        raise ValueError("pkv_pool_copy_page_bytes: err needs one int32")
    for t, n in ((pool_a, "pool_a"), (pool_b, "pool_b"), (src, "src"), (dst, "dst")):
        _need(t, t.dtype if n.startswith("pool") else torch.int32, n)
    P = pool_a.shape[0]
    page_bytes = pool_a.numel() * pool_a.element_size() // P
    rc = LIB.pkv_pool_copy_page_bytes(_ptr(pool_a), _ptr(pool_b), _ptr(src), _ptr(dst), src.numel(), P, page_bytes,
                                      _ptr(err), _stream(stream))
    _check(rc, "pkv_pool_copy_page_bytes")


def pkv_table_remap(block_table, remap, err=None, stream=None):
    """block_table int32 [B, W] rewritten in place; remap int32 [P] (device)."""
    _need(block_table, torch.int32, "block_table")
    _need(remap, torch.int32, "remap")
    B, W = block_table.shape
    rc = LIB.pkv_table_remap(_ptr(block_table), B, W, _ptr(remap), remap.numel(), _ptr(err), _stream(stream))
    _check(rc, "pkv_table_remap")
