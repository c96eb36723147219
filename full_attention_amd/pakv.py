"""ctypes binding of libpakv.so, with the C ABI's names minus the ``pakv_`` prefix.

Argument marshalling only: tensors become device addresses, the current torch
stream becomes the hipStream_t.  Every computation runs in the library's HIP
kernels; if the library is missing, importing this module fails.
"""

import ctypes
import os

# torch's ROCm build ships its own HIP runtime.  It has to be in the process
# before libpakv.so is loaded, so that the library's libamdhip64.so.7
# dependency resolves (by soname) to that same runtime: one HIP runtime per
# process, and torch's stream handles are valid for the library's launches.
import torch  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
# PAKV_LIBRARY selects another build of the library (the diagnostic builds
# beside libpakv.so: libpakv_bounds.so, libpakv_hostsan.so)
LIB_PATH = os.environ.get("PAKV_LIBRARY") or os.path.join(_HERE, "libpakv.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                      "(or python -m full_attention_amd.build)")
lib = ctypes.CDLL(LIB_PATH)

OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_ALIAS, ERR_WORKSPACE, ERR_HIP = range(6)
KV_BF16, KV_INT8_PTH, KV_FP8_PTH = 0, 1, 2
PAGE_SIZE = 16

EXPORTED = (
    "pakv_last_error", "pakv_resolve_kv_sources", "pakv_layer_map_create", "pakv_layer_map_destroy",
    "pakv_layer_map_bind_slab", "pakv_layer_map_source", "pakv_kv_bytes_per_token", "pakv_slab_bytes",
    "pakv_paged_kv_store", "pakv_decode_workspace_bytes", "pakv_paged_attn_decode",
    "pakv_decode_plan_bytes", "pakv_decode_plan", "pakv_paged_attn_decode_planned",
    "pakv_paged_attn_decode_append",
    "pakv_paged_attn_extend", "pakv_set_timing_events", "pakv_timing_pairs_used", "pakv_workgroup_xcds",
    "pakv_paged_attn_decode_noalloc", "pakv_decode_noalloc_max_bytes", "pakv_paged_attn_extend_packed",
    "pakv_page_pool_create", "pakv_page_pool_destroy", "pakv_page_pool_reserve", "pakv_page_pool_release_seq",
    "pakv_page_pool_table", "pakv_page_pool_free_pages", "pakv_page_pool_released", "pakv_pool_tokens",
    "pakv_decode_step_workspace_bytes", "pakv_decode_step_create", "pakv_decode_step_run",
    "pakv_decode_step_bucket", "pakv_decode_step_destroy", "pakv_set_decode_checks",
    "pakv_debug_bounds_counts", "pakv_debug_bounds_reset", "pakv_extend_staging_bytes",
    "pakv_paged_attn_extend_staged",
)

TIME_STORE, TIME_DECODE, TIME_EXTEND, TIME_STAGE = 1, 2, 8, 16
DECODE_PLAN_MISMATCH, DECODE_XCD_SPLIT = 1, 2     # bits of the decode workspace's status word
CHECK_XCD_PLACEMENT = 1
DEBUG_COUNTS = 3                                  # decode plans, stores, extend calls


class LayerDesc(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("window", ctypes.c_int32),
                ("kv_source", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("sm_scale", ctypes.c_float), ("k_eq_v", ctypes.c_int32),
                ("v_norm_eps", ctypes.c_float)]


class Slab(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
                ("num_pages", ctypes.c_int32), ("page_size", ctypes.c_int32)]


class StepLayer(ctypes.Structure):
    _fields_ = [("layer", ctypes.c_int32), ("q", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p)]


class Pages(ctypes.Structure):
    _fields_ = [("page_table", ctypes.c_void_p), ("num_seqs", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32)]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_S = ctypes.c_size_t

lib.pakv_last_error.restype = ctypes.c_char_p
lib.pakv_last_error.argtypes = []
lib.pakv_resolve_kv_sources.restype = _I
lib.pakv_resolve_kv_sources.argtypes = [_I, _P, _I, _P]
lib.pakv_layer_map_create.restype = _I
lib.pakv_layer_map_create.argtypes = [_P, _I, ctypes.POINTER(_P)]
lib.pakv_layer_map_destroy.restype = None
lib.pakv_layer_map_destroy.argtypes = [_P]
lib.pakv_layer_map_bind_slab.restype = _I
lib.pakv_layer_map_bind_slab.argtypes = [_P, _I, ctypes.POINTER(Slab)]
lib.pakv_layer_map_source.restype = _I
lib.pakv_layer_map_source.argtypes = [_P, _I, ctypes.POINTER(_I)]
lib.pakv_kv_bytes_per_token.restype = _I
lib.pakv_kv_bytes_per_token.argtypes = [_P, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]
lib.pakv_slab_bytes.restype = _I
lib.pakv_slab_bytes.argtypes = [_P, _I, _I, ctypes.POINTER(_S), ctypes.POINTER(_S)]
lib.pakv_paged_kv_store.restype = _I
lib.pakv_paged_kv_store.argtypes = [_P, _I, ctypes.POINTER(Pages), _P, _P, _P, _P, _I, _I, _P]
lib.pakv_decode_workspace_bytes.restype = _S
lib.pakv_decode_workspace_bytes.argtypes = [_P, _I, _I, _I]
lib.pakv_paged_attn_decode.restype = _I
lib.pakv_paged_attn_decode.argtypes = [_P, _I, ctypes.POINTER(Pages), _P, _P, _P, _I, _I, _P, _S, _P]
lib.pakv_decode_plan_bytes.restype = _S
lib.pakv_decode_plan_bytes.argtypes = [_P, _I, _I, _I]
lib.pakv_decode_plan.restype = _I
lib.pakv_decode_plan.argtypes = [_P, _I, ctypes.POINTER(Pages), _P, _I, _I, _P, _S, _P]
lib.pakv_paged_attn_decode_planned.restype = _I
lib.pakv_paged_attn_decode_planned.argtypes = [_P, _I, ctypes.POINTER(Pages), _P, _S, _P, _P, _I, _I, _P, _S, _P]
lib.pakv_paged_attn_decode_append.restype = _I
lib.pakv_paged_attn_decode_append.argtypes = [_P, _I, ctypes.POINTER(Pages), _P, _S, _P, _P, _P, _P, _I, _I, _P, _S,
                                              _P]
lib.pakv_paged_attn_decode_noalloc.restype = _I
lib.pakv_paged_attn_decode_noalloc.argtypes = [_P, _I, ctypes.POINTER(Pages), _P, _P, _P, _I, _I, _P]
lib.pakv_decode_noalloc_max_bytes.restype = _S
lib.pakv_decode_noalloc_max_bytes.argtypes = []
lib.pakv_paged_attn_extend.restype = _I
lib.pakv_paged_attn_extend.argtypes = [_P, _I, ctypes.POINTER(Pages), _P, _P, _P, _P, _I, _I, _I, _I, _P]
lib.pakv_paged_attn_extend_packed.restype = _I
lib.pakv_paged_attn_extend_packed.argtypes = [_P, _I, ctypes.POINTER(Pages), _P, _P, _P, _P, _P, _P, _I, _I, _I, _I,
                                              _P]
lib.pakv_extend_staging_bytes.restype = _S
lib.pakv_extend_staging_bytes.argtypes = [_P, _I, _I, _I, _I, _I]
lib.pakv_paged_attn_extend_staged.restype = _I
lib.pakv_paged_attn_extend_staged.argtypes = [_P, _I, ctypes.POINTER(Pages), _P, _P, _P, _P, _P, _P, _I, _I, _I, _I,
                                              _P, _S, _I, _P]
lib.pakv_page_pool_create.restype = _I
lib.pakv_page_pool_create.argtypes = [_I, _I, _I, _I, ctypes.POINTER(_P)]
lib.pakv_page_pool_destroy.restype = None
lib.pakv_page_pool_destroy.argtypes = [_P]
lib.pakv_page_pool_reserve.restype = _I
lib.pakv_page_pool_reserve.argtypes = [_P, _I, _I, _I]
lib.pakv_page_pool_release_seq.restype = _I
lib.pakv_page_pool_release_seq.argtypes = [_P, _I]
lib.pakv_page_pool_table.restype = ctypes.POINTER(_I)
lib.pakv_page_pool_table.argtypes = [_P]
lib.pakv_page_pool_free_pages.restype = _I
lib.pakv_page_pool_free_pages.argtypes = [_P]
lib.pakv_page_pool_released.restype = _I
lib.pakv_page_pool_released.argtypes = [_P, _P, _I]
lib.pakv_pool_tokens.restype = _I
lib.pakv_pool_tokens.argtypes = [_P, ctypes.c_int64, ctypes.c_double, ctypes.POINTER(ctypes.c_int64),
                                 ctypes.POINTER(ctypes.c_int64)]
lib.pakv_decode_step_workspace_bytes.restype = _S
lib.pakv_decode_step_workspace_bytes.argtypes = [_P, _P, _I, _I, _I]
lib.pakv_decode_step_create.restype = _I
lib.pakv_decode_step_create.argtypes = [_P, ctypes.POINTER(Pages), ctypes.POINTER(Pages), _P, _I, _I, _P, _I, _P, _I,
                                        _P, _S, ctypes.POINTER(_P)]
lib.pakv_decode_step_run.restype = _I
lib.pakv_decode_step_run.argtypes = [_P, _I, _P]
lib.pakv_decode_step_bucket.restype = _I
lib.pakv_decode_step_bucket.argtypes = [_P, _I]
lib.pakv_decode_step_destroy.restype = None
lib.pakv_decode_step_destroy.argtypes = [_P]
lib.pakv_set_decode_checks.restype = _I
lib.pakv_set_decode_checks.argtypes = [_I]
lib.pakv_set_timing_events.restype = _I
lib.pakv_set_timing_events.argtypes = [_P, _I, _I]
lib.pakv_timing_pairs_used.restype = _I
lib.pakv_timing_pairs_used.argtypes = []
lib.pakv_workgroup_xcds.restype = _I
lib.pakv_workgroup_xcds.argtypes = [_P, _I, _P]
lib.pakv_debug_bounds_counts.restype = _I
lib.pakv_debug_bounds_counts.argtypes = [ctypes.POINTER(ctypes.c_uint32)]
lib.pakv_debug_bounds_reset.restype = _I
lib.pakv_debug_bounds_reset.argtypes = []


class PakvError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"pakv status {status}: {message}")
        self.status = status


def last_error():
    return lib.pakv_last_error().decode()


def _check(status):
    if status != OK:
        raise PakvError(status, last_error())
    return status


def _ptr(x):
    """Device (or host) address of a tensor, an int, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    if torch.cuda.is_available():
        return torch.cuda.current_stream().cuda_stream
    return None


def resolve_kv_sources(layer_types, first_shared):
    n = len(layer_types)
    types = (ctypes.c_int32 * max(n, 1))(*layer_types)
    out = (ctypes.c_int32 * max(n, 1))()
    _check(lib.pakv_resolve_kv_sources(n, ctypes.cast(types, _P), first_shared, ctypes.cast(out, _P)))
    return list(out)[:n]


class LayerMap:
    """Owner of a pakv_layer_map*.  ``descs`` is a list of LayerDesc."""

    def __init__(self, descs):
        arr = (LayerDesc * len(descs))(*descs)
        handle = _P()
        _check(lib.pakv_layer_map_create(ctypes.cast(arr, _P), len(descs), ctypes.byref(handle)))
        self.handle = handle
        self.n = len(descs)
        self._slabs = {}

    def close(self):
        if self.handle:
            lib.pakv_layer_map_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def bind_slab(self, layer, k, v, num_pages, k_scale=None, v_scale=None):
        slab = Slab(_ptr(k), _ptr(v), _ptr(k_scale), _ptr(v_scale), num_pages, PAGE_SIZE)
        _check(lib.pakv_layer_map_bind_slab(self.handle, layer, ctypes.byref(slab)))
        self._slabs[layer] = (k, v, k_scale, v_scale)   # keep the buffers alive

    def source(self, layer):
        out = _I()
        _check(lib.pakv_layer_map_source(self.handle, layer, ctypes.byref(out)))
        return out.value

    def kv_bytes_per_token(self):
        f, w = ctypes.c_int64(), ctypes.c_int64()
        _check(lib.pakv_kv_bytes_per_token(self.handle, ctypes.byref(f), ctypes.byref(w)))
        return f.value, w.value

    def slab_bytes(self, layer, num_pages):
        c, s = _S(), _S()
        _check(lib.pakv_slab_bytes(self.handle, layer, num_pages, ctypes.byref(c), ctypes.byref(s)))
        return c.value, s.value


def make_pages(page_table, num_seqs=None, max_pages_per_seq=None):
    """pakv_pages for a device int32 [B, max_pages] tensor.  The struct holds
    the tensor's address, so it also keeps the tensor alive: a temporary table
    freed while its pages struct is in use would let later allocations reuse
    the memory the kernels read page ids from."""
    if num_seqs is None:
        num_seqs, max_pages_per_seq = page_table.shape
    pages = Pages(_ptr(page_table), num_seqs, max_pages_per_seq)
    pages._table = page_table
    return pages


def paged_kv_store(layer_map, layer, pages, cu_tokens, start_pos, k, v, num_seqs, total_tokens, stream=None):
    return _check(lib.pakv_paged_kv_store(layer_map.handle, layer, ctypes.byref(pages), _ptr(cu_tokens),
                                          _ptr(start_pos), _ptr(k), _ptr(v), num_seqs, total_tokens,
                                          _stream(stream)))


def decode_workspace_bytes(layer_map, layer, num_seqs, max_kv_len):
    return lib.pakv_decode_workspace_bytes(layer_map.handle, layer, num_seqs, max_kv_len)


def paged_attn_decode(layer_map, layer, pages, kv_lens, q, out, num_seqs, max_kv_len,
                      workspace, workspace_bytes, stream=None):
    return _check(lib.pakv_paged_attn_decode(layer_map.handle, layer, ctypes.byref(pages), _ptr(kv_lens),
                                             _ptr(q), _ptr(out), num_seqs, max_kv_len, _ptr(workspace),
                                             workspace_bytes, _stream(stream)))


def decode_plan_bytes(layer_map, layer, num_seqs, max_kv_len):
    return lib.pakv_decode_plan_bytes(layer_map.handle, layer, num_seqs, max_kv_len)


def decode_plan(layer_map, layer, pages, kv_lens, num_seqs, max_kv_len, plan, plan_bytes, stream=None):
    return _check(lib.pakv_decode_plan(layer_map.handle, layer, ctypes.byref(pages), _ptr(kv_lens), num_seqs,
                                       max_kv_len, _ptr(plan), plan_bytes, _stream(stream)))


def paged_attn_decode_planned(layer_map, layer, pages, plan, plan_bytes, q, out, num_seqs, max_kv_len,
                              workspace, workspace_bytes, stream=None):
    return _check(lib.pakv_paged_attn_decode_planned(layer_map.handle, layer, ctypes.byref(pages), _ptr(plan),
                                                     plan_bytes, _ptr(q), _ptr(out), num_seqs, max_kv_len,
                                                     _ptr(workspace), workspace_bytes, _stream(stream)))


def paged_attn_decode_append(layer_map, layer, pages, plan, plan_bytes, k_new, v_new, q, out, num_seqs,
                             max_kv_len, workspace, workspace_bytes, stream=None):
    return _check(lib.pakv_paged_attn_decode_append(layer_map.handle, layer, ctypes.byref(pages), _ptr(plan),
                                                    plan_bytes, _ptr(k_new), _ptr(v_new), _ptr(q), _ptr(out),
                                                    num_seqs, max_kv_len, _ptr(workspace), workspace_bytes,
                                                    _stream(stream)))


def paged_attn_decode_noalloc(layer_map, layer, pages, kv_lens, q, out, num_seqs, max_kv_len, stream=None):
    return _check(lib.pakv_paged_attn_decode_noalloc(layer_map.handle, layer, ctypes.byref(pages), _ptr(kv_lens),
                                                     _ptr(q), _ptr(out), num_seqs, max_kv_len, _stream(stream)))


def decode_noalloc_max_bytes():
    return lib.pakv_decode_noalloc_max_bytes()


def paged_attn_extend(layer_map, layer, pages, cu_q, prefix_lens, q, out, num_seqs, total_q, max_q_len,
                      max_kv_len, stream=None):
    return _check(lib.pakv_paged_attn_extend(layer_map.handle, layer, ctypes.byref(pages), _ptr(cu_q),
                                             _ptr(prefix_lens), _ptr(q), _ptr(out), num_seqs, total_q,
                                             max_q_len, max_kv_len, _stream(stream)))


def extend_staging_bytes(layer_map, layer, num_seqs, max_q_len, max_kv_len, packed):
    return lib.pakv_extend_staging_bytes(layer_map.handle, layer, num_seqs, max_q_len, max_kv_len, 1 if packed else 0)


def paged_attn_extend_staged(layer_map, layer, pages, cu_q, prefix_lens, q, k_ext, v_ext, out, num_seqs, total_q,
                             max_q_len, max_kv_len, workspace, workspace_bytes, stage=True, stream=None):
    return _check(lib.pakv_paged_attn_extend_staged(layer_map.handle, layer, ctypes.byref(pages), _ptr(cu_q),
                                                    _ptr(prefix_lens), _ptr(q), _ptr(k_ext), _ptr(v_ext), _ptr(out),
                                                    num_seqs, total_q, max_q_len, max_kv_len, _ptr(workspace),
                                                    workspace_bytes, 1 if stage else 0, _stream(stream)))


def paged_attn_extend_packed(layer_map, layer, pages, cu_q, prefix_lens, q, k_ext, v_ext, out, num_seqs, total_q,
                             max_q_len, max_kv_len, stream=None):
    return _check(lib.pakv_paged_attn_extend_packed(layer_map.handle, layer, ctypes.byref(pages), _ptr(cu_q),
                                                    _ptr(prefix_lens), _ptr(q), _ptr(k_ext), _ptr(v_ext), _ptr(out),
                                                    num_seqs, total_q, max_q_len, max_kv_len, _stream(stream)))


class PagePool:
    """Owner of a pakv_page_pool* (host bookkeeping of which pages each
    sequence holds, for one group of layers)."""

    def __init__(self, num_pages, max_seqs, max_pages_per_seq, window):
        handle = _P()
        _check(lib.pakv_page_pool_create(num_pages, max_seqs, max_pages_per_seq, window, ctypes.byref(handle)))
        self.handle = handle
        self.shape = (max_seqs, max_pages_per_seq)

    def close(self):
        if self.handle:
            lib.pakv_page_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def reserve(self, seq, first_query, end):
        _check(lib.pakv_page_pool_reserve(self.handle, seq, first_query, end))

    def release_seq(self, seq):
        _check(lib.pakv_page_pool_release_seq(self.handle, seq))

    def table(self):
        """A copy of the host table, int32 [max_seqs, max_pages_per_seq]."""
        import numpy as np
        p = lib.pakv_page_pool_table(self.handle)
        n = self.shape[0] * self.shape[1]
        return np.ctypeslib.as_array(p, shape=(n,)).reshape(self.shape).copy()

    def free_pages(self):
        return lib.pakv_page_pool_free_pages(self.handle)

    def released(self):
        n = lib.pakv_page_pool_released(self.handle, None, 0)
        buf = (_I * max(n, 1))()
        lib.pakv_page_pool_released(self.handle, ctypes.cast(buf, _P), n)
        return list(buf)[:n]


def pool_tokens(layer_map, budget_bytes, window_share):
    f, w = ctypes.c_int64(), ctypes.c_int64()
    _check(lib.pakv_pool_tokens(layer_map.handle, int(budget_bytes), float(window_share), ctypes.byref(f),
                                ctypes.byref(w)))
    return f.value, w.value


class DecodeStep:
    """Owner of a pakv_decode_step*: the decode step of a layer stack captured
    into one HIP graph per batch-size bucket.  layers: list of (layer, q, out,
    k_new, v_new) with tensors sized for max_batch (k_new / v_new None where
    the rows are stored beforehand); every buffer is kept referenced here, as
    the graphs hold their addresses."""

    def __init__(self, layer_map, pages_full, kv_lens, max_batch, max_kv_len, layers, buckets, workspace,
                 pages_sliding=None):
        arr = (StepLayer * len(layers))(*[StepLayer(l, _ptr(q), _ptr(o), _ptr(kn), _ptr(vn))
                                          for l, q, o, kn, vn in layers])
        bk = (_I * len(buckets))(*buckets)
        handle = _P()
        _check(lib.pakv_decode_step_create(layer_map.handle, ctypes.byref(pages_full),
                                           ctypes.byref(pages_sliding) if pages_sliding is not None else None,
                                           _ptr(kv_lens), max_batch, max_kv_len, ctypes.cast(arr, _P), len(layers),
                                           ctypes.cast(bk, _P), len(buckets), _ptr(workspace), workspace.numel(),
                                           ctypes.byref(handle)))
        self.handle = handle
        self._keep = (layer_map, pages_full, pages_sliding, kv_lens, layers, workspace)

    @staticmethod
    def workspace_bytes(layer_map, layers, max_batch, max_kv_len):
        arr = (StepLayer * len(layers))(*[StepLayer(l, 1, 1, None, None) for l, *_ in layers])
        return lib.pakv_decode_step_workspace_bytes(layer_map.handle, ctypes.cast(arr, _P), len(layers), max_batch,
                                                    max_kv_len)

    def run(self, batch, stream=None):
        _check(lib.pakv_decode_step_run(self.handle, batch, _stream(stream)))

    def bucket(self, batch):
        return lib.pakv_decode_step_bucket(self.handle, batch)

    def close(self):
        if self.handle:
            lib.pakv_decode_step_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def workgroup_xcds(out, num_workgroups, stream=None):
    """out: device int32 [num_workgroups]; out[i] = the XCD workgroup i ran on."""
    return _check(lib.pakv_workgroup_xcds(_ptr(out), num_workgroups, _stream(stream)))


def set_decode_checks(flags):
    return _check(lib.pakv_set_decode_checks(flags))


def debug_bounds_counts():
    """Page-table entries outside the pool met on the current device since the
    last reset: (decode plans, stores, extend calls).  PAKV_DEBUG_BOUNDS builds
    only (PakvError with ERR_UNSUPPORTED otherwise)."""
    out = (ctypes.c_uint32 * DEBUG_COUNTS)()
    _check(lib.pakv_debug_bounds_counts(out))
    return tuple(int(x) for x in out)


def debug_bounds_reset():
    return _check(lib.pakv_debug_bounds_reset())


def set_timing_events(events, kernel_mask):
    """events: ctypes array of 2*n hipEvent_t handles (or None to clear)."""
    if events is None:
        return _check(lib.pakv_set_timing_events(None, 0, 0))
    return _check(lib.pakv_set_timing_events(ctypes.cast(events, _P), len(events) // 2, kernel_mask))


def timing_pairs_used():
    return lib.pakv_timing_pairs_used()
