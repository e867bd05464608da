"""ctypes binding of libdcpkv.so: argument marshalling only.

Every function keeps the C name of the entry point it wraps (include/dcpkv.h)
and only turns tensors into device pointers, Python lists into host arrays
and status codes into exceptions.  All arithmetic runs in the library's HIP
kernels; there is no other path.  If the library is missing, importing this
module raises.
"""

from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# DCPKV_LIBRARY may point at another build of the same library (same ABI)
LIB_PATH = os.environ.get("DCPKV_LIBRARY") or os.path.join(_HERE, "libdcpkv.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m context_paged_kv_amd.build` "
        "(this package has no fallback path)")

# DCPKV_HOST_ONLY=1 binds a build of the host part alone (the page map, block
# tables, filters and checks; used to run the host tests under the address and
# undefined-behaviour sanitizers): no HIP runtime, and no device entry point.
HOST_ONLY = os.environ.get("DCPKV_HOST_ONLY") == "1"

# One HIP runtime per process: torch ships its own libamdhip64 (same SONAME as
# ROCm's).  Importing torch first makes the loader bind this library to the
# runtime torch already uses; loading ours first would bring up a second HIP/HSA
# runtime that sees no device.
if not HOST_ONLY:
    import torch  # noqa: E402,F401

_lib = C.CDLL(LIB_PATH)

# the include/dcpkv.h revision these signatures follow; a library of another revision is refused
ABI_VERSION = 7
_lib.dcpkv_abi_version.restype = C.c_int
if _lib.dcpkv_abi_version() != ABI_VERSION:
    raise ImportError(f"{LIB_PATH} has ABI version {_lib.dcpkv_abi_version()}, this binding needs {ABI_VERSION}: "
                      "rebuild it with `python -m context_paged_kv_amd.build`")

DCPKV_OK = 0
DCPKV_EDEVICE = -5
DCPKV_ENOMEM = -12
DCPKV_EINVAL = -22
DCPKV_ENOSPC = -28
DCPKV_ENOTSUP = -95
KV_F32, KV_BF16, KV_FP8E4M3 = 0, 1, 2
LAYOUT_SPLIT, LAYOUT_MLA = 0, 1
Q_F32, Q_BF16 = 0, 1
OWN_PAGE, OWN_TOKEN = 0, 1

EXPORTED = (
    "dcpkv_last_error", "dcpkv_abi_version", "cp_layersplit_layer_range", "dcp_filter_kv_indices",
    "dcp_pagemap_create", "dcp_pagemap_destroy", "dcp_pagemap_num_free", "dcp_pagemap_alloc",
    "dcp_pagemap_release", "dcp_build_block_tables", "kv_reshard_pages", "kv_check_unique_pages",
    "kv_path_entries", "kv_pack_pages", "kv_unpack_pages", "kv_reshard_tokens",
    "dcp_decode_partial_workspace", "dcp_decode_partial", "dcp_decode_partial_noalloc", "dcp_lse_merge",
    "dcpkv_probe_mfma", "dcpkv_probe_copy", "dcpkv_probe_copy_pages",
)
NOALLOC_SCRATCH_BYTES = 64 << 20  # DCPKV_NOALLOC_SCRATCH_BYTES


class DcpkvError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class kv_reshard_desc(C.Structure):
    _fields_ = [("num_sources", C.c_int32), ("num_layers", C.c_int32), ("dcp_size", C.c_int32),
                ("dst_filter", C.c_int32), ("page_bytes", C.c_int64), ("src_pages", C.c_int64),
                ("dst_pages", C.c_int64)]


class kv_token_reshard_desc(C.Structure):
    _fields_ = [("num_sources", C.c_int32), ("num_layers", C.c_int32), ("dcp_size", C.c_int32),
                ("page_size", C.c_int32), ("token_rows", C.c_int32), ("row_bytes", C.c_int32),
                ("src_pages", C.c_int64), ("dst_pages", C.c_int64)]


class dcp_attn_desc(C.Structure):
    _fields_ = [("kv_dtype", C.c_int32), ("kv_layout", C.c_int32), ("q_dtype", C.c_int32),
                ("num_q_heads", C.c_int32), ("num_kv_heads", C.c_int32),
                ("head_dim_qk", C.c_int32), ("head_dim_v", C.c_int32), ("page_size", C.c_int32),
                ("dcp_size", C.c_int32), ("batch", C.c_int32), ("q_len", C.c_int32),
                ("max_local_pages", C.c_int32), ("layer", C.c_int32), ("num_layers", C.c_int32),
                ("pages_per_layer", C.c_int64), ("softmax_scale", C.c_float), ("token_interleave", C.c_int32)]


_P = C.c_void_p
_I32P = C.POINTER(C.c_int32)
_I64P = C.POINTER(C.c_int64)

# (argtypes, restype) of every entry point; the host part comes first
_SIGS = {
    "dcpkv_last_error": ([], C.c_char_p),
    "dcpkv_abi_version": ([], C.c_int),
    "cp_layersplit_layer_range": ([C.c_int32, C.c_int32, C.c_int32, _I32P, _I32P], C.c_int),
    "dcp_filter_kv_indices": ([_I64P, C.c_int64, C.c_int32, C.c_int32, _I64P, _I64P], C.c_int),
    "dcp_pagemap_create": ([C.c_int32, C.c_int32, C.c_int64, _I64P, C.POINTER(_P)], C.c_int),
    "dcp_pagemap_destroy": ([_P], None),
    "dcp_pagemap_num_free": ([_P], C.c_int64),
    "dcp_pagemap_alloc": ([_P, C.c_int64, _I64P, C.c_int64], C.c_int),
    "dcp_pagemap_release": ([_P, _I64P, C.c_int64], C.c_int),
    "dcp_build_block_tables": ([C.c_int32, C.c_int32, _I64P, _I64P, C.c_int32, C.c_int32, _I32P, _I32P], C.c_int),
    "kv_check_unique_pages": ([_I64P, C.c_int64, C.c_int64, _I64P], C.c_int),
    "kv_reshard_pages": ([C.POINTER(kv_reshard_desc), C.POINTER(_P), C.POINTER(_P), C.POINTER(_P), C.POINTER(_P),
                          _P, _P, C.c_int64, C.c_int64, _P, _P, _P], C.c_int),
    "kv_path_entries": ([C.POINTER(kv_reshard_desc), C.c_int32, _P, _P, C.c_int64, C.c_int64, _P, _P, _P], C.c_int),
    "kv_pack_pages": ([C.POINTER(kv_reshard_desc), C.c_int32, _P, _P, _P, _P, _P, C.c_int64, C.c_int64, _P, _P, _P,
                       _P], C.c_int),
    "kv_unpack_pages": ([C.POINTER(kv_reshard_desc), C.c_int32, C.c_int32, _P, _P, _P, _P, _P, C.c_int64, C.c_int64,
                         _P, _P, _P], C.c_int),
    "kv_reshard_tokens": ([C.POINTER(kv_token_reshard_desc), C.POINTER(_P), C.POINTER(_P), _P, _P, C.c_int64, _P,
                           C.c_int32, C.c_int64, _P, _P], C.c_int),
    "dcp_decode_partial_workspace": ([C.POINTER(dcp_attn_desc), C.c_int64], C.c_size_t),
    "dcp_decode_partial": ([C.POINTER(dcp_attn_desc), _P, C.POINTER(_P), C.POINTER(_P), _P, _P, C.c_int64, C.c_int32,
                            C.c_int32, _P, _P, _P, C.c_size_t, _P], C.c_int),
    "dcp_decode_partial_noalloc": ([C.POINTER(dcp_attn_desc), _P, C.POINTER(_P), C.POINTER(_P), _P, _P, C.c_int64,
                                    C.c_int32, C.c_int32, _P, _P, _P], C.c_int),
    "dcp_lse_merge": ([C.c_int32, C.c_int64, C.c_int32, _P, _P, _P, _P, _P], C.c_int),
    "dcpkv_probe_mfma": ([C.c_int32, C.c_int32, _P, C.c_int64, _I64P, _P], C.c_int),
    "dcpkv_probe_copy": ([_P, _P, C.c_int64, _P], C.c_int),
    "dcpkv_probe_copy_pages": ([_P, _P, _P, _P, C.c_int64, C.c_int64, C.c_int64, C.c_int64, _P], C.c_int),
}
HOST_SYMBOLS = ("dcpkv_last_error", "dcpkv_abi_version", "cp_layersplit_layer_range", "dcp_filter_kv_indices",
                "dcp_pagemap_create", "dcp_pagemap_destroy", "dcp_pagemap_num_free", "dcp_pagemap_alloc",
                "dcp_pagemap_release", "dcp_build_block_tables", "kv_check_unique_pages")
for _name, (_args, _res) in _SIGS.items():
    if HOST_ONLY and _name not in HOST_SYMBOLS:
        continue
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res


def _check(rc: int) -> None:
    if rc != DCPKV_OK:
        raise DcpkvError(rc, _lib.dcpkv_last_error().decode(errors="replace"))


def _i64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64))


def _ptr64(a: np.ndarray):
    return a.ctypes.data_as(_I64P)


def _ptr32(a: np.ndarray):
    return a.ctypes.data_as(_I32P)


def _dptr(t) -> Optional[int]:
    """Device pointer of a tensor (None passes NULL)."""
    if t is None:
        return None
    if not getattr(t, "is_cuda", False):
        raise ValueError("expected a tensor in GPU memory")
    return t.data_ptr()


def _ptr_array(ts):
    if ts is None:
        return None
    arr = (_P * len(ts))(*[_dptr(t) for t in ts])
    return arr


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return int(stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


def dcpkv_last_error() -> str:
    return _lib.dcpkv_last_error().decode(errors="replace")


def dcpkv_abi_version() -> int:
    return _lib.dcpkv_abi_version()


def cp_layersplit_layer_range(num_layers: int, num_sources: int, r: int):
    b, e = C.c_int32(), C.c_int32()
    _check(_lib.cp_layersplit_layer_range(num_layers, num_sources, r, C.byref(b), C.byref(e)))
    return b.value, e.value


def dcp_filter_kv_indices(kv_indices: Sequence[int], dcp_size: int, dcp_rank: int) -> np.ndarray:
    idx = _i64(kv_indices)
    out = np.empty(max(1, idx.size), dtype=np.int64)
    cnt = C.c_int64()
    _check(_lib.dcp_filter_kv_indices(_ptr64(idx), idx.size, dcp_size, dcp_rank, _ptr64(out), C.byref(cnt)))
    return out[: cnt.value].copy()


def dcp_pagemap_create(dcp_size: int, page_size: int, num_virtual_pages: int, free_order=None) -> int:
    h = _P()
    fo = None if free_order is None else _i64(free_order)
    _check(_lib.dcp_pagemap_create(dcp_size, page_size, num_virtual_pages,
                                   None if fo is None else _ptr64(fo), C.byref(h)))
    return h.value


def dcp_pagemap_destroy(handle: int) -> None:
    _lib.dcp_pagemap_destroy(handle)


def dcp_pagemap_num_free(handle: int) -> int:
    return _lib.dcp_pagemap_num_free(handle)


def dcp_pagemap_alloc(handle: int, num_tokens: int, page_size: int) -> np.ndarray:
    cap = max(1, -(-num_tokens // page_size))
    out = np.empty(cap, dtype=np.int64)
    _check(_lib.dcp_pagemap_alloc(handle, num_tokens, _ptr64(out), cap))
    return out


def dcp_pagemap_release(handle: int, global_pages: Sequence[int]) -> None:
    g = _i64(global_pages)
    _check(_lib.dcp_pagemap_release(handle, _ptr64(g) if g.size else None, g.size))


class PageMap:
    """Owning handle around dcp_pagemap_* (frees the host object on close)."""

    def __init__(self, dcp_size: int, page_size: int, num_virtual_pages: int, free_order=None):
        self.dcp_size, self.page_size = dcp_size, page_size
        self.handle = dcp_pagemap_create(dcp_size, page_size, num_virtual_pages, free_order)

    def alloc(self, num_tokens: int) -> np.ndarray:
        return dcp_pagemap_alloc(self.handle, num_tokens, self.page_size)

    def release(self, global_pages) -> None:
        dcp_pagemap_release(self.handle, global_pages)

    def num_free(self) -> int:
        return dcp_pagemap_num_free(self.handle)

    def close(self) -> None:
        if self.handle:
            dcp_pagemap_destroy(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def dcp_build_block_tables(dcp_size: int, pages_per_request: Sequence[Sequence[int]], max_local_pages: int,
                           token_interleave: int = 0):
    """Returns (tables int32 [N][B][max_local_pages], counts int32 [N][B])."""
    batch = len(pages_per_request)
    offs = np.zeros(batch + 1, dtype=np.int64)
    for b, pg in enumerate(pages_per_request):
        offs[b + 1] = offs[b] + len(pg)
    flat = _i64(np.concatenate([np.asarray(p, dtype=np.int64) for p in pages_per_request])
                if batch else np.zeros(0, np.int64))
    tables = np.empty((dcp_size, batch, max_local_pages), dtype=np.int32)
    counts = np.empty((dcp_size, batch), dtype=np.int32)
    _check(_lib.dcp_build_block_tables(dcp_size, batch, _ptr64(flat) if flat.size else None, _ptr64(offs),
                                       max_local_pages, token_interleave, _ptr32(tables), _ptr32(counts)))
    return tables, counts


def kv_reshard_pages(*, num_layers: int, dcp_size: int, page_bytes: int, src_pages: int, dst_pages: int,
                     src_pools, dst_pools, src_page_ids, dst_global_pages, first_uncached: int = 0,
                     dst_filter: int = -1, src_scales=None, dst_scales=None, bad_entries=None,
                     pages_per_dst=None, num_pages: Optional[int] = None, stream=None) -> None:
    """Enqueue the page-level 2D reshard (see include/dcpkv.h)."""
    desc = kv_reshard_desc(len(src_pools), num_layers, dcp_size, dst_filter, page_bytes, src_pages, dst_pages)
    n = src_page_ids.numel() if num_pages is None else num_pages
    _check(_lib.kv_reshard_pages(C.byref(desc), _ptr_array(src_pools), _ptr_array(dst_pools),
                                 _ptr_array(src_scales), _ptr_array(dst_scales), _dptr(src_page_ids),
                                 _dptr(dst_global_pages), n, first_uncached, _dptr(bad_entries),
                                 _dptr(pages_per_dst), _stream(stream)))


def kv_check_unique_pages(dst_global_pages: Sequence[int], first_uncached: int = 0) -> int:
    """-1 when the destination pages past first_uncached are distinct (host list), else raises
    DcpkvError; the error's `first_duplicate` is the first list position that repeats a page."""
    g = _i64(dst_global_pages)
    dup = C.c_int64(-2)
    rc = _lib.kv_check_unique_pages(_ptr64(g) if g.size else None, g.size, first_uncached, C.byref(dup))
    if rc != DCPKV_OK:
        err = DcpkvError(rc, _lib.dcpkv_last_error().decode(errors="replace"))
        err.first_duplicate = dup.value
        raise err
    return dup.value


def kv_reshard_tokens(*, num_layers: int, dcp_size: int, page_size: int, token_rows: int, row_bytes: int,
                      src_pages: int, dst_pages: int, src_pools, dst_pools, src_page_ids, dst_global_pages,
                      first_uncached: int = 0, request_offsets=None, num_requests: Optional[int] = None,
                      bad_entries=None, num_pages: Optional[int] = None, stream=None) -> None:
    """Enqueue the token scatter reshard for pools under token ownership (see include/dcpkv.h).
    request_offsets: device int64 [B + 1] delimiting the requests in the lists (None: one request)."""
    desc = kv_token_reshard_desc(len(src_pools), num_layers, dcp_size, page_size, token_rows, row_bytes,
                                 src_pages, dst_pages)
    n = src_page_ids.numel() if num_pages is None else num_pages
    if num_requests is None:
        num_requests = request_offsets.numel() - 1 if request_offsets is not None else 1
    _check(_lib.kv_reshard_tokens(C.byref(desc), _ptr_array(src_pools), _ptr_array(dst_pools), _dptr(src_page_ids),
                                  _dptr(dst_global_pages), n, _dptr(request_offsets), num_requests, first_uncached,
                                  _dptr(bad_entries), _stream(stream)))


def _path_desc(num_sources: int, num_layers: int, dcp_size: int, page_bytes: int, src_pages: int,
               dst_pages: int) -> kv_reshard_desc:
    return kv_reshard_desc(num_sources, num_layers, dcp_size, -1, page_bytes, src_pages, dst_pages)


def kv_path_entries(*, num_sources: int, num_layers: int, dcp_size: int, page_bytes: int, src_pages: int,
                    dst_pages: int, dest: int, src_page_ids, dst_global_pages, out_positions, out_count,
                    first_uncached: int = 0, num_pages: Optional[int] = None, stream=None) -> None:
    """Enqueue the entry list of the path to `dest` (see include/dcpkv.h)."""
    desc = _path_desc(num_sources, num_layers, dcp_size, page_bytes, src_pages, dst_pages)
    n = src_page_ids.numel() if num_pages is None else num_pages
    _check(_lib.kv_path_entries(C.byref(desc), dest, _dptr(src_page_ids), _dptr(dst_global_pages), n,
                                first_uncached, _dptr(out_positions), _dptr(out_count), _stream(stream)))


def kv_pack_pages(*, num_sources: int, num_layers: int, dcp_size: int, page_bytes: int, src_pages: int,
                  dst_pages: int, source: int, src_pool, src_page_ids, positions, count, unit_begin: int,
                  cap_units: int, staging, src_scales=None, staging_scales=None, out_units=None,
                  stream=None) -> None:
    """Enqueue the packing of one window of units of path (source, .) (see include/dcpkv.h)."""
    desc = _path_desc(num_sources, num_layers, dcp_size, page_bytes, src_pages, dst_pages)
    _check(_lib.kv_pack_pages(C.byref(desc), source, _dptr(src_pool), _dptr(src_scales), _dptr(src_page_ids),
                              _dptr(positions), _dptr(count), unit_begin, cap_units, _dptr(staging),
                              _dptr(staging_scales), _dptr(out_units), _stream(stream)))


def kv_unpack_pages(*, num_sources: int, num_layers: int, dcp_size: int, page_bytes: int, src_pages: int,
                    dst_pages: int, source: int, dest: int, dst_pool, dst_global_pages, positions, count,
                    unit_begin: int, cap_units: int, staging, dst_scales=None, staging_scales=None,
                    stream=None) -> None:
    """Enqueue the unpacking of one window of units into destination `dest` (see include/dcpkv.h)."""
    desc = _path_desc(num_sources, num_layers, dcp_size, page_bytes, src_pages, dst_pages)
    _check(_lib.kv_unpack_pages(C.byref(desc), source, dest, _dptr(dst_pool), _dptr(dst_scales),
                                _dptr(dst_global_pages), _dptr(positions), _dptr(count), unit_begin, cap_units,
                                _dptr(staging), _dptr(staging_scales), _stream(stream)))


def make_attn_desc(*, kv_dtype: int, kv_layout: int, q_dtype: int, num_q_heads: int, num_kv_heads: int,
                   head_dim_qk: int, head_dim_v: int, page_size: int, dcp_size: int, batch: int,
                   q_len: int, max_local_pages: int, layer: int, num_layers: int, pages_per_layer: int,
                   softmax_scale: float, token_interleave: int = 0) -> dcp_attn_desc:
    return dcp_attn_desc(kv_dtype, kv_layout, q_dtype, num_q_heads, num_kv_heads, head_dim_qk, head_dim_v,
                         page_size, dcp_size, batch, q_len, max_local_pages, layer, num_layers, pages_per_layer,
                         softmax_scale, token_interleave)


def dcp_decode_partial_workspace(desc: dcp_attn_desc, total_tokens: int) -> int:
    n = _lib.dcp_decode_partial_workspace(C.byref(desc), total_tokens)
    if n == 0:
        raise DcpkvError(DCPKV_EINVAL, "bad attention descriptor")
    return n


def dcp_decode_partial(desc: dcp_attn_desc, *, q, kv_pools, kv_scales, block_tables, seq_lens,
                       total_tokens: int, partial_out, partial_lse, workspace, shard_begin: int = 0,
                       shard_count: Optional[int] = None, stream=None) -> None:
    """Enqueue per-shard partial attention (see include/dcpkv.h)."""
    sc = desc.dcp_size - shard_begin if shard_count is None else shard_count
    _check(_lib.dcp_decode_partial(C.byref(desc), _dptr(q), _ptr_array(kv_pools), _ptr_array(kv_scales),
                                   _dptr(block_tables), _dptr(seq_lens), total_tokens, shard_begin, sc,
                                   _dptr(partial_out), _dptr(partial_lse), _dptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)))


def dcp_decode_partial_noalloc(desc: dcp_attn_desc, *, q, kv_pools, kv_scales, block_tables, seq_lens,
                               total_tokens: int, partial_out, partial_lse, shard_begin: int = 0,
                               shard_count: Optional[int] = None, stream=None) -> None:
    """Enqueue per-shard partial attention without a workspace (the library's scratch; see
    include/dcpkv.h)."""
    sc = desc.dcp_size - shard_begin if shard_count is None else shard_count
    _check(_lib.dcp_decode_partial_noalloc(C.byref(desc), _dptr(q), _ptr_array(kv_pools), _ptr_array(kv_scales),
                                           _dptr(block_tables), _dptr(seq_lens), total_tokens, shard_begin, sc,
                                           _dptr(partial_out), _dptr(partial_lse), _stream(stream)))


def dcp_lse_merge(dcp_size: int, rows: int, head_dim_v: int, partial_out, partial_lse, out, out_lse=None,
                  stream=None) -> None:
    """Enqueue the exact LSE merge of dcp_size partials (see include/dcpkv.h)."""
    _check(_lib.dcp_lse_merge(dcp_size, rows, head_dim_v, _dptr(partial_out), _dptr(partial_lse), _dptr(out),
                              _dptr(out_lse), _stream(stream)))


PROBE_SINK_FLOATS = 1024 * 512


def dcpkv_probe_mfma(kind: int, iters: int, sink, stream=None) -> int:
    """Enqueue the MFMA rate probe (see include/dcpkv.h); returns the launch's flops."""
    flops = C.c_int64(0)
    _check(_lib.dcpkv_probe_mfma(kind, iters, _dptr(sink), sink.numel(), C.byref(flops), _stream(stream)))
    return flops.value


def dcpkv_probe_copy(src, dst, nbytes: Optional[int] = None, stream=None) -> None:
    """Enqueue the streaming copy the reshard is read against (see include/dcpkv.h)."""
    n = src.numel() * src.element_size() if nbytes is None else nbytes
    _check(_lib.dcpkv_probe_copy(_dptr(src), _dptr(dst), n, _stream(stream)))


def dcpkv_probe_copy_pages(src, dst, src_pages, dst_pages, page_bytes: int, stream=None) -> None:
    """Enqueue the page-list copy (see include/dcpkv.h): page src_pages[i] of src to page
    dst_pages[i] of dst; the capacities are the buffers' sizes in pages."""
    sb, db = src.numel() * src.element_size(), dst.numel() * dst.element_size()
    _check(_lib.dcpkv_probe_copy_pages(_dptr(src), _dptr(dst), _dptr(src_pages), _dptr(dst_pages), src_pages.numel(),
                                       sb // page_bytes, db // page_bytes, page_bytes, _stream(stream)))
