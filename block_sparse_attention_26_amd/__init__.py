"""Python binding of libcosa, the MI355X CoSA prefill-attention library.

Argument marshalling only: every computation runs in the HIP kernels of
``libcosa.so`` (built in-tree by ``block_sparse_attention_26_amd.build``).
There is no fallback: if the library is missing or fails to load, every entry
point raises.

Low-level functions carry the C names (``cosa_kap_order``,
``cosa_osk_attention``, ``cosa_dense_attention``, ``cosa_mask_from_order``,
``cosa_order_from_mask``, ``cosa_osk_attention_masked``, ``cosa_block_mass``,
``cosa_union_order``, ``cosa_osk_decode``, ``cosa_osk_decode_workspace_size``,
``cosa_kap_rank``, ``cosa_cobs_scores``, ``cosa_cobs_workspace_size``, ``cosa_kap_pool_keys``,
``cosa_kap_order_pooled``,
``cosa_validate``,
``cosa_dims``, ``cosa_kap_workspace_size``) and take integer device pointers.
The ``Problem`` class and the ``kap_order`` / ``osk_attention`` /
``dense_attention`` / ``mask_from_order`` / ``order_from_mask`` /
``osk_attention_masked`` / ``block_mass`` / ``union_order`` / ``osk_decode`` / ``kap_rank`` / ``cobs_scores`` / ``pool_keys`` helpers accept torch tensors that already live on the
GPU and allocate the outputs with torch.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

__all__ = [
    "CosaError", "Problem", "load", "library_path",
    "cosa_validate", "cosa_dims", "cosa_kap_workspace_size", "cosa_kap_order",
    "cosa_osk_attention", "cosa_dense_attention", "cosa_status_string",
    "cosa_last_error", "cosa_version", "cosa_mask_from_order", "cosa_order_from_mask",
    "cosa_osk_attention_masked", "cosa_block_mass", "cosa_union_order",
    "cosa_osk_decode", "cosa_osk_decode_workspace_size", "cosa_kap_rank", "cosa_cobs_scores",
    "cosa_cobs_workspace_size", "cosa_kap_pool_keys", "cosa_kap_order_pooled", "cosa_kap_kmax",
    "cosa_osk_decode_noalloc", "kap_order", "pool_keys", "osk_attention", "dense_attention", "mask_from_order", "order_from_mask",
    "osk_attention_masked", "mask_words_for", "block_mass", "union_order", "osk_decode", "kap_rank",
    "cobs_scores",
    "COSA_F32", "COSA_BF16", "EXPORTED_SYMBOLS",
]

COSA_F32, COSA_BF16 = 0, 1
_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB = None

# Every symbol include/cosa.h declares.
EXPORTED_SYMBOLS = (
    "cosa_validate", "cosa_dims", "cosa_kap_workspace_size", "cosa_kap_order",
    "cosa_osk_attention", "cosa_dense_attention", "cosa_status_string",
    "cosa_last_error", "cosa_version", "cosa_mask_from_order", "cosa_order_from_mask",
    "cosa_osk_attention_masked", "cosa_block_mass", "cosa_union_order",
    "cosa_osk_decode", "cosa_osk_decode_workspace_size", "cosa_kap_rank", "cosa_cobs_scores",
    "cosa_cobs_workspace_size", "cosa_kap_pool_keys", "cosa_kap_order_pooled", "cosa_kap_kmax",
    "cosa_osk_decode_noalloc",
)


class CosaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libcosa status {status}: {message}")
        self.status = status


class cosa_problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("h_q", ctypes.c_int32), ("h_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("block", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float), ("num_pages", ctypes.c_int32),
        ("max_blocks_k", ctypes.c_int32),
        ("cu_seqlens_q", ctypes.c_void_p), ("seqlens_k", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("host_cu_seqlens_q", ctypes.c_void_p), ("host_seqlens_k", ctypes.c_void_p),
        ("q_stride_tok", ctypes.c_int64), ("q_stride_head", ctypes.c_int64),
        ("o_stride_tok", ctypes.c_int64), ("o_stride_head", ctypes.c_int64),
    ]


class cosa_dims_t(ctypes.Structure):
    _fields_ = [("total_q", ctypes.c_int32), ("max_nq", ctypes.c_int32),
                ("max_nk", ctypes.c_int32), ("max_nr", ctypes.c_int32),
                ("kmax", ctypes.c_int32)]


def library_path() -> str:
    return os.environ.get("COSA_LIBRARY", os.path.join(_PKG, "libcosa.so"))


def load():
    """Load libcosa.so (once). Raises if it is not built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"libcosa.so not found at {path}; build it with "
            "`python -m block_sparse_attention_26_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(cosa_problem)
    vp, i32, f32, f64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_double, ctypes.c_size_t
    sigs = {
        "cosa_validate": (i32, [P]),
        "cosa_dims": (i32, [P, i32, f64, ctypes.POINTER(cosa_dims_t)]),
        "cosa_kap_workspace_size": (sz, [P, i32, i32]),
        "cosa_kap_kmax": (sz, [P, f64]),
        "cosa_kap_order": (i32, [P, vp, vp, i32, f64, vp, vp, vp, i32, vp, vp, vp, sz, vp]),
        "cosa_osk_attention": (i32, [P, vp, vp, vp, vp, vp, i32, i32, f32, vp, vp, vp, vp, vp, vp]),
        "cosa_dense_attention": (i32, [P, vp, vp, vp, vp, vp, vp]),
        "cosa_mask_from_order": (i32, [P, vp, vp, i32, vp, i32, vp]),
        "cosa_order_from_mask": (i32, [P, vp, i32, vp, vp, i32, vp]),
        "cosa_osk_attention_masked": (i32, [P, vp, vp, vp, vp, i32, i32, f32, vp, vp, vp, vp, vp]),
        "cosa_block_mass": (i32, [P, vp, vp, vp, vp, vp]),
        "cosa_union_order": (i32, [P, vp, vp, i32, vp, vp, i32, vp]),
        "cosa_osk_decode_workspace_size": (sz, [P, i32]),
        "cosa_kap_rank": (i32, [P, i32, f64, vp, vp, vp, vp, i32, vp, vp]),
        "cosa_kap_pool_keys": (i32, [P, vp, i32, vp, i32, vp]),
        "cosa_kap_order_pooled": (i32, [P, vp, vp, i32, f64, vp, vp, vp, i32, vp, vp, vp, sz, vp]),
        "cosa_cobs_workspace_size": (sz, [P, i32]),
        "cosa_cobs_scores": (i32, [P, vp, vp, i32, vp, vp, sz, vp]),
        "cosa_osk_decode": (i32, [P, vp, vp, vp, vp, vp, i32, i32, f32, i32, vp, vp, vp, vp, vp, sz, vp]),
        "cosa_osk_decode_noalloc": (i32, [P, vp, vp, vp, vp, vp, i32, i32, f32, i32, vp, vp, vp, vp, vp]),
        "cosa_status_string": (ctypes.c_char_p, [i32]),
        "cosa_last_error": (ctypes.c_char_p, []),
        "cosa_version": (i32, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        lib = load()
        raise CosaError(status, lib.cosa_last_error().decode())


# ---- raw C entry points (same names as include/cosa.h) ---------------------

def cosa_status_string(status: int) -> str:
    return load().cosa_status_string(status).decode()


def cosa_last_error() -> str:
    return load().cosa_last_error().decode()


def cosa_version() -> int:
    return load().cosa_version()


def cosa_validate(problem: "cosa_problem") -> int:
    return load().cosa_validate(ctypes.byref(problem))


def cosa_dims(problem: "cosa_problem", pool: int, budget: float) -> "cosa_dims_t":
    d = cosa_dims_t()
    _check(load().cosa_dims(ctypes.byref(problem), int(pool), float(budget), ctypes.byref(d)))
    return d


def cosa_kap_kmax(problem: "cosa_problem", budget: float) -> int:
    return load().cosa_kap_kmax(ctypes.byref(problem), float(budget))


def cosa_kap_workspace_size(problem: "cosa_problem", pool: int, with_scores: bool) -> int:
    return load().cosa_kap_workspace_size(ctypes.byref(problem), int(pool), 1 if with_scores else 0)


def cosa_kap_order(problem, q, k_pages, pool, budget, order, hrm, count, kmax,
                   proxy_scores, block_scores, workspace, workspace_bytes, stream) -> None:
    _check(load().cosa_kap_order(ctypes.byref(problem), q, k_pages, int(pool), float(budget),
                                 order, hrm, count, int(kmax), proxy_scores, block_scores,
                                 workspace, int(workspace_bytes), stream))


def cosa_osk_attention(problem, q, k_pages, v_pages, order, count, kmax, group,
                       skip_threshold, o, visited, skipped, skip_bits, lse, stream) -> None:
    _check(load().cosa_osk_attention(ctypes.byref(problem), q, k_pages, v_pages, order, count,
                                     int(kmax), int(group), float(skip_threshold), o, visited,
                                     skipped, skip_bits, lse, stream))


def cosa_dense_attention(problem, q, k_pages, v_pages, o, lse, stream) -> None:
    _check(load().cosa_dense_attention(ctypes.byref(problem), q, k_pages, v_pages, o, lse, stream))


def cosa_mask_from_order(problem, order, count, kmax, mask, mask_words, stream) -> None:
    _check(load().cosa_mask_from_order(ctypes.byref(problem), order, count, int(kmax), mask,
                                       int(mask_words), stream))


def cosa_order_from_mask(problem, mask, mask_words, order, count, kmax, stream) -> None:
    _check(load().cosa_order_from_mask(ctypes.byref(problem), mask, int(mask_words), order, count,
                                       int(kmax), stream))


def cosa_osk_attention_masked(problem, q, k_pages, v_pages, mask, mask_words, group,
                              skip_threshold, o, visited, skipped, lse, stream) -> None:
    _check(load().cosa_osk_attention_masked(ctypes.byref(problem), q, k_pages, v_pages, mask,
                                            int(mask_words), int(group), float(skip_threshold), o,
                                            visited, skipped, lse, stream))


def cosa_kap_pool_keys(problem, k_pages, pool, pooled_keys, last_block_only, stream) -> None:
    _check(load().cosa_kap_pool_keys(ctypes.byref(problem), k_pages, int(pool), pooled_keys,
                                     1 if last_block_only else 0, stream))


def cosa_kap_order_pooled(problem, q, pooled_keys, pool, budget, order, hrm, count, kmax,
                          proxy_scores, block_scores, workspace, workspace_bytes, stream) -> None:
    _check(load().cosa_kap_order_pooled(ctypes.byref(problem), q, pooled_keys, int(pool), float(budget),
                                        order, hrm, count, int(kmax), proxy_scores, block_scores,
                                        workspace, int(workspace_bytes), stream))


def cosa_kap_rank(problem, pool, budget, scores, order, hrm, count, kmax, block_scores, stream) -> None:
    _check(load().cosa_kap_rank(ctypes.byref(problem), int(pool), float(budget), scores, order, hrm, count,
                                int(kmax), block_scores, stream))


def cosa_cobs_workspace_size(problem, pool) -> int:
    return load().cosa_cobs_workspace_size(ctypes.byref(problem), int(pool))


def cosa_cobs_scores(problem, q, k_pages, pool, scores, workspace, workspace_bytes, stream) -> None:
    _check(load().cosa_cobs_scores(ctypes.byref(problem), q, k_pages, int(pool), scores, workspace,
                                   int(workspace_bytes), stream))


def cosa_osk_decode_workspace_size(problem, n_splits) -> int:
    return load().cosa_osk_decode_workspace_size(ctypes.byref(problem), int(n_splits))


def cosa_osk_decode(problem, q, k_pages, v_pages, order, count, kmax, group, skip_threshold, n_splits,
                    o, visited, skipped, lse, workspace, workspace_bytes, stream) -> None:
    _check(load().cosa_osk_decode(ctypes.byref(problem), q, k_pages, v_pages, order, count, int(kmax),
                                  int(group), float(skip_threshold), int(n_splits), o, visited, skipped,
                                  lse, workspace, int(workspace_bytes), stream))


def cosa_osk_decode_noalloc(problem, q, k_pages, v_pages, order, count, kmax, group, skip_threshold, n_splits,
                            o, visited, skipped, lse, stream) -> None:
    _check(load().cosa_osk_decode_noalloc(ctypes.byref(problem), q, k_pages, v_pages, order, count, int(kmax),
                                          int(group), float(skip_threshold), int(n_splits), o, visited, skipped,
                                          lse, stream))


def cosa_union_order(problem, order, count, kmax, union_order, union_count, union_kmax, stream) -> None:
    _check(load().cosa_union_order(ctypes.byref(problem), order, count, int(kmax), union_order,
                                   union_count, int(union_kmax), stream))


def cosa_block_mass(problem, q, k_pages, lse, mass, stream) -> None:
    _check(load().cosa_block_mass(ctypes.byref(problem), q, k_pages, lse, mass, stream))


# ---- torch-facing helpers ---------------------------------------------------

def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t, name, *, shape=None, dtype=None, device=None, contiguous=True):
    """Raise ValueError unless tensor t matches what the library will assume."""
    if t is None:
        raise ValueError(f"{name} is None")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


class Problem:
    """A cosa_problem plus the device and host metadata it points at.

    ``cu_seqlens_q`` / ``seqlens_k`` / ``block_table`` are int32 device
    tensors; ``host_cu_seqlens_q`` / ``host_seqlens_k`` are the same values as
    Python sequences (they are copied into host arrays owned here).
    """

    def __init__(self, *, h_q: int, h_kv: int, head_dim: int, block: int, dtype: int,
                 softmax_scale: float, num_pages: int, cu_seqlens_q, seqlens_k, block_table,
                 host_cu_seqlens_q: Sequence[int], host_seqlens_k: Sequence[int]):
        batch = len(host_seqlens_k)
        self._hcu = (ctypes.c_int32 * (batch + 1))(*[int(x) for x in host_cu_seqlens_q])
        self._hlk = (ctypes.c_int32 * batch)(*[int(x) for x in host_seqlens_k])
        self._dev = (cu_seqlens_q, seqlens_k, block_table)  # keep alive
        self.c = cosa_problem(
            batch=batch, h_q=h_q, h_kv=h_kv, head_dim=head_dim, block=block, dtype=dtype,
            softmax_scale=softmax_scale, num_pages=num_pages,
            max_blocks_k=int(block_table.shape[1]),
            cu_seqlens_q=cu_seqlens_q.data_ptr(), seqlens_k=seqlens_k.data_ptr(),
            block_table=block_table.data_ptr(),
            host_cu_seqlens_q=ctypes.cast(self._hcu, ctypes.c_void_p),
            host_seqlens_k=ctypes.cast(self._hlk, ctypes.c_void_p),
        )
        self.group = h_q // h_kv
        self._dims = {}

    # -- tensor checks (shapes and dtypes the C ABI assumes) --------------------
    def torch_dtype(self):
        import torch
        return torch.bfloat16 if self.c.dtype == COSA_BF16 else torch.float32

    def _rows_view(self, t, name):
        """q or o: a [total_q, h_q, head_dim] view whose head_dim is contiguous
        (token and head strides are passed to the library)."""
        c = self.c
        _need(t, name, shape=(self.dims().total_q, c.h_q, c.head_dim), dtype=self.torch_dtype(),
              contiguous=False)
        if t.stride(2) != 1:
            raise ValueError(f"{name} must have a contiguous head_dim (stride {t.stride(2)})")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        return t

    def check_pages(self, k_pages, name="k_pages"):
        c = self.c
        _need(k_pages, name, shape=(c.num_pages, c.h_kv, c.block, c.head_dim), dtype=self.torch_dtype())
        if not k_pages.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        return k_pages

    def check_lists(self, order, count, device=None):
        import torch
        c = self.c
        d = self.dims()
        if order.dim() != 4:
            raise ValueError(f"order must be [batch, h_kv, max_nq, kmax], got shape {tuple(order.shape)}")
        _need(order, "order", shape=(c.batch, c.h_kv, d.max_nq, order.shape[3]), dtype=torch.int32,
              device=device)
        _need(count, "count", shape=(c.batch, c.h_kv, d.max_nq), dtype=torch.int32, device=device)
        return int(order.shape[3])

    def for_tensors(self, q, o=None) -> "cosa_problem":
        """A copy of the problem struct carrying q's (and o's) element strides."""
        c = cosa_problem.from_buffer_copy(self.c)
        self._rows_view(q, "q")
        c.q_stride_tok, c.q_stride_head = q.stride(0), q.stride(1)
        if o is not None:
            self._rows_view(o, "o")
            if o.device != q.device:
                raise ValueError("o and q must be on the same device")
            c.o_stride_tok, c.o_stride_head = o.stride(0), o.stride(1)
        return c

    def new_rows(self, q):
        """A contiguous output tensor shaped like q."""
        import torch
        return torch.empty(tuple(q.shape), dtype=q.dtype, device=q.device)

    @classmethod
    def from_case(cls, case, device="cuda"):
        """Build from a ``synthetic.Case``, copying its metadata to the device."""
        dt = COSA_BF16 if case.dtype == "bf16" else COSA_F32
        return cls(h_q=case.h_q, h_kv=case.h_kv, head_dim=case.head_dim, block=case.block,
                   dtype=dt, softmax_scale=case.scale, num_pages=int(case.k_pages.shape[0]),
                   cu_seqlens_q=case.cu_seqlens_q.to(device), seqlens_k=case.seqlens_k.to(device),
                   block_table=case.block_table.to(device),
                   host_cu_seqlens_q=case.cu_seqlens_q.tolist(),
                   host_seqlens_k=case.seqlens_k.tolist())

    def dims(self, pool: int = 0, budget: float = 0.0) -> cosa_dims_t:
        """Padded extents (cached: a Problem's shape does not change after construction)."""
        key = (int(pool), float(budget))
        d = self._dims.get(key)
        if d is None:
            d = self._dims[key] = cosa_dims(self.c, pool, budget)
        return d

    def validate(self) -> int:
        return cosa_validate(self.c)


def pool_keys(problem: Problem, k_pages, pool: int, *, out=None, last_block_only: bool = False, stream=None):
    """Pooled keys [num_pages, h_kv, B/p, d] (into ``out`` when given)."""
    import torch
    c = problem.c
    problem.check_pages(k_pages)
    if out is None:
        out = torch.zeros((c.num_pages, c.h_kv, c.block // pool, c.head_dim), dtype=k_pages.dtype,
                          device=k_pages.device)
    _need(out, "out", shape=(c.num_pages, c.h_kv, c.block // pool, c.head_dim), dtype=k_pages.dtype,
          device=k_pages.device)
    cosa_kap_pool_keys(c, k_pages.data_ptr(), pool, out.data_ptr(), last_block_only, _stream(stream))
    return out


def kap_order(problem: Problem, q, k_pages, pool: int, budget: float, *, kmax=None,
              export_scores: bool = False, export_block_scores: bool = False,
              workspace=None, pooled_keys=None, stream=None):
    """Run the proxy; returns dict(order, hrm, count, kmax[, P][, s]). With
    ``pooled_keys`` (from ``pool_keys``) the keys are not pooled again."""
    import torch
    dev = q.device
    c = problem.for_tensors(q)
    if pooled_keys is None:
        problem.check_pages(k_pages)
    d = problem.dims(pool, budget)
    kmax = d.kmax if kmax is None else int(kmax)
    order = torch.empty((problem.c.batch, problem.c.h_kv, d.max_nq, kmax), dtype=torch.int32, device=dev)
    hrm = torch.empty(order.shape, dtype=torch.uint8, device=dev)
    count = torch.empty(order.shape[:3], dtype=torch.int32, device=dev)
    P = (torch.empty((problem.c.batch, problem.c.h_q, d.max_nr, d.max_nk), dtype=torch.float32, device=dev)
         if export_scores else None)
    s = (torch.empty((problem.c.batch, problem.c.h_kv, d.max_nq, d.max_nk), dtype=torch.float32, device=dev)
         if export_block_scores else None)
    ws_bytes = cosa_kap_workspace_size(problem.c, pool, P is None)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    if pooled_keys is None:
        cosa_kap_order(c, q.data_ptr(), k_pages.data_ptr(), pool, budget, order.data_ptr(),
                       hrm.data_ptr(), count.data_ptr(), kmax, _ptr(P), _ptr(s), workspace.data_ptr(),
                       workspace.numel(), _stream(stream))
    else:
        pc = problem.c
        _need(pooled_keys, "pooled_keys", shape=(pc.num_pages, pc.h_kv, pc.block // pool, pc.head_dim),
              dtype=problem.torch_dtype(), device=dev)
        cosa_kap_order_pooled(c, q.data_ptr(), pooled_keys.data_ptr(), pool, budget, order.data_ptr(),
                              hrm.data_ptr(), count.data_ptr(), kmax, _ptr(P), _ptr(s), workspace.data_ptr(),
                              workspace.numel(), _stream(stream))
    out = {"order": order, "hrm": hrm, "count": count, "kmax": kmax, "workspace": workspace}
    if P is not None:
        out["P"] = P
    if s is not None:
        out["s"] = s
    return out


def osk_attention(problem: Problem, q, k_pages, v_pages, order, count, tau: float, *,
                  skip_bits: bool = False, lse: bool = False, out=None, stream=None):
    """Run the ordered-skipping kernel; returns dict(O, visited, skipped[, skip_bits][, lse])."""
    import torch
    dev = q.device
    d = problem.dims()
    problem.check_pages(k_pages)
    problem.check_pages(v_pages, "v_pages")
    kmax = problem.check_lists(order, count, dev)
    o = problem.new_rows(q) if out is None else out
    c = problem.for_tensors(q, o)
    vis = torch.empty((problem.c.batch, problem.c.h_q, d.max_nq), dtype=torch.int32, device=dev)
    skp = torch.empty_like(vis)
    bits = (torch.empty((problem.c.batch, problem.c.h_q, d.max_nq, kmax), dtype=torch.uint8, device=dev)
            if skip_bits else None)
    ls = torch.empty((problem.c.h_q, d.total_q), dtype=torch.float32, device=dev) if lse else None
    cosa_osk_attention(c, q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(),
                       order.data_ptr(), count.data_ptr(), kmax, problem.group, tau, o.data_ptr(),
                       vis.data_ptr(), skp.data_ptr(), _ptr(bits), _ptr(ls), _stream(stream))
    res = {"O": o, "visited": vis, "skipped": skp}
    if bits is not None:
        res["skip_bits"] = bits
    if ls is not None:
        res["lse"] = ls
    return res


def dense_attention(problem: Problem, q, k_pages, v_pages, *, lse: bool = False, out=None,
                    stream=None):
    """Dense causal attention; returns dict(O[, lse])."""
    import torch
    d = problem.dims()
    problem.check_pages(k_pages)
    problem.check_pages(v_pages, "v_pages")
    o = problem.new_rows(q) if out is None else out
    c = problem.for_tensors(q, o)
    ls = torch.empty((problem.c.h_q, d.total_q), dtype=torch.float32, device=q.device) if lse else None
    cosa_dense_attention(c, q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(),
                         o.data_ptr(), _ptr(ls), _stream(stream))
    res = {"O": o}
    if ls is not None:
        res["lse"] = ls
    return res


def mask_words_for(problem: Problem) -> int:
    return max(1, (problem.dims().max_nk + 63) // 64)


def mask_from_order(problem: Problem, order, count, *, mask_words=None, stream=None):
    """Binary block mask (int64 view of the uint64 words) of the listed blocks."""
    import torch
    d = problem.dims()
    problem.check_lists(order, count, order.device)
    mw = mask_words_for(problem) if mask_words is None else int(mask_words)
    mask = torch.empty((problem.c.batch, problem.c.h_kv, d.max_nq, mw), dtype=torch.int64, device=order.device)
    cosa_mask_from_order(problem.c, order.data_ptr(), count.data_ptr(), int(order.shape[3]),
                         mask.data_ptr(), mw, _stream(stream))
    return mask


def order_from_mask(problem: Problem, mask, kmax: int, *, device=None, stream=None):
    """Ascending list of the selected causal blocks (mask None: every causal block);
    returns dict(order, count)."""
    import torch
    d = problem.dims()
    dev = mask.device if mask is not None else device
    if mask is not None:
        if mask.dim() != 4:
            raise ValueError(f"mask must be [batch, h_kv, max_nq, mask_words], got shape {tuple(mask.shape)}")
        _need(mask, "mask", shape=(problem.c.batch, problem.c.h_kv, d.max_nq, mask.shape[3]), dtype=torch.int64)
    order = torch.empty((problem.c.batch, problem.c.h_kv, d.max_nq, int(kmax)), dtype=torch.int32, device=dev)
    count = torch.empty(order.shape[:3], dtype=torch.int32, device=dev)
    mw = int(mask.shape[3]) if mask is not None else 0
    cosa_order_from_mask(problem.c, _ptr(mask), mw, order.data_ptr(), count.data_ptr(), int(kmax),
                         _stream(stream))
    return {"order": order, "count": count}


def osk_attention_masked(problem: Problem, q, k_pages, v_pages, mask, tau: float, *, lse: bool = False,
                         out=None, stream=None):
    """Control-flow-skipping walk over a binary block mask; returns dict(O, visited, skipped[, lse])."""
    import torch
    dev = q.device
    d = problem.dims()
    problem.check_pages(k_pages)
    problem.check_pages(v_pages, "v_pages")
    if mask.dim() != 4:
        raise ValueError(f"mask must be [batch, h_kv, max_nq, mask_words], got shape {tuple(mask.shape)}")
    _need(mask, "mask", shape=(problem.c.batch, problem.c.h_kv, d.max_nq, mask.shape[3]), dtype=torch.int64,
          device=dev)
    o = problem.new_rows(q) if out is None else out
    c = problem.for_tensors(q, o)
    vis = torch.empty((problem.c.batch, problem.c.h_q, d.max_nq), dtype=torch.int32, device=dev)
    skp = torch.empty_like(vis)
    ls = torch.empty((problem.c.h_q, d.total_q), dtype=torch.float32, device=dev) if lse else None
    cosa_osk_attention_masked(c, q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(),
                              mask.data_ptr(), int(mask.shape[3]), problem.group, tau, o.data_ptr(),
                              vis.data_ptr(), skp.data_ptr(), _ptr(ls), _stream(stream))
    res = {"O": o, "visited": vis, "skipped": skp}
    if ls is not None:
        res["lse"] = ls
    return res


def kap_rank(problem: Problem, scores, pool: int, budget: float, *, kmax=None, export_block_scores=False,
             stream=None):
    """Rank/sort pass over given scores; returns dict(order, hrm, count, kmax[, s])."""
    import torch
    dev = scores.device
    d = problem.dims(pool, budget)
    _need(scores, "scores", shape=(problem.c.batch, problem.c.h_q, d.max_nr, d.max_nk), dtype=torch.float32)
    kmax = d.kmax if kmax is None else int(kmax)
    order = torch.empty((problem.c.batch, problem.c.h_kv, d.max_nq, kmax), dtype=torch.int32, device=dev)
    hrm = torch.empty(order.shape, dtype=torch.uint8, device=dev)
    count = torch.empty(order.shape[:3], dtype=torch.int32, device=dev)
    s = (torch.empty((problem.c.batch, problem.c.h_kv, d.max_nq, d.max_nk), dtype=torch.float32, device=dev)
         if export_block_scores else None)
    cosa_kap_rank(problem.c, pool, budget, scores.data_ptr(), order.data_ptr(), hrm.data_ptr(),
                  count.data_ptr(), kmax, _ptr(s), _stream(stream))
    out = {"order": order, "hrm": hrm, "count": count, "kmax": kmax}
    if s is not None:
        out["s"] = s
    return out


def cobs_scores(problem: Problem, q, k_pages, pool: int, *, workspace=None, stream=None):
    """Second-order block scores [batch, h_q, max_nr, max_nk] fp32."""
    import torch
    d = problem.dims(pool, 0.0)
    c = problem.for_tensors(q)
    problem.check_pages(k_pages)
    out = torch.empty((problem.c.batch, problem.c.h_q, d.max_nr, d.max_nk), dtype=torch.float32, device=q.device)
    ws_bytes = cosa_cobs_workspace_size(problem.c, pool)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    cosa_cobs_scores(c, q.data_ptr(), k_pages.data_ptr(), pool, out.data_ptr(), workspace.data_ptr(),
                     workspace.numel(), _stream(stream))
    return out


def osk_decode(problem: Problem, q, k_pages, v_pages, order, count, tau: float, n_splits: int, *,
               lse: bool = False, out=None, workspace=None, stream=None):
    """Decode step over the proxy's lists, split into n_splits segments;
    returns dict(O, visited, skipped[, lse])."""
    import torch
    dev = q.device
    d = problem.dims()
    problem.check_pages(k_pages)
    problem.check_pages(v_pages, "v_pages")
    problem.check_lists(order, count, dev)
    o = problem.new_rows(q) if out is None else out
    c = problem.for_tensors(q, o)
    vis = torch.empty((problem.c.batch, problem.c.h_q, d.max_nq), dtype=torch.int32, device=dev)
    skp = torch.empty_like(vis)
    ls = torch.empty((problem.c.h_q, d.total_q), dtype=torch.float32, device=dev) if lse else None
    ws_bytes = cosa_osk_decode_workspace_size(problem.c, n_splits)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    cosa_osk_decode(c, q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), order.data_ptr(),
                    count.data_ptr(), int(order.shape[3]), problem.group, tau, n_splits, o.data_ptr(),
                    vis.data_ptr(), skp.data_ptr(), _ptr(ls), workspace.data_ptr(), workspace.numel(),
                    _stream(stream))
    res = {"O": o, "visited": vis, "skipped": skp}
    if ls is not None:
        res["lse"] = ls
    return res


def union_order(problem: Problem, order, count, *, union_kmax=None, stream=None):
    """Block-union lists (one table per sequence and KV group, cut causally per
    query block); returns dict(order, count)."""
    import torch
    d = problem.dims()
    problem.check_lists(order, count, order.device)
    uk = d.max_nk if union_kmax is None else int(union_kmax)
    uo = torch.empty((problem.c.batch, problem.c.h_kv, d.max_nq, uk), dtype=torch.int32, device=order.device)
    uc = torch.empty(uo.shape[:3], dtype=torch.int32, device=order.device)
    cosa_union_order(problem.c, order.data_ptr(), count.data_ptr(), int(order.shape[3]), uo.data_ptr(),
                     uc.data_ptr(), uk, _stream(stream))
    return {"order": uo, "count": uc}


def block_mass(problem: Problem, q, k_pages, lse, *, stream=None):
    """Exact attention mass [batch, h_q, max_nq, max_nk] of every causal block,
    given the rows' log-sum-exp from ``dense_attention(..., lse=True)``."""
    import torch
    d = problem.dims()
    c = problem.for_tensors(q)
    problem.check_pages(k_pages)
    _need(lse, "lse", shape=(problem.c.h_q, d.total_q), dtype=torch.float32, device=q.device)
    mass = torch.empty((problem.c.batch, problem.c.h_q, d.max_nq, d.max_nk), dtype=torch.float32,
                       device=q.device)
    cosa_block_mass(c, q.data_ptr(), k_pages.data_ptr(), lse.data_ptr(), mass.data_ptr(),
                    _stream(stream))
    return mass


def dense_causal_flops(seqlens_q: Sequence[int], seqlens_k: Sequence[int], h_q: int, head_dim: int) -> float:
    """4 * d * (number of causal (query, key) pairs) * h_q: QK^T and PV of dense attention."""
    pairs = 0
    for lq, lk in zip(seqlens_q, seqlens_k):
        off = lk - lq
        pairs += lq * (off + 1) + lq * (lq - 1) // 2
    return 4.0 * head_dim * pairs * h_q


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
