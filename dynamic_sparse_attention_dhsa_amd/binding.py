"""Python binding of the DHSA C ABI (include/dhsa.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream, every stage runs in the gfx950 kernels of ``libdhsa.so``.  There is
no fallback: if the library is missing or a tensor is not on the GPU, these
functions raise.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdhsa.so")

DHSA_OK = 0
DHSA_F32 = 0
DHSA_BF16 = 1
STATUS_NAMES = {0: "DHSA_OK", 1: "DHSA_ERR_NULL_ARG", 2: "DHSA_ERR_BAD_SHAPE", 3: "DHSA_ERR_BAD_LAYOUT",
                4: "DHSA_ERR_BAD_BUDGET", 5: "DHSA_ERR_UNSUPPORTED", 6: "DHSA_ERR_LAUNCH", 7: "DHSA_ERR_WORKSPACE"}

# every entry point declared in include/dhsa.h
EXPORTS = ("dhsa_abi_version", "dhsa_status_str", "dhsa_validate_layout", "dhsa_route_plan",
           "dhsa_chunk_summarize", "dhsa_route", "dhsa_route_grouped", "dhsa_sparse_prefill",
           "dhsa_adjacent_similarity", "dhsa_chunk_boundaries", "dhsa_decode_workspace_bytes",
           "dhsa_decode_load_prefix", "dhsa_decode_step", "dhsa_route_plan_tokens", "dhsa_route_tokens",
           "dhsa_decode_step_noalloc")


class DhsaError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: {message}")
        self.status = status
        self.name = STATUS_NAMES.get(status, str(status))


class DecodeStateStruct(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
                ("max_chunks", ctypes.c_int32), ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
                ("seq_len", ctypes.c_void_p), ("num_closed", ctypes.c_void_p), ("chunk_start", ctypes.c_void_p),
                ("k_sum", ctypes.c_void_p), ("q_run", ctypes.c_void_p), ("k_run", ctypes.c_void_p),
                ("status", ctypes.c_void_p)]


class LayoutStruct(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("total_tokens", ctypes.c_int32),
                ("total_chunks", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("cu_seqlens", ctypes.c_void_p), ("cu_chunks", ctypes.c_void_p),
                ("seq_chunk_start", ctypes.c_void_p), ("h_cu_seqlens", ctypes.c_void_p),
                ("h_cu_chunks", ctypes.c_void_p), ("h_seq_chunk_start", ctypes.c_void_p)]


_LIB = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdhsa.so (after torch, so both share torch's HIP runtime)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with dynamic_sparse_attention_dhsa_amd.build.build()")
    lib = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lp = ctypes.POINTER(LayoutStruct)
    lib.dhsa_abi_version.restype = i32
    lib.dhsa_status_str.restype = ctypes.c_char_p
    lib.dhsa_status_str.argtypes = [i32]
    lib.dhsa_validate_layout.restype = i32
    lib.dhsa_validate_layout.argtypes = [lp]
    lib.dhsa_route_plan.restype = i32
    lib.dhsa_route_plan.argtypes = [lp, vp, vp, ctypes.POINTER(i64)]
    lib.dhsa_route_plan_tokens.restype = i32
    lib.dhsa_route_plan_tokens.argtypes = [lp, vp, vp, ctypes.POINTER(i64)]
    lib.dhsa_route_tokens.restype = i32
    lib.dhsa_route_tokens.argtypes = [lp, vp, vp, vp, vp, vp, vp, i64, i32, vp, vp]
    lib.dhsa_chunk_summarize.restype = i32
    lib.dhsa_chunk_summarize.argtypes = [lp, vp, vp, vp, vp, vp]
    for name in ("dhsa_route", "dhsa_route_grouped"):
        getattr(lib, name).restype = i32
        getattr(lib, name).argtypes = [lp, vp, vp, vp, vp, i64, vp, vp]
    lib.dhsa_sparse_prefill.restype = i32
    lib.dhsa_sparse_prefill.argtypes = [lp, vp, vp, vp, vp, vp, i64, vp, ctypes.c_float, vp, vp, vp]
    lib.dhsa_adjacent_similarity.restype = i32
    lib.dhsa_adjacent_similarity.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, ctypes.c_float, vp, vp, vp]
    lib.dhsa_chunk_boundaries.restype = i32
    lib.dhsa_chunk_boundaries.argtypes = [i32, i32, vp, vp, vp, i32, i32, vp, vp, vp, vp]
    dsp = ctypes.POINTER(DecodeStateStruct)
    lib.dhsa_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.dhsa_decode_workspace_bytes.argtypes = [dsp, i32, i32]
    lib.dhsa_decode_load_prefix.restype = i32
    lib.dhsa_decode_load_prefix.argtypes = [dsp, lp, vp, vp, vp, vp]
    lib.dhsa_decode_step.restype = i32
    lib.dhsa_decode_step.argtypes = [dsp, vp, vp, vp, i32, i32, ctypes.c_float, i32, i32, ctypes.c_float, vp, vp,
                                     vp, ctypes.c_size_t, vp]
    lib.dhsa_decode_step_noalloc.restype = i32
    lib.dhsa_decode_step_noalloc.argtypes = [dsp, vp, vp, vp, i32, i32, ctypes.c_float, i32, i32, ctypes.c_float, vp,
                                             vp, vp]
    if lib.dhsa_abi_version() != 1:
        raise RuntimeError("libdhsa.so ABI version mismatch")
    _LIB = lib
    return lib


def _check(status: int, where: str) -> None:
    if status != DHSA_OK:
        msg = load_library().dhsa_status_str(status).decode()
        raise DhsaError(status, where, msg)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _on_gpu(t: torch.Tensor) -> bool:
    """A GPU tensor on the current device (the library launches on that device's current stream)."""
    return t.is_cuda and t.device.index == torch.cuda.current_device()


def _require(t: Optional[torch.Tensor], name: str, shape, dtype: torch.dtype) -> None:
    """A caller-supplied tensor the kernels read or write in full: contiguous, of this dtype and exact
    shape, on the current GPU (None: the binding allocates it)."""
    if t is None:
        return
    if not _on_gpu(t) or t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise DhsaError(2, name, f"expected a contiguous {dtype} tensor {list(shape)} on the current GPU, "
                                 f"got {t.dtype} {list(t.shape)} on {t.device}")


def _host_i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


class Layout:
    """A packed varlen batch: device offsets plus their host mirrors, as the C ABI wants them."""

    def __init__(self, cu_seqlens, cu_chunks, seq_chunk_start, num_q_heads: int, num_kv_heads: int,
                 head_dim: int, dtype: torch.dtype, device="cuda"):
        self.h_cu_seqlens = _host_i32(cu_seqlens)
        self.h_cu_chunks = _host_i32(cu_chunks)
        self.h_seq_chunk_start = _host_i32(seq_chunk_start)
        if dtype == torch.bfloat16:
            code = DHSA_BF16
        elif dtype == torch.float32:
            code = DHSA_F32
        else:
            raise DhsaError(5, "Layout", f"unsupported dtype {dtype}")
        self.dtype = dtype
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.d_cu_seqlens = torch.from_numpy(self.h_cu_seqlens).to(self.device)
        self.d_cu_chunks = torch.from_numpy(self.h_cu_chunks).to(self.device)
        self.d_seq_chunk_start = torch.from_numpy(self.h_seq_chunk_start).to(self.device)
        self.num_seqs = self.h_cu_seqlens.size - 1
        self.total_tokens = int(self.h_cu_seqlens[-1])
        self.total_chunks = int(self.h_cu_chunks.size - 1)
        self.num_q_heads, self.num_kv_heads, self.head_dim = num_q_heads, num_kv_heads, head_dim
        self.struct = LayoutStruct(self.num_seqs, self.total_tokens, self.total_chunks, num_q_heads,
                                   num_kv_heads, head_dim, code, self.d_cu_seqlens.data_ptr(),
                                   self.d_cu_chunks.data_ptr(), self.d_seq_chunk_start.data_ptr(),
                                   self.h_cu_seqlens.ctypes.data, self.h_cu_chunks.ctypes.data,
                                   self.h_seq_chunk_start.ctypes.data)

    def validate(self) -> None:
        _check(load_library().dhsa_validate_layout(ctypes.byref(self.struct)), "dhsa_validate_layout")

    def _check_tensor(self, t: torch.Tensor, heads: int, name: str) -> None:
        if not _on_gpu(t):
            raise DhsaError(1, name, "tensor is not on the current GPU")
        if self.device.index != t.device.index:
            raise DhsaError(1, name, f"layout is on {self.device}, the current device is {t.device}")
        if t.dtype != self.dtype:
            raise DhsaError(2, name, f"dtype {t.dtype} != layout dtype {self.dtype}")
        if tuple(t.shape) != (self.total_tokens, heads, self.head_dim) or not t.is_contiguous():
            raise DhsaError(2, name, f"expected contiguous [{self.total_tokens}, {heads}, {self.head_dim}], "
                                     f"got {tuple(t.shape)}")


class RoutePlan:
    """CSR row pointers (host and device) for a per-chunk budget."""

    def __init__(self, layout: Layout, topk):
        lib = load_library()
        self.h_topk = _host_i32(topk)
        if self.h_topk.shape != (layout.total_chunks,):
            raise DhsaError(2, "route_plan", "topk needs one entry per chunk")
        self.h_row_ptr = np.zeros(layout.total_chunks + 1, np.int32)
        nnz = ctypes.c_int64(0)
        _check(lib.dhsa_route_plan(ctypes.byref(layout.struct), self.h_topk.ctypes.data,
                                   self.h_row_ptr.ctypes.data, ctypes.byref(nnz)), "dhsa_route_plan")
        self.nnz = int(nnz.value)
        self.d_row_ptr = torch.from_numpy(self.h_row_ptr).to(layout.device)

    @classmethod
    def from_row_ptr(cls, layout: Layout, row_ptr) -> "RoutePlan":
        self = cls.__new__(cls)
        self.h_topk = None
        self.h_row_ptr = _host_i32(row_ptr)
        self.nnz = int(self.h_row_ptr[-1])
        self.d_row_ptr = torch.from_numpy(self.h_row_ptr).to(layout.device)
        return self


class TokenPlan(RoutePlan):
    """CSR row pointers for a per-chunk token budget (dhsa_route_plan_tokens): row i holds the most
    chunks any ranking could keep, so rows carry -1 padding after their diagonal."""

    def __init__(self, layout: Layout, token_budget):
        lib = load_library()
        self.h_topk = None
        self.h_token_budget = _host_i32(token_budget)
        if self.h_token_budget.shape != (layout.total_chunks,):
            raise DhsaError(2, "route_plan_tokens", "token_budget needs one entry per chunk")
        self.h_row_ptr = np.zeros(layout.total_chunks + 1, np.int32)
        nnz = ctypes.c_int64(0)
        _check(lib.dhsa_route_plan_tokens(ctypes.byref(layout.struct), self.h_token_budget.ctypes.data,
                                          self.h_row_ptr.ctypes.data, ctypes.byref(nnz)), "dhsa_route_plan_tokens")
        self.nnz = int(nnz.value)
        self.d_row_ptr = torch.from_numpy(self.h_row_ptr).to(layout.device)
        self.d_token_budget = torch.from_numpy(self.h_token_budget).to(layout.device)


def chunk_summarize(layout: Layout, q: torch.Tensor, k: torch.Tensor,
                    q_sum: Optional[torch.Tensor] = None, k_sum: Optional[torch.Tensor] = None
                    ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Stage 1 (dhsa_chunk_summarize): fp32 q_sum [C, Hq, d], k_sum [C, Hkv, d]."""
    layout._check_tensor(q, layout.num_q_heads, "q")
    layout._check_tensor(k, layout.num_kv_heads, "k")
    C = layout.total_chunks
    _require(q_sum, "q_sum", (C, layout.num_q_heads, layout.head_dim), torch.float32)
    _require(k_sum, "k_sum", (C, layout.num_kv_heads, layout.head_dim), torch.float32)
    if q_sum is None:
        q_sum = torch.empty((C, layout.num_q_heads, layout.head_dim), dtype=torch.float32, device=q.device)
    if k_sum is None:
        k_sum = torch.empty((C, layout.num_kv_heads, layout.head_dim), dtype=torch.float32, device=q.device)
    _check(load_library().dhsa_chunk_summarize(ctypes.byref(layout.struct), _ptr(q), _ptr(k), _ptr(q_sum),
                                               _ptr(k_sum), _stream()), "dhsa_chunk_summarize")
    return q_sum, k_sum


def route(layout: Layout, plan: RoutePlan, q_sum: torch.Tensor, k_sum: torch.Tensor,
          block_idx: Optional[torch.Tensor] = None, grouped: bool = False) -> torch.Tensor:
    """Stage 2 (dhsa_route, or dhsa_route_grouped when ``grouped``: one selection per KV head, shared
    by its query heads): kept key chunks, int32 [Hq, nnz], rows ascending with the diagonal last."""
    if block_idx is None:
        block_idx = torch.empty((layout.num_q_heads, plan.nnz), dtype=torch.int32, device=q_sum.device)
    C = layout.total_chunks
    _require(q_sum, "q_sum", (C, layout.num_q_heads, layout.head_dim), torch.float32)
    _require(k_sum, "k_sum", (C, layout.num_kv_heads, layout.head_dim), torch.float32)
    _require(block_idx, "block_idx", (layout.num_q_heads, plan.nnz), torch.int32)
    name = "dhsa_route_grouped" if grouped else "dhsa_route"
    _check(getattr(load_library(), name)(ctypes.byref(layout.struct), _ptr(q_sum), _ptr(k_sum),
                                         _ptr(plan.d_row_ptr), plan.h_row_ptr.ctypes.data, plan.nnz,
                                         _ptr(block_idx), _stream()),
           name)
    return block_idx


def route_tokens(layout: Layout, plan: TokenPlan, q_sum: torch.Tensor, k_sum: torch.Tensor,
                 block_idx: Optional[torch.Tensor] = None, grouped: bool = False) -> torch.Tensor:
    """Stage 2 under a token budget (dhsa_route_tokens): int32 [Hq, nnz], each row its kept chunks
    ascending, the diagonal, then -1 up to the row's capacity."""
    if not isinstance(plan, TokenPlan):
        raise DhsaError(2, "route_tokens", "needs a TokenPlan")
    if block_idx is None:
        block_idx = torch.empty((layout.num_q_heads, plan.nnz), dtype=torch.int32, device=q_sum.device)
    C = layout.total_chunks
    _require(q_sum, "q_sum", (C, layout.num_q_heads, layout.head_dim), torch.float32)
    _require(k_sum, "k_sum", (C, layout.num_kv_heads, layout.head_dim), torch.float32)
    _require(block_idx, "block_idx", (layout.num_q_heads, plan.nnz), torch.int32)
    _check(load_library().dhsa_route_tokens(ctypes.byref(layout.struct), _ptr(q_sum), _ptr(k_sum),
                                            _ptr(plan.d_token_budget), plan.h_token_budget.ctypes.data,
                                            _ptr(plan.d_row_ptr), plan.h_row_ptr.ctypes.data, plan.nnz,
                                            int(bool(grouped)), _ptr(block_idx), _stream()), "dhsa_route_tokens")
    return block_idx


def sparse_prefill(layout: Layout, plan: RoutePlan, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                   block_idx: torch.Tensor, softmax_scale: Optional[float] = None, return_lse: bool = False,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """Stage 3 (dhsa_sparse_prefill): out [T, Hq, d] in q's dtype, optional lse [Hq, T] fp32."""
    layout._check_tensor(q, layout.num_q_heads, "q")
    layout._check_tensor(k, layout.num_kv_heads, "k")
    layout._check_tensor(v, layout.num_kv_heads, "v")
    _require(block_idx, "block_idx", (layout.num_q_heads, plan.nnz), torch.int32)
    _require(out, "out", (layout.total_tokens, layout.num_q_heads, layout.head_dim), layout.dtype)
    _require(lse, "lse", (layout.num_q_heads, layout.total_tokens), torch.float32)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(layout.head_dim)
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((layout.num_q_heads, layout.total_tokens), dtype=torch.float32, device=q.device)
    _check(load_library().dhsa_sparse_prefill(ctypes.byref(layout.struct), _ptr(q), _ptr(k), _ptr(v),
                                              _ptr(plan.d_row_ptr), plan.h_row_ptr.ctypes.data, plan.nnz,
                                              _ptr(block_idx), float(softmax_scale), _ptr(out), _ptr(lse),
                                              _stream()), "dhsa_sparse_prefill")
    return (out, lse) if return_lse else out


def prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens, cu_chunks, seq_chunk_start, topk=None,
            softmax_scale: Optional[float] = None, return_lse: bool = False, grouped: bool = False,
            token_budget=None):
    """The whole path: summaries, routing (per query head, or per KV head when ``grouped``; a chunk
    budget ``topk`` or a token budget ``token_budget``, one entry per chunk), sparse attention.
    Returns a dict of device tensors."""
    if (topk is None) == (token_budget is None):
        raise DhsaError(2, "prefill", "give exactly one of topk and token_budget")
    layout = Layout(cu_seqlens, cu_chunks, seq_chunk_start, q.shape[1], k.shape[1], q.shape[2], q.dtype,
                    device=q.device)
    q_sum, k_sum = chunk_summarize(layout, q, k)
    if token_budget is None:
        plan = RoutePlan(layout, topk)
        block_idx = route(layout, plan, q_sum, k_sum, grouped=grouped)
    else:
        plan = TokenPlan(layout, token_budget)
        block_idx = route_tokens(layout, plan, q_sum, k_sum, grouped=grouped)
    res = sparse_prefill(layout, plan, q, k, v, block_idx, softmax_scale, return_lse=return_lse)
    out, lse = res if return_lse else (res, None)
    return dict(out=out, lse=lse, q_sum=q_sum, k_sum=k_sum, row_ptr=plan.h_row_ptr, block_idx=block_idx,
                layout=layout, plan=plan)


# ----------------------------------------------------------------------------- online chunking (own rule)

class SeqLayout:
    """Token offsets of a batch for the chunking calls: device copy plus host mirror (built once)."""

    def __init__(self, cu_seqlens, device="cuda"):
        self.h_cu_seqlens = _host_i32(cu_seqlens)
        self.d_cu_seqlens = torch.from_numpy(self.h_cu_seqlens).to(torch.device(device))
        self.num_seqs = self.h_cu_seqlens.size - 1
        self.total_tokens = int(self.h_cu_seqlens[-1])


def _seq_layout(cu_seqlens, device) -> SeqLayout:
    return cu_seqlens if isinstance(cu_seqlens, SeqLayout) else SeqLayout(cu_seqlens, device)


def adjacent_similarity(k: torch.Tensor, cu_seqlens, tau: float, sim: Optional[torch.Tensor] = None,
                        cut_bits: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """dhsa_adjacent_similarity: sim float32 [T] (cosine of adjacent key rows over all KV heads, 1 at
    sequence starts and zero rows) and cut_bits int64 [ceil(T/64)] (bit t set when sim[t] < tau).
    ``cu_seqlens``: a SeqLayout, or host offsets (copied to the device on each call)."""
    if not _on_gpu(k) or k.dim() != 3 or not k.is_contiguous():
        raise DhsaError(2, "k", "expected a contiguous GPU tensor [T, Hkv, d]")
    if k.dtype == torch.bfloat16:
        code = DHSA_BF16
    elif k.dtype == torch.float32:
        code = DHSA_F32
    else:
        raise DhsaError(5, "k", f"unsupported dtype {k.dtype}")
    sl = _seq_layout(cu_seqlens, k.device)
    T = k.shape[0]
    if sim is None:
        sim = torch.empty(T, dtype=torch.float32, device=k.device)
    if cut_bits is None:
        cut_bits = torch.empty((T + 63) // 64, dtype=torch.int64, device=k.device)
    if sim.numel() < T or cut_bits.numel() < (T + 63) // 64:
        raise DhsaError(2, "sim/cut_bits", "output buffers too small")
    for t, name, dt in ((sim, "sim", torch.float32), (cut_bits, "cut_bits", torch.int64)):
        if not _on_gpu(t) or t.dtype != dt or not t.is_contiguous():
            raise DhsaError(2, name, f"expected a contiguous {dt} tensor on the current GPU")
    _check(load_library().dhsa_adjacent_similarity(sl.num_seqs, T, k.shape[1], k.shape[2], code,
                                                   _ptr(sl.d_cu_seqlens), sl.h_cu_seqlens.ctypes.data, _ptr(k),
                                                   float(tau), _ptr(sim), _ptr(cut_bits), _stream()),
           "dhsa_adjacent_similarity")
    return sim, cut_bits


def chunk_boundaries(cut_bits: torch.Tensor, cu_seqlens, lo: int, hi: int,
                     out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None
                     ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """dhsa_chunk_boundaries: device cu_chunks int32 [T+1] (entries 0..C valid), seq_chunk_start
    int32 [B+1] and num_chunks int32 [1] (``out`` supplies them preallocated)."""
    if not _on_gpu(cut_bits) or cut_bits.dtype != torch.int64 or not cut_bits.is_contiguous():
        raise DhsaError(2, "cut_bits", "expected a contiguous int64 tensor on the current GPU")
    sl = _seq_layout(cu_seqlens, cut_bits.device)
    T = sl.total_tokens
    if cut_bits.numel() != (T + 63) // 64:
        raise DhsaError(2, "cut_bits", f"expected {(T + 63) // 64} words")
    if out is None:
        out = (torch.empty(T + 1, dtype=torch.int32, device=cut_bits.device),
               torch.empty(sl.num_seqs + 1, dtype=torch.int32, device=cut_bits.device),
               torch.empty(1, dtype=torch.int32, device=cut_bits.device))
    cu_chunks, scs, nch = out
    _require(cu_chunks, "cu_chunks", (T + 1,), torch.int32)
    _require(scs, "seq_chunk_start", (sl.num_seqs + 1,), torch.int32)
    _require(nch, "num_chunks", (1,), torch.int32)
    _check(load_library().dhsa_chunk_boundaries(sl.num_seqs, T, _ptr(sl.d_cu_seqlens), sl.h_cu_seqlens.ctypes.data,
                                                _ptr(cut_bits), int(lo), int(hi), _ptr(cu_chunks), _ptr(scs),
                                                _ptr(nch), _stream()), "dhsa_chunk_boundaries")
    return cu_chunks, scs, nch


def online_chunks(k: torch.Tensor, cu_seqlens, lo: int, hi: int, tau: float) -> Tuple[np.ndarray, np.ndarray]:
    """Both chunking steps, then the host copies a Layout needs: (cu_chunks [C+1], seq_chunk_start [B+1])."""
    sl = _seq_layout(cu_seqlens, k.device)
    _, bits = adjacent_similarity(k, sl, tau)
    cu_chunks, scs, nch = chunk_boundaries(bits, sl, lo, hi)
    C = int(nch.cpu().item())
    return cu_chunks[:C + 1].cpu().numpy(), scs.cpu().numpy()


# ----------------------------------------------------------------------------- decode

class DecodeState:
    """Decode state of a batch (dhsa_decode_state): caches, chunk tables and running sums, all device
    tensors owned here; ``load_prefix`` hands a chunked prefill batch over, ``step`` appends one token
    per sequence and returns its attention output."""

    def __init__(self, num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int, dtype: torch.dtype,
                 max_tokens: int, max_chunks: int, device="cuda"):
        dev = torch.device(device)
        if dtype == torch.bfloat16:
            code = DHSA_BF16
        elif dtype == torch.float32:
            code = DHSA_F32
        else:
            raise DhsaError(5, "DecodeState", f"unsupported dtype {dtype}")
        B, Hq, Hkv, d, L, C = num_seqs, num_q_heads, num_kv_heads, head_dim, max_tokens, max_chunks
        self.dtype, self.device = dtype, dev
        self.num_q_heads, self.num_kv_heads, self.head_dim = Hq, Hkv, d
        self.k_cache = torch.zeros((B, L, Hkv, d), dtype=dtype, device=dev)
        self.v_cache = torch.zeros((B, L, Hkv, d), dtype=dtype, device=dev)
        self.seq_len = torch.zeros(B, dtype=torch.int32, device=dev)
        self.num_closed = torch.zeros(B, dtype=torch.int32, device=dev)
        self.chunk_start = torch.zeros((B, C + 1), dtype=torch.int32, device=dev)
        self.k_sum = torch.zeros((B, C, Hkv, d), dtype=torch.float32, device=dev)
        self.q_run = torch.zeros((B, Hq, d), dtype=torch.float32, device=dev)
        self.k_run = torch.zeros((B, Hkv, d), dtype=torch.float32, device=dev)
        self.status = torch.zeros(B, dtype=torch.int32, device=dev)
        self.struct = DecodeStateStruct(B, Hq, Hkv, d, code, L, C, *(t.data_ptr() for t in (
            self.k_cache, self.v_cache, self.seq_len, self.num_closed, self.chunk_start, self.k_sum, self.q_run,
            self.k_run, self.status)))
        self._ws = {}

    def workspace(self, topk: int, grouped: bool) -> torch.Tensor:
        key = (int(topk), bool(grouped))
        if key not in self._ws:
            n = load_library().dhsa_decode_workspace_bytes(ctypes.byref(self.struct), int(topk), int(grouped))
            if n == 0:
                raise DhsaError(2, "dhsa_decode_workspace_bytes", "state or budget not supported")
            self._ws[key] = torch.empty(n, dtype=torch.uint8, device=self.device)
        return self._ws[key]

    def _check_device(self) -> None:
        if not _on_gpu(self.k_cache):
            raise DhsaError(1, "decode state", f"state is on {self.k_cache.device}, the current device is "
                                               f"cuda:{torch.cuda.current_device()}")

    def load_prefix(self, layout: "Layout", q: torch.Tensor, k: torch.Tensor, v: torch.Tensor) -> None:
        self._check_device()
        layout._check_tensor(q, layout.num_q_heads, "q")
        layout._check_tensor(k, layout.num_kv_heads, "k")
        layout._check_tensor(v, layout.num_kv_heads, "v")
        _check(load_library().dhsa_decode_load_prefix(ctypes.byref(self.struct), ctypes.byref(layout.struct), _ptr(q),
                                                      _ptr(k), _ptr(v), _stream()), "dhsa_decode_load_prefix")

    def step(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, lo: int, hi: int, tau: float, topk: int,
             grouped: bool = False, softmax_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
             kept: Optional[torch.Tensor] = None) -> torch.Tensor:
        """dhsa_decode_step with a workspace this object allocates once per (topk, grouped)."""
        return self._step(q, k, v, lo, hi, tau, topk, grouped, softmax_scale, out, kept, noalloc=False)

    def step_noalloc(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, lo: int, hi: int, tau: float,
                     topk: int, grouped: bool = False, softmax_scale: Optional[float] = None,
                     out: torch.Tensor = None, kept: Optional[torch.Tensor] = None) -> torch.Tensor:
        """dhsa_decode_step_noalloc: the library's static scratch instead of a workspace.  ``out`` is
        required, so that nothing is allocated on this path either."""
        if out is None:
            raise DhsaError(1, "step_noalloc", "out must be given (this path allocates nothing)")
        return self._step(q, k, v, lo, hi, tau, topk, grouped, softmax_scale, out, kept, noalloc=True)

    def _step(self, q, k, v, lo, hi, tau, topk, grouped, softmax_scale, out, kept, noalloc: bool) -> torch.Tensor:
        self._check_device()
        B = self.seq_len.numel()
        for t, name, heads in ((q, "q", self.num_q_heads), (k, "k", self.num_kv_heads), (v, "v", self.num_kv_heads)):
            if not _on_gpu(t) or t.dtype != self.dtype or tuple(t.shape) != (B, heads, self.head_dim) \
                    or not t.is_contiguous():
                raise DhsaError(2, name, f"expected contiguous {self.dtype} [{B}, {heads}, {self.head_dim}] on the current GPU")
        _require(out, "out", (B, self.num_q_heads, self.head_dim), self.dtype)
        _require(kept, "kept", (B, self.num_q_heads, topk), torch.int32)
        if softmax_scale is None:
            softmax_scale = 1.0 / math.sqrt(self.head_dim)
        if noalloc:
            _check(load_library().dhsa_decode_step_noalloc(ctypes.byref(self.struct), _ptr(q), _ptr(k), _ptr(v),
                                                           int(lo), int(hi), float(tau), int(topk), int(grouped),
                                                           float(softmax_scale), _ptr(out), _ptr(kept), _stream()),
                   "dhsa_decode_step_noalloc")
            return out
        if out is None:
            out = torch.empty_like(q)
        ws = self.workspace(topk, grouped)
        _check(load_library().dhsa_decode_step(ctypes.byref(self.struct), _ptr(q), _ptr(k), _ptr(v), int(lo), int(hi),
                                               float(tau), int(topk), int(grouped), float(softmax_scale), _ptr(out),
                                               _ptr(kept), _ptr(ws), ws.numel(), _stream()), "dhsa_decode_step")
        return out
