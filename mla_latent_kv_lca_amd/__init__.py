"""Python binding of liblca.so (latent-condensed MLA kernels for MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of include/lca.h. torch provides device memory and
the current stream. There is no fallback: if the library is not built, every
call raises.

Entry points (same names as the C ABI):
  lca_plan, lca_condense (and lca_condense_mode), mla_latent_attn_decode,
  mla_latent_attn_prefill_chunk, mla_up_proj,
  lca_condense_workspace_size, mla_latent_attn_decode_workspace_size,
  lca_version, lca_last_error
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_int64, c_size_t, c_void_p

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblca.so")

LCA_OK, LCA_ERR_INVALID_ARG, LCA_ERR_UNSUPPORTED, LCA_ERR_WORKSPACE, LCA_ERR_HIP = 0, -1, -2, -3, -4
LCA_BF16, LCA_F32 = 0, 1
# condensation modes: the method, and the two variants of the pages' ablation table
LCA_MODE_LCA, LCA_MODE_POOL_ROPE, LCA_MODE_ANCHOR = 0, 1, 2
D_C, D_R, D_ROW, D_V = 512, 64, 576, 128

# every symbol include/lca.h declares
EXPORTS = ("lca_version", "lca_last_error", "lca_plan", "lca_condense_workspace_size",
           "lca_condense", "lca_condense_mode", "lca_condense_paged", "lca_condense_step",
           "mla_latent_attn_decode_workspace_size",
           "mla_latent_attn_decode", "mla_latent_attn_decode_paged", "mla_latent_attn_decode_paged_up",
           "mla_latent_attn_decode_paged_up_step",
           "mla_latent_attn_decode_up", "mla_latent_attn_decode_up_noalloc", "mla_latent_attn_prefill_chunk",
           "mla_latent_attn_prefill_chunk_paged", "mla_latent_attn_prefill_chunk_sched",
           "mla_latent_attn_prefill_chunk_paged_sched",
           "mla_up_proj",
           "lca_project_workspace_size", "lca_project")


class LcaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"lca status {status}: {msg}")
        self.status = status


class LatentT(ctypes.Structure):
    _fields_ = [("c", c_void_p), ("kr", c_void_p), ("c_seq_stride", c_int64),
                ("c_tok_stride", c_int64), ("kr_seq_stride", c_int64),
                ("kr_tok_stride", c_int64), ("dtype", c_int32)]


class PagedT(ctypes.Structure):
    _fields_ = [("pages", c_void_p), ("row_stride", c_int64), ("page_rows", c_int32),
                ("block_table", c_void_p), ("table_stride", c_int64)]


class StepT(ctypes.Structure):
    _fields_ = [("w", c_int64), ("g", c_int32), ("q_ring", c_void_p), ("q_ring_seq_stride", c_int64),
                ("anchor_idx", c_void_p), ("anchor_seq_stride", c_int64), ("pos", c_void_p), ("dst_row", c_void_p)]


class PlanT(ctypes.Structure):
    _fields_ = [("m", c_int64), ("raw_begin", c_int64), ("raw_end", c_int64),
                ("n_entries", c_int64)]


_lib = None


def load() -> ctypes.CDLL:
    """Load liblca.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m mla_latent_kv_lca_amd.build` (or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    P = POINTER
    lib.lca_version.restype = c_int32
    lib.lca_version.argtypes = []
    lib.lca_last_error.restype = c_char_p
    lib.lca_last_error.argtypes = []
    lib.lca_plan.restype = c_int32
    lib.lca_plan.argtypes = [c_int64, c_int64, c_int32, P(PlanT)]
    lib.lca_condense_workspace_size.restype = c_size_t
    lib.lca_condense_workspace_size.argtypes = [c_int32, c_int64, c_int64]
    lib.lca_condense.restype = c_int32
    lib.lca_condense.argtypes = [P(LatentT), c_int32, c_int32, c_int64, c_int64, c_void_p, c_int32,
                                 c_int64, c_int64, c_int64, c_int32, c_int64, c_int64, c_float,
                                 P(LatentT), c_void_p, c_int64, c_void_p, c_int64, c_void_p,
                                 c_size_t, c_void_p]
    lib.lca_condense_mode.restype = c_int32
    lib.lca_condense_mode.argtypes = [P(LatentT), c_int32, c_int32, c_int64, c_int64, c_void_p, c_int32,
                                      c_int64, c_int64, c_int64, c_int32, c_int64, c_int64, c_float,
                                      P(LatentT), c_void_p, c_int64, c_void_p, c_int64, c_void_p,
                                      c_size_t, c_int32, c_void_p]
    lib.mla_latent_attn_decode_workspace_size.restype = c_size_t
    lib.mla_latent_attn_decode_workspace_size.argtypes = [c_int32, c_int32, c_int64]
    lib.mla_latent_attn_decode.restype = c_int32
    lib.mla_latent_attn_decode.argtypes = [c_void_p, c_int32, c_int64, c_int32, c_int32, P(LatentT),
                                           c_int64, P(LatentT), c_int64, c_int64, c_float,
                                           c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.lca_condense_paged.restype = c_int32
    lib.lca_condense_paged.argtypes = [P(PagedT), c_int32, c_int32, c_void_p, c_void_p, c_int64, c_void_p, c_int32,
                                       c_int64, c_int64, c_int64, c_int32, c_int64, c_int64, c_float, P(LatentT),
                                       c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_size_t, c_void_p]
    lib.lca_condense_step.restype = c_int32
    lib.lca_condense_step.argtypes = [P(PagedT), c_int32, c_int64, c_int32, c_void_p, c_int32, c_int64, c_int32,
                                      c_void_p, c_int64, c_float, P(LatentT), c_void_p, c_int64, c_void_p,
                                      c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
    lib.mla_latent_attn_decode_paged.restype = c_int32
    lib.mla_latent_attn_decode_paged.argtypes = [c_void_p, c_int32, c_int64, c_int32, c_int32, P(LatentT),
                                                 c_void_p, P(PagedT), c_void_p, c_void_p, c_int64, c_float,
                                                 c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.mla_latent_attn_decode_paged_up.restype = c_int32
    lib.mla_latent_attn_decode_paged_up.argtypes = [c_void_p, c_int32, c_int64, c_int32, c_int32, P(LatentT),
                                                    c_void_p, P(PagedT), c_void_p, c_void_p, c_int64, c_float,
                                                    c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_int32,
                                                    c_void_p, c_size_t, c_void_p]
    lib.mla_latent_attn_decode_paged_up_step.restype = c_int32
    lib.mla_latent_attn_decode_paged_up_step.argtypes = [c_void_p, c_int32, c_int64, c_int32, c_int32, P(LatentT),
                                                         c_void_p, P(PagedT), c_void_p, c_void_p, c_int64, c_float,
                                                         c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_int32,
                                                         P(StepT), c_void_p, c_size_t, c_void_p]
    lib.mla_latent_attn_prefill_chunk_paged.restype = c_int32
    lib.mla_latent_attn_prefill_chunk_paged.argtypes = [c_void_p, c_int32, c_int64, c_int64, c_int32, c_int32,
                                                        P(LatentT), c_int64, P(PagedT), c_int32, c_int64, c_float,
                                                        c_void_p, c_int32, c_void_p, c_void_p]
    lib.mla_latent_attn_decode_up.restype = c_int32
    lib.mla_latent_attn_decode_up.argtypes = [c_void_p, c_int32, c_int64, c_int32, c_int32, P(LatentT),
                                              c_int64, P(LatentT), c_int64, c_int64, c_float,
                                              c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_int32,
                                              c_void_p, c_size_t, c_void_p]
    lib.mla_latent_attn_decode_up_noalloc.restype = c_int32
    lib.mla_latent_attn_decode_up_noalloc.argtypes = [c_void_p, c_int32, c_int64, c_int32, c_int32, P(LatentT),
                                                      c_int64, P(LatentT), c_int64, c_int64, c_float,
                                                      c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_int32,
                                                      c_void_p]
    lib.mla_latent_attn_prefill_chunk.restype = c_int32
    lib.mla_latent_attn_prefill_chunk.argtypes = [c_void_p, c_int32, c_int64, c_int64, c_int32,
                                                  c_int32, P(LatentT), c_int64, P(LatentT),
                                                  c_int64, c_float, c_void_p, c_int32, c_void_p,
                                                  c_void_p]
    lib.mla_latent_attn_prefill_chunk_sched.restype = c_int32
    lib.mla_latent_attn_prefill_chunk_sched.argtypes = lib.mla_latent_attn_prefill_chunk.argtypes[:-1] + [
        c_void_p, c_void_p]
    lib.mla_latent_attn_prefill_chunk_paged_sched.restype = c_int32
    lib.mla_latent_attn_prefill_chunk_paged_sched.argtypes = lib.mla_latent_attn_prefill_chunk_paged.argtypes[:-1] + [
        c_void_p, c_void_p]
    lib.mla_up_proj.restype = c_int32
    lib.mla_up_proj.argtypes = [c_void_p, c_int32, c_int64, c_int32, c_void_p, c_int32, c_void_p,
                                c_int32, c_void_p]
    lib.lca_project_workspace_size.restype = ctypes.c_size_t
    lib.lca_project_workspace_size.argtypes = [c_int64, c_int32]
    lib.lca_project.restype = c_int32
    lib.lca_project.argtypes = [c_void_p, c_int64, c_int64, c_int32, c_void_p, ctypes.c_double, c_void_p,
                                c_void_p, c_int32, c_void_p, c_int64, c_void_p, c_void_p, c_int32, c_int64,
                                c_void_p, ctypes.c_size_t, c_void_p]
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != LCA_OK:
        raise LcaError(status, load().lca_last_error().decode())


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return LCA_BF16
    if t.dtype == torch.float32:
        return LCA_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use bfloat16 or float32")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check_lse(lse, rows: int, H: int) -> None:
    """lse is optional; when given it receives rows * H fp32 values written
    at lse[row * H + head], so it must be a contiguous fp32 tensor of exactly
    that many elements (the kernels index it without bounds)."""
    if lse is None:
        return
    if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != rows * H:
        raise ValueError(f"lse must be a contiguous fp32 tensor of {rows} x {H} elements")


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def latent(c: torch.Tensor, kr: torch.Tensor) -> LatentT:
    """Describe c_KV [B, L, 512] (or [L, 512]) and k_R [B, L, 64] views. The
    description holds references to both tensors, so their memory lives as
    long as it does."""
    if c.dtype != kr.dtype:
        raise TypeError("c and kr must share a dtype")
    if c.shape[-1] != D_C or kr.shape[-1] != D_R or c.stride(-1) != 1 or kr.stride(-1) != 1:
        raise ValueError("c must end in a contiguous 512-wide axis and kr in a 64-wide axis")
    cs = c.stride(0) if c.dim() == 3 else 0
    ks = kr.stride(0) if kr.dim() == 3 else 0
    d = LatentT(c.data_ptr(), kr.data_ptr(), cs, c.stride(-2), ks, kr.stride(-2), dtype_code(c))
    d._tensors = (c, kr)  # the descriptor keeps its tensors (e.g. temporary copies) alive
    return d


def packed_latent(cache: torch.Tensor) -> LatentT:
    """Describe a packed [B, L, 576] (or [L, 576]) cache: c = [..., :512], kr = [..., 512:]."""
    return latent(cache[..., :D_C], cache[..., D_C:])


def paged_latent(pool: torch.Tensor, block_table: torch.Tensor) -> PagedT:
    """Describe a paged cache: pool [n_pages, page_rows, 576] bf16 (packed rows),
    block_table int32 [B, pages per sequence] on the device. The description holds
    references to both tensors."""
    if pool.dim() != 3 or pool.shape[-1] != D_ROW or pool.stride(-1) != 1:
        raise ValueError("pool must be [n_pages, page_rows, 576] with contiguous rows")
    if pool.stride(0) != pool.shape[1] * pool.stride(1):
        raise ValueError("pages must be contiguous in the pool")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("block_table must be an int32 [B, n] tensor with contiguous rows")
    d = PagedT(pool.data_ptr(), pool.stride(1), pool.shape[1], block_table.data_ptr(), block_table.stride(0))
    d._tensors = (pool, block_table)
    return d


# ----------------------------------------------------------------- calls ---
def lca_version() -> int:
    return load().lca_version()


def lca_last_error() -> str:
    return load().lca_last_error().decode()


def lca_plan(L: int, w: int, g: int) -> dict:
    out = PlanT()
    _check(load().lca_plan(L, w, g, ctypes.byref(out)))
    return {"m": out.m, "raw_begin": out.raw_begin, "raw_end": out.raw_end,
            "n_entries": out.n_entries}


def gqa_sequences(q: torch.Tensor, n_kv: int) -> torch.Tensor:
    """GQA as independent sequences (the reading that the pages' "extends to
    GQA" leaves open: n_kv latent caches, the H query heads in n_kv groups of
    Hg = H / n_kv consecutive heads, group k attending and condensing cache
    k). With caches and representatives laid out [B, n_kv, L, 576] (used as
    [B * n_kv, L, 576]) every entry point runs GQA unchanged on B * n_kv
    sequences of Hg heads. This reorders queries [B, T, H, 576] kv-major into
    [B * n_kv, T, Hg, 576]; decode queries [B, H, 576] are already kv-major
    and only need .view(B * n_kv, Hg, 576)."""
    B, T, H, D = q.shape
    if H % n_kv:
        raise ValueError("H must be a multiple of n_kv")
    return q.view(B, T, n_kv, H // n_kv, D).transpose(1, 2).contiguous().view(B * n_kv, T, H // n_kv, D)


def lca_condense_workspace_size(B: int, n_groups: int, q_row_step: int) -> int:
    return load().lca_condense_workspace_size(B, n_groups, q_row_step)


def mla_latent_attn_decode_workspace_size(B: int, H: int, max_entries: int) -> int:
    return load().mla_latent_attn_decode_workspace_size(B, H, max_entries)


def _workspace(nbytes: int, like: torch.Tensor, ws):
    """Caller's workspace, or a fresh one (no initialisation is needed)."""
    if ws is not None:
        return ws
    return torch.empty(max(16, (nbytes + 15) // 16 * 16), dtype=torch.uint8, device=like.device)


def decode_workspace(B: int, H: int, max_entries: int, device="cuda") -> torch.Tensor:
    """Workspace for mla_latent_attn_decode (any contents), reusable across
    calls that do not overlap."""
    n = mla_latent_attn_decode_workspace_size(B, H, max_entries)
    return torch.empty(max(16, (n + 15) // 16 * 16), dtype=torch.uint8, device=device)


def lca_condense(cache: LatentT, B: int, g: int, group_begin: int, n_groups: int,
                 q: torch.Tensor, q_row0: int, q_row_step: int, sm_scale: float,
                 reps: LatentT, anchor: torch.Tensor, alpha: torch.Tensor | None = None,
                 workspace: torch.Tensor | None = None, stream=None, mode: int = LCA_MODE_LCA) -> None:
    """Condense groups [group_begin, group_begin + n_groups) (q: [B, T, H, 576];
    anchor: int32 [B, *]; alpha: fp32 [B, *, g] or None). mode != LCA_MODE_LCA
    calls lca_condense_mode (the ablation variants)."""
    if q.dim() != 4 or q.shape[-1] != D_ROW or q.stride(-1) != 1 or q.stride(-2) != D_ROW:
        raise ValueError("q must be [B, T, H, 576] with contiguous heads")
    if anchor.dtype != torch.int32:
        raise TypeError("anchor must be int32")
    ws = _workspace(lca_condense_workspace_size(B, n_groups, q_row_step), q, workspace)
    args = (ctypes.byref(cache), B, g, group_begin, n_groups, q.data_ptr(), dtype_code(q), q.stride(0),
            q.stride(1), q.shape[1], q.shape[2], q_row0, q_row_step, sm_scale, ctypes.byref(reps),
            anchor.data_ptr(), anchor.stride(0), _ptr(alpha), 0 if alpha is None else alpha.stride(0),
            ws.data_ptr(), ws.numel() * ws.element_size())
    if mode == LCA_MODE_LCA:
        _check(load().lca_condense(*args, _stream(stream)))
    else:
        _check(load().lca_condense_mode(*args, mode, _stream(stream)))


def lca_condense_paged(cache: PagedT, B: int, g: int, seq_group_begin: torch.Tensor, seq_n_groups: torch.Tensor,
                       max_groups: int, q: torch.Tensor, q_row0: int, sm_scale: float, reps: LatentT,
                       anchor: torch.Tensor, alpha: torch.Tensor | None = None,
                       workspace: torch.Tensor | None = None, stream=None, q_row_step: int = 0) -> None:
    """Ragged condensation over a paged cache; q [B, T, H, 576]; per-sequence
    int32 [B] device arrays; group seq_group_begin[b] + n of sequence b uses
    query rows [q_row0 + n * q_row_step, + g) (q_row_step = 0: one summary
    query per sequence)."""
    if q.dim() != 4 or q.shape[-1] != D_ROW or q.stride(-1) != 1 or q.stride(-2) != D_ROW:
        raise ValueError("q must be [B, T, H, 576] with contiguous heads")
    if anchor.dtype != torch.int32:
        raise TypeError("anchor must be int32")
    for t in (seq_group_begin, seq_n_groups):
        if t.dtype != torch.int32 or not t.is_contiguous() or t.numel() != B:
            raise ValueError("per-sequence arrays must be contiguous int32 [B] tensors")
    ws = _workspace(lca_condense_workspace_size(B, max_groups, q_row_step), q, workspace)
    _check(load().lca_condense_paged(
        ctypes.byref(cache), B, g, seq_group_begin.data_ptr(), seq_n_groups.data_ptr(), max_groups, q.data_ptr(),
        dtype_code(q), q.stride(0), q.stride(1), q.shape[1], q.shape[2], q_row0, q_row_step, sm_scale,
        ctypes.byref(reps),
        anchor.data_ptr(), anchor.stride(0), _ptr(alpha), 0 if alpha is None else alpha.stride(0),
        ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream)))


def lca_condense_step(cache: PagedT, w: int, g: int, q: torch.Tensor, q_ring: torch.Tensor, sm_scale: float,
                      reps: LatentT, anchor: torch.Tensor, seq_m: torch.Tensor, seq_raw_begin: torch.Tensor,
                      seq_raw_end: torch.Tensor, pos: torch.Tensor | None = None,
                      dst_row: torch.Tensor | None = None, stream=None) -> None:
    """One decode step's incremental condensation with device-side state:
    q [B, H, 576] (this step's queries), q_ring [B, g, H, 576] (same dtype);
    seq_m, seq_raw_begin, seq_raw_end int32 [B] (rewritten); pos int32 [B] and
    dst_row int64 [B] (optional) receive the next token's position and pool row."""
    if q.dim() != 3 or q.shape[-1] != D_ROW or q.stride(-1) != 1 or q.stride(-2) != D_ROW:
        raise ValueError("q must be [B, H, 576] with contiguous heads")
    B, H = q.shape[0], q.shape[1]
    if q_ring.dtype != q.dtype or q_ring.dim() != 4 or q_ring.shape[1:] != (g, H, D_ROW) or q_ring.shape[0] != B \
            or q_ring.stride(1) != H * D_ROW or q_ring.stride(2) != D_ROW or q_ring.stride(3) != 1:
        raise ValueError("q_ring must be [B, g, H, 576] of q's dtype with contiguous rows")
    if anchor.dtype != torch.int32:
        raise TypeError("anchor must be int32")
    for t in (seq_m, seq_raw_begin, seq_raw_end) + ((pos,) if pos is not None else ()):
        if t.dtype != torch.int32 or not t.is_contiguous() or t.numel() != B:
            raise ValueError("per-sequence arrays must be contiguous int32 [B] tensors")
    if dst_row is not None and (dst_row.dtype != torch.int64 or not dst_row.is_contiguous() or dst_row.numel() != B):
        raise ValueError("dst_row must be a contiguous int64 [B] tensor")
    _check(load().lca_condense_step(
        ctypes.byref(cache), B, w, g, q.data_ptr(), dtype_code(q), q.stride(0), H, q_ring.data_ptr(),
        q_ring.stride(0), sm_scale, ctypes.byref(reps), anchor.data_ptr(), anchor.stride(0), seq_m.data_ptr(),
        seq_raw_begin.data_ptr(), seq_raw_end.data_ptr(), _ptr(pos), _ptr(dst_row), _stream(stream)))


def mla_latent_attn_decode_paged(q: torch.Tensor, reps: LatentT, seq_m: torch.Tensor, cache: PagedT,
                                 seq_raw_begin: torch.Tensor, seq_raw_end: torch.Tensor, max_entries: int,
                                 sm_scale: float, o_latent: torch.Tensor, lse: torch.Tensor | None = None,
                                 workspace: torch.Tensor | None = None, stream=None) -> None:
    """Ragged batch over a paged cache: q [B, H, 576]; seq_m, seq_raw_begin,
    seq_raw_end int32 [B] device tensors; o_latent fp32 [B, H, 512]."""
    if q.dim() != 3 or q.shape[-1] != D_ROW or q.stride(-1) != 1 or q.stride(-2) != D_ROW:
        raise ValueError("q must be [B, H, 576] with contiguous heads")
    B, H = q.shape[0], q.shape[1]
    if o_latent.dtype != torch.float32 or not o_latent.is_contiguous() or o_latent.shape != (B, H, D_C):
        raise ValueError("o_latent must be a contiguous fp32 [B, H, 512] tensor")
    for t in (seq_m, seq_raw_begin, seq_raw_end):
        if t.dtype != torch.int32 or not t.is_contiguous() or t.numel() != B:
            raise ValueError("per-sequence arrays must be contiguous int32 [B] tensors")
    _check_lse(lse, B, H)
    ws = _workspace(mla_latent_attn_decode_workspace_size(B, H, max_entries), q, workspace)
    _check(load().mla_latent_attn_decode_paged(
        q.data_ptr(), dtype_code(q), q.stride(0), B, H, ctypes.byref(reps), seq_m.data_ptr(),
        ctypes.byref(cache), seq_raw_begin.data_ptr(), seq_raw_end.data_ptr(), max_entries, sm_scale,
        o_latent.data_ptr(), _ptr(lse), ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream)))


def mla_latent_attn_decode_paged_up(q: torch.Tensor, reps: LatentT, seq_m: torch.Tensor, cache: PagedT,
                                    seq_raw_begin: torch.Tensor, seq_raw_end: torch.Tensor, max_entries: int,
                                    sm_scale: float, o_latent: torch.Tensor, w_uv: torch.Tensor, out: torch.Tensor,
                                    lse: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                                    stream=None) -> None:
    """Paged decode plus W_UV up-projection: arguments of
    mla_latent_attn_decode_paged, w_uv [H, 512, 128], out [B, H, 128]."""
    if q.dim() != 3 or q.shape[-1] != D_ROW or q.stride(-1) != 1 or q.stride(-2) != D_ROW:
        raise ValueError("q must be [B, H, 576] with contiguous heads")
    B, H = q.shape[0], q.shape[1]
    if o_latent.dtype != torch.float32 or not o_latent.is_contiguous() or o_latent.shape != (B, H, D_C):
        raise ValueError("o_latent must be a contiguous fp32 [B, H, 512] tensor")
    for t in (seq_m, seq_raw_begin, seq_raw_end):
        if t.dtype != torch.int32 or not t.is_contiguous() or t.numel() != B:
            raise ValueError("per-sequence arrays must be contiguous int32 [B] tensors")
    _check_lse(lse, B, H)
    if not w_uv.is_contiguous() or tuple(w_uv.shape) != (H, D_C, D_V):
        raise ValueError("w_uv must be a contiguous [H, 512, 128] tensor")
    if not out.is_contiguous() or tuple(out.shape) != (B, H, D_V):
        raise ValueError("out must be a contiguous [B, H, 128] tensor")
    ws = _workspace(mla_latent_attn_decode_workspace_size(B, H, max_entries), q, workspace)
    _check(load().mla_latent_attn_decode_paged_up(
        q.data_ptr(), dtype_code(q), q.stride(0), B, H, ctypes.byref(reps), seq_m.data_ptr(),
        ctypes.byref(cache), seq_raw_begin.data_ptr(), seq_raw_end.data_ptr(), max_entries, sm_scale,
        o_latent.data_ptr(), _ptr(lse), w_uv.data_ptr(), dtype_code(w_uv), out.data_ptr(), dtype_code(out),
        ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream)))


def mla_latent_attn_decode_paged_up_step(q: torch.Tensor, reps: LatentT, seq_m: torch.Tensor, cache: PagedT,
                                         seq_raw_begin: torch.Tensor, seq_raw_end: torch.Tensor, max_entries: int,
                                         sm_scale: float, o_latent: torch.Tensor, w_uv: torch.Tensor,
                                         out: torch.Tensor, w: int, g: int, q_ring: torch.Tensor,
                                         anchor: torch.Tensor, pos: torch.Tensor | None = None,
                                         dst_row: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                                         workspace: torch.Tensor | None = None, stream=None) -> None:
    """mla_latent_attn_decode_paged_up followed by lca_condense_step (the step
    condensation inside the merge / W_UV launch): arguments of the two."""
    if q.dim() != 3 or q.shape[-1] != D_ROW or q.stride(-1) != 1 or q.stride(-2) != D_ROW:
        raise ValueError("q must be [B, H, 576] with contiguous heads")
    B, H = q.shape[0], q.shape[1]
    if o_latent.dtype != torch.float32 or not o_latent.is_contiguous() or o_latent.shape != (B, H, D_C):
        raise ValueError("o_latent must be a contiguous fp32 [B, H, 512] tensor")
    for t in (seq_m, seq_raw_begin, seq_raw_end) + ((pos,) if pos is not None else ()):
        if t.dtype != torch.int32 or not t.is_contiguous() or t.numel() != B:
            raise ValueError("per-sequence arrays must be contiguous int32 [B] tensors")
    if dst_row is not None and (dst_row.dtype != torch.int64 or not dst_row.is_contiguous() or dst_row.numel() != B):
        raise ValueError("dst_row must be a contiguous int64 [B] tensor")
    if q_ring.dtype != q.dtype or q_ring.dim() != 4 or q_ring.shape[1:] != (g, H, D_ROW) or q_ring.shape[0] != B \
            or q_ring.stride(1) != H * D_ROW or q_ring.stride(2) != D_ROW or q_ring.stride(3) != 1:
        raise ValueError("q_ring must be [B, g, H, 576] of q's dtype with contiguous rows")
    if anchor.dtype != torch.int32:
        raise TypeError("anchor must be int32")
    _check_lse(lse, B, H)
    if not w_uv.is_contiguous() or tuple(w_uv.shape) != (H, D_C, D_V):
        raise ValueError("w_uv must be a contiguous [H, 512, 128] tensor")
    if not out.is_contiguous() or tuple(out.shape) != (B, H, D_V):
        raise ValueError("out must be a contiguous [B, H, 128] tensor")
    step = StepT(w, g, q_ring.data_ptr(), q_ring.stride(0), anchor.data_ptr(), anchor.stride(0), _ptr(pos),
                 _ptr(dst_row))
    ws = _workspace(mla_latent_attn_decode_workspace_size(B, H, max_entries), q, workspace)
    _check(load().mla_latent_attn_decode_paged_up_step(
        q.data_ptr(), dtype_code(q), q.stride(0), B, H, ctypes.byref(reps), seq_m.data_ptr(),
        ctypes.byref(cache), seq_raw_begin.data_ptr(), seq_raw_end.data_ptr(), max_entries, sm_scale,
        o_latent.data_ptr(), _ptr(lse), w_uv.data_ptr(), dtype_code(w_uv), out.data_ptr(), dtype_code(out),
        ctypes.byref(step), ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream)))


def mla_latent_attn_decode(q: torch.Tensor, reps: LatentT | None, m: int, raw: LatentT | None,
                           raw_begin: int, raw_end: int, sm_scale: float, o_latent: torch.Tensor,
                           lse: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                           stream=None) -> None:
    """q [B, H, 576]; o_latent fp32 [B, H, 512] contiguous; lse fp32 [B, H] or None."""
    if q.dim() != 3 or q.shape[-1] != D_ROW or q.stride(-1) != 1 or q.stride(-2) != D_ROW:
        raise ValueError("q must be [B, H, 576] with contiguous heads")
    B, H = q.shape[0], q.shape[1]
    if o_latent.dtype != torch.float32 or not o_latent.is_contiguous() or o_latent.shape != (B, H, D_C):
        raise ValueError("o_latent must be a contiguous fp32 [B, H, 512] tensor")
    _check_lse(lse, B, H)
    n = m + raw_end - raw_begin
    ws = _workspace(mla_latent_attn_decode_workspace_size(B, H, max(n, 1)), q, workspace)
    _check(load().mla_latent_attn_decode(
        q.data_ptr(), dtype_code(q), q.stride(0), B, H,
        None if reps is None else ctypes.byref(reps), m,
        None if raw is None else ctypes.byref(raw), raw_begin, raw_end, sm_scale,
        o_latent.data_ptr(), _ptr(lse), ws.data_ptr(), ws.numel() * ws.element_size(),
        _stream(stream)))


def mla_latent_attn_decode_up(q: torch.Tensor, reps: LatentT | None, m: int, raw: LatentT | None,
                              raw_begin: int, raw_end: int, sm_scale: float, o_latent: torch.Tensor,
                              w_uv: torch.Tensor, out: torch.Tensor, lse: torch.Tensor | None = None,
                              workspace: torch.Tensor | None = None, stream=None) -> None:
    """Decode plus W_UV up-projection: q [B, H, 576]; o_latent fp32 [B, H, 512];
    w_uv [H, 512, 128]; out [B, H, 128]; all contiguous."""
    if q.dim() != 3 or q.shape[-1] != D_ROW or q.stride(-1) != 1 or q.stride(-2) != D_ROW:
        raise ValueError("q must be [B, H, 576] with contiguous heads")
    B, H = q.shape[0], q.shape[1]
    if o_latent.dtype != torch.float32 or not o_latent.is_contiguous() or o_latent.shape != (B, H, D_C):
        raise ValueError("o_latent must be a contiguous fp32 [B, H, 512] tensor")
    _check_lse(lse, B, H)
    if not w_uv.is_contiguous() or tuple(w_uv.shape) != (H, D_C, D_V):
        raise ValueError("w_uv must be a contiguous [H, 512, 128] tensor")
    if not out.is_contiguous() or tuple(out.shape) != (B, H, D_V):
        raise ValueError("out must be a contiguous [B, H, 128] tensor")
    n = m + raw_end - raw_begin
    ws = _workspace(mla_latent_attn_decode_workspace_size(B, H, max(n, 1)), q, workspace)
    _check(load().mla_latent_attn_decode_up(
        q.data_ptr(), dtype_code(q), q.stride(0), B, H,
        None if reps is None else ctypes.byref(reps), m,
        None if raw is None else ctypes.byref(raw), raw_begin, raw_end, sm_scale,
        o_latent.data_ptr(), _ptr(lse), w_uv.data_ptr(), dtype_code(w_uv), out.data_ptr(),
        dtype_code(out), ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream)))


def mla_latent_attn_decode_up_noalloc(q: torch.Tensor, reps: LatentT | None, m: int, raw: LatentT | None,
                                      raw_begin: int, raw_end: int, sm_scale: float, o_latent: torch.Tensor,
                                      w_uv: torch.Tensor, out: torch.Tensor, lse: torch.Tensor | None = None,
                                      stream=None) -> None:
    """mla_latent_attn_decode_up with the library's fixed device scratch
    instead of a workspace (the call allocates nothing). Calls that overlap
    on one GPU must not be issued (they share the scratch)."""
    if q.dim() != 3 or q.shape[-1] != D_ROW or q.stride(-1) != 1 or q.stride(-2) != D_ROW:
        raise ValueError("q must be [B, H, 576] with contiguous heads")
    B, H = q.shape[0], q.shape[1]
    if o_latent.dtype != torch.float32 or not o_latent.is_contiguous() or o_latent.shape != (B, H, D_C):
        raise ValueError("o_latent must be a contiguous fp32 [B, H, 512] tensor")
    _check_lse(lse, B, H)
    if not w_uv.is_contiguous() or tuple(w_uv.shape) != (H, D_C, D_V):
        raise ValueError("w_uv must be a contiguous [H, 512, 128] tensor")
    if not out.is_contiguous() or tuple(out.shape) != (B, H, D_V):
        raise ValueError("out must be a contiguous [B, H, 128] tensor")
    _check(load().mla_latent_attn_decode_up_noalloc(
        q.data_ptr(), dtype_code(q), q.stride(0), B, H,
        None if reps is None else ctypes.byref(reps), m,
        None if raw is None else ctypes.byref(raw), raw_begin, raw_end, sm_scale,
        o_latent.data_ptr(), _ptr(lse), w_uv.data_ptr(), dtype_code(w_uv), out.data_ptr(),
        dtype_code(out), _stream(stream)))


def mla_latent_attn_prefill_chunk(q: torch.Tensor, chunk_start: int, reps: LatentT | None, m: int,
                                  raw: LatentT, raw_begin: int, sm_scale: float,
                                  o_latent: torch.Tensor, lse: torch.Tensor | None = None,
                                  stream=None, sched: torch.Tensor | None = None) -> None:
    """q [C, H, 576] (queries at positions chunk_start ..); o_latent [C, H, 512].
    sched (int32 [2] on the device, zeroed once, see prefill_sched()) selects
    mla_latent_attn_prefill_chunk_sched."""
    if q.dim() != 3 or q.shape[-1] != D_ROW or q.stride(-1) != 1 or q.stride(-2) != D_ROW:
        raise ValueError("q must be [C, H, 576] with contiguous heads")
    C, H = q.shape[0], q.shape[1]
    if not o_latent.is_contiguous() or o_latent.shape != (C, H, D_C):
        raise ValueError("o_latent must be a contiguous [C, H, 512] tensor")
    _check_lse(lse, C, H)
    args = (q.data_ptr(), dtype_code(q), q.stride(0), chunk_start, C, H,
            None if reps is None else ctypes.byref(reps), m, ctypes.byref(raw), raw_begin, sm_scale,
            o_latent.data_ptr(), dtype_code(o_latent), _ptr(lse))
    if sched is None:
        _check(load().mla_latent_attn_prefill_chunk(*args, _stream(stream)))
    else:
        _check_sched(sched)
        _check(load().mla_latent_attn_prefill_chunk_sched(*args, sched.data_ptr(), _stream(stream)))


def mla_latent_attn_prefill_chunk_paged(q: torch.Tensor, chunk_start: int, reps: LatentT | None, m: int,
                                        cache: PagedT, seq: int, raw_begin: int, sm_scale: float,
                                        o_latent: torch.Tensor, lse: torch.Tensor | None = None,
                                        stream=None, sched: torch.Tensor | None = None) -> None:
    """Chunked prefill of sequence `seq` of a paged cache: q [C, H, 576]
    (queries at positions chunk_start ..), o_latent [C, H, 512]. sched as in
    mla_latent_attn_prefill_chunk."""
    if q.dim() != 3 or q.shape[-1] != D_ROW or q.stride(-1) != 1 or q.stride(-2) != D_ROW:
        raise ValueError("q must be [C, H, 576] with contiguous heads")
    C, H = q.shape[0], q.shape[1]
    if not o_latent.is_contiguous() or o_latent.shape != (C, H, D_C):
        raise ValueError("o_latent must be a contiguous [C, H, 512] tensor")
    _check_lse(lse, C, H)
    args = (q.data_ptr(), dtype_code(q), q.stride(0), chunk_start, C, H,
            None if reps is None else ctypes.byref(reps), m, ctypes.byref(cache), seq, raw_begin, sm_scale,
            o_latent.data_ptr(), dtype_code(o_latent), _ptr(lse))
    if sched is None:
        _check(load().mla_latent_attn_prefill_chunk_paged(*args, _stream(stream)))
    else:
        _check_sched(sched)
        _check(load().mla_latent_attn_prefill_chunk_paged_sched(*args, sched.data_ptr(), _stream(stream)))


def prefill_sched(device="cuda") -> torch.Tensor:
    """A zeroed scheduling counter for the *_sched prefill calls (int32 [2];
    every call leaves it zeroed, so it is reused; one per concurrent stream)."""
    return torch.zeros(2, dtype=torch.int32, device=device)


def _check_sched(sched: torch.Tensor) -> None:
    if sched.dtype != torch.int32 or sched.numel() < 2 or not sched.is_contiguous():
        raise ValueError("sched must be a contiguous int32 tensor of at least 2 elements")


def mla_up_proj(o_latent: torch.Tensor, w_uv: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    """o_latent [T, H, 512], w_uv [H, 512, 128], out [T, H, 128], all contiguous."""
    for name, t in (("o_latent", o_latent), ("w_uv", w_uv), ("out", out)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    T, H = o_latent.shape[0], o_latent.shape[1]
    if o_latent.shape[2] != D_C or tuple(w_uv.shape) != (H, D_C, D_V) or tuple(out.shape) != (T, H, D_V):
        raise ValueError("shapes must be o_latent [T,H,512], w_uv [H,512,128], out [T,H,128]")
    _check(load().mla_up_proj(o_latent.data_ptr(), dtype_code(o_latent), T, H, w_uv.data_ptr(),
                              dtype_code(w_uv), out.data_ptr(), dtype_code(out), _stream(stream)))


def lca_project_workspace_size(T: int, H: int) -> int:
    return load().lca_project_workspace_size(T, H)


def lca_project(x: torch.Tensor, pos: torch.Tensor, w_proj: torch.Tensor, w_uk: torch.Tensor,
                rows: torch.Tensor, dst_row: torch.Tensor, q: torch.Tensor, rope_base: float = 10000.0,
                workspace=None, stream=None) -> None:
    """Hidden states x [T, d] (bf16, rows contiguous) at positions pos (int32
    [T]) -> cache rows written at rows.view(-1, row_stride)[dst_row[t]] (bf16,
    last dim contiguous) and absorbed queries q [T, H, 576] (bf16 or f32,
    token stride q.stride(0)). w_proj bf16 [576 + 192 H, d], w_uk bf16
    [H, 512, 128], dst_row int64 [T]."""
    T, d = x.shape
    H = w_uk.shape[0]
    if x.stride(1) != 1 or not w_proj.is_contiguous() or not w_uk.is_contiguous():
        raise ValueError("x rows, w_proj and w_uk must be contiguous")
    if tuple(w_proj.shape) != (D_ROW + 192 * H, d) or tuple(w_uk.shape[1:]) != (D_C, D_V):
        raise ValueError("w_proj must be [576 + 192 H, d] and w_uk [H, 512, 128]")
    if q.dim() != 3 or tuple(q.shape[1:]) != (H, D_ROW) or q.stride(2) != 1 or q.stride(1) != D_ROW:
        raise ValueError("q must be [T, H, 576] with contiguous heads")
    if pos.dtype != torch.int32 or dst_row.dtype != torch.int64:
        raise ValueError("pos must be int32 and dst_row int64")
    if rows.stride(-1) != 1:
        raise ValueError("rows must have a contiguous last dim")
    row_stride = rows.stride(-2) if rows.dim() >= 2 else D_ROW
    ws = _workspace(lca_project_workspace_size(T, H), x, workspace)
    _check(load().lca_project(x.data_ptr(), x.stride(0), T, d, pos.data_ptr(), rope_base, w_proj.data_ptr(),
                              w_uk.data_ptr(), H, rows.data_ptr(), row_stride, dst_row.data_ptr(),
                              q.data_ptr(), dtype_code(q), q.stride(0), ws.data_ptr(),
                              ws.numel() * ws.element_size(), _stream(stream)))
