"""MI355X-native FlashPrefill block-sparse prefill attention.

Thin Python binding over libflashprefill.so (C ABI in include/flashprefill.h).
Every step of the path runs in the HIP kernels; this module only marshals
arguments: it takes torch tensors for device memory, passes their data
pointers, strides and the current HIP stream, and allocates outputs with
torch.  There is no CPU fallback: if the library is missing, loading fails.

Stages (FlashPrefill, Methods 1-3; FlashPrefill V2 for FP8 and paged KV):
    discover            -> pooled Q/K block means (fp64)
    threshold_compact   -> per-(head, query block) ascending key-block lists
    sparse_attn         -> causal GQA attention over the listed blocks (bf16 out)
and dense_attn, plus *_paged / *_varlen variants for packed batches.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

from ._lib import (FP_BF16, FP_FP8_E4M3, FlashPrefillError, call, load)

__all__ = [
    "FlashPrefillError", "load", "discover", "threshold_compact", "sparse_attn", "dense_attn", "prefill",
    "VarlenBatch", "discover_paged", "threshold_compact_varlen", "sparse_attn_paged", "idx_capacity",
    "BLOCK", "HEAD_DIM",
]

BLOCK = 128
HEAD_DIM = 128


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return FP_BF16
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return FP_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype} (bf16, float8_e4m3fn or uint8 e4m3fn codes)")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _nb(L: int) -> int:
    return -(-int(L) // BLOCK)


def idx_capacity(hq: int, nb: int) -> int:
    return hq * nb * (nb + 1) // 2


def default_scale(d: int = HEAD_DIM) -> float:
    return 1.0 / math.sqrt(d)


# ------------------------------------------------------------- argument checks
# The C ABI takes raw pointers and sizes, so it cannot see how large a caller's
# buffer is.  Every wrapper below checks shapes, dtypes, strides and devices of
# its tensors against the sizes it passes down and raises ValueError before
# anything is enqueued.


def _require(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _rows(name: str, t: torch.Tensor, tokens: Optional[int] = None, heads: Optional[int] = None) -> None:
    """A [tokens, heads, 128] operand with a unit innermost stride."""
    _require(isinstance(t, torch.Tensor), f"{name} must be a torch tensor")
    _require(t.dim() == 3, f"{name} must be [tokens, heads, {HEAD_DIM}], got shape {tuple(t.shape)}")
    _require(t.shape[2] == HEAD_DIM, f"{name} head dim is {t.shape[2]}, needs {HEAD_DIM}")
    _require(t.stride(2) == 1, f"{name} needs a unit innermost stride (got {t.stride(2)})")
    if tokens is not None:
        _require(t.shape[0] == tokens, f"{name} has {t.shape[0]} tokens, expected {tokens}")
    if heads is not None:
        _require(t.shape[1] == heads, f"{name} has {t.shape[1]} heads, expected {heads}")


def _pages(name: str, t: torch.Tensor, heads: Optional[int] = None) -> None:
    """A page cache [pages, 128, heads, 128] with a unit innermost stride."""
    _require(t.dim() == 4 and t.shape[1] == BLOCK and t.shape[3] == HEAD_DIM,
             f"{name} must be [pages, {BLOCK}, heads, {HEAD_DIM}], got shape {tuple(t.shape)}")
    _require(t.stride(3) == 1, f"{name} needs a unit innermost stride (got {t.stride(3)})")
    if heads is not None:
        _require(t.shape[2] == heads, f"{name} has {t.shape[2]} heads, expected {heads}")


def _same_dtype(q: torch.Tensor, *others) -> int:
    code = _dtype_code(q)
    for name, t in others:
        _require(_dtype_code(t) == code, f"{name} dtype {t.dtype} does not match q dtype {q.dtype}")
    return code


def _exact(name: str, t: Optional[torch.Tensor], shape, dtype, contiguous: bool = True) -> None:
    """A buffer of exactly `shape` and `dtype` (contiguous unless stated otherwise)."""
    if t is None:
        return
    _require(isinstance(t, torch.Tensor), f"{name} must be a torch tensor")
    _require(tuple(t.shape) == tuple(shape), f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    _require(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    if contiguous:
        _require(t.is_contiguous(), f"{name} must be contiguous")


def _capacity(name: str, t: torch.Tensor, n: int, dtype=torch.int32) -> None:
    """A flat buffer of at least n elements of `dtype`."""
    _require(isinstance(t, torch.Tensor), f"{name} must be a torch tensor")
    _require(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    _require(t.is_contiguous(), f"{name} must be contiguous")
    _require(t.numel() >= n, f"{name} holds {t.numel()} elements, needs at least {n}")


def _scales(code: int, **named) -> None:
    """fp8 needs one fp32 scale per head for each operand passed (name=(tensor, heads))."""
    if code != FP_FP8_E4M3:
        return
    for name, (t, heads) in named.items():
        _require(t is not None, f"fp8 inputs need {name}")
        _exact(name, t, (heads,), torch.float32)


def _device(*tensors) -> None:
    """Every tensor given lives on one CUDA device."""
    ts = [t for t in tensors if t is not None]
    dev = ts[0].device
    _require(dev.type == "cuda", f"tensors must be on a CUDA device, got {dev}")
    for t in ts[1:]:
        _require(t.device == dev, f"tensors on different devices: {dev} and {t.device}")


def _out_rows(out: torch.Tensor, tokens: int, heads: int) -> None:
    _rows("out", out, tokens, heads)
    _require(out.dtype == torch.bfloat16, f"out must be bfloat16, got {out.dtype}")


def _lists(idx, counts, heads: int, rows_total: int, tri_total: int) -> None:
    """idx (triangular-packed lists) and counts [heads, rows_total] int32."""
    _capacity("idx", idx, heads * tri_total)
    _exact("counts", counts, (heads, rows_total), torch.int32)


def _pooled(name: str, t: torch.Tensor, heads: int, blocks: int) -> None:
    _exact(name, t, (heads, blocks, HEAD_DIM), torch.float64)


def _heads(hq: int, hkv: int) -> None:
    _require(hkv >= 1 and hq % hkv == 0, f"query heads {hq} must be a multiple of KV heads {hkv}")


# ------------------------------------------------------------- single sequence
def discover(q: torch.Tensor, k: torch.Tensor, q_scale=None, k_scale=None, pooled_q=None, pooled_k=None):
    """Mean-pool Q [L, hq, 128] and K [L, hkv, 128] per 128-token block -> fp64
    ([hq, nb, 128], [hkv, nb, 128])."""
    _rows("q", q)
    L, hq, d = q.shape
    _rows("k", k, tokens=L)
    hkv = k.shape[1]
    _heads(hq, hkv)
    code = _same_dtype(q, ("k", k))
    _scales(code, q_scale=(q_scale, hq), k_scale=(k_scale, hkv))
    nb = _nb(L)
    if pooled_q is None:
        pooled_q = torch.empty((hq, nb, d), dtype=torch.float64, device=q.device)
    if pooled_k is None:
        pooled_k = torch.empty((hkv, nb, d), dtype=torch.float64, device=q.device)
    _pooled("pooled_q", pooled_q, hq, nb)
    _pooled("pooled_k", pooled_k, hkv, nb)
    _device(q, k, q_scale, k_scale, pooled_q, pooled_k)
    call("fp_discover", _ptr(q), _ptr(k), _dtype_code(q), _ptr(q_scale), _ptr(k_scale), L, hq, hkv, d, BLOCK,
         q.stride(0), q.stride(1), k.stride(0), k.stride(1), _ptr(pooled_q), _ptr(pooled_k), _stream(q))
    return pooled_q, pooled_k


def threshold_compact(pooled_q: torch.Tensor, pooled_k: torch.Tensor, alpha: float, n_sink: int, n_local: int,
                      softmax_scale: Optional[float] = None, idx=None, counts=None, scores=None):
    """Block scores, alpha x row-max threshold with sink/local blocks, ascending
    lists -> (idx int32 triangular-packed [hq * nb(nb+1)/2], counts int32 [hq, nb]).
    scores: optional fp64 [hq, nb, nb] tensor that receives the scaled pooled
    scores s_ij for j <= i (a debug output; entries j > i are left as they are)."""
    hq, nb, d = pooled_q.shape
    hkv = pooled_k.shape[0]
    _heads(hq, hkv)
    _pooled("pooled_q", pooled_q, hq, nb)
    _pooled("pooled_k", pooled_k, hkv, nb)
    if softmax_scale is None:
        softmax_scale = default_scale(d)
    if idx is None:
        idx = torch.zeros(idx_capacity(hq, nb), dtype=torch.int32, device=pooled_q.device)
    if counts is None:
        counts = torch.empty((hq, nb), dtype=torch.int32, device=pooled_q.device)
    _lists(idx, counts, hq, nb, nb * (nb + 1) // 2)
    _exact("scores", scores, (hq, nb, nb), torch.float64)
    _device(pooled_q, pooled_k, idx, counts, scores)
    call("fp_threshold_compact", _ptr(pooled_q), _ptr(pooled_k), nb, hq, hkv, d, float(softmax_scale),
         float(alpha), int(n_sink), int(n_local), _ptr(idx), _ptr(counts), _ptr(scores), _stream(pooled_q))
    return idx, counts


def mask_words(nb: int) -> int:
    """32-bit words per row of a bit-packed block mask."""
    return (nb + 31) // 32


def threshold_mask(pooled_q: torch.Tensor, pooled_k: torch.Tensor, alpha: float, n_sink: int, n_local: int,
                   softmax_scale: Optional[float] = None, mask=None):
    """The threshold decisions as a bit-packed block mask (int32 words holding uint32
    bits) [hq, nb, ceil(nb/32)]: bit j%32 of word j//32 of row (h, i) = keep(h, i, j).
    Words never written are left as allocated (zeros here)."""
    hq, nb, d = pooled_q.shape
    hkv = pooled_k.shape[0]
    if softmax_scale is None:
        softmax_scale = default_scale(d)
    _heads(hq, hkv)
    _pooled("pooled_q", pooled_q, hq, nb)
    _pooled("pooled_k", pooled_k, hkv, nb)
    if mask is None:
        mask = torch.zeros((hq, nb, mask_words(nb)), dtype=torch.int32, device=pooled_q.device)
    _exact("mask", mask, (hq, nb, mask_words(nb)), torch.int32)
    _device(pooled_q, pooled_k, mask)
    call("fp_threshold_mask", _ptr(pooled_q), _ptr(pooled_k), nb, hq, hkv, d, float(softmax_scale),
         float(alpha), int(n_sink), int(n_local), _ptr(mask), _stream(pooled_q))
    return mask


def _lse_buffer(lse, return_lse, heads, tokens, device):
    """The caller's LSE buffer [heads, tokens] fp32, a new one, or None."""
    if lse is not None:
        _exact("lse", lse, (heads, tokens), torch.float32)
        return lse
    return torch.empty((heads, tokens), dtype=torch.float32, device=device) if return_lse else None


def _attn(name, q, k, v, idx, counts, q_scale, k_scale, v_scale, softmax_scale, out, return_lse, lse=None):
    _rows("q", q)
    L, hq, d = q.shape
    _rows("k", k, tokens=L)
    hkv = k.shape[1]
    _rows("v", v, tokens=L, heads=hkv)
    _heads(hq, hkv)
    code = _same_dtype(q, ("k", k), ("v", v))
    _scales(code, q_scale=(q_scale, hq), k_scale=(k_scale, hkv), v_scale=(v_scale, hkv))
    nb = _nb(L)
    if name == "fp_sparse_attn":
        _lists(idx, counts, hq, nb, nb * (nb + 1) // 2)
    elif name == "fp_sparse_attn_grouped":
        _lists(idx, counts, hkv, nb, nb * (nb + 1) // 2)
    elif name == "fp_sparse_attn_masked":
        _exact("mask", idx, (hq, nb, mask_words(nb)), torch.int32)
    if softmax_scale is None:
        softmax_scale = default_scale(d)
    if out is None:
        out = torch.empty((L, hq, d), dtype=torch.bfloat16, device=q.device)
    _out_rows(out, L, hq)
    return_lse = return_lse or lse is not None
    lse = _lse_buffer(lse, return_lse, hq, L, q.device)
    _device(q, k, v, q_scale, k_scale, v_scale, idx, counts, out, lse)
    args = [_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(q_scale), _ptr(k_scale), _ptr(v_scale),
            L, hq, hkv, d, BLOCK, q.stride(0), q.stride(1), k.stride(0), k.stride(1),
            v.stride(0), v.stride(1), out.stride(0), out.stride(1)]
    if name in ("fp_sparse_attn", "fp_sparse_attn_grouped"):
        args += [_ptr(idx), _ptr(counts)]
    elif name == "fp_sparse_attn_masked":
        args += [_ptr(idx)]
    args += [float(softmax_scale), _ptr(out), _ptr(lse), _stream(q)]
    call(name, *args)
    return (out, lse) if return_lse else out


def sparse_attn(q, k, v, idx, counts, q_scale=None, k_scale=None, v_scale=None, softmax_scale=None,
                out=None, return_lse=False, lse=None):
    """Causal GQA attention of Q [L, hq, 128] over the listed K/V blocks -> bf16 [L, hq, 128]
    (and the natural-log LSE [hq, L] fp32 when return_lse or an lse buffer is given)."""
    return _attn("fp_sparse_attn", q, k, v, idx, counts, q_scale, k_scale, v_scale, softmax_scale, out, return_lse,
                 lse)


def pool(x, scale=None, pooled=None):
    """Block means of x [L, H, 128] (bf16, or e4m3 codes with per-head scale)
    -> [H, nb, 128] fp64."""
    _rows("x", x)
    L, H, d = x.shape
    code = _dtype_code(x)
    _scales(code, scale=(scale, H))
    if pooled is None:
        pooled = torch.empty((H, _nb(L), d), dtype=torch.float64, device=x.device)
    _pooled("pooled", pooled, H, _nb(L))
    _device(x, scale, pooled)
    call("fp_pool", _ptr(x), _dtype_code(x), _ptr(scale), L, H, d, BLOCK, x.stride(0), x.stride(1), _ptr(pooled),
         _stream(x))
    return pooled


def mean_correct_workspace(L: int, hkv: int, device) -> torch.Tensor:
    """Scratch for mean_correct: fp_mean_correct_workspace_bytes(L, hkv) bytes."""
    n = int(load().fp_mean_correct_workspace_bytes(L, hkv))
    if n < 0:
        raise ValueError(f"invalid L={L} / hkv={hkv}")
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def mean_correct(q, pooled_k, pooled_v, idx, counts, out, lse, q_scale=None, softmax_scale=None, workspace=None):
    """The V2 mean correction as implemented here (an assumption, off unless called):
    fold every pruned block, as 128 copies of its mean key and value, into the output
    and LSE of sparse_attn(..., return_lse=True), in place.  workspace: a buffer from
    mean_correct_workspace (allocated here when None)."""
    _rows("q", q)
    L, hq, d = q.shape
    hkv = pooled_k.shape[0]
    _heads(hq, hkv)
    nb = _nb(L)
    code = _dtype_code(q)
    _scales(code, q_scale=(q_scale, hq))
    _pooled("pooled_k", pooled_k, hkv, nb)
    _pooled("pooled_v", pooled_v, hkv, nb)
    _lists(idx, counts, hq, nb, nb * (nb + 1) // 2)
    _out_rows(out, L, hq)
    _exact("lse", lse, (hq, L), torch.float32)
    _require(lse is not None, "lse is required (the sparse call's return_lse=True output)")
    if softmax_scale is None:
        softmax_scale = default_scale(d)
    if workspace is None:
        workspace = mean_correct_workspace(L, hkv, q.device)
    _capacity("workspace", workspace, int(load().fp_mean_correct_workspace_bytes(L, hkv)), torch.uint8)
    _device(q, q_scale, pooled_k, pooled_v, idx, counts, out, lse, workspace)
    call("fp_mean_correct", _ptr(q), _dtype_code(q), _ptr(q_scale), _ptr(pooled_k), _ptr(pooled_v), L, hq, hkv,
         d, BLOCK, q.stride(0), q.stride(1), out.stride(0), out.stride(1), _ptr(idx), _ptr(counts),
         float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), _stream(q))
    return out, lse


def mean_correct_noalloc(q, pooled_k, pooled_v, idx, counts, out, lse, q_scale=None, softmax_scale=None):
    """mean_correct without a workspace: the library's static per-GPU scratch (8 MiB)
    holds the tile images, so nothing is allocated.  Calls that overlap on one GPU
    race; sizes beyond the scratch raise FlashPrefillError (FP_EUNSUPPORTED)."""
    _rows("q", q)
    L, hq, d = q.shape
    hkv = pooled_k.shape[0]
    _heads(hq, hkv)
    nb = _nb(L)
    _scales(_dtype_code(q), q_scale=(q_scale, hq))
    _pooled("pooled_k", pooled_k, hkv, nb)
    _pooled("pooled_v", pooled_v, hkv, nb)
    _lists(idx, counts, hq, nb, nb * (nb + 1) // 2)
    _out_rows(out, L, hq)
    _exact("lse", lse, (hq, L), torch.float32)
    _require(lse is not None, "lse is required (the sparse call's return_lse=True output)")
    if softmax_scale is None:
        softmax_scale = default_scale(d)
    _device(q, q_scale, pooled_k, pooled_v, idx, counts, out, lse)
    call("fp_mean_correct_noalloc", _ptr(q), _dtype_code(q), _ptr(q_scale), _ptr(pooled_k), _ptr(pooled_v), L, hq,
         hkv, d, BLOCK, q.stride(0), q.stride(1), out.stride(0), out.stride(1), _ptr(idx), _ptr(counts),
         float(softmax_scale), _ptr(out), _ptr(lse), _stream(q))
    return out, lse


def union_compact(mask, hkv: int, idx=None, counts=None):
    """Group-shared lists: the union of the per-head masks (from threshold_mask) of
    every KV group, as ascending lists -> (idx [hkv * nb(nb+1)/2] int32,
    counts [hkv, nb] int32)."""
    _require(mask.dim() == 3, f"mask must be [hq, nb, words], got shape {tuple(mask.shape)}")
    hq, nb, _ = mask.shape
    _heads(hq, hkv)
    _exact("mask", mask, (hq, nb, mask_words(nb)), torch.int32)
    if idx is None:
        idx = torch.zeros(idx_capacity(hkv, nb), dtype=torch.int32, device=mask.device)
    if counts is None:
        counts = torch.empty((hkv, nb), dtype=torch.int32, device=mask.device)
    _lists(idx, counts, hkv, nb, nb * (nb + 1) // 2)
    _device(mask, idx, counts)
    call("fp_union_compact", _ptr(mask), nb, hq, hkv, _ptr(idx), _ptr(counts), _stream(mask))
    return idx, counts


def sparse_attn_grouped(q, k, v, idx, counts, q_scale=None, k_scale=None, v_scale=None, softmax_scale=None,
                        out=None, return_lse=False, lse=None):
    """sparse_attn with one list per KV group (from union_compact): every query head
    attends over its group's list."""
    return _attn("fp_sparse_attn_grouped", q, k, v, idx, counts, q_scale, k_scale, v_scale, softmax_scale, out,
                 return_lse, lse)


def sparse_attn_masked(q, k, v, mask, q_scale=None, k_scale=None, v_scale=None, softmax_scale=None,
                       out=None, return_lse=False, lse=None):
    """Logical-skip form of sparse_attn: loops over every causal key block and skips
    those whose mask bit is 0 (mask from threshold_mask).  Same output as sparse_attn
    on the lists of the same decisions."""
    return _attn("fp_sparse_attn_masked", q, k, v, mask, None, q_scale, k_scale, v_scale, softmax_scale, out,
                 return_lse, lse)


def dense_attn(q, k, v, q_scale=None, k_scale=None, v_scale=None, softmax_scale=None, out=None, return_lse=False,
               lse=None):
    """Dense causal GQA attention with the same kernel (implicit full lists)."""
    return _attn("fp_dense_attn", q, k, v, None, None, q_scale, k_scale, v_scale, softmax_scale, out, return_lse,
                 lse)


def prefill(q, k, v, alpha: float, n_sink: int = 1, n_local: int = 4, q_scale=None, k_scale=None, v_scale=None,
            softmax_scale=None, return_lse=False):
    """discover -> threshold_compact -> sparse_attn on one sequence."""
    pq, pk = discover(q, k, q_scale, k_scale)
    idx, counts = threshold_compact(pq, pk, alpha, n_sink, n_local, softmax_scale)
    res = sparse_attn(q, k, v, idx, counts, q_scale, k_scale, v_scale, softmax_scale, return_lse=return_lse)
    return res, idx, counts


# ------------------------------------------------------------ packed batches
@dataclass
class VarlenBatch:
    """Host-side description of a packed batch; cu_seqlens lives on the device."""
    lengths: Sequence[int]
    device: torch.device

    def __post_init__(self):
        self.lengths = [int(x) for x in self.lengths]
        cu = [0]
        for n in self.lengths:
            cu.append(cu[-1] + n)
        self.cu_seqlens = torch.tensor(cu, dtype=torch.int32, device=self.device)
        nbs = [_nb(n) for n in self.lengths]
        self.seq_blocks = nbs
        self.cu_blocks = [0]
        self.cu_tri = [0]
        for nb in nbs:
            self.cu_blocks.append(self.cu_blocks[-1] + nb)
            self.cu_tri.append(self.cu_tri[-1] + nb * (nb + 1) // 2)
        self.n_seqs = len(self.lengths)
        self.max_seqlen = max(self.lengths) if self.lengths else 0
        self.total_tokens = cu[-1]
        self.total_blocks = self.cu_blocks[-1]
        self.total_tri = self.cu_tri[-1]


def _kv_batch(name, t, page_table, tokens, heads=None):
    """Packed K/V [tokens, heads, 128] (page_table None) or a page cache."""
    if page_table is None:
        _rows(name, t, tokens=tokens, heads=heads)
    else:
        _pages(name, t, heads=heads)


def _page_table(page_table, n_seqs: int, need_pages: int) -> None:
    if page_table is None:
        return
    _require(page_table.dim() == 2 and page_table.shape[0] == n_seqs,
             f"page_table must be [n_seqs={n_seqs}, max_pages], got shape {tuple(page_table.shape)}")
    _require(page_table.dtype == torch.int32 and page_table.is_contiguous(), "page_table must be contiguous int32")
    _require(page_table.shape[1] >= need_pages,
             f"page_table has {page_table.shape[1]} pages per sequence, needs {need_pages}")


def discover_paged(q, k, batch: VarlenBatch, page_table=None, q_scale=None, k_scale=None,
                   pooled_q=None, pooled_k=None):
    """Per-sequence pooling of packed Q [T, hq, 128] and K, either packed [T, hkv, 128]
    (page_table None) or a page cache [P, 128, hkv, 128] -> ([hq, total_blocks, 128],
    [hkv, total_blocks, 128]) fp64."""
    _rows("q", q, tokens=batch.total_tokens)
    T, hq, d = q.shape
    _kv_batch("k", k, page_table, batch.total_tokens)
    _page_table(page_table, batch.n_seqs, _nb(batch.max_seqlen))
    if page_table is not None:
        P, _, hkv, _ = k.shape
        k_sp, k_st, k_sh = k.stride(0), k.stride(1), k.stride(2)
        max_pages = page_table.shape[1]
    else:
        P, hkv = 0, k.shape[1]
        k_sp, k_st, k_sh = 0, k.stride(0), k.stride(1)
        max_pages = 0
    _heads(hq, hkv)
    code = _same_dtype(q, ("k", k))
    _scales(code, q_scale=(q_scale, hq), k_scale=(k_scale, hkv))
    if pooled_q is None:
        pooled_q = torch.empty((hq, batch.total_blocks, d), dtype=torch.float64, device=q.device)
    if pooled_k is None:
        pooled_k = torch.empty((hkv, batch.total_blocks, d), dtype=torch.float64, device=q.device)
    _pooled("pooled_q", pooled_q, hq, batch.total_blocks)
    _pooled("pooled_k", pooled_k, hkv, batch.total_blocks)
    _device(q, k, page_table, q_scale, k_scale, pooled_q, pooled_k, batch.cu_seqlens)
    call("fp_discover_paged", _ptr(q), _ptr(k), _dtype_code(q), _ptr(q_scale), _ptr(k_scale),
         _ptr(batch.cu_seqlens), batch.n_seqs, batch.max_seqlen, batch.total_tokens, batch.total_blocks,
         _ptr(page_table), max_pages, P, hq, hkv, d, BLOCK, q.stride(0), q.stride(1), k_sp, k_st, k_sh,
         _ptr(pooled_q), _ptr(pooled_k), _stream(q))
    return pooled_q, pooled_k


def threshold_compact_varlen(pooled_q, pooled_k, batch: VarlenBatch, alpha: float, n_sink: int, n_local: int,
                             softmax_scale=None, idx=None, counts=None):
    """Per-sequence lists -> (idx [hq * total_tri] int32, counts [hq, total_blocks] int32)."""
    hq, _, d = pooled_q.shape
    hkv = pooled_k.shape[0]
    if softmax_scale is None:
        softmax_scale = default_scale(d)
    _heads(hq, hkv)
    _pooled("pooled_q", pooled_q, hq, batch.total_blocks)
    _pooled("pooled_k", pooled_k, hkv, batch.total_blocks)
    if idx is None:
        idx = torch.zeros(hq * batch.total_tri, dtype=torch.int32, device=pooled_q.device)
    if counts is None:
        counts = torch.empty((hq, batch.total_blocks), dtype=torch.int32, device=pooled_q.device)
    _lists(idx, counts, hq, batch.total_blocks, batch.total_tri)
    _device(pooled_q, pooled_k, idx, counts, batch.cu_seqlens)
    call("fp_threshold_compact_varlen", _ptr(pooled_q), _ptr(pooled_k), _ptr(batch.cu_seqlens), batch.n_seqs,
         batch.max_seqlen, batch.total_blocks, batch.total_tri, hq, hkv, d, float(softmax_scale), float(alpha),
         int(n_sink), int(n_local), _ptr(idx), _ptr(counts), _stream(pooled_q))
    return idx, counts


def sparse_attn_paged(q, k, v, batch: VarlenBatch, idx=None, counts=None, page_table=None, q_scale=None,
                      k_scale=None, v_scale=None, softmax_scale=None, out=None, return_lse=False, lse=None):
    """Per-sequence causal attention of packed Q over listed blocks (idx/counts None =
    dense) with K/V packed or paged -> bf16 [T, hq, 128]."""
    _rows("q", q, tokens=batch.total_tokens)
    T, hq, d = q.shape
    _kv_batch("k", k, page_table, batch.total_tokens)
    _page_table(page_table, batch.n_seqs, _nb(batch.max_seqlen))
    if page_table is not None:
        P, _, hkv, _ = k.shape
        _pages("v", v, heads=hkv)
        _require(v.shape[0] == P, f"v has {v.shape[0]} pages, k has {P}")
        ks = (k.stride(0), k.stride(1), k.stride(2))
        vs = (v.stride(0), v.stride(1), v.stride(2))
        max_pages = page_table.shape[1]
    else:
        P, hkv = 0, k.shape[1]
        _rows("v", v, tokens=batch.total_tokens, heads=hkv)
        ks = (0, k.stride(0), k.stride(1))
        vs = (0, v.stride(0), v.stride(1))
        max_pages = 0
    _heads(hq, hkv)
    code = _same_dtype(q, ("k", k), ("v", v))
    _scales(code, q_scale=(q_scale, hq), k_scale=(k_scale, hkv), v_scale=(v_scale, hkv))
    _require((idx is None) == (counts is None), "idx and counts must both be given or both be None")
    if idx is not None:
        _lists(idx, counts, hq, batch.total_blocks, batch.total_tri)
    if softmax_scale is None:
        softmax_scale = default_scale(d)
    if out is None:
        out = torch.empty((T, hq, d), dtype=torch.bfloat16, device=q.device)
    _out_rows(out, T, hq)
    return_lse = return_lse or lse is not None
    lse = _lse_buffer(lse, return_lse, hq, T, q.device)
    _device(q, k, v, page_table, q_scale, k_scale, v_scale, idx, counts, out, lse, batch.cu_seqlens)
    call("fp_sparse_attn_paged", _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(q_scale), _ptr(k_scale),
         _ptr(v_scale), _ptr(batch.cu_seqlens), batch.n_seqs, batch.max_seqlen, batch.total_tokens,
         batch.total_blocks, batch.total_tri, _ptr(page_table), max_pages, P, hq, hkv, d, BLOCK,
         q.stride(0), q.stride(1), *ks, *vs, out.stride(0), out.stride(1), _ptr(idx), _ptr(counts),
         float(softmax_scale), _ptr(out), _ptr(lse), _stream(q))
    return (out, lse) if return_lse else out


def pool_varlen(x, batch: VarlenBatch, page_table=None, scale=None, pooled=None):
    """Per-sequence block means of packed x [T, H, 128] or of a page cache [P, 128, H, 128]
    -> [H, total_blocks, 128] fp64 (used to pool V for mean_correct_varlen)."""
    _kv_batch("x", x, page_table, batch.total_tokens)
    _page_table(page_table, batch.n_seqs, _nb(batch.max_seqlen))
    if page_table is not None:
        P, _, H, d = x.shape
        st = (x.stride(0), x.stride(1), x.stride(2))
        max_pages = page_table.shape[1]
    else:
        P, H, d = 0, x.shape[1], x.shape[2]
        st = (0, x.stride(0), x.stride(1))
        max_pages = 0
    _scales(_dtype_code(x), scale=(scale, H))
    if pooled is None:
        pooled = torch.empty((H, batch.total_blocks, d), dtype=torch.float64, device=x.device)
    _pooled("pooled", pooled, H, batch.total_blocks)
    _device(x, page_table, scale, pooled, batch.cu_seqlens)
    call("fp_pool_varlen", _ptr(x), _dtype_code(x), _ptr(scale), _ptr(batch.cu_seqlens), batch.n_seqs,
         batch.max_seqlen, batch.total_tokens, batch.total_blocks, _ptr(page_table), max_pages, P, H, d, BLOCK, *st,
         _ptr(pooled), _stream(x))
    return pooled


def mean_correct_varlen(q, pooled_k, pooled_v, batch: VarlenBatch, idx, counts, out, lse, q_scale=None,
                        softmax_scale=None, workspace=None):
    """mean_correct applied to every sequence of a packed batch, in place on the output
    and LSE of sparse_attn_paged(..., return_lse=True).  pooled_k from discover_paged,
    pooled_v from pool_varlen, idx/counts from threshold_compact_varlen."""
    _rows("q", q, tokens=batch.total_tokens)
    T, hq, d = q.shape
    hkv = pooled_k.shape[0]
    _heads(hq, hkv)
    _scales(_dtype_code(q), q_scale=(q_scale, hq))
    _pooled("pooled_k", pooled_k, hkv, batch.total_blocks)
    _pooled("pooled_v", pooled_v, hkv, batch.total_blocks)
    _lists(idx, counts, hq, batch.total_blocks, batch.total_tri)
    _out_rows(out, T, hq)
    _require(lse is not None, "lse is required (the sparse call's return_lse=True output)")
    _exact("lse", lse, (hq, T), torch.float32)
    if softmax_scale is None:
        softmax_scale = default_scale(d)
    need = int(load().fp_mean_correct_varlen_workspace_bytes(batch.total_blocks, max(batch.n_seqs, 1), hkv))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _capacity("workspace", workspace, need, torch.uint8)
    _device(q, q_scale, pooled_k, pooled_v, idx, counts, out, lse, workspace, batch.cu_seqlens)
    call("fp_mean_correct_varlen", _ptr(q), _dtype_code(q), _ptr(q_scale), _ptr(pooled_k), _ptr(pooled_v),
         _ptr(batch.cu_seqlens), batch.n_seqs, batch.max_seqlen, batch.total_tokens, batch.total_blocks,
         batch.total_tri, hq, hkv, d, BLOCK, q.stride(0), q.stride(1), out.stride(0), out.stride(1), _ptr(idx),
         _ptr(counts), float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), _stream(q))
    return out, lse


# --------------------------------------------------------------- chunked prefill
@dataclass
class ChunkedBatch:
    """Chunked / prefix-cached prefill batch: sequence s brings q_lengths[s] new
    queries against a K/V cache of k_lengths[s] >= q_lengths[s] tokens; its queries
    are the last q_lengths[s] positions.  Query blocks follow absolute positions
    (block I = positions 128I .. 128I+127), so sequence s has query blocks
    I0 .. I0+nq-1 with I0 = (k - q) // 128, and list row I has I + 1 slots."""
    q_lengths: Sequence[int]
    k_lengths: Sequence[int]
    device: torch.device

    def __post_init__(self):
        self.q_lengths = [int(x) for x in self.q_lengths]
        self.k_lengths = [int(x) for x in self.k_lengths]
        assert len(self.q_lengths) == len(self.k_lengths)
        assert all(0 <= q <= k for q, k in zip(self.q_lengths, self.k_lengths)), "need 0 <= len_q <= len_k"
        cq, ck = [0], [0]
        for q, k in zip(self.q_lengths, self.k_lengths):
            cq.append(cq[-1] + q)
            ck.append(ck[-1] + k)
        self.cu_seqlens_q = torch.tensor(cq, dtype=torch.int32, device=self.device)
        self.cu_seqlens_k = torch.tensor(ck, dtype=torch.int32, device=self.device)
        self.I0, self.nq, self.nk = [], [], []
        self.cu_qblocks, self.cu_kblocks, self.cu_tri = [0], [0], [0]
        for q, k in zip(self.q_lengths, self.k_lengths):
            off = k - q
            i0 = off // BLOCK
            nq = (off + q - 1) // BLOCK - i0 + 1 if q > 0 else 0
            nk = _nb(k)
            self.I0.append(i0)
            self.nq.append(nq)
            self.nk.append(nk)
            self.cu_qblocks.append(self.cu_qblocks[-1] + nq)
            self.cu_kblocks.append(self.cu_kblocks[-1] + nk)
            self.cu_tri.append(self.cu_tri[-1] + nq * (i0 + 1) + nq * (nq - 1) // 2)
        self.n_seqs = len(self.q_lengths)
        self.max_seqlen_q = max(self.q_lengths) if self.q_lengths else 0
        self.max_seqlen_k = max(self.k_lengths) if self.k_lengths else 0
        self.total_q = cq[-1]
        self.total_k = ck[-1]
        self.total_qblocks = self.cu_qblocks[-1]
        self.total_kblocks = self.cu_kblocks[-1]
        self.total_tri = self.cu_tri[-1]

    def row_offset(self, s: int, I: int) -> int:
        """Start of list row (s, absolute query block I) within one head's lists."""
        r = I - self.I0[s]
        return self.cu_tri[s] + r * (self.I0[s] + 1) + r * (r - 1) // 2


def _kv_strides(k, page_table):
    if page_table is not None:
        return k.shape[0], k.shape[2], (k.stride(0), k.stride(1), k.stride(2)), page_table.shape[1]
    return 0, k.shape[1], (0, k.stride(0), k.stride(1)), 0


def discover_chunked(q, k, batch: ChunkedBatch, page_table=None, q_scale=None, k_scale=None,
                     pooled_q=None, pooled_k=None):
    """Pooled means of the query blocks of every chunk (absolute block alignment) and
    of the key blocks of every cache -> (pooled_q [hq, total_qblocks, 128],
    pooled_k [hkv, total_kblocks, 128]) fp64."""
    _rows("q", q, tokens=batch.total_q)
    hq, d = q.shape[1], q.shape[2]
    _kv_batch("k", k, page_table, batch.total_k)
    _page_table(page_table, batch.n_seqs, _nb(batch.max_seqlen_k))
    P, hkv, ks, max_pages = _kv_strides(k, page_table)
    _heads(hq, hkv)
    code = _same_dtype(q, ("k", k))
    _scales(code, q_scale=(q_scale, hq), k_scale=(k_scale, hkv))
    if pooled_q is None:
        pooled_q = torch.empty((hq, batch.total_qblocks, d), dtype=torch.float64, device=q.device)
    if pooled_k is None:
        pooled_k = torch.empty((hkv, batch.total_kblocks, d), dtype=torch.float64, device=q.device)
    _pooled("pooled_q", pooled_q, hq, batch.total_qblocks)
    _pooled("pooled_k", pooled_k, hkv, batch.total_kblocks)
    _device(q, k, page_table, q_scale, k_scale, pooled_q, pooled_k, batch.cu_seqlens_q, batch.cu_seqlens_k)
    call("fp_discover_chunked", _ptr(q), _ptr(k), _dtype_code(q), _ptr(q_scale), _ptr(k_scale),
         _ptr(batch.cu_seqlens_q), _ptr(batch.cu_seqlens_k), batch.n_seqs, batch.max_seqlen_q, batch.max_seqlen_k,
         batch.total_q, batch.total_k, batch.total_qblocks, batch.total_kblocks, _ptr(page_table), max_pages, P,
         hq, hkv, d, BLOCK, q.stride(0), q.stride(1), *ks, _ptr(pooled_q), _ptr(pooled_k), _stream(q))
    return pooled_q, pooled_k


def threshold_compact_chunked(pooled_q, pooled_k, batch: ChunkedBatch, alpha: float, n_sink: int, n_local: int,
                              softmax_scale=None, idx=None, counts=None):
    """Lists of every (head, sequence, query block) -> (idx [hq * total_tri] int32,
    counts [hq, total_qblocks] int32); row layout as in ChunkedBatch.row_offset."""
    hq, _, d = pooled_q.shape
    hkv = pooled_k.shape[0]
    if softmax_scale is None:
        softmax_scale = default_scale(d)
    _heads(hq, hkv)
    _pooled("pooled_q", pooled_q, hq, batch.total_qblocks)
    _pooled("pooled_k", pooled_k, hkv, batch.total_kblocks)
    if idx is None:
        idx = torch.zeros(hq * batch.total_tri, dtype=torch.int32, device=pooled_q.device)
    if counts is None:
        counts = torch.empty((hq, batch.total_qblocks), dtype=torch.int32, device=pooled_q.device)
    _lists(idx, counts, hq, batch.total_qblocks, batch.total_tri)
    _device(pooled_q, pooled_k, idx, counts, batch.cu_seqlens_q, batch.cu_seqlens_k)
    call("fp_threshold_compact_chunked", _ptr(pooled_q), _ptr(pooled_k), _ptr(batch.cu_seqlens_q),
         _ptr(batch.cu_seqlens_k), batch.n_seqs, batch.max_seqlen_q, batch.max_seqlen_k, batch.total_qblocks,
         batch.total_kblocks, batch.total_tri, hq, hkv, d, float(softmax_scale), float(alpha), int(n_sink),
         int(n_local), _ptr(idx), _ptr(counts), _stream(pooled_q))
    return idx, counts


def sparse_attn_chunked(q, k, v, batch: ChunkedBatch, idx=None, counts=None, page_table=None, q_scale=None,
                        k_scale=None, v_scale=None, softmax_scale=None, out=None, return_lse=False, lse=None):
    """Chunk queries attend causally (bottom-right aligned) to their cache over the
    listed key blocks (idx/counts None = every block) -> bf16 [total_q, hq, 128]."""
    _rows("q", q, tokens=batch.total_q)
    T, hq, d = q.shape
    _kv_batch("k", k, page_table, batch.total_k)
    _page_table(page_table, batch.n_seqs, _nb(batch.max_seqlen_k))
    P, hkv, ks, max_pages = _kv_strides(k, page_table)
    _kv_batch("v", v, page_table, batch.total_k, heads=hkv)
    if page_table is not None:
        _require(v.shape[0] == P, f"v has {v.shape[0]} pages, k has {P}")
    _, _, vs, _ = _kv_strides(v, page_table)
    _heads(hq, hkv)
    code = _same_dtype(q, ("k", k), ("v", v))
    _scales(code, q_scale=(q_scale, hq), k_scale=(k_scale, hkv), v_scale=(v_scale, hkv))
    _require((idx is None) == (counts is None), "idx and counts must both be given or both be None")
    if idx is not None:
        _lists(idx, counts, hq, batch.total_qblocks, batch.total_tri)
    if softmax_scale is None:
        softmax_scale = default_scale(d)
    if out is None:
        out = torch.empty((T, hq, d), dtype=torch.bfloat16, device=q.device)
    _out_rows(out, T, hq)
    return_lse = return_lse or lse is not None
    lse = _lse_buffer(lse, return_lse, hq, T, q.device)
    _device(q, k, v, page_table, q_scale, k_scale, v_scale, idx, counts, out, lse,
            batch.cu_seqlens_q, batch.cu_seqlens_k)
    call("fp_sparse_attn_chunked", _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(q_scale), _ptr(k_scale),
         _ptr(v_scale), _ptr(batch.cu_seqlens_q), _ptr(batch.cu_seqlens_k), batch.n_seqs, batch.max_seqlen_q,
         batch.max_seqlen_k, batch.total_q, batch.total_k, batch.total_qblocks, batch.total_kblocks,
         batch.total_tri, _ptr(page_table), max_pages, P, hq, hkv, d, BLOCK, q.stride(0), q.stride(1), *ks, *vs,
         out.stride(0), out.stride(1), _ptr(idx), _ptr(counts), float(softmax_scale), _ptr(out), _ptr(lse),
         _stream(q))
    return (out, lse) if return_lse else out
