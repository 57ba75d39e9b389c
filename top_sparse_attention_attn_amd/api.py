"""Python binding of libsparse_attn.so (declared in include/sparse_attn.h).

Argument marshalling only: every entry point checks dtypes/devices/contiguity of
the torch tensors, passes their device pointers and the current HIP stream to
the C ABI, and raises SparseAttnError on a nonzero status. All computation runs
in the library's kernels; if the library cannot be loaded the first call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsparse_attn.so")
_lib = None
_lock = threading.Lock()

SA_STATUS = {0: "SA_OK", 1: "SA_ERR_NULL", 2: "SA_ERR_SHAPE", 3: "SA_ERR_ALIGN", 4: "SA_ERR_UNSUPPORTED",
             5: "SA_ERR_WORKSPACE", 6: "SA_ERR_HIP"}

EXPORTED = ["sa_status_string", "sparse_attn_workspace_bytes", "sparse_attn_num_splits", "sparse_attn_head_groups",
            "sparse_attn_fp8_num_splits", "sparse_attn_fwd",
            "sparse_attn_fwd_noalloc",
            "sparse_attn_split_fwd", "sparse_attn_merge_fwd", "sparse_attn_fp8_fwd", "sparse_attn_fp8_split_fwd",
            "sparse_attn_fp8_merge_fwd", "topk_bitmask_shape", "topk_bitmask_build",
            "masked_attn_fwd", "masked_attn_offset_fwd", "candidate_mask_apply", "candidate_mask_grid"]


class SparseAttnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = _load().sa_status_string(status).decode() if _lib is not None else ""
        super().__init__(f"{fn} failed: {SA_STATUS.get(status, status)} ({msg})")


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with `python -m top_sparse_attention_attn_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        P, I64, I, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
        lib.sa_status_string.argtypes = [I]
        lib.sa_status_string.restype = ctypes.c_char_p
        lib.sparse_attn_workspace_bytes.argtypes = [I64, I64, I64, I64, I64, I]
        lib.sparse_attn_workspace_bytes.restype = ctypes.c_size_t
        lib.sparse_attn_num_splits.argtypes = [I64, I64, I64, I64, I64]
        lib.sparse_attn_num_splits.restype = I
        lib.sparse_attn_head_groups.argtypes = [I64, I64, I64, I64, I64, I]
        lib.sparse_attn_head_groups.restype = I
        lib.sparse_attn_fp8_num_splits.argtypes = [I64, I64, I64, I64]
        lib.sparse_attn_fp8_num_splits.restype = I
        for name in ("sparse_attn_fwd", "sparse_attn_split_fwd", "sparse_attn_merge_fwd"):
            getattr(lib, name).argtypes = [P, P, P, P, P, I64, I64, I64, I64, I64, I64, F, I, P, ctypes.c_size_t, P]
            getattr(lib, name).restype = I
        lib.sparse_attn_fwd_noalloc.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I64, I64, F, I, P]
        lib.sparse_attn_fwd_noalloc.restype = I
        for name in ("sparse_attn_fp8_fwd", "sparse_attn_fp8_split_fwd", "sparse_attn_fp8_merge_fwd"):
            getattr(lib, name).argtypes = [P, P, P, P, P, I64, I64, I64, I64, I64, F, I, P, ctypes.c_size_t, P]
            getattr(lib, name).restype = I
        lib.topk_bitmask_shape.argtypes = [I64, I64, I64, I, P]
        lib.topk_bitmask_shape.restype = I
        lib.topk_bitmask_build.argtypes = [P, P, P, P, I64, I64, I64, I64, I64, I64, P]
        lib.topk_bitmask_build.restype = I
        lib.masked_attn_fwd.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I64, I64, I64, I64, F, I, P]
        lib.masked_attn_fwd.restype = I
        lib.masked_attn_offset_fwd.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, I64, I64, I64, I64, F, P]
        lib.masked_attn_offset_fwd.restype = I
        lib.candidate_mask_apply.argtypes = [P, P, P, P, I64, I64, I64, I64, I64, I64, I64, I64, P]
        lib.candidate_mask_apply.restype = I
        lib.candidate_mask_grid.argtypes = [I64, I64]
        lib.candidate_mask_grid.restype = I
        _lib = lib
        return lib


def _stream_ptr(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t: torch.Tensor, name: str, dtype, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_strided(t: torch.Tensor, name: str, dtype, dim: int, device=None):
    """Like _check, but any (non-negative) element strides are accepted."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dim() != dim:
        raise ValueError(f"{name} must be {dim}-D")
    if any(st < 0 for st in t.stride()):
        raise ValueError(f"{name} has a negative stride")


def _call(fn_name: str, *args):
    rc = getattr(_load(), fn_name)(*args)
    if rc != 0:
        raise SparseAttnError(fn_name, rc)


# --------------------------------------------------------------------------- sparse attention
_ws_cache: dict = {}


def sparse_attn_num_splits(B: int, S: int, H: int, D: int, K: int) -> int:
    return int(_load().sparse_attn_num_splits(B, S, H, D, K))


def sparse_attn_head_groups(B: int, S: int, H: int, D: int, K: int, fp8: bool = False) -> int:
    return int(_load().sparse_attn_head_groups(B, S, H, D, K, int(bool(fp8))))


def sparse_attn_fp8_num_splits(B: int, S: int, H: int, K: int) -> int:
    return int(_load().sparse_attn_fp8_num_splits(B, S, H, K))


def sparse_attn_workspace_bytes(B: int, S: int, H: int, D: int, K: int, num_splits: int = 0) -> int:
    return int(_load().sparse_attn_workspace_bytes(B, S, H, D, K, num_splits))


def new_workspace(nbytes: int, device) -> torch.Tensor:
    """A 256-byte aligned uint8 device buffer of `nbytes` bytes, usable as sparse_attn's workspace."""
    ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws[off:off + nbytes]


def _workspace(device: torch.device, nbytes: int, workspace: torch.Tensor | None):
    if nbytes == 0:
        return None, 0
    if workspace is not None:
        _check(workspace, "workspace", torch.uint8, device)
        return workspace, workspace.numel()
    key = (device, torch.cuda.current_stream(device).cuda_stream)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes + 256:
        ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    off = (-ws.data_ptr()) % 256
    view = ws[off:off + nbytes]
    return view, view.numel()


def sparse_attn(q: torch.Tensor, kv: torch.Tensor, attn_sink: torch.Tensor, topk_idxs: torch.Tensor,
                scale: float, out: torch.Tensor | None = None, num_splits: int = 0,
                workspace: torch.Tensor | None = None) -> torch.Tensor:
    """o = sparse_attn(q, kv, attn_sink, topk_idxs, scale).

    q [B,S,H,D] bf16, kv [B,T,D] bf16, attn_sink [H] fp32, topk_idxs [B,S,K] int32
    (-1 = empty slot); returns o [B,S,H,D] bf16. num_splits = 0 lets the library choose;
    `workspace` (uint8, 256-byte aligned, see new_workspace) overrides the cached one.
    """
    return _sparse_call("sparse_attn_fwd", q, kv, attn_sink, topk_idxs, scale, out, num_splits, workspace)


def sparse_attn_noalloc(q: torch.Tensor, kv: torch.Tensor, attn_sink: torch.Tensor, topk_idxs: torch.Tensor,
                        scale: float, out: torch.Tensor | None = None, num_splits: int = 0) -> torch.Tensor:
    """sparse_attn through sparse_attn_fwd_noalloc: the split partials go to the library's own
    40 MiB device array (shared by every call on the GPU), so no workspace is allocated. With
    `out` given the call allocates nothing at all."""
    return _sparse_call("sparse_attn_fwd_noalloc", q, kv, attn_sink, topk_idxs, scale, out, num_splits, None)


def sparse_attn_split(q, kv, attn_sink, topk_idxs, scale, out=None, num_splits: int = 0, workspace=None):
    """First phase of sparse_attn (sparse_attn_split_fwd): split partials into `workspace`,
    or the full output when the call has one split. Pass the same workspace to sparse_attn_merge."""
    return _sparse_call("sparse_attn_split_fwd", q, kv, attn_sink, topk_idxs, scale, out, num_splits, workspace)


def sparse_attn_merge(q, kv, attn_sink, topk_idxs, scale, out, num_splits: int = 0, workspace=None):
    """Second phase of sparse_attn (sparse_attn_merge_fwd): merge the partials into `out`."""
    return _sparse_call("sparse_attn_merge_fwd", q, kv, attn_sink, topk_idxs, scale, out, num_splits, workspace)


def sparse_attn_fp8(q: torch.Tensor, kv8: torch.Tensor, attn_sink: torch.Tensor, topk_idxs: torch.Tensor,
                    scale: float, out: torch.Tensor | None = None, num_splits: int = 0,
                    workspace: torch.Tensor | None = None) -> torch.Tensor:
    """sparse_attn over FP8 rows: kv8 [B,T,584] uint8 in the MODEL1 row layout (448 e4m3 bytes,
    64 bf16 RoPE dims, 7 scale bytes + 1 pad; dim d < 448 = e4m3 * 2^(scale[d // 64] - 127)).
    q [B,S,H,512] bf16; otherwise as sparse_attn."""
    return _sparse_call("sparse_attn_fp8_fwd", q, kv8, attn_sink, topk_idxs, scale, out, num_splits, workspace)


def sparse_attn_fp8_split(q, kv8, attn_sink, topk_idxs, scale, out=None, num_splits: int = 0, workspace=None):
    """First phase of sparse_attn_fp8 (sparse_attn_fp8_split_fwd): split partials into `workspace`,
    or the full output when the call has one split. Pass the same workspace to sparse_attn_fp8_merge."""
    return _sparse_call("sparse_attn_fp8_split_fwd", q, kv8, attn_sink, topk_idxs, scale, out, num_splits, workspace)


def sparse_attn_fp8_merge(q, kv8, attn_sink, topk_idxs, scale, out, num_splits: int = 0, workspace=None):
    """Second phase of sparse_attn_fp8 (sparse_attn_fp8_merge_fwd): merge the partials into `out`."""
    return _sparse_call("sparse_attn_fp8_merge_fwd", q, kv8, attn_sink, topk_idxs, scale, out, num_splits, workspace)


def _sparse_call(entry, q, kv, attn_sink, topk_idxs, scale, out, num_splits, workspace):
    dev = q.device
    fp8 = entry.startswith("sparse_attn_fp8_")
    _check(q, "q", torch.bfloat16)
    _check(kv, "kv", torch.uint8 if fp8 else torch.bfloat16, dev)
    _check(attn_sink, "attn_sink", torch.float32, dev)
    _check(topk_idxs, "topk_idxs", torch.int32, dev)
    if q.dim() != 4 or kv.dim() != 3 or topk_idxs.dim() != 3 or attn_sink.dim() != 1:
        raise ValueError("expected q [B,S,H,D], kv [B,T,D], attn_sink [H], topk_idxs [B,S,K]")
    B, S, H, D = q.shape
    T = kv.shape[1]
    K = topk_idxs.shape[2]
    if kv.shape[0] != B or kv.shape[2] != (584 if fp8 else D) or attn_sink.shape[0] != H or \
            tuple(topk_idxs.shape[:2]) != (B, S) or (fp8 and D != 512):
        raise ValueError("inconsistent shapes")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", torch.bfloat16, dev)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    if entry == "sparse_attn_fwd_noalloc":
        _call(entry, _ptr(q), _ptr(kv), _ptr(attn_sink), _ptr(topk_idxs), _ptr(out), B, S, H, D, T, K,
              float(scale), int(num_splits), _stream_ptr(dev))
        return out
    need = sparse_attn_workspace_bytes(B, S, H, D, K, num_splits)
    ws, ws_bytes = _workspace(dev, need, workspace)
    if fp8:
        _call(entry, _ptr(q), _ptr(kv), _ptr(attn_sink), _ptr(topk_idxs), _ptr(out), B, S, H, T, K,
              float(scale), int(num_splits), _ptr(ws), ws_bytes, _stream_ptr(dev))
    else:
        _call(entry, _ptr(q), _ptr(kv), _ptr(attn_sink), _ptr(topk_idxs), _ptr(out), B, S, H, D, T, K,
              float(scale), int(num_splits), _ptr(ws), ws_bytes, _stream_ptr(dev))
    return out


# --------------------------------------------------------------------------- bit mask
def topk_bitmask_shape(B: int, max_q_len: int, max_key_len: int, reserve_key_start_word: bool = False):
    arr = (ctypes.c_int64 * 3)()
    _call("topk_bitmask_shape", B, max_q_len, max_key_len, int(bool(reserve_key_start_word)), arr)
    return int(arr[0]), int(arr[1]), int(arr[2])


def topk_bitmask_build(topk_idxs: torch.Tensor, key_len: int, q_lens: torch.Tensor | None = None,
                       key_starts: torch.Tensor | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """Bit-packed mask [B, padded_q, words] (uint32 bits stored as int32) for topk_idxs [B, Q, topk] int32."""
    dev = topk_idxs.device
    _check(topk_idxs, "topk_idxs", torch.int32)
    if topk_idxs.dim() != 3:
        raise ValueError("topk_idxs must be [B, Q, topk]")
    B, Q, topk = topk_idxs.shape
    if q_lens is not None:
        _check(q_lens, "q_lens", torch.int32, dev)
    if key_starts is not None:
        _check(key_starts, "key_starts", torch.int32, dev)
    if out is None:
        shape = topk_bitmask_shape(B, Q, key_len, key_starts is not None)
        out = torch.empty(shape, dtype=torch.int32, device=dev)
    else:
        _check(out, "out", torch.int32, dev)
        if out.dim() != 3 or out.shape[0] != B:
            raise ValueError("out must be [B, padded_q, words]")
    _call("topk_bitmask_build", _ptr(topk_idxs), _ptr(q_lens), _ptr(key_starts), _ptr(out), B, Q, topk, int(key_len),
          out.shape[1], out.shape[2], _stream_ptr(dev))
    return out


# --------------------------------------------------------------------------- masked attention
def masked_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask: torch.Tensor | None, scale: float,
                mask_load_bits: int = 128, out: torch.Tensor | None = None) -> torch.Tensor:
    """Dense attention over the keys whose mask bit is set (mask None = all keys).

    q [B,Q,H,192], k [B,KV,H,192], v [B,KV,H,128] bf16; mask [B,padded_q,words] int32/uint32 bits.
    """
    return _masked_call("masked_attn_fwd", q, k, v, mask, scale, out, (int(mask_load_bits),))


def masked_attn_offset(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask: torch.Tensor, scale: float,
                       out: torch.Tensor | None = None, return_lse: bool = False):
    """Chunked-context form: k, v are a chunk of KV keys and chunk key j reads mask bit
    key_start + j, with key_start = mask[b, 0, words-1] (written by topk_bitmask_build from
    key_starts). Shapes as masked_attn; the mask is required. With return_lse, also returns
    lse [B, Q, H] fp32 (natural log, -inf for no visible key), for merging the chunks of one
    context: o = sum_c exp(lse_c - LSE) o_c, LSE = logsumexp_c lse_c."""
    if mask is None:
        raise ValueError("masked_attn_offset needs the mask (it carries key_start)")
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_lse else None
    out = _masked_call("masked_attn_offset_fwd", q, k, v, mask, scale, out, (), lse=lse)
    return (out, lse) if return_lse else out


def _masked_call(entry, q, k, v, mask, scale, out, extra, lse=False):
    dev = q.device
    _check(q, "q", torch.bfloat16)
    _check(k, "k", torch.bfloat16, dev)
    _check(v, "v", torch.bfloat16, dev)
    B, Q, H, Dqk = q.shape
    KV, Dv = k.shape[1], v.shape[3]
    if k.shape != (B, KV, H, Dqk) or tuple(v.shape[:3]) != (B, KV, H):
        raise ValueError("inconsistent shapes")
    padded_q = words = 0
    if mask is not None:
        _check(mask, "mask", torch.int32, dev)
        if mask.dim() != 3 or mask.shape[0] != B:
            raise ValueError("mask must be [B, padded_q, words]")
        padded_q, words = mask.shape[1], mask.shape[2]
    if out is None:
        out = torch.empty((B, Q, H, Dv), dtype=torch.bfloat16, device=dev)
    else:
        _check(out, "out", torch.bfloat16, dev)
        if tuple(out.shape) != (B, Q, H, Dv):
            raise ValueError(f"out must be [{B}, {Q}, {H}, {Dv}]")
    lse_arg = () if lse is False else (_ptr(lse),)  # only the chunked-context entry takes lse
    _call(entry, _ptr(q), _ptr(k), _ptr(v), _ptr(mask), _ptr(out), *lse_arg, B, Q, KV, H, Dqk, Dv, padded_q, words,
          float(scale), *extra, _stream_ptr(dev))
    return out


# --------------------------------------------------------------------------- candidate mask
def candidate_mask_grid(rows: int, width: int) -> int:
    """Workgroups candidate_mask_apply launches for these shapes (a function of the shapes only)."""
    return int(_load().candidate_mask_grid(int(rows), int(width)))


def candidate_mask_apply(logits: torch.Tensor, ends: torch.Tensor, flags: torch.Tensor, block_size: int,
                         starts: torch.Tensor | None = None, row_repeat: int = 1) -> torch.Tensor:
    """Mask the indexer's decode logits in place: for row r (sharing starts/ends with the other
    rows of r // row_repeat), columns [start, end) keep their value where the block flag
    flags[r, (c - start) // block_size] (or, for the last column, the edge flag flags[r, nblocks])
    is set and become -inf otherwise; columns below start become -inf; columns at or past end
    are left as they are.

    logits float32 [rows, width] (any strides); ends / starts int32 1-D with ceil(rows /
    row_repeat) entries (any stride); flags uint8 [rows, ceil(width / block_size) + 1] contiguous.
    Returns logits.
    """
    dev = logits.device
    _check_strided(logits, "logits", torch.float32, 2)
    _check_strided(ends, "ends", torch.int32, 1, dev)
    if starts is not None:
        _check_strided(starts, "starts", torch.int32, 1, dev)
    _check(flags, "flags", torch.uint8, dev)
    rows, width = logits.shape
    block_size, row_repeat = int(block_size), int(row_repeat)
    if block_size < 1 or row_repeat < 1:
        raise ValueError("block_size and row_repeat must be >= 1")
    nb = -(-width // block_size)
    if tuple(flags.shape) != (rows, nb + 1):
        raise ValueError(f"flags must be [{rows}, {nb + 1}]")
    need = -(-rows // row_repeat)
    if ends.shape[0] < need or (starts is not None and starts.shape[0] < need):
        raise ValueError(f"ends / starts need {need} entries")
    _call("candidate_mask_apply", _ptr(logits), _ptr(starts), _ptr(ends), _ptr(flags), rows, width,
          logits.stride(0), logits.stride(1), 0 if starts is None else starts.stride(0), ends.stride(0), block_size,
          row_repeat, _stream_ptr(dev))
    return logits
