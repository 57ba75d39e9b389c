"""CPU oracle for top-k sparse attention and its bit-packed-mask form.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package's smoke check and the
benchmark's CPU-baseline leg may import this module. The GPU library never
imports, links or calls it, and it shares no code with the GPU library.

The arithmetic lives in ``sparse_attn_oracle.c`` (plain C, IEEE double). This
module compiles it with gcc when no built copy exists, loads it with ctypes and
marshals numpy arrays. bf16 tensors cross this boundary as their raw 16-bit
patterns (numpy ``uint16``).

Sources, per function:
  sparse_attn          "DeepSeek V4 源码剖析" ch. 5, sections 5.1, 5.2, 5.4, 5.5
  topk_mask_shape      prhub summary of vLLM PR #52217, key source (_topk_mask_shape)
  topk_mask_build      same page (_build_topk_mask + its test) and prhub summary of
                       vLLM PR #48770, key source (dense_mask_mod, offset_dense_mask_mod)
  masked_attn          prhub summary of vLLM PR #48770 (masked-MHA path) and PR #52217
  masked_attn_offset   prhub summary of vLLM PR #48770, key source (offset_dense_mask_mod:
                       chunked context, key index + key_start from the reserved word)
  candidate_mask       prhub summary of vLLM PR #56628 (the indexer's candidate-mask rule)
  sparse_attn_fp8      as sparse_attn, over FP8 rows in the MODEL1 layout of "DeepSeek V4
                       源码剖析" ch. 5, section 5.7 (448 e4m3 + 64 bf16 + 8 scale bytes)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "sparse_attn_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

_lock = threading.Lock()
_libs: dict[str, ctypes.CDLL] = {}


def build(path: str = LIBRARY, mutant: int = 0, openmp: bool = True) -> str:
    """Compile the C oracle into a shared library at ``path`` (always recompiles).

    ``mutant`` > 0 plants one of the numbered mistakes in the source; it exists only
    so the mutation test can show that the pins catch each of them.
    """
    cmd = ["gcc", "-O2", "-std=c11", "-shared", "-fPIC", "-o", path + ".tmp", SOURCE, "-lm"]
    if openmp:
        cmd.insert(1, "-fopenmp")
    if mutant:
        cmd.insert(1, f"-DORACLE_MUTANT={int(mutant)}")
    subprocess.run(cmd, check=True)
    os.replace(path + ".tmp", path)
    return path


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    P = ctypes.c_void_p
    I = ctypes.c_int64
    lib.oracle_sparse_attn.argtypes = [P, P, P, P, P, I, I, I, I, I, I, ctypes.c_double, P, I]
    lib.oracle_sparse_attn.restype = ctypes.c_int
    lib.oracle_topk_mask_shape.argtypes = [I, I, I, ctypes.c_int, P]
    lib.oracle_topk_mask_shape.restype = ctypes.c_int
    lib.oracle_topk_mask_build.argtypes = [P, P, P, P, I, I, I, I, I, I]
    lib.oracle_topk_mask_build.restype = ctypes.c_int
    lib.oracle_masked_attn.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, I, ctypes.c_double, P, I]
    lib.oracle_masked_attn.restype = ctypes.c_int
    lib.oracle_masked_attn_offset.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, I, ctypes.c_double, P, I]
    lib.oracle_masked_attn_offset.restype = ctypes.c_int
    lib.oracle_sparse_attn_fp8.argtypes = [P, P, P, P, P, I, I, I, I, I, ctypes.c_double, P, I]
    lib.oracle_sparse_attn_fp8.restype = ctypes.c_int
    lib.oracle_fp8_dequant.argtypes = [P, P, I]
    lib.oracle_fp8_dequant.restype = ctypes.c_int
    lib.oracle_candidate_mask.argtypes = [P, P, P, P, I, I, I, I, I, I, I, I]
    lib.oracle_candidate_mask.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_num_threads.restype = None
    return lib


def load(path: str = LIBRARY) -> ctypes.CDLL:
    """Load (building first only when missing) the oracle library at ``path``."""
    with _lock:
        lib = _libs.get(path)
        if lib is None:
            if not os.path.exists(path):
                build(path)
            lib = _bind(ctypes.CDLL(path))
            _libs[path] = lib
        return lib


class Oracle:
    """The oracle's operations, bound to one compiled copy of the C source."""

    def __init__(self, lib: ctypes.CDLL | None = None):
        self.lib = lib if lib is not None else load()

    @staticmethod
    def _ptr(a: np.ndarray | None) -> int | None:
        return None if a is None else a.ctypes.data

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def set_num_threads(self, n: int) -> None:
        """OpenMP threads for later calls (timing on fewer cores)."""
        self.lib.oracle_set_num_threads(int(n))

    def sparse_attn(self, q_bits, kv_bits, sink, idx, scale, tokens=None) -> np.ndarray:
        """o[t, h, :] for the flat tokens t = b*S + s listed in ``tokens`` (all when None).

        q_bits [B,S,H,D] uint16 (bf16 patterns), kv_bits [B,T,D] uint16, sink [H] float32,
        idx [B,S,K] int32. Returns float64 [len(tokens), H, D].
        """
        q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
        kv_bits = np.ascontiguousarray(kv_bits, dtype=np.uint16)
        sink = np.ascontiguousarray(sink, dtype=np.float32)
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        B, S, H, D = q_bits.shape
        Bk, T, Dk = kv_bits.shape
        K = idx.shape[2]
        if Bk != B or Dk != D or sink.shape != (H,) or idx.shape[:2] != (B, S):
            raise ValueError("sparse_attn oracle: inconsistent shapes")
        if tokens is None:
            tokens = np.arange(B * S, dtype=np.int64)
        tokens = np.ascontiguousarray(tokens, dtype=np.int64)
        out = np.empty((len(tokens), H, D), dtype=np.float64)
        rc = self.lib.oracle_sparse_attn(
            self._ptr(q_bits), self._ptr(kv_bits), self._ptr(sink), self._ptr(idx), self._ptr(out),
            B, S, H, D, T, K, float(scale), self._ptr(tokens), len(tokens))
        if rc != 0:
            raise ValueError("sparse_attn oracle rejected its arguments")
        return out

    def sparse_attn_fp8(self, q_bits, kv8, sink, idx, scale, tokens=None) -> np.ndarray:
        """sparse_attn over FP8 rows: kv8 [B,T,584] uint8 (D = 512). Returns float64 [len(tokens), H, 512]."""
        q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
        kv8 = np.ascontiguousarray(kv8, dtype=np.uint8)
        sink = np.ascontiguousarray(sink, dtype=np.float32)
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        B, S, H, D = q_bits.shape
        Bk, T, R = kv8.shape
        K = idx.shape[2]
        if D != 512 or R != 584 or Bk != B or sink.shape != (H,) or idx.shape[:2] != (B, S):
            raise ValueError("sparse_attn_fp8 oracle: inconsistent shapes")
        if tokens is None:
            tokens = np.arange(B * S, dtype=np.int64)
        tokens = np.ascontiguousarray(tokens, dtype=np.int64)
        out = np.empty((len(tokens), H, D), dtype=np.float64)
        rc = self.lib.oracle_sparse_attn_fp8(
            self._ptr(q_bits), self._ptr(kv8), self._ptr(sink), self._ptr(idx), self._ptr(out),
            B, S, H, T, K, float(scale), self._ptr(tokens), len(tokens))
        if rc != 0:
            raise ValueError("sparse_attn_fp8 oracle rejected its arguments")
        return out

    def fp8_dequant(self, kv8) -> np.ndarray:
        """Dequantized rows: kv8 [..., 584] uint8 -> float64 [..., 512]."""
        kv8 = np.ascontiguousarray(kv8, dtype=np.uint8)
        if kv8.shape[-1] != 584:
            raise ValueError("fp8_dequant oracle: rows are 584 bytes")
        n = kv8.size // 584
        out = np.empty(kv8.shape[:-1] + (512,), dtype=np.float64)
        if self.lib.oracle_fp8_dequant(self._ptr(kv8), self._ptr(out), n) != 0:
            raise ValueError("fp8_dequant oracle rejected its arguments")
        return out

    def topk_mask_shape(self, B, max_q, max_key, reserve_key_start_word=False) -> tuple[int, int, int]:
        out = np.zeros(3, dtype=np.int64)
        rc = self.lib.oracle_topk_mask_shape(int(B), int(max_q), int(max_key), int(bool(reserve_key_start_word)),
                                             self._ptr(out))
        if rc != 0:
            raise ValueError("topk_mask_shape oracle rejected its arguments")
        return int(out[0]), int(out[1]), int(out[2])

    def topk_mask_build(self, idx, key_len, q_lens=None, key_starts=None, padded_q=None, words=None) -> np.ndarray:
        """The whole [B, padded_q, words] uint32 mask for idx [B, Q, topk] int32.

        padded_q / words default to the shape rule (with the reserved word when
        key_starts is given).
        """
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        B, Q, topk = idx.shape
        _, pq, w = self.topk_mask_shape(B, Q, key_len, key_starts is not None)
        padded_q = pq if padded_q is None else int(padded_q)
        words = w if words is None else int(words)
        ql = None if q_lens is None else np.ascontiguousarray(q_lens, dtype=np.int32)
        ks = None if key_starts is None else np.ascontiguousarray(key_starts, dtype=np.int32)
        mask = np.empty((B, padded_q, words), dtype=np.uint32)
        rc = self.lib.oracle_topk_mask_build(self._ptr(idx), self._ptr(ql), self._ptr(ks), self._ptr(mask),
                                             B, Q, topk, int(key_len), padded_q, words)
        if rc != 0:
            raise ValueError("topk_mask_build oracle rejected its arguments")
        return mask

    def masked_attn(self, q_bits, k_bits, v_bits, mask, scale, rows=None) -> np.ndarray:
        """o[r, h, :] for flat query rows r = b*Q + q listed in ``rows`` (all when None).

        q_bits [B,Q,H,Dqk], k_bits [B,KV,H,Dqk], v_bits [B,KV,H,Dv] uint16; mask
        [B,padded_q,W] uint32 or None (every key visible). Returns float64 [len(rows), H, Dv].
        """
        return self._masked(self.lib.oracle_masked_attn, q_bits, k_bits, v_bits, mask, scale, rows)

    def masked_attn_offset(self, q_bits, k_bits, v_bits, mask, scale, rows=None) -> np.ndarray:
        """The chunked-context form: chunk key j is mask key key_start[b] + j, with key_start[b]
        the reserved word mask[b, 0, W-1]; keys at or past that word are never visible.
        Arguments and result as masked_attn (mask required)."""
        if mask is None:
            raise ValueError("masked_attn_offset oracle: the mask is required")
        return self._masked(self.lib.oracle_masked_attn_offset, q_bits, k_bits, v_bits, mask, scale, rows)

    def _masked(self, fn, q_bits, k_bits, v_bits, mask, scale, rows):
        q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
        k_bits = np.ascontiguousarray(k_bits, dtype=np.uint16)
        v_bits = np.ascontiguousarray(v_bits, dtype=np.uint16)
        B, Q, H, Dqk = q_bits.shape
        _, KV, _, Dv = v_bits.shape
        if k_bits.shape != (B, KV, H, Dqk) or v_bits.shape[:3] != (B, KV, H):
            raise ValueError("masked_attn oracle: inconsistent shapes")
        if mask is not None:
            mask = np.ascontiguousarray(mask, dtype=np.uint32)
            if mask.shape[0] != B:
                raise ValueError("masked_attn oracle: mask batch mismatch")
            padded_q, W = mask.shape[1], mask.shape[2]
        else:
            padded_q, W = Q, 0
        if rows is None:
            rows = np.arange(B * Q, dtype=np.int64)
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        out = np.empty((len(rows), H, Dv), dtype=np.float64)
        rc = fn(
            self._ptr(q_bits), self._ptr(k_bits), self._ptr(v_bits), self._ptr(mask), self._ptr(out),
            B, Q, KV, H, Dqk, Dv, padded_q, W, float(scale), self._ptr(rows), len(rows))
        if rc != 0:
            raise ValueError("masked_attn oracle rejected its arguments")
        return out


    def candidate_mask(self, logits, ends, flags, block_size, starts=None, row_repeat=1) -> np.ndarray:
        """The whole-row candidate mask applied to a copy of ``logits`` (float32 [rows, width], any
        element strides that are multiples of 4 bytes). ends / starts int32 1-D (strided views
        allowed), flags uint8 [rows, nblocks + 1]. Returns the masked copy."""
        out = np.array(logits, dtype=np.float32, copy=True)
        if out.ndim != 2:
            raise ValueError("candidate_mask oracle: logits must be 2-D")
        rows, width = out.shape
        flags = np.ascontiguousarray(flags, dtype=np.uint8)
        ends = np.asarray(ends)
        if ends.dtype != np.int32 or (starts is not None and np.asarray(starts).dtype != np.int32):
            raise ValueError("candidate_mask oracle: starts / ends must be int32")
        st = None if starts is None else np.asarray(starts)
        sr, sc = out.strides[0] // 4, out.strides[1] // 4
        rc = self.lib.oracle_candidate_mask(
            out.ctypes.data, None if st is None else st.ctypes.data, ends.ctypes.data, flags.ctypes.data,
            rows, width, sr, sc, 0 if st is None else st.strides[0] // 4, ends.strides[0] // 4, int(block_size),
            int(row_repeat))
        if rc != 0:
            raise ValueError("candidate_mask oracle rejected its arguments")
        return out


def bf16_bits(x) -> np.ndarray:
    """Raw 16-bit patterns of a torch bfloat16 tensor (any device) as numpy uint16."""
    import torch  # local: the oracle itself needs no torch

    t = x.detach().to("cpu").contiguous()
    if t.dtype != torch.bfloat16:
        raise TypeError("bf16_bits expects a bfloat16 tensor")
    return t.view(torch.int16).numpy().view(np.uint16)


def bits_to_float(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float64 (exact)."""
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def float_to_bits(x: np.ndarray) -> np.ndarray:
    """Round float values to bf16 (nearest-even) and return the bit patterns (used for fixtures)."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(f)
    out = rounded.astype(np.uint16)
    out[nan] = 0x7FC0
    return out
