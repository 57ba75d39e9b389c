"""Helpers shared by the GPU parity tests (test harness only)."""
from __future__ import annotations

import numpy as np
import torch

import oracle

# Tolerance for bf16 outputs against the fp64 oracle: |gpu - ref| <= ATOL + RTOL * |ref|.
ATOL = 2e-2
RTOL = 2e-2


def bits(t: torch.Tensor) -> np.ndarray:
    return oracle.bf16_bits(t)


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_close(got: np.ndarray, ref: np.ndarray, what: str = ""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan_ref), f"{what}: NaN pattern differs"
    g, r = got[~nan_ref], ref[~nan_ref]
    err = np.abs(g - r)
    bad = err > ATOL + RTOL * np.abs(r)
    if bad.any():
        i = int(np.argmax(err - (ATOL + RTOL * np.abs(r))))
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; worst err {err[i]:.4g} "
                             f"at ref {r[i]:.4g}; max abs err {err.max():.4g}")


def compact_rows(kv: torch.Tensor, idx: torch.Tensor, tokens: np.ndarray, S: int):
    """For sampled tokens, gather only the kv rows they reference (test harness, not method
    arithmetic): returns kv_c [n, T_c, D] bf16 (CPU), idx_c [n, 1, K] int32 with indices
    remapped into kv_c (empty slots stay -1) so the oracle sees the same rows."""
    T = kv.shape[1]
    rows_kv, rows_idx = [], []
    for t in tokens:
        b, s = int(t) // S, int(t) % S
        sl = idx[b, s].cpu().to(torch.int64)
        valid = (sl >= 0) & (sl < T)
        uniq, inv = torch.unique(sl[valid], return_inverse=True)
        remap = torch.full_like(sl, -1)
        remap[valid] = inv
        rows_kv.append(kv[b, uniq.to(kv.device)].cpu() if uniq.numel() else torch.zeros(0, kv.shape[2], dtype=kv.dtype))
        rows_idx.append(remap.to(torch.int32))
    Tc = max(1, max(r.shape[0] for r in rows_kv))
    kv_c = torch.zeros(len(tokens), Tc, kv.shape[2], dtype=kv.dtype)
    for i, r in enumerate(rows_kv):
        kv_c[i, : r.shape[0]] = r
    idx_c = torch.stack(rows_idx).unsqueeze(1)
    return kv_c, idx_c


def sparse_reference(orc, q, kv, sink, idx, scale, tokens=None):
    """Oracle output [ntok, H, D] for the listed flat tokens (all when None)."""
    B, S, H, D = q.shape
    if tokens is None:
        return orc.sparse_attn(bits(q), bits(kv), sink.cpu().numpy(), idx.cpu().numpy(), scale)
    tokens = np.asarray(tokens, dtype=np.int64)
    kv_c, idx_c = compact_rows(kv, idx, tokens, S)
    qs = q.reshape(B * S, H, D)[torch.as_tensor(tokens, device=q.device)].unsqueeze(1)
    return orc.sparse_attn(bits(qs), bits(kv_c), sink.cpu().numpy(), idx_c.numpy(), scale)
