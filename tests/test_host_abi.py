"""The C-ABI library without a GPU: it loads, exports what include/sparse_attn.h declares,
computes the mask shape on the host, and rejects bad arguments before touching HIP."""
import ctypes
import os
import re

import pytest

import top_sparse_attention_attn_amd as sa
from top_sparse_attention_attn_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"if", "defined"})


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(api.library_path())
    names = declared_functions()
    assert set(names) >= set(api.EXPORTED), names
    for name in names:
        assert hasattr(lib, name), name


def test_mask_shape_rule_matches_pages_example():
    # prhub summary of vLLM PR #52217, test_topk_mask_rows_are_aligned_for_vectorized_loads
    assert sa.topk_bitmask_shape(2, 129, 129) == (2, 256, 8)
    assert sa.topk_bitmask_shape(2, 129, 129, True) == (2, 256, 8)
    assert sa.topk_bitmask_shape(1, 1, 129)[2] == 8


def test_mask_shape_matches_oracle(oracle_impl):
    for args in [(1, 0, 0, False), (3, 128, 8192, False), (3, 129, 8192, True), (2, 257, 31, True), (1, 1, 1, False),
                 (4, 2048, 8192, False), (2, 100, 262144, True)]:
        assert sa.topk_bitmask_shape(*args) == oracle_impl.topk_mask_shape(*args), args


def _lib():
    return api._load()


FAKE = ctypes.c_void_p(1 << 20)      # never dereferenced: every call below is rejected first
FAKE_ODD = ctypes.c_void_p((1 << 20) + 8)


def _sparse(q=FAKE, kv=FAKE, sink=FAKE, idx=FAKE, out=FAKE, B=1, S=1, H=8, D=64, T=16, K=8, splits=0, ws=None, wsb=0):
    return _lib().sparse_attn_fwd(q, kv, sink, idx, out, B, S, H, D, T, K, 0.125, splits, ws, wsb, None)


def test_sparse_rejects_before_any_hip_call():
    assert _sparse(D=100) == 4                      # unsupported head dim
    assert _sparse(H=129) == 4                      # too many heads
    assert _sparse(B=-1) == 2
    assert _sparse(splits=-1) == 2
    assert _sparse(q=None) == 1
    assert _sparse(idx=None) == 1
    assert _sparse(q=FAKE_ODD) == 3                 # q not 16-byte aligned
    # decode-like shape that needs a workspace, none given
    assert _sparse(B=64, H=128, D=512, T=8320, K=1152) == 5
    # empty work is accepted without a launch
    assert _sparse(B=0) == 0
    assert _sparse(S=0, q=None, out=None) == 0
    # 2^30 tokens in 16 splits: 2^34 (token, split) pairs do not fit the launch
    assert _sparse(B=1 << 30, D=512, T=1 << 20, K=1024, splits=16) == 2


def test_size_limits_before_any_hip_call():
    # T = 2^31 would wrap to a negative int inside the kernel
    assert _sparse(T=1 << 31) == 2
    # topk beyond int32
    assert _mask(topk=1 << 31, Q=1, B=1) == 2
    # masked: too many heads for the kernel's 32-bit tile offsets; too many mask words
    assert _masked(H=4097) == 4
    assert _masked(W=(1 << 21) + 4, KV=64) == 2
    assert _masked(Q=1 << 31, pq=1 << 31) == 2


def test_noalloc_rejects_oversize_before_any_hip_call():
    lib = _lib()
    # 2048 tokens x 8 splits of 128 heads x 512: partials far beyond the 40 MiB scratch array
    rc = lib.sparse_attn_fwd_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, 2048, 1, 128, 512, 4096, 1152, 0.1, 8, None)
    assert rc == 5
    # the ordinary argument checks come first
    assert lib.sparse_attn_fwd_noalloc(None, FAKE, FAKE, FAKE, FAKE, 1, 1, 8, 64, 16, 8, 0.1, 0, None) == 1
    assert lib.sparse_attn_fwd_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 8, 100, 16, 8, 0.1, 0, None) == 4


def test_workspace_policy():
    # bf16 rows, 128 heads at D = 512: two head groups of 64 at <= 32 tokens and at 40, 56 and 64 tokens
    # (where they keep >= 2 splits and as many workgroups), so the split count is per (token, head
    # group); one group at 48 and from 72 tokens on
    for ntok, want in ((4, 9), (8, 8), (16, 6), (24, 5), (32, 4), (40, 3), (48, 5), (56, 2), (64, 2), (72, 3),
                       (80, 3), (96, 2), (128, 2), (192, 1)):
        assert sa.sparse_attn_num_splits(ntok, 1, 128, 512, 1152) == want, ntok
    # no head groups below 64 heads or at D = 64: the split count is the token's own
    assert sa.sparse_attn_num_splits(8, 1, 32, 512, 1152) == 9
    assert sa.sparse_attn_num_splits(8, 1, 128, 64, 1152) == 9
    for ntok, g16, g8 in ((8, 2, 2), (32, 2, 2), (40, 2, 1), (48, 1, 1), (56, 2, 1), (64, 2, 1), (72, 1, 1), (4096, 1, 1)):
        assert sa.sparse_attn_head_groups(ntok, 1, 128, 512, 1152) == g16, ntok
        assert sa.sparse_attn_head_groups(ntok, 1, 128, 512, 1152, fp8=True) == g8, ntok
    assert sa.sparse_attn_head_groups(8, 1, 96, 512, 1152) == 2 and sa.sparse_attn_head_groups(8, 1, 48, 512, 1152) == 1
    assert sa.sparse_attn_head_groups(8, 1, 100, 512, 1152) == 1  # not a multiple of 32
    # FP8 rows keep one group at 64 tokens: 4 splits, and the workspace query covers both row formats
    assert sa.sparse_attn_fp8_num_splits(64, 1, 128, 1152) == 4
    assert sa.sparse_attn_workspace_bytes(64, 1, 128, 512, 1152) == 64 * 4 * 128 * (512 * 2 + 8)
    # never more than one workgroup per CU (256) in all, never more than the tiles or 16
    for ntok in range(1, 300):
        for K in (1, 32, 100, 512, 1152, 2048, 65536):
            n = sa.sparse_attn_num_splits(ntok, 1, 128, 512, K)
            assert 1 <= n <= max(1, min(16, -(-K // 32), 256 // ntok)), (ntok, K, n)
    assert sa.sparse_attn_num_splits(1, 4096, 128, 512, 1152) == 1
    assert sa.sparse_attn_num_splits(1, 4, 8, 64, 32) == 1
    assert sa.sparse_attn_workspace_bytes(1, 4096, 128, 512, 1152) == 0
    def r256(x):
        return (x + 255) // 256 * 256
    for n in (4, 2):  # bf16 partials, fp32 (m, l) per head
        want = 64 * n * 128 * 512 * 2 + 64 * n * 128 * 8
        assert sa.sparse_attn_workspace_bytes(64, 1, 128, 512, 1152, n) == want
    assert sa.sparse_attn_workspace_bytes(64, 1, 128, 512, 1152) == sa.sparse_attn_workspace_bytes(64, 1, 128, 512, 1152, 4)


def _mask(idx=FAKE, ql=None, ks=None, m=FAKE, B=1, Q=4, topk=8, key_len=100, pq=128, W=4):
    return _lib().topk_bitmask_build(idx, ql, ks, m, B, Q, topk, key_len, pq, W, None)


def test_bitmask_rejects_before_any_hip_call():
    assert _mask(W=6) == 2            # words not a multiple of 4
    assert _mask(key_len=200) == 2    # 32 * words < key_len
    assert _mask(pq=2) == 2           # padded_q < Q
    assert _mask(ks=FAKE, key_len=128) == 2  # no room for the reserved word
    assert _mask(m=None) == 1
    assert _mask(m=FAKE_ODD) == 3
    assert _mask(B=0) == 0


def _masked(q=FAKE, k=FAKE, v=FAKE, m=FAKE, o=FAKE, B=1, Q=4, KV=64, H=2, Dqk=192, Dv=128, pq=128, W=4, bits=128):
    return _lib().masked_attn_fwd(q, k, v, m, o, B, Q, KV, H, Dqk, Dv, pq, W, 0.1, bits, None)


def test_masked_rejects_before_any_hip_call():
    assert _masked(Dqk=128) == 4
    assert _masked(bits=64) == 2
    assert _masked(W=1) == 2
    assert _masked(KV=200) == 2       # mask too narrow for the keys
    assert _masked(o=None) == 1
    assert _masked(k=FAKE_ODD) == 3
    assert _masked(Q=0) == 0


def _offset(q=FAKE, k=FAKE, v=FAKE, m=FAKE, o=FAKE, lse=None, B=1, Q=4, KV=64, H=2, Dqk=192, Dv=128, pq=128, W=8):
    return _lib().masked_attn_offset_fwd(q, k, v, m, o, lse, B, Q, KV, H, Dqk, Dv, pq, W, 0.1, None)


def test_masked_offset_rejects_before_any_hip_call():
    assert _offset(m=None) == 1      # the mask carries key_start
    assert _offset(W=0) == 2         # no reserved word
    assert _offset(W=6) == 2         # rows are whole 16-byte chunks
    assert _offset(pq=2) == 2
    assert _offset(Dqk=128) == 4
    assert _offset(o=None) == 1
    assert _offset(v=FAKE_ODD) == 3
    assert _offset(m=FAKE_ODD) == 3
    assert _offset(lse=ctypes.c_void_p((1 << 20) + 2)) == 3  # lse must be 4-byte aligned
    assert _offset(H=0) == 0


def _cand(lg=FAKE, st=None, en=FAKE, fl=FAKE, rows=4, width=1000, sr=1000, sc=1, ss=1, se=1, bs=16, rr=1):
    return _lib().candidate_mask_apply(lg, st, en, fl, rows, width, sr, sc, ss, se, bs, rr, None)


def test_candidate_mask_rejects_before_any_hip_call():
    assert _cand(bs=0) == 2
    assert _cand(rr=0) == 2
    assert _cand(sc=0) == 2
    assert _cand(sr=-1) == 2
    assert _cand(width=1 << 31) == 2
    assert _cand(en=None) == 1
    assert _cand(fl=None) == 1
    assert _cand(lg=ctypes.c_void_p((1 << 20) + 2)) == 3
    assert _cand(rows=0) == 0 and _cand(width=0) == 0


def test_candidate_grid_depends_on_shapes_only():
    assert sa.candidate_mask_grid(96, 1 << 20) == 96 * (4096 // 96)
    assert sa.candidate_mask_grid(1, 8192) == 8          # one workgroup per 1024-column tile at most
    assert sa.candidate_mask_grid(8192, 1 << 20) == 8192  # at least one per row
    assert sa.candidate_mask_grid(0, 100) == 0


def _fp8(q=FAKE, kv=FAKE, sink=FAKE, idx=FAKE, out=FAKE, B=1, S=1, H=8, T=16, K=8, ws=None, wsb=0):
    return _lib().sparse_attn_fp8_fwd(q, kv, sink, idx, out, B, S, H, T, K, 0.1, 0, ws, wsb, None)


def test_sparse_fp8_rejects_before_any_hip_call():
    assert _fp8(T=(1 << 31) // 584 + 1) == 2   # rows past 2^31 bytes
    assert _fp8(kv=ctypes.c_void_p((1 << 20) + 4)) == 3  # rows need 8-byte alignment
    assert _fp8(H=129) == 4
    assert _fp8(idx=None) == 1
    assert _fp8(B=0) == 0


def test_status_strings():
    for s in range(7):
        assert _lib().sa_status_string(s)
    assert _lib().sa_status_string(99) == b"unknown status"


def test_binding_raises_without_gpu_tensors():
    import torch

    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sa.sparse_attn(q, torch.zeros(1, 4, 64, dtype=torch.bfloat16), torch.zeros(8), torch.zeros(1, 1, 2, dtype=torch.int32),
                       0.125)
