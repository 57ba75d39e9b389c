"""Checks that pin the CPU oracle to facts fixed outside it.

Each check takes an ``oracle.Oracle`` and raises AssertionError when the oracle
disagrees with something the pages or the mathematics fix: values the pages
print, closed forms, invariants, special cases that reduce to a library routine
(torch's scaled_dot_product_attention in float64 on the CPU) and brute force on
tiny inputs. The checks are plain functions so that the mutation test can run
them against deliberately broken builds of the oracle as well.

Sources: "DeepSeek V4 源码剖析" ch. 5 (sections 5.1, 5.2, 5.4, 5.5); prhub
summaries of vLLM PR #52217 (mask shape rule, worked example), PR #48770
(bit order, masked-MHA form) and PR #56628 (candidate-mask rule, its test ends).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# --------------------------------------------------------------------------- helpers
def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _f64(t: torch.Tensor) -> torch.Tensor:
    return t.to(torch.float64)


def _bf16(x) -> torch.Tensor:
    return torch.as_tensor(x, dtype=torch.float32).to(torch.bfloat16)


def _tiny(seed=0, B=2, S=3, H=4, D=16, T=40, K=12, holes=3):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, S, H, D, generator=g).to(torch.bfloat16)
    kv = torch.randn(B, T, D, generator=g).to(torch.bfloat16)
    sink = torch.randn(H, generator=g, dtype=torch.float32)
    idx = torch.stack([torch.randperm(T, generator=g)[:K] for _ in range(B * S)]).view(B, S, K).to(torch.int32)
    for b in range(B):
        for s in range(S):
            idx[b, s, torch.randperm(K, generator=g)[:holes]] = -1
    return q, kv, sink, idx


def _run_sparse(o, q, kv, sink, idx, scale):
    return o.sparse_attn(_bits(q), _bits(kv), sink.numpy(), idx.numpy(), scale)


def pages_loop(q, kv, sink, idx, scale):
    """The semantics that "DeepSeek V4 源码剖析" section 5.2 states for sparse_attn, written out
    independently of the oracle as one batched float64 computation: for every token and head
    the logits of the gathered rows are scale * q.k; a slot is empty when its index is negative
    (it gets no weight); with M the largest of the token's valid logits and the head's sink, each
    valid slot weighs exp(x - M) and the sink adds exp(sink - M) to the denominator only."""
    B, S, H, D = q.shape
    qf = _f64(q)                                             # [B,S,H,D]
    valid = idx >= 0                                         # [B,S,K]
    safe = idx.clamp(min=0).long()
    rows = torch.stack([_f64(kv[b])[safe[b]] for b in range(B)])   # [B,S,K,D]
    logits = torch.einsum("bshd,bskd->bshk", qf, rows) * scale      # [B,S,H,K]
    logits = logits.masked_fill(~valid[:, :, None, :], float("-inf"))
    sk = _f64(sink).view(1, 1, H, 1)
    top = torch.maximum(logits.amax(dim=-1, keepdim=True), sk)      # [B,S,H,1]
    w = torch.exp(logits - top)                                     # empty slots: exp(-inf) = 0
    denom = w.sum(dim=-1, keepdim=True) + torch.exp(sk - top)
    return (torch.einsum("bshk,bskd->bshd", w, rows) / denom).numpy()


def sdpa_with_sink(qv, keys, sink_value, scale):
    """softmax over {scale*q.k_j} plus one extra logit `sink_value` whose row is zero,
    via torch's scaled_dot_product_attention (float64): the extra key is the zero vector
    with an additive bias equal to the sink."""
    qv = _f64(qv).view(1, 1, 1, -1)
    n, D = keys.shape
    k = torch.cat([_f64(keys), torch.zeros(1, D, dtype=torch.float64)]).view(1, 1, n + 1, D)
    bias = torch.zeros(1, 1, 1, n + 1, dtype=torch.float64)
    bias[..., n] = sink_value
    return F.scaled_dot_product_attention(qv, k, k, attn_mask=bias, scale=scale).view(-1).numpy()


# --------------------------------------------------------------------------- sparse_attn pins
def check_loop_semantics(o):
    """The oracle equals the stated semantics of section 5.2 (pages_loop) on tiny inputs, with
    and without duplicate slots."""
    q, kv, sink, idx = _tiny(seed=1)
    scale = 16 ** -0.5
    got = _run_sparse(o, q, kv, sink, idx, scale).reshape(q.shape)
    ref = pages_loop(q, kv, sink, idx, scale)
    assert np.abs(got - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max()), np.abs(got - ref).max()
    idx2 = idx.clone()
    idx2[:, :, 1] = idx2[:, :, 0].clamp(min=0)  # a duplicated valid row in every token
    got = _run_sparse(o, q, kv, sink, idx2, scale).reshape(q.shape)
    ref = pages_loop(q, kv, sink, idx2, scale)
    assert np.abs(got - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max()), np.abs(got - ref).max()


def check_all_invalid_zero(o):
    """Every slot -1 with finite sinks gives exactly 0."""
    q, kv, sink, idx = _tiny(seed=2)
    idx[:] = -1
    got = _run_sparse(o, q, kv, sink, idx, 0.25)
    assert np.all(got == 0.0)


def check_order_invariance(o):
    """Permuting the K slots leaves the output unchanged."""
    q, kv, sink, idx = _tiny(seed=3)
    g = torch.Generator().manual_seed(33)
    perm = torch.randperm(idx.shape[-1], generator=g)
    a = _run_sparse(o, q, kv, sink, idx, 0.25)
    b = _run_sparse(o, q, kv, sink, idx[:, :, perm].contiguous(), 0.25)
    assert np.abs(a - b).max() <= 1e-13 * max(1.0, np.abs(a).max())


def check_dense_equivalence(o):
    """Sink -inf and the full index set reduce to dense softmax attention
    (torch scaled_dot_product_attention, float64)."""
    B, S, H, D, T = 1, 3, 4, 16, 24
    g = torch.Generator().manual_seed(4)
    q = torch.randn(B, S, H, D, generator=g).to(torch.bfloat16)
    kv = torch.randn(B, T, D, generator=g).to(torch.bfloat16)
    sink = torch.full((H,), float("-inf"))
    idx = torch.stack([torch.randperm(T, generator=g) for _ in range(S)]).view(B, S, T).to(torch.int32)
    scale = 0.3
    got = _run_sparse(o, q, kv, sink, idx, scale).reshape(B, S, H, D)
    kk = _f64(kv[0]).view(1, 1, T, D)
    ref = F.scaled_dot_product_attention(_f64(q[0]).permute(1, 0, 2).unsqueeze(0), kk, kk, scale=scale)
    ref = ref[0].permute(1, 0, 2).numpy()
    assert np.abs(got[0] - ref).max() <= 1e-12


def check_sink_extra_key(o):
    """The sink is one more softmax logit whose row is zero: sink in the denominator
    only (section 5.5). Checked against SDPA with a zero key biased by the sink."""
    q, kv, sink, idx = _tiny(seed=5)
    scale = 16 ** -0.5
    got = _run_sparse(o, q, kv, sink, idx, scale).reshape(q.shape)
    B, S, H, _ = q.shape
    for b in range(B):
        for s in range(S):
            v = idx[b, s][idx[b, s] >= 0].long()
            for h in range(H):
                ref = sdpa_with_sink(q[b, s, h], kv[b, v], float(sink[h]), scale)
                assert np.abs(got[b, s, h] - ref).max() <= 1e-12, (b, s, h)


def check_exact_mean(o):
    """q = 0, sink -inf, 64 valid slots over rows with entries in {-1, 0, 1}: every weight
    is exactly 1/64, so o is the plain mean of the selected rows (exact in float64)."""
    g = torch.Generator().manual_seed(6)
    T, D, K = 100, 8, 70
    kv = torch.randint(-1, 2, (1, T, D), generator=g).to(torch.bfloat16)
    q = torch.zeros(1, 1, 2, D, dtype=torch.bfloat16)
    idx = torch.full((1, 1, K), -1, dtype=torch.int32)
    sel = torch.randperm(T, generator=g)[:64]
    pos = torch.randperm(K, generator=g)[:64]
    idx[0, 0, pos] = sel.to(torch.int32)
    sink = torch.full((2,), float("-inf"))
    got = _run_sparse(o, q, kv, sink, idx, 1.0)
    mean = kv[0, sel].to(torch.float64).sum(0).numpy() / 64.0
    assert np.array_equal(got[0, 0], mean) and np.array_equal(got[0, 1], mean)


def check_sink_halves(o):
    """q = 0 and sink = ln(n): the sink weighs as much as all n rows together, so o is
    half the mean of the rows."""
    g = torch.Generator().manual_seed(7)
    T, D, n = 50, 8, 20
    kv = torch.randn(1, T, D, generator=g).to(torch.bfloat16)
    q = torch.zeros(1, 1, 1, D, dtype=torch.bfloat16)
    idx = torch.randperm(T, generator=g)[:n].view(1, 1, n).to(torch.int32)
    sink = torch.tensor([math.log(n)], dtype=torch.float32)
    got = _run_sparse(o, q, kv, sink, idx, 1.0)[0, 0]
    # float32 sink: the exact weight of the sink is exp(float32(ln n)) / n
    ws = math.exp(float(sink[0])) / n
    ref = kv[0, idx[0, 0].long()].to(torch.float64).mean(0).numpy() / (1.0 + ws)
    assert np.abs(got - ref).max() <= 1e-14


def check_single_row(o):
    """One valid slot and sink -inf: the output is that row exactly."""
    q, kv, sink, idx = _tiny(seed=8)
    idx[:] = -1
    idx[:, :, 5] = 7
    sink[:] = float("-inf")
    got = _run_sparse(o, q, kv, sink, idx, 0.25).reshape(q.shape)
    row = kv[:, 7].to(torch.float64).numpy()
    for s in range(q.shape[1]):
        for h in range(q.shape[2]):
            assert np.array_equal(got[:, s, h], row)


def check_inf_nan_sink(o):
    """sink +inf: every real weight is 0, o = 0. sink NaN: NaN row (section 5.5 boundary
    cases; NaN from an uninitialised sink, section 5.14)."""
    q, kv, sink, idx = _tiny(seed=9)
    sink[0] = float("inf")
    sink[1] = float("nan")
    got = _run_sparse(o, q, kv, sink, idx, 0.25).reshape(q.shape)
    assert np.all(got[:, :, 0] == 0.0)
    assert np.all(np.isnan(got[:, :, 1]))
    assert np.all(np.isfinite(got[:, :, 2:]))


def check_huge_sink(o):
    """A large sink (100) stays finite and matches SDPA with the sink key."""
    q, kv, sink, idx = _tiny(seed=10)
    sink[:] = 100.0
    scale = 16 ** -0.5
    got = _run_sparse(o, q, kv, sink, idx, scale).reshape(q.shape)
    assert np.all(np.isfinite(got))
    v = idx[0, 0][idx[0, 0] >= 0].long()
    ref = sdpa_with_sink(q[0, 0, 0], kv[0, v], 100.0, scale)
    assert np.abs(got[0, 0, 0] - ref).max() <= 1e-12 * np.abs(ref).max()


def check_duplicates_count(o):
    """q = 0, sink -inf, row a in two slots and row b in one: o = (2a + b) / 3."""
    g = torch.Generator().manual_seed(11)
    kv = torch.randn(1, 10, 8, generator=g).to(torch.bfloat16)
    q = torch.zeros(1, 1, 1, 8, dtype=torch.bfloat16)
    idx = torch.tensor([[[3, -1, 3, 6]]], dtype=torch.int32)
    sink = torch.tensor([float("-inf")])
    got = _run_sparse(o, q, kv, sink, idx, 1.0)[0, 0]
    a, b = kv[0, 3].to(torch.float64), kv[0, 6].to(torch.float64)
    ref = ((2 * a + b) / 3).numpy()
    assert np.abs(got - ref).max() <= 1e-15


def check_scale_closed_form(o):
    """Two valid rows, e0 and 0, q = c*e0: logits scale*c and 0, so
    o[0] = e^{scale c} / (e^{scale c} + 1 + e^{sink}) and o[1:] = 0."""
    D = 8
    kv = torch.zeros(1, 4, D, dtype=torch.bfloat16)
    kv[0, 1, 0] = 1.0
    q = torch.zeros(1, 1, 1, D, dtype=torch.bfloat16)
    q[0, 0, 0, 0] = 3.0
    idx = torch.tensor([[[1, 2]]], dtype=torch.int32)
    sink = torch.tensor([0.5])
    scale = 0.7
    got = _run_sparse(o, q, kv, sink, idx, scale)[0, 0]
    e = math.exp(scale * 3.0)
    assert abs(got[0] - e / (e + 1.0 + math.exp(0.5))) <= 1e-15
    assert np.all(got[1:] == 0.0)


def check_out_of_range_is_empty(o):
    """Indices outside [0, T) other than -1 behave exactly like -1 (empty slot)."""
    q, kv, sink, idx = _tiny(seed=12)
    T = kv.shape[1]
    bad = idx.clone()
    bad[:, :, 0] = T
    bad[:, :, 1] = -7
    ref_idx = bad.clone()
    ref_idx[:, :, :2] = -1
    a = _run_sparse(o, q, kv, sink, bad, 0.25)
    b = _run_sparse(o, q, kv, sink, ref_idx, 0.25)
    assert np.array_equal(a, b)


# --------------------------------------------------------------------------- bitmask pins
def check_mask_worked_example(o):
    """The page's printed example: (2,129,129) -> (2,256,8) with and
    without the reserved word; 129 keys -> 8 words; indices {0,128} -> row [1,0,0,0,1,0,0,0]
    with the padding kept."""
    with open(os.path.join(GOLDEN, "bitmask_worked_example.json")) as f:
        ex = json.load(f)
    for case in ex["shapes"]:
        B, mq, mk, res = case["args"]
        shape = o.topk_mask_shape(B, mq, mk, res)
        if "expect" in case:
            assert shape == tuple(case["expect"]), (case, shape)
        else:
            assert shape[2] == case["expect_words"], (case, shape)
    b = ex["build"]
    idx = np.array(b["topk_idxs"], dtype=np.int32)
    mask = o.topk_mask_build(idx, b["key_len"], q_lens=np.array(b["q_lens"], dtype=np.int32))
    assert mask.shape[2] == 8
    assert mask[0, 0].tolist() == b["row0_expect"]
    assert not mask[0, 1:].any()


def _brute_mask(idx, key_len, padded_q, W, q_lens=None, key_starts=None):
    B, Q, _ = idx.shape
    out = np.zeros((B, padded_q, W), dtype=np.uint64)
    for b in range(B):
        live = Q if q_lens is None else max(0, min(Q, int(q_lens[b])))
        for q in range(live):
            keys = {int(j) for j in idx[b, q] if 0 <= int(j) < key_len}
            for j in keys:
                out[b, q, j // 32] += 2 ** (j % 32)
        if key_starts is not None:
            out[b, 0, W - 1] = int(np.uint32(key_starts[b]))
    return out.astype(np.uint32)


def check_mask_brute_force(o):
    """Bit j of row (b,q) set iff j is among that row's indices (set semantics), with -1,
    duplicates and out-of-range indices mixed in; padding rows and words are zero."""
    g = np.random.default_rng(13)
    B, Q, topk, key_len = 3, 37, 50, 300
    idx = g.integers(-3, key_len + 40, size=(B, Q, topk)).astype(np.int32)
    idx[:, :, 10] = idx[:, :, 11]  # duplicates
    q_lens = np.array([37, 5, 0], dtype=np.int32)
    mask = o.topk_mask_build(idx, key_len, q_lens=q_lens)
    _, pq, W = o.topk_mask_shape(B, Q, key_len)
    assert mask.shape == (B, pq, W) == (3, 128, 12)
    assert np.array_equal(mask, _brute_mask(idx, key_len, pq, W, q_lens))


def check_mask_single_equals_batched(o):
    """A one-request build equals the same request's slice of a batched build."""
    g = np.random.default_rng(14)
    idx = g.integers(-1, 200, size=(2, 20, 16)).astype(np.int32)
    full = o.topk_mask_build(idx, 200)
    one = o.topk_mask_build(idx[1:2], 200)
    assert np.array_equal(full[1:2], one)


def check_mask_reserved_word(o):
    """key_starts go to word W-1 of query row 0; W = 8 for 129 keys and 260 for 8192 keys."""
    g = np.random.default_rng(15)
    for key_len, W in ((129, 8), (8192, 260)):
        idx = g.integers(0, key_len, size=(2, 3, 8)).astype(np.int32)
        ks = np.array([1234, 7], dtype=np.int32)
        mask = o.topk_mask_build(idx, key_len, key_starts=ks)
        assert mask.shape[2] == W
        assert mask[0, 0, W - 1] == 1234 and mask[1, 0, W - 1] == 7
        assert not mask[:, 1:, W - 1].any()
        assert np.array_equal(mask, _brute_mask(idx, key_len, mask.shape[1], W, key_starts=ks))


# --------------------------------------------------------------------------- masked attention pins
def _masked_tiny(seed, B=2, Q=5, KV=40, H=3, Dqk=24, Dv=16):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Q, H, Dqk, generator=g).to(torch.bfloat16)
    k = torch.randn(B, KV, H, Dqk, generator=g).to(torch.bfloat16)
    v = torch.randn(B, KV, H, Dv, generator=g).to(torch.bfloat16)
    return q, k, v


def _pack(bool_mask, W):
    B, Q, KV = bool_mask.shape
    out = np.zeros((B, Q, W), dtype=np.uint64)
    for j in range(KV):
        out[:, :, j // 32] += bool_mask[:, :, j].astype(np.uint64) << np.uint64(j % 32)
    return out.astype(np.uint32)


def check_masked_dense(o):
    """A mask with every key set, and no mask at all, both equal dense attention (SDPA)."""
    q, k, v = _masked_tiny(16)
    B, Q, KV, H = q.shape[0], q.shape[1], k.shape[1], q.shape[2]
    scale = 24 ** -0.5
    ones = _pack(np.ones((B, Q, KV), dtype=bool), 4)
    got = o.masked_attn(_bits(q), _bits(k), _bits(v), ones, scale).reshape(B, Q, H, -1)
    none = o.masked_attn(_bits(q), _bits(k), _bits(v), None, scale).reshape(B, Q, H, -1)
    assert np.array_equal(got, none)
    ref = F.scaled_dot_product_attention(_f64(q).permute(0, 2, 1, 3), _f64(k).permute(0, 2, 1, 3),
                                         _f64(v).permute(0, 2, 1, 3), scale=scale).permute(0, 2, 1, 3).numpy()
    assert np.abs(got - ref).max() <= 1e-12


def check_masked_random(o):
    """A random mask equals SDPA with the same boolean mask; an empty row gives 0; a row
    with one key set gives that key's value exactly (LSB-first bit order)."""
    q, k, v = _masked_tiny(17)
    B, Q, KV, H = q.shape[0], q.shape[1], k.shape[1], q.shape[2]
    g = np.random.default_rng(17)
    bm = g.random((B, Q, KV)) < 0.3
    bm[0, 2, :] = False           # empty row
    bm[1, 3, :] = False
    bm[1, 3, 33] = True           # single key
    bm[0, 0, :] = False
    bm[0, 0, 0] = True
    bm[0, 0, 31] = True
    scale = 24 ** -0.5
    got = o.masked_attn(_bits(q), _bits(k), _bits(v), _pack(bm, 4), scale).reshape(B, Q, H, -1)
    assert np.all(got[0, 2] == 0.0)
    assert np.array_equal(got[1, 3], _f64(v[1, 33]).numpy())
    attn = torch.from_numpy(bm).unsqueeze(1)  # [B,1,Q,KV]
    ref = F.scaled_dot_product_attention(_f64(q).permute(0, 2, 1, 3), _f64(k).permute(0, 2, 1, 3),
                                         _f64(v).permute(0, 2, 1, 3), attn_mask=attn, scale=scale)
    ref = ref.permute(0, 2, 1, 3).numpy()
    live = bm.any(axis=2)
    assert np.abs(got[live] - ref[live]).max() <= 1e-12


def check_two_forms_agree(o):
    """Distinct top-k lists scattered into a mask and fed to masked attention with one head
    and k = v = kv give the same result as sparse attention with sink -inf."""
    g = torch.Generator().manual_seed(18)
    B, Q, KV, D, topk = 2, 6, 70, 16, 9
    q = torch.randn(B, Q, 1, D, generator=g).to(torch.bfloat16)
    kv = torch.randn(B, KV, D, generator=g).to(torch.bfloat16)
    idx = torch.stack([torch.randperm(KV, generator=g)[:topk] for _ in range(B * Q)]).view(B, Q, topk).to(torch.int32)
    idx[0, 1, 3] = -1
    mask = o.topk_mask_build(idx.numpy(), KV)
    kvh = kv.unsqueeze(2).contiguous()
    a = o.masked_attn(_bits(q), _bits(kvh), _bits(kvh), mask, D ** -0.5)
    b = o.sparse_attn(_bits(q), _bits(kv), np.array([-np.inf], dtype=np.float32), idx.numpy(), D ** -0.5)
    assert np.abs(a - b).max() <= 1e-13


def _offset_case(seed, key_len, key_start, KV, B=2, Q=4, H=2, Dqk=24, Dv=16, W=None, density=0.4):
    """Random boolean visibility over a global context of key_len keys, packed by hand
    (not by the oracle's builder) with key_start in the reserved word, and a chunk of KV
    keys' k and v."""
    g = np.random.default_rng(seed)
    W = W if W is not None else 4 * -(-(-(-key_len // 32) + 1) // 4)
    bm = g.random((B, Q, key_len)) < density
    mask = _pack(bm, W)
    mask[:, 0, W - 1] = np.uint32(key_start)
    q, k, v = _masked_tiny(seed, B=B, Q=Q, KV=KV, H=H, Dqk=Dqk, Dv=Dv)
    return q, k, v, bm, mask, W


def _sdpa_masked(q, k, v, bm, scale):
    attn = torch.from_numpy(bm).unsqueeze(1)
    ref = F.scaled_dot_product_attention(_f64(q).permute(0, 2, 1, 3), _f64(k).permute(0, 2, 1, 3),
                                         _f64(v).permute(0, 2, 1, 3), attn_mask=attn, scale=scale)
    return ref.permute(0, 2, 1, 3).numpy()


def check_offset_chunk_is_sdpa(o):
    """Chunked-context form: with key_start = 37 (not a multiple of 32) chunk key j sees global
    key 37 + j; the result equals SDPA over the chunk with the global mask's columns 37..37+KV-1,
    for every query row (row 0 holds the start; the other rows' last word is zero)."""
    key_len, ks, KV = 200, 37, 100
    q, k, v, bm, mask, W = _offset_case(21, key_len, ks, KV)
    scale = 24 ** -0.5
    B, Q, H = q.shape[0], q.shape[1], q.shape[2]
    got = o.masked_attn_offset(_bits(q), _bits(k), _bits(v), mask, scale).reshape(B, Q, H, -1)
    sub = bm[:, :, ks:ks + KV]
    ref = _sdpa_masked(q, k, v, sub, scale)
    live = sub.any(axis=2)
    assert live.all()
    assert np.abs(got[live] - ref[live]).max() <= 1e-12


def check_offset_zero_start_is_plain(o):
    """key_start = 0 reduces the chunked form to the plain masked form (same mask bits)."""
    q, k, v, bm, mask, W = _offset_case(22, 96, 0, 96)
    scale = 24 ** -0.5
    a = o.masked_attn_offset(_bits(q), _bits(k), _bits(v), mask, scale)
    b = o.masked_attn(_bits(q), _bits(k), _bits(v), mask, scale)
    assert np.array_equal(a, b)


def check_offset_stops_at_reserved_word(o):
    """Chunk keys whose global position falls at or past the reserved word are not visible:
    with W = 8 (bit words 0..6 = keys 0..223), key_start 200 and a chunk of 40 keys, only chunk
    keys 0..23 can be seen, although the reserved word's own bits (the start, 200) are set; a
    start past every bit word leaves every row empty (o = 0)."""
    key_len, ks, KV = 224, 200, 40
    q, k, v, bm, mask, W = _offset_case(23, key_len, ks, KV, W=8, density=1.0)
    assert W == 8 and mask[0, 0, 7] == 200
    scale = 24 ** -0.5
    B, Q, H = q.shape[0], q.shape[1], q.shape[2]
    got = o.masked_attn_offset(_bits(q), _bits(k), _bits(v), mask, scale).reshape(B, Q, H, -1)
    sub = np.zeros((B, Q, KV), dtype=bool)
    sub[:, :, :224 - ks] = True
    ref = _sdpa_masked(q, k, v, sub, scale)
    assert np.abs(got - ref).max() <= 1e-12
    mask[:, 0, 7] = np.uint32(5000)
    empty = o.masked_attn_offset(_bits(q), _bits(k), _bits(v), mask, scale)
    assert np.all(empty == 0.0)


# --------------------------------------------------------------------------- candidate mask pins
def _kept(row):
    return np.flatnonzero(row != -np.inf)


def check_candmask_closed_forms(o):
    """All block flags set with start 0 and end = width keeps the row as it is; no flag at all
    masks every column; an end <= 0 masks everything; an end past width acts as width; the edge
    flag alone keeps exactly column width-1, and only when that column is live (end = width)."""
    g = np.random.default_rng(31)
    rows, width, bs = 6, 100, 16
    nb = -(-width // bs)
    x = g.standard_normal((rows, width)).astype(np.float32)
    ends = np.array([width, width, 0, -5, width + 40, width - 1], dtype=np.int32)
    flags = np.zeros((rows, nb + 1), dtype=np.uint8)
    flags[0, :nb] = 1
    flags[2, :] = 1
    flags[3, :] = 1
    flags[4, :nb] = 1
    flags[5, nb] = 1
    flags[1, nb] = 1
    got = o.candidate_mask(x, ends, flags, bs)
    assert np.array_equal(got[0], x[0])
    assert np.array_equal(_kept(got[1]), [width - 1]) and got[1, width - 1] == x[1, width - 1]
    assert not np.isfinite(got[2]).any() and not np.isfinite(got[3]).any()
    assert np.array_equal(got[4], x[4])
    assert len(_kept(got[5])) == 0  # end = width - 1: column width-1 is not live


def check_candmask_single_block(o):
    """One block flag b with start s keeps exactly columns [s + b*bs, min(s + (b+1)*bs, e)):
    blocks are counted from the row's start, not from column 0."""
    g = np.random.default_rng(32)
    width, bs = 200, 8
    nb = -(-width // bs)
    cases = [(0, 200, 3), (13, 200, 0), (13, 40, 3), (50, 150, 11), (7, 190, 22)]
    x = g.standard_normal((len(cases), width)).astype(np.float32)
    starts = np.array([c[0] for c in cases], dtype=np.int32)
    ends = np.array([c[1] for c in cases], dtype=np.int32)
    flags = np.zeros((len(cases), nb + 1), dtype=np.uint8)
    for r, (_, _, b) in enumerate(cases):
        flags[r, b] = 1
    got = o.candidate_mask(x, ends, flags, bs, starts=starts)
    for r, (st, en, b) in enumerate(cases):
        lo, hi = st + b * bs, min(st + (b + 1) * bs, en)
        assert np.array_equal(_kept(got[r]), np.arange(lo, max(lo, hi))), (r, _kept(got[r]))
        assert np.array_equal(got[r, lo:hi], x[r, lo:hi])


def check_candmask_row_repeat_and_page_ends(o):
    """With every flag set, row r keeps exactly [0, e) for the page's test ends (0, 1, the
    1024-column tile edges, width-1, width, width/2); with row_repeat 2, rows 2i and 2i+1 share
    ends[i]."""
    width = 4096
    ends_list = [0, 1, 1023, 1024, 1025, width - 1, width, width // 2]
    rows = len(ends_list)
    x = np.ones((rows, width), dtype=np.float32)
    flags = np.ones((rows, width // 16 + 1), dtype=np.uint8)
    got = o.candidate_mask(x, np.array(ends_list, dtype=np.int32), flags, 16)
    for r, e in enumerate(ends_list):
        assert np.array_equal(_kept(got[r]), np.arange(e)), r
    half = np.array(ends_list[::2], dtype=np.int32)
    got2 = o.candidate_mask(x, half, flags, 16, row_repeat=2)
    for r in range(rows):
        assert np.array_equal(_kept(got2[r]), np.arange(half[r // 2])), r


# --------------------------------------------------------------------------- FP8 row pins
def _fp8_rows(seed, n, scale_lo=118, scale_hi=136):
    """Random FP8 rows (584 bytes: 448 e4m3, 64 bf16, 7 scales + pad) without NaN bytes."""
    g = np.random.default_rng(seed)
    rows = g.integers(0, 256, size=(n, 584), dtype=np.uint8)
    nan = (rows[:, :448] & 0x7F) == 0x7F
    rows[:, :448][nan] ^= 0x01
    rope = torch.randn(n, 64, generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16)
    rows[:, 448:576] = rope.view(torch.int16).numpy().view(np.uint8).reshape(n, 128)
    rows[:, 576:583] = g.integers(scale_lo, scale_hi + 1, size=(n, 7), dtype=np.uint8)
    rows[:, 583] = 0
    return rows


def _fp8_decode_torch(rows):
    """Dequantized rows through torch's float8_e4m3fn and bfloat16 decoders (float64)."""
    t = torch.from_numpy(rows)
    fp8 = t[:, :448].contiguous().view(torch.float8_e4m3fn).to(torch.float64)
    sc = torch.pow(2.0, t[:, 576:583].to(torch.float64) - 127.0).repeat_interleave(64, dim=1)
    rope = t[:, 448:576].contiguous().view(torch.bfloat16).to(torch.float64)
    return torch.cat([fp8 * sc, rope], dim=1).numpy()


def check_fp8_decode_matches_torch(o):
    """Every non-NaN e4m3 byte, at several scale bytes, and the bf16 RoPE dims decode as torch's
    float8_e4m3fn / bfloat16 do, times 2^(scale - 127) per 64-dim tile (MODEL1 row layout)."""
    rows = _fp8_rows(41, 6, scale_lo=100, scale_hi=160)
    allb = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], dtype=np.uint8)
    rows[0, :len(allb)] = allb
    rows[1, :len(allb)] = allb[::-1]
    assert np.array_equal(o.fp8_dequant(rows), _fp8_decode_torch(rows))
    one = np.zeros((1, 584), dtype=np.uint8)
    one[0, [0, 1, 2, 64]] = [0x38, 0x7E, 0x01, 0x40]   # 1, 448, 2^-9 (subnormal), 2
    one[0, 576:583] = [127, 128, 127, 127, 127, 127, 127]
    d = o.fp8_dequant(one)[0]
    assert d[0] == 1.0 and d[1] == 448.0 and d[2] == 2.0 ** -9 and d[64] == 4.0


def check_fp8_attention_equals_bf16_rows(o):
    """Sparse attention over FP8 rows equals it over the same rows written as bf16 (exact: the
    scaled e4m3 values fit bf16), and one valid slot with sink -inf returns that row."""
    g = torch.Generator().manual_seed(42)
    B, S, H, T, K = 2, 2, 3, 30, 10
    rows = _fp8_rows(43, B * T)
    dec = _fp8_decode_torch(rows)
    kv16 = torch.from_numpy(dec).to(torch.bfloat16)
    assert np.array_equal(kv16.to(torch.float64).numpy(), dec)
    q = torch.randn(B, S, H, 512, generator=g).to(torch.bfloat16)
    idx = torch.stack([torch.randperm(T, generator=g)[:K] for _ in range(B * S)]).view(B, S, K).to(torch.int32)
    idx[0, 1, 2] = -1
    sink = torch.randn(H, generator=g)
    scale = 512 ** -0.5
    a = o.sparse_attn_fp8(_bits(q), rows.reshape(B, T, 584), sink.numpy(), idx.numpy(), scale)
    b = o.sparse_attn(_bits(q), _bits(kv16.view(B, T, 512)), sink.numpy(), idx.numpy(), scale)
    assert np.abs(a - b).max() <= 1e-12 * max(1.0, np.abs(b).max())
    one = np.full((B, S, K), -1, dtype=np.int32)
    one[1, 0, 4] = 7
    c = o.sparse_attn_fp8(_bits(q), rows.reshape(B, T, 584), np.full(H, -np.inf, dtype=np.float32), one, scale)
    assert np.array_equal(c[2], np.broadcast_to(dec[T + 7], (H, 512)))


SPARSE_PINS = [check_loop_semantics, check_all_invalid_zero, check_order_invariance, check_dense_equivalence,
               check_sink_extra_key, check_exact_mean, check_sink_halves, check_single_row, check_inf_nan_sink,
               check_huge_sink, check_duplicates_count, check_scale_closed_form, check_out_of_range_is_empty]
MASK_PINS = [check_mask_worked_example, check_mask_brute_force, check_mask_single_equals_batched,
             check_mask_reserved_word]
MASKED_PINS = [check_masked_dense, check_masked_random, check_two_forms_agree, check_offset_chunk_is_sdpa,
               check_offset_zero_start_is_plain, check_offset_stops_at_reserved_word]
CANDIDATE_PINS = [check_candmask_closed_forms, check_candmask_single_block, check_candmask_row_repeat_and_page_ends]
FP8_PINS = [check_fp8_decode_matches_torch, check_fp8_attention_equals_bf16_rows]
ALL_PINS = SPARSE_PINS + MASK_PINS + MASKED_PINS + CANDIDATE_PINS + FP8_PINS
