"""Seeded synthetic inputs shaped like the workloads the pages describe.

This module only draws random numbers and lays out index lists; it holds none
of the attention arithmetic, so both the GPU path and the CPU oracle can be fed
from it. Index lists are drawn on the CPU with a seeded torch generator; large
dense tensors (q, kv) are drawn on the target device with a seeded generator of
that device, so a given (config, seed, device) always yields the same data.

Shapes follow "DeepSeek V4 源码剖析" ch. 5: q [B,S,128,512] bf16, kv [B,T,512]
bf16 with T = window + compressed rows, attn_sink [128] fp32, topk_idxs
[B,S,1152] int32 with -1 for an empty slot (section 5.1); the masked form follows
the prhub summaries of vLLM PRs #48770 / #52217 (8 heads, qk 192, v 128).
"""
from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class SparseConfig:
    name: str
    B: int
    S: int
    H: int
    D: int
    T: int
    K: int
    kind: str  # "tiny" | "decode" | "prefill" | "ragged"
    window: int = 128


SPARSE_CONFIGS = {
    # 1 Tiny: parity only.
    "tiny": SparseConfig("tiny", B=1, S=4, H=8, D=64, T=256, K=32, kind="tiny"),
    # 2 Decode (the headline workload): 128 window rows + 8192 compressed rows.
    "decode": SparseConfig("decode", B=64, S=1, H=128, D=512, T=128 + 8192, K=1152, kind="decode"),
    # 3 Prefill: 4096 raw tokens + 1024 compressed rows, causal indices.
    "prefill": SparseConfig("prefill", B=1, S=4096, H=128, D=512, T=4096 + 1024, K=1152, kind="prefill"),
    # 5 Ragged long decode: 1M-token context at ratio 4 -> 262144 compressed rows + window.
    "ragged": SparseConfig("ragged", B=32, S=1, H=128, D=512, T=128 + 262144, K=1152, kind="ragged"),
}


@dataclass(frozen=True)
class MaskedConfig:
    name: str
    B: int
    Q: int
    KV: int
    H: int
    Dqk: int
    Dv: int
    topk: int


MASKED_CONFIGS = {
    # 4 Bitmask / masked form.
    "masked": MaskedConfig("masked", B=2, Q=2048, KV=8192, H=8, Dqk=192, Dv=128, topk=2048),
    "masked_small": MaskedConfig("masked_small", B=2, Q=80, KV=300, H=2, Dqk=192, Dv=128, topk=64),
}


@dataclass(frozen=True)
class CandidateConfig:
    name: str
    rows: int          # decode rows (batch x next_n)
    width: int         # logits workspace width (the engine's longest context)
    block_size: int
    end_lo: int        # live ends ~ U[end_lo, end_hi]
    end_hi: int


CANDIDATE_CONFIGS = {
    # The indexer's decode logits at a 1M-token workspace with ~128 live columns per row and 96
    # rows (the case the ROCm candidate-mask change was measured on), and a long-context mix.
    "candidate": CandidateConfig("candidate", rows=96, width=1 << 20, block_size=16, end_lo=64, end_hi=192),
    "candidate_long": CandidateConfig("candidate_long", rows=96, width=1 << 20, block_size=16, end_lo=0,
                                      end_hi=1 << 20),
}


def _cpu_gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _dev_gen(seed: int, device) -> torch.Generator:
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def randn_bf16(shape, seed: int, device="cpu") -> torch.Tensor:
    """N(0,1) drawn in fp32 on `device` with a seeded generator, rounded to bf16."""
    g = _dev_gen(seed, device)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def _distinct(n_pick: int, pool: int, g: torch.Generator) -> torch.Tensor:
    return torch.randperm(pool, generator=g)[:n_pick]


def sparse_indices(cfg: SparseConfig, seed: int) -> torch.Tensor:
    """topk_idxs [B,S,K] int32 on the CPU, following the config's recipe.

    tiny:    K distinct uniform rows of [0,T); 3 random slots per token set to -1.
    decode:  slots 0..127 = window rows 0..127, then 1024 distinct rows of
             [128, T); each slot independently -1 with probability 0.05.
    prefill: token s sees the window max(0,s-127)..s, then min(1024, pool)
             distinct rows drawn from the pool {raw rows < s-127} and
             {compressed rows 4096+c : c < (s+1)//4}; remaining slots -1.
    ragged:  live_len ~ U[128, T], n ~ U[1, K], n <- min(n, live_len);
             slots 0..n-1 hold n distinct rows of [0, live_len), the rest -1.
    """
    g = _cpu_gen(seed)
    B, S, K, T = cfg.B, cfg.S, cfg.K, cfg.T
    idx = torch.full((B, S, K), -1, dtype=torch.int32)
    if cfg.kind == "tiny":
        for b in range(B):
            for s in range(S):
                idx[b, s] = _distinct(K, T, g).to(torch.int32)
                holes = _distinct(3, K, g)
                idx[b, s, holes] = -1
    elif cfg.kind == "decode":
        w = cfg.window
        for b in range(B):
            for s in range(S):
                idx[b, s, :w] = torch.arange(w, dtype=torch.int32)
                idx[b, s, w:] = (w + _distinct(K - w, T - w, g)).to(torch.int32)
        holes = torch.rand((B, S, K), generator=g) < 0.05
        idx[holes] = -1
    elif cfg.kind == "prefill":
        w = cfg.window
        raw = T - 1024  # 4096 raw token rows, then the compressed rows
        for b in range(B):
            for s in range(S):
                lo = max(0, s - (w - 1))
                win = torch.arange(lo, s + 1, dtype=torch.int32)
                n_raw = lo  # raw rows strictly before the window
                n_cmp = (s + 1) // 4
                pool = n_raw + n_cmp
                n_pick = min(K - w, pool)
                picks = _distinct(n_pick, pool, g) if pool > 0 else torch.zeros(0, dtype=torch.int64)
                picks = torch.where(picks < n_raw, picks, raw + (picks - n_raw))
                row = torch.cat([win, picks.to(torch.int32)])
                idx[b, s, : row.numel()] = row
    elif cfg.kind == "ragged":
        for b in range(B):
            for s in range(S):
                live = int(torch.randint(128, T + 1, (1,), generator=g))
                n = int(torch.randint(1, K + 1, (1,), generator=g))
                n = min(n, live)
                idx[b, s, :n] = _distinct(n, live, g).to(torch.int32)
    else:
        raise ValueError(cfg.kind)
    return idx


def sparse_inputs(cfg: SparseConfig | str, seed: int, device="cpu") -> dict:
    """q, kv, attn_sink, topk_idxs, scale for one config; dense tensors on `device`."""
    if isinstance(cfg, str):
        cfg = SPARSE_CONFIGS[cfg]
    q = randn_bf16((cfg.B, cfg.S, cfg.H, cfg.D), seed * 4 + 1, device)
    kv = randn_bf16((cfg.B, cfg.T, cfg.D), seed * 4 + 2, device)
    sink = torch.randn((cfg.H,), generator=_cpu_gen(seed * 4 + 3), dtype=torch.float32).to(device)
    idx = sparse_indices(cfg, seed * 4 + 4).to(device)
    return {"q": q, "kv": kv, "attn_sink": sink, "topk_idxs": idx, "scale": cfg.D ** -0.5, "config": cfg,
            "seed": seed}


def topk_lists(B: int, Q: int, topk: int, key_len: int, seed: int, hole_prob: float = 0.0) -> torch.Tensor:
    """[B,Q,topk] int32 on the CPU: each row holds `topk` distinct keys of [0, key_len);
    with hole_prob > 0 each slot is independently replaced by -1."""
    g = _cpu_gen(seed)
    idx = torch.empty((B, Q, topk), dtype=torch.int32)
    # distinct per row: argsort of uniform keys is a uniform random permutation
    for b in range(B):
        keys = torch.rand((Q, key_len), generator=g)
        idx[b] = torch.argsort(keys, dim=1)[:, :topk].to(torch.int32)
    if hole_prob > 0:
        holes = torch.rand((B, Q, topk), generator=g) < hole_prob
        idx[holes] = -1
    return idx


def masked_inputs(cfg: MaskedConfig | str, seed: int, device="cpu") -> dict:
    """q, k, v for the masked form (bf16 N(0,1)), scale = Dqk^-0.5, and the top-k lists."""
    if isinstance(cfg, str):
        cfg = MASKED_CONFIGS[cfg]
    q = randn_bf16((cfg.B, cfg.Q, cfg.H, cfg.Dqk), seed * 4 + 1, device)
    k = randn_bf16((cfg.B, cfg.KV, cfg.H, cfg.Dqk), seed * 4 + 2, device)
    v = randn_bf16((cfg.B, cfg.KV, cfg.H, cfg.Dv), seed * 4 + 3, device)
    idx = topk_lists(cfg.B, cfg.Q, cfg.topk, cfg.KV, seed * 4 + 4).to(device)
    return {"q": q, "k": k, "v": v, "topk_idxs": idx, "scale": cfg.Dqk ** -0.5, "config": cfg, "seed": seed}


def candidate_inputs(cfg: CandidateConfig | str, seed: int, device="cpu", keep_prob: float = 0.5) -> dict:
    """logits [rows, width] fp32 N(0,1), ends ~ U[end_lo, end_hi] int32, random keep flags
    [rows, nblocks + 1] uint8 (each block kept with keep_prob; the edge flag likewise)."""
    if isinstance(cfg, str):
        cfg = CANDIDATE_CONFIGS[cfg]
    g = _cpu_gen(seed)
    nb = -(-cfg.width // cfg.block_size)
    ends = torch.randint(cfg.end_lo, cfg.end_hi + 1, (cfg.rows,), generator=g, dtype=torch.int64).to(torch.int32)
    flags = (torch.rand((cfg.rows, nb + 1), generator=g) < keep_prob).to(torch.uint8)
    logits = torch.randn((cfg.rows, cfg.width), generator=_dev_gen(seed * 3 + 1, device), device=device)
    return {"logits": logits, "ends": ends.to(device), "flags": flags.to(device), "block_size": cfg.block_size,
            "config": cfg, "seed": seed}


def fp8_kv_rows(B: int, T: int, seed: int, device="cpu") -> torch.Tensor:
    """[B, T, 584] uint8 FP8 rows in the MODEL1 layout: N(0,1) values of dims 0..447 quantised
    per 64-dim tile with a power-of-two scale byte (the smallest 2^e with amax / 2^e <= 448,
    stored as e + 127) through torch's float8_e4m3fn, N(0,1) bf16 dims 448..511, a zero pad byte."""
    g = _dev_gen(seed, device)
    n = B * T
    rows = torch.empty((n, 584), dtype=torch.uint8, device=device)
    step = 1 << 18
    for a in range(0, n, step):
        m = min(step, n - a)
        x = torch.randn((m, 7, 64), generator=g, device=device)
        e = torch.ceil(torch.log2(x.abs().amax(dim=2).clamp_min(1e-30) / 448.0)).clamp(-120, 120)
        qv = (x / torch.pow(2.0, e).unsqueeze(2)).to(torch.float8_e4m3fn)
        rows[a:a + m, :448] = qv.view(torch.uint8).reshape(m, 448)
        rope = torch.randn((m, 64), generator=g, device=device).to(torch.bfloat16)
        rows[a:a + m, 448:576] = rope.view(torch.uint8).reshape(m, 128)
        rows[a:a + m, 576:583] = (e + 127).to(torch.uint8)
        rows[a:a + m, 583] = 0
    return rows.view(B, T, 584)
