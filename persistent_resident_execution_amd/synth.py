"""Seeded synthetic inputs shared by the GPU engine's callers and the oracle.

This module holds workload shapes and input generation only -- none of the
decode step's arithmetic.  Both sides consume the same buffers it returns:
weights ~N(0, 0.02) rounded to bf16 (routed and shared experts quantised to
fp8 e4m3 with bf16 128x128 block scales), norm gains 1.0, prompt tokens
uniform over the vocabulary, and (where a test hands a cache over as an input)
K/V values ~N(0, 1) rounded to bf16.

Each tensor draws from its own torch generator, seeded from (seed, tensor
name), so any tensor can be regenerated alone and generation order does not
matter.  Generation runs on whatever device is asked for; a test that needs
host copies for the oracle copies the very same bytes back.
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass, field, replace

import torch

# --------------------------------------------------------------------------
# shapes


@dataclass(frozen=True)
class ModelConfig:
    name: str
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    vocab: int
    max_ctx: int
    batch: int = 1
    rope_theta: float = 10000.0
    rms_eps: float = 1e-5
    n_experts: int = 0
    top_k: int = 0
    n_shared: int = 0
    expert_ffn: int = 0
    kv_fp8: bool = False  # K/V cache as fp8 e4m3 codes with one fp32 scale per row

    @property
    def is_moe(self) -> bool:
        return self.n_experts > 0


@dataclass(frozen=True)
class Workload:
    """A model, the prefilled context of each sequence and the decode steps."""
    name: str
    model: ModelConfig
    contexts: tuple
    steps: int
    note: str = ""


TINY = ModelConfig("tiny", n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                   ffn_dim=768, vocab=1024, max_ctx=256)
DENSE8B = ModelConfig("dense8b", n_layers=32, hidden=4096, n_q_heads=32, n_kv_heads=8,
                      head_dim=128, ffn_dim=14336, vocab=128256, max_ctx=1536)
MOE = ModelConfig("moe", n_layers=12, hidden=6144, n_q_heads=48, n_kv_heads=8, head_dim=128,
                  ffn_dim=0, vocab=151552, max_ctx=4352, n_experts=128, top_k=8, n_shared=1,
                  expert_ffn=2048)

WORKLOADS = {
    "tiny": Workload("tiny", TINY, (128,), 64,
                     "tiny dense decoder, batch 1, 128 prefilled random tokens, 64 greedy steps"),
    "dense8b_ctx1024": Workload("dense8b_ctx1024", DENSE8B, (1024,), 256,
                                "8B-shape dense decoder, batch 1, context 1024, 256 greedy steps"),
    "dense8b_ctx8192": Workload("dense8b_ctx8192", replace(DENSE8B, max_ctx=8192 + 256), (8192,),
                                256, "8B-shape dense decoder, batch 1, context 8192, 256 steps"),
    "dense8b_mb8": Workload("dense8b_mb8", replace(DENSE8B, batch=8, max_ctx=8192 + 128),
                            (512, 1024, 1536, 2048, 3072, 4096, 6144, 8192), 128,
                            "8B-shape dense decoder, micro-batch 8, unequal contexts, 128 steps"),
    "dense8b_ctx8192_kv8": Workload("dense8b_ctx8192_kv8", replace(DENSE8B, max_ctx=8192 + 256, kv_fp8=True),
                                    (8192,), 256, "8B-shape dense decoder, batch 1, context 8192, fp8 e4m3 K/V "
                                                  "cache (one fp32 scale per row), 256 steps"),
    "moe": Workload("moe", MOE, (4096,), 128,
                    "MoE decoder (128 experts top-8 + 1 shared, fp8 experts), context 4096, "
                    "128 greedy steps"),
}

# Test-only shapes: several tiles per operator with ragged tails everywhere
# (hidden not a multiple of 512, ffn and vocab not multiples of the row tile).
SMALL_DENSE = ModelConfig("small_dense", n_layers=3, hidden=384, n_q_heads=6, n_kv_heads=2,
                          head_dim=64, ffn_dim=1000, vocab=2003, max_ctx=320)
SMALL_MOE = ModelConfig("small_moe", n_layers=2, hidden=384, n_q_heads=6, n_kv_heads=2,
                        head_dim=64, ffn_dim=0, vocab=1500, max_ctx=192, n_experts=16, top_k=4,
                        n_shared=1, expert_ffn=256)
# One query head per KV head (plain multi-head attention, G = 1).
SMALL_MHA = ModelConfig("small_mha", n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=4,
                        head_dim=64, ffn_dim=512, vocab=1024, max_ctx=160)
# Eight KV heads (one per XCD, as in the 8B and MoE shapes), so the XCD-local
# hand-offs are in use; ragged hidden and ffn.
SMALL_GQA8 = ModelConfig("small_gqa8", n_layers=2, hidden=640, n_q_heads=16, n_kv_heads=8,
                         head_dim=64, ffn_dim=1200, vocab=1777, max_ctx=288)
# Micro-batch shapes (GEMM inputs in whole 32-column blocks, as the packed
# matrix-core layout needs; rows still ragged against the 16-row groups and
# the workgroup split): 8 sequences, and 3.
SMALL_MB = ModelConfig("small_mb", n_layers=2, hidden=384, n_q_heads=6, n_kv_heads=2,
                       head_dim=64, ffn_dim=1056, vocab=2003, max_ctx=320, batch=8)
SMALL_MB3 = ModelConfig("small_mb3", n_layers=2, hidden=256, n_q_heads=8, n_kv_heads=4,
                        head_dim=64, ffn_dim=544, vocab=1500, max_ctx=200, batch=3)
# Seven query heads per KV head and 128-dim heads: the micro-batch attention
# variant that reads q from LDS (more than four query heads per KV head).
SMALL_MB_G7 = ModelConfig("small_mb_g7", n_layers=2, hidden=512, n_q_heads=14, n_kv_heads=2,
                          head_dim=128, ffn_dim=832, vocab=1201, max_ctx=240, batch=5)


# --------------------------------------------------------------------------
# generators

def _tensor_seed(seed: int, name: str) -> int:
    return (int(seed) * 1_000_003 + zlib.crc32(name.encode())) & 0x7FFF_FFFF_FFFF_FFFF


def _gen(seed: int, name: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_tensor_seed(seed, name))
    return g


def normal_bf16(shape, std, seed, name, device="cpu") -> torch.Tensor:
    """N(0, std) rounded to bf16 (round to nearest even, torch's cast)."""
    g = _gen(seed, name, device)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    t.mul_(std)
    return t.to(torch.bfloat16)


def quantize_fp8_blocks(w: torch.Tensor):
    """Encode fp32 matrices [..., out, in] as fp8 e4m3 codes with one bf16 scale
    per 128x128 block: scale = bf16(amax / 448) (1.0 for an all-zero block),
    code = e4m3(clamp(w / scale, -448, 448)).  Input construction only."""
    *lead, m, k = w.shape
    mb, kb = (m + 127) // 128, (k + 127) // 128
    pad = torch.zeros(*lead, mb * 128, kb * 128, dtype=torch.float32, device=w.device)
    pad[..., :m, :k] = w
    blk = pad.reshape(*lead, mb, 128, kb, 128)
    amax = blk.abs().amax(dim=(-1, -3))                       # [..., mb, kb]
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax)).to(torch.bfloat16)
    s = scale.float()[..., :, None, :, None]
    q = (blk / s).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    q = q.reshape(*lead, mb * 128, kb * 128)[..., :m, :k].contiguous()
    return q, scale.contiguous()


def fp8_expert_stack(n, rows, cols, seed, name, device):
    """n matrices [rows][cols] ~N(0, 0.02), fp8-quantised per 128x128 block
    (drawn and quantised as one [n][rows][cols] tensor: a handful of device
    operations per stack instead of a dozen per expert)."""
    g = _gen(seed, name, device)
    w = torch.randn((n, rows, cols), generator=g, device=device, dtype=torch.float32).mul_(0.02)
    q, s = quantize_fp8_blocks(w)
    del w
    return q, s


def gen_weights(cfg: ModelConfig, seed: int = 0, device="cpu") -> dict:
    """All weights of cfg as torch tensors on device (see module docstring)."""
    h, d, std = cfg.hidden, cfg.head_dim, 0.02
    ones = lambda n: torch.ones(n, dtype=torch.bfloat16, device=device)  # noqa: E731
    W = {
        "embed": normal_bf16((cfg.vocab, h), std, seed, "embed", device),
        "final_norm": ones(h),
        "lm_head": normal_bf16((cfg.vocab, h), std, seed, "lm_head", device),
        "layers": [],
    }
    for l in range(cfg.n_layers):
        p = f"layer{l}."
        L = {
            "attn_norm": ones(h),
            "wq": normal_bf16((cfg.n_q_heads * d, h), std, seed, p + "wq", device),
            "wk": normal_bf16((cfg.n_kv_heads * d, h), std, seed, p + "wk", device),
            "wv": normal_bf16((cfg.n_kv_heads * d, h), std, seed, p + "wv", device),
            "wo": normal_bf16((h, cfg.n_q_heads * d), std, seed, p + "wo", device),
            "ffn_norm": ones(h),
        }
        if cfg.is_moe:
            f, E = cfg.expert_ffn, cfg.n_experts
            L["router"] = normal_bf16((E, h), std, seed, p + "router", device)
            L["e_wg"], L["e_sg"] = fp8_expert_stack(E, f, h, seed, p + "e_wg", device)
            L["e_wu"], L["e_su"] = fp8_expert_stack(E, f, h, seed, p + "e_wu", device)
            L["e_wd"], L["e_sd"] = fp8_expert_stack(E, h, f, seed, p + "e_wd", device)
            S = cfg.n_shared
            L["s_wg"], L["s_sg"] = fp8_expert_stack(S, f, h, seed, p + "s_wg", device)
            L["s_wu"], L["s_su"] = fp8_expert_stack(S, f, h, seed, p + "s_wu", device)
            L["s_wd"], L["s_sd"] = fp8_expert_stack(S, h, f, seed, p + "s_wd", device)
        else:
            f = cfg.ffn_dim
            L["wg"] = normal_bf16((f, h), std, seed, p + "wg", device)
            L["wu"] = normal_bf16((f, h), std, seed, p + "wu", device)
            L["wd"] = normal_bf16((h, f), std, seed, p + "wd", device)
        W["layers"].append(L)
    return W


def gen_tokens(vocab: int, n: int, seed: int = 0, seq: int = 0, device="cpu") -> torch.Tensor:
    """n prompt tokens uniform over [0, vocab), int32, one stream per sequence."""
    g = _gen(seed, f"tokens.{seq}", device)
    return torch.randint(0, vocab, (n,), generator=g, device=device, dtype=torch.int64).to(
        torch.int32)


def empty_kv_cache(cfg: ModelConfig, device="cpu"):
    """A zeroed cache of cfg's format: (k, v, k_scale, v_scale); bf16
    [n_layers][batch][n_kv_heads][max_ctx][head_dim] and no scales, or, for an
    fp8 cache, uint8 codes of that shape and fp32 row scales
    [n_layers][batch][n_kv_heads][max_ctx]."""
    shape = (cfg.n_layers, cfg.batch, cfg.n_kv_heads, cfg.max_ctx, cfg.head_dim)
    if not cfg.kv_fp8:
        return (torch.zeros(shape, dtype=torch.bfloat16, device=device),
                torch.zeros(shape, dtype=torch.bfloat16, device=device), None, None)
    return (torch.zeros(shape, dtype=torch.uint8, device=device), torch.zeros(shape, dtype=torch.uint8, device=device),
            torch.zeros(shape[:4], dtype=torch.float32, device=device),
            torch.zeros(shape[:4], dtype=torch.float32, device=device))


def gen_kv_cache(cfg: ModelConfig, ctx: int, seed: int = 0, device="cpu"):
    """A synthetic cache for tests that take the cache as an input: bf16
    [n_layers][batch][n_kv_heads][max_ctx][head_dim], positions < ctx ~N(0,1),
    the rest zero."""
    shape = (cfg.n_layers, cfg.batch, cfg.n_kv_heads, cfg.max_ctx, cfg.head_dim)
    k = torch.zeros(shape, dtype=torch.bfloat16, device=device)
    v = torch.zeros(shape, dtype=torch.bfloat16, device=device)
    k[..., :ctx, :] = normal_bf16(shape[:3] + (ctx, cfg.head_dim), 1.0, seed, "cache.k", device)
    v[..., :ctx, :] = normal_bf16(shape[:3] + (ctx, cfg.head_dim), 1.0, seed, "cache.v", device)
    return k, v


# --------------------------------------------------------------------------
# host views

def to_bits(t: torch.Tensor):
    """Raw bits of a bf16 / fp8 tensor as a host numpy array (uint16 / uint8)."""
    import numpy as np
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    raise TypeError(t.dtype)


def weights_to_numpy(W: dict) -> dict:
    out = {k: to_bits(W[k]) for k in ("embed", "final_norm", "lm_head")}
    out["layers"] = [{k: to_bits(v) for k, v in L.items()} for L in W["layers"]]
    return out


def weight_bytes(cfg: ModelConfig) -> dict:
    """Bytes of each weight group read once per decode step (all rows)."""
    h, d = cfg.hidden, cfg.head_dim
    qkv = (cfg.n_q_heads + 2 * cfg.n_kv_heads) * d * h * 2
    o = h * cfg.n_q_heads * d * 2
    out = {"qkv": qkv * cfg.n_layers, "o": o * cfg.n_layers, "lm": cfg.vocab * h * 2,
           "embed_row": h * 2 * cfg.batch, "norms": (2 * cfg.n_layers + 1) * h * 2}
    if cfg.is_moe:
        f = cfg.expert_ffn
        blocks = lambda m, k: ((m + 127) // 128) * ((k + 127) // 128) * 2  # noqa: E731
        per_expert = 3 * f * h + 2 * blocks(f, h) + blocks(h, f)
        out["router"] = cfg.n_experts * h * 2 * cfg.n_layers
        out["experts_active"] = (cfg.top_k + cfg.n_shared) * per_expert * cfg.n_layers
    else:
        out["ffn"] = 3 * cfg.ffn_dim * h * 2 * cfg.n_layers
    return out
