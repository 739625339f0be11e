"""Seeded synthetic inputs for paged grouped-query decode attention.

This module only draws inputs: slot lists (CSR ``kv_indptr`` / ``kv_indices``
over a token-granular pool), query rows and K/V pools.  It holds none of the
attention arithmetic, and both the GPU path and the CPU oracle consume what it
produces.

Workload shapes follow the source pages:
  * page size 1, one pool shared by the whole batch: Agent-Infer page
    ("Agent-Infer: 纯 Rust 编写的高性能 LLM 推理引擎"), section "分页 KV 缓存";
  * 32 query heads over 8 KV heads with head_dim 128 (Qwen3-4B/8B, 36 layers)
    and head_dim 256 for the Qwen3.5 full-attention layers: Pegainfer page
    ("Pegainfer: 纯Rust+CUDA构建的LLM推理引擎"), section "关键技术实现" items 1
    and 2 and the table in "支持的模型架构";
  * prefill chunks of 512 tokens, 64 while decodes are running: Agent-Infer
    page, section "连续批处理";
  * shared prompt prefixes across requests (radix prefix cache): Agent-Infer
    page, section "前缀缓存".
The pages publish no benchmark dataset; every input here is drawn from seeded
generators.

Recipe (applies to every workload):
  * lengths: ``numpy.random.Generator(PCG64(seed))`` integers, inclusive range;
  * slot ids: a seeded ``permutation(num_slots)`` handed out in request order
    (distinct across requests), except shared prefixes, which are drawn once
    per group and repeated in every request of that group;
  * Q, K, V: float32 N(0, 1) from ``torch.Generator(device).manual_seed``,
    drawn in chunks of 2**28 values and rounded to bfloat16
    (round-to-nearest-even); Q uses ``seed``; layer l of a multi-layer workload
    has its own pools, K from ``2 * s`` and V from ``2 * s + 1`` with
    ``s = seed * 1000 + 1 + l``; the draws depend on the device type;
  * softmax scale: the float32 value nearest 1/sqrt(head_dim).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np

try:  # torch is needed for the tensors, not for the slot lists
    import torch
except ImportError:  # pragma: no cover
    torch = None


@dataclasses.dataclass(frozen=True)
class DecodeSpec:
    name: str
    batch: int
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    num_slots: int
    len_lo: int
    len_hi: int
    seed: int
    prefix_group_size: int = 0   # requests per shared-prefix group (0 = no sharing)
    prefix_len: int = 0          # shared leading slot ids per group
    num_layers: int = 1


@dataclasses.dataclass(frozen=True)
class PrefillSpec:
    name: str
    batch: int
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    num_slots: int
    cached_len: int
    chunk_len: int
    seed: int


# Workloads, named by what they are.
SINGLE_REQUEST_256 = DecodeSpec(
    "single_request_b1_l256", batch=1, num_qo_heads=32, num_kv_heads=8, head_dim=128,
    num_slots=4096, len_lo=256, len_hi=256, seed=1000)
QWEN3_4B_BATCH8 = DecodeSpec(
    "qwen3_4b_b8_l512_4096", batch=8, num_qo_heads=32, num_kv_heads=8, head_dim=128,
    num_slots=65536, len_lo=512, len_hi=4096, seed=1001)
BATCH64_SHARED_PREFIX = DecodeSpec(
    "b64_l2048_8192_prefix16x4x1024_36layers", batch=64, num_qo_heads=32, num_kv_heads=8,
    head_dim=128, num_slots=600_000, len_lo=2048, len_hi=8192, seed=1002,
    prefix_group_size=4, prefix_len=1024, num_layers=36)
# The batch-64 workload with every list in the 4k-8k range (the same shared
# prefixes and pool): the spec point of batch 64 at 4-8k context.
BATCH64_4K_8K = DecodeSpec(
    "b64_l4096_8192_prefix16x4x1024_36layers", batch=64, num_qo_heads=32, num_kv_heads=8,
    head_dim=128, num_slots=600_000, len_lo=4096, len_hi=8192, seed=1007,
    prefix_group_size=4, prefix_len=1024, num_layers=36)
HEADDIM256_BATCH32 = DecodeSpec(
    "hd256_b32_l1024_16384", batch=32, num_qo_heads=16, num_kv_heads=4, head_dim=256,
    num_slots=400_000, len_lo=1024, len_hi=16384, seed=1003)
# Not one of the benchmark configurations: one system prompt shared by a whole
# batch, the case a cascade plan (shared prefix read once) is made for.
SYSTEM_PROMPT_B64 = DecodeSpec(
    "b64_system_prompt4096_suffix256_2048", batch=64, num_qo_heads=32, num_kv_heads=8,
    head_dim=128, num_slots=250_000, len_lo=4096 + 256, len_hi=4096 + 2048, seed=1006,
    prefix_group_size=64, prefix_len=4096, num_layers=36)
PREFILL_CHUNK512 = PrefillSpec(
    "prefill_8x4096_chunk512", batch=8, num_qo_heads=32, num_kv_heads=8, head_dim=128,
    num_slots=131072, cached_len=4096, chunk_len=512, seed=1004)
PREFILL_CHUNK64 = PrefillSpec(
    "prefill_8x4096_chunk64", batch=8, num_qo_heads=32, num_kv_heads=8, head_dim=128,
    num_slots=131072, cached_len=4096, chunk_len=64, seed=1005)

DECODE_SPECS = [SINGLE_REQUEST_256, QWEN3_4B_BATCH8, BATCH64_SHARED_PREFIX, BATCH64_4K_8K, HEADDIM256_BATCH32]
PREFILL_SPECS = [PREFILL_CHUNK512, PREFILL_CHUNK64]


def softmax_scale(head_dim: int) -> float:
    """The float32 value nearest 1/sqrt(head_dim), returned as a Python float."""
    return float(np.float32(1.0 / math.sqrt(head_dim)))


# ----------------------------------------------------------------------------
# slot lists (host, numpy)
# ----------------------------------------------------------------------------
def draw_lengths(rng: np.random.Generator, batch: int, lo: int, hi: int) -> np.ndarray:
    return rng.integers(lo, hi + 1, size=batch).astype(np.int64)


def slot_lists(lengths, num_slots: int, rng: np.random.Generator,
               prefix_group_size: int = 0, prefix_len: int = 0):
    """CSR slot lists for the given per-request lengths.

    Slot ids come from one seeded permutation of the pool and are distinct
    across requests, except that consecutive groups of ``prefix_group_size``
    requests repeat the same ``prefix_len`` leading ids.
    Returns (kv_indptr int32 [B+1], kv_indices int32 [sum(lengths)]).
    """
    lengths = np.asarray(lengths, dtype=np.int64)
    B = lengths.size
    perm = rng.permutation(num_slots)
    cursor = 0
    pieces: List[np.ndarray] = []
    prefix: Optional[np.ndarray] = None
    for b in range(B):
        L = int(lengths[b])
        if prefix_group_size and prefix_len:
            if b % prefix_group_size == 0:
                prefix = perm[cursor:cursor + prefix_len]
                cursor += prefix_len
            if L < prefix_len:
                raise ValueError("request shorter than its shared prefix")
            own = perm[cursor:cursor + (L - prefix_len)]
            cursor += L - prefix_len
            ids = np.concatenate([prefix, own])
        else:
            ids = perm[cursor:cursor + L]
            cursor += L
        if cursor > num_slots:
            raise ValueError("pool too small for the drawn lengths")
        pieces.append(ids)
    indptr = np.zeros(B + 1, dtype=np.int64)
    indptr[1:] = np.cumsum(lengths)
    if indptr[-1] > np.iinfo(np.int32).max:
        raise ValueError("slot list too long for int32 offsets")
    indices = np.concatenate(pieces) if pieces else np.zeros(0, np.int64)
    return indptr.astype(np.int32), indices.astype(np.int32)


def decode_lists(spec: DecodeSpec):
    """(kv_indptr, kv_indices) of a decode workload, deterministic in spec.seed."""
    rng = np.random.Generator(np.random.PCG64(spec.seed))
    lengths = draw_lengths(rng, spec.batch, spec.len_lo, spec.len_hi)
    return slot_lists(lengths, spec.num_slots, rng, spec.prefix_group_size, spec.prefix_len)


def prefill_lists(spec: PrefillSpec):
    """(qo_indptr, kv_indptr, kv_indices) of a chunked-prefill workload."""
    rng = np.random.Generator(np.random.PCG64(spec.seed))
    L = spec.cached_len + spec.chunk_len
    lengths = np.full(spec.batch, L, dtype=np.int64)
    kv_indptr, kv_indices = slot_lists(lengths, spec.num_slots, rng)
    qo_indptr = (np.arange(spec.batch + 1) * spec.chunk_len).astype(np.int32)
    return qo_indptr, kv_indptr, kv_indices


# ----------------------------------------------------------------------------
# tensors (torch, on any device)
# ----------------------------------------------------------------------------
def _generator(device, seed: int):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal_bf16(shape, seed: int, device="cpu", chunk_elems: int = 1 << 28):
    """bf16 tensor of N(0,1) float32 draws rounded to nearest-even, filled in chunks."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    g = _generator(device, seed)
    n = flat.numel()
    for start in range(0, n, chunk_elems):
        stop = min(n, start + chunk_elems)
        flat[start:stop] = torch.randn(stop - start, generator=g, device=device,
                                       dtype=torch.float32).to(torch.bfloat16)
    return out


def make_pools(num_slots: int, num_kv_heads: int, head_dim: int, seed: int, device="cpu"):
    """(K, V) pools, each bf16 [num_slots, Hkv, D]."""
    k = normal_bf16((num_slots, num_kv_heads, head_dim), seed * 2 + 0, device)
    v = normal_bf16((num_slots, num_kv_heads, head_dim), seed * 2 + 1, device)
    return k, v


# Per-pool scales of the 8-bit workloads: codes hold value / scale.
FP8_K_SCALE = 0.25
FP8_V_SCALE = 0.5


def normal_e4m3(shape, seed: int, scale: float, device="cpu", chunk_elems: int = 1 << 28):
    """OCP FP8 E4M3 codes (torch.float8_e4m3fn) of N(0,1) float32 draws divided
    by `scale`, rounded to nearest-even, filled in chunks."""
    out = torch.empty(shape, dtype=torch.float8_e4m3fn, device=device)
    flat = out.view(-1)
    g = _generator(device, seed)
    n = flat.numel()
    for start in range(0, n, chunk_elems):
        stop = min(n, start + chunk_elems)
        x = torch.randn(stop - start, generator=g, device=device, dtype=torch.float32)
        flat[start:stop] = (x / scale).to(torch.float8_e4m3fn)
    return out


def make_pools_e4m3(num_slots: int, num_kv_heads: int, head_dim: int, seed: int, device="cpu",
                    k_scale: float = FP8_K_SCALE, v_scale: float = FP8_V_SCALE):
    """(K, V) pools of E4M3 codes, each [num_slots, Hkv, D]."""
    k = normal_e4m3((num_slots, num_kv_heads, head_dim), seed * 2 + 0, k_scale, device)
    v = normal_e4m3((num_slots, num_kv_heads, head_dim), seed * 2 + 1, v_scale, device)
    return k, v


def layer_seed(seed: int, layer: int) -> int:
    return seed * 1000 + 1 + layer


@dataclasses.dataclass
class DecodeCase:
    spec: DecodeSpec
    kv_indptr: np.ndarray       # int32 [B+1], host
    kv_indices: np.ndarray      # int32 [nnz], host
    q: "torch.Tensor"           # bf16 [B, Hq, D]
    k_pools: list               # per layer, bf16 [N, Hkv, D]
    v_pools: list
    sm_scale: float


def make_decode_case(spec: DecodeSpec, device="cpu", layers: Optional[int] = None) -> DecodeCase:
    """Slot lists, Q and per-layer pools of a decode workload."""
    kv_indptr, kv_indices = decode_lists(spec)
    n_layers = spec.num_layers if layers is None else layers
    q = normal_bf16((spec.batch, spec.num_qo_heads, spec.head_dim), spec.seed, device)
    ks, vs = [], []
    for layer in range(n_layers):
        k, v = make_pools(spec.num_slots, spec.num_kv_heads, spec.head_dim,
                          layer_seed(spec.seed, layer), device)
        ks.append(k)
        vs.append(v)
    return DecodeCase(spec, kv_indptr, kv_indices, q, ks, vs, softmax_scale(spec.head_dim))


@dataclasses.dataclass
class PrefillCase:
    spec: PrefillSpec
    qo_indptr: np.ndarray
    kv_indptr: np.ndarray
    kv_indices: np.ndarray
    q: "torch.Tensor"           # bf16 [T, Hq, D]
    k_pool: "torch.Tensor"
    v_pool: "torch.Tensor"
    sm_scale: float


def make_prefill_case(spec: PrefillSpec, device="cpu") -> PrefillCase:
    qo_indptr, kv_indptr, kv_indices = prefill_lists(spec)
    T = int(qo_indptr[-1])
    q = normal_bf16((T, spec.num_qo_heads, spec.head_dim), spec.seed, device)
    k, v = make_pools(spec.num_slots, spec.num_kv_heads, spec.head_dim,
                      layer_seed(spec.seed, 0), device)
    return PrefillCase(spec, qo_indptr, kv_indptr, kv_indices, q, k, v,
                       softmax_scale(spec.head_dim))


def bits(t: "torch.Tensor") -> np.ndarray:
    """uint16 bit patterns of a bf16 tensor, on the host."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def codes(t: "torch.Tensor") -> np.ndarray:
    """uint8 codes of an 8-bit (E4M3) tensor, on the host."""
    return t.detach().contiguous().view(torch.uint8).cpu().numpy()


def poison_unreferenced(pool: "torch.Tensor", kv_indices) -> None:
    """Write NaN into every slot of ``pool`` that no list references."""
    idx = torch.as_tensor(np.asarray(kv_indices, dtype=np.int64), device=pool.device)
    keep = torch.zeros(pool.shape[0], dtype=torch.bool, device=pool.device)
    if idx.numel():
        keep[idx] = True
    pool[~keep] = float("nan")


def random_small_decode(seed: int, batch: int, num_qo_heads: int, num_kv_heads: int,
                        head_dim: int, len_lo: int, len_hi: int, num_slots: int,
                        device="cpu"):
    """A small decode case with scattered slots: (indptr, indices, q, k, v, scale)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = draw_lengths(rng, batch, len_lo, len_hi)
    indptr, indices = slot_lists(lengths, num_slots, rng)
    q = normal_bf16((batch, num_qo_heads, head_dim), seed * 7 + 1, device)
    k, v = make_pools(num_slots, num_kv_heads, head_dim, seed * 7 + 2, device)
    return indptr, indices, q, k, v, softmax_scale(head_dim)
