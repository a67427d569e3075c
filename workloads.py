"""Seeded synthetic inputs for split-KV decode attention.

This module only draws inputs; it holds none of the attention arithmetic, so
both the CPU oracle and the HIP library can be fed from it. The shapes follow
the workloads on the pages this project implements:

  * "04_flash_decoding.py" (CS349E lecture 11), demo 1: one KV sequence of
    10,000 cached keys, head dim 128, 8 packed query heads, split into 7.
  * "flash_decode_splitk.py" (MiniInfer): MHA in [batch, heads, seqlen, dim]
    layout, head dims {16, 32, 64, 128}, default split count
    min(16, max(1, ceil(kv_len / 256))).
  * "04_flash_decoding.py", demo 3: the flash-decoding blog's A100
    microbenchmark shape, 16 query heads / 2 KV heads, head dim 128, fp16,
    with batch x KV length held at 65,536 (plus 1 x 131,072).
  * "04_flash_decoding.py", demo 4: Llama-3.1-8B decode attention, 32 query
    heads / 8 KV heads, head dim 128, KV length {1K, 8K, 32K, 128K} x batch
    {1, 16}, and a split-count sweep {1, 2, ..., 128} at batch 1 / 64K.
  * "decode_attention_splitkv.py" (TileLang tutorial): varlen packed GQA,
    Qwen2.5-7B's 28 query heads / 4 KV heads (group 7), head dim 128,
    [total_kv, kv_heads, dim] with int32 cu_seqlens_k.

Recipe: per-sequence KV lengths, when they vary, are integers uniform in
[64, 32768] drawn by a CPU torch.Generator seeded with ``seed`` (0 by
default); then a torch.Generator with the same seed on the target device
draws q, K, V, in this order, as N(0, 1) in float32; the
values are then cast to the workload dtype, so every consumer sees identical
rounded values. Layout "packed" is [total_kv, kv_heads, dim]; layout "bhsd"
is [batch, kv_heads, max_len, dim]. Optional padding rows past the data are
filled with NaN so that any read outside a sequence shows up in the output.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    kv_heads: int
    dim: int
    dtype: str                 # "f32" | "f16" | "bf16"
    kv_len: int | None = None  # uniform length; None -> varlen draw
    varlen_range: tuple[int, int] | None = None
    layout: str = "packed"     # "packed" | "bhsd"
    num_splits: int | None = None   # None -> use the planner
    scale: float | None = None      # None -> 1/sqrt(dim)
    notes: str = ""

    @property
    def group(self) -> int:
        return self.heads // self.kv_heads

    @property
    def sm_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.dim)

    @property
    def elem_bytes(self) -> int:
        return {"f32": 4, "f16": 2, "bf16": 2}[self.dtype]


def mha_default_splits(kv_len: int) -> int:
    """min(16, max(1, ceil(kv_len / 256))), the default split count of
    flash_decode_splitk.py."""
    return min(16, max(1, -(-kv_len // 256)))


def tiny() -> Workload:
    return Workload("tiny_gqa8_d128_l10000_f32", 1, 8, 1, 128, "f32", kv_len=10000,
                    num_splits=7, notes="exactness case, 04_flash_decoding.py demo 1")


def mha(dim: int) -> Workload:
    return Workload(f"mha_b4_h32_l4096_d{dim}_f16", 4, 32, 32, dim, "f16", kv_len=4096,
                    layout="bhsd", num_splits=mha_default_splits(4096),
                    notes="MHA head-dim sweep, flash_decode_splitk.py")


FD_UBENCH_SHAPES = [(256, 256), (128, 512), (64, 1024), (32, 2048), (16, 4096), (8, 8192),
                    (4, 16384), (2, 32768), (1, 65536), (1, 131072)]


def fd_ubench(batch: int, kv_len: int) -> Workload:
    return Workload(f"fd_ubench_b{batch}_l{kv_len}_h16kv2_d128_f16", batch, 16, 2, 128, "f16",
                    kv_len=kv_len, notes="flash-decoding blog shape, 04_flash_decoding.py demo 3")


# 04_flash_decoding.py demo 4: the split-count sweep at 16/2 heads
DEMO4_SHAPES = [(1, 65536), (8, 8192), (64, 2048)]
DEMO4_SPLITS = [1, 2, 4, 8, 16, 32, 64, 128]

LLAMA_LENS = [1024, 8192, 32768, 131072]
LLAMA_BATCHES = [1, 16]
LLAMA_SWEEP_SPLITS = [1, 2, 4, 8, 16, 32, 64, 128]


def llama(batch: int, kv_len: int, num_splits: int | None = None) -> Workload:
    tag = f"_ns{num_splits}" if num_splits is not None else ""
    return Workload(f"llama8b_b{batch}_l{kv_len}_h32kv8_d128_bf16{tag}", batch, 32, 8, 128,
                    "bf16", kv_len=kv_len, num_splits=num_splits,
                    notes="Llama-3.1-8B shape, 04_flash_decoding.py demo 4")


def varlen_qwen() -> Workload:
    return Workload("varlen_qwen7b_b32_h28kv4_d128_f16", 32, 28, 4, 128, "f16",
                    varlen_range=(64, 32768), num_splits=8,
                    notes="varlen packed GQA, decode_attention_splitkv.py")


def all_workloads() -> list[Workload]:
    out = [tiny()] + [mha(d) for d in (16, 32, 64, 128)]
    out += [fd_ubench(b, s) for b, s in FD_UBENCH_SHAPES]
    out += [fd_ubench(b, s) for b, s in DEMO4_SHAPES if (b, s) not in FD_UBENCH_SHAPES]
    out += [llama(b, s) for s in LLAMA_LENS for b in LLAMA_BATCHES]
    out += [llama(1, 65536, ns) for ns in LLAMA_SWEEP_SPLITS]
    out.append(varlen_qwen())
    return out


def draw_lengths(w: Workload, gen: torch.Generator) -> list[int]:
    if w.kv_len is not None:
        return [int(w.kv_len)] * w.batch
    lo, hi = w.varlen_range
    return [int(x) for x in torch.randint(lo, hi + 1, (w.batch,), generator=gen,
                                          device=gen.device).tolist()]


def varlen_splits(w: Workload, lengths: list[int]) -> int:
    """num_splits=8, falling back to 1 when the shortest sequence has fewer
    keys than splits (the rule stated for the varlen workload)."""
    ns = w.num_splits
    return ns if min(lengths) >= ns else 1


@dataclass
class Inputs:
    workload: Workload
    q: torch.Tensor            # [B, H, D]
    k: torch.Tensor            # packed [T(+pad), Hkv, D] or bhsd [B, Hkv, S(+pad), D]
    v: torch.Tensor
    cu_seqlens_k: torch.Tensor  # int32 [B+1] on the same device
    lengths: list[int] = field(default_factory=list)

    @property
    def kv_bytes(self) -> int:
        """Bytes of K and V that one pass must read: sum_b L_b * Hkv * D * 2 * e."""
        w = self.workload
        return sum(self.lengths) * w.kv_heads * w.dim * 2 * w.elem_bytes


def _randn(shape, gen, device, dtype, chunk_elems=1 << 28):
    """N(0,1) drawn in float32 and cast to dtype, in bounded chunks."""
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk_elems):
        e = min(n, s + chunk_elems)
        flat[s:e] = torch.randn(e - s, generator=gen, device=device, dtype=torch.float32).to(dtype)
    return out


def make_inputs(w: Workload, device="cpu", seed: int = 0, pad_rows: int = 0,
                lengths: list[int] | None = None) -> Inputs:
    """Draw the inputs of workload ``w`` on ``device``.

    ``pad_rows`` extra rows filled with NaN follow the data (packed: after
    total_kv; bhsd: after each sequence's max_len). ``lengths`` overrides the
    drawn lengths (for edge-case tests).
    """
    device = torch.device(device)
    if lengths is None:
        # lengths come from a CPU generator so they do not depend on the device
        lgen = torch.Generator(device="cpu")
        lgen.manual_seed(seed)
        lengths = draw_lengths(w, lgen)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    lengths = [int(x) for x in lengths]
    if len(lengths) != w.batch:
        raise ValueError("one length per sequence")
    dt = DTYPES[w.dtype]
    B, H, Hkv, D = w.batch, w.heads, w.kv_heads, w.dim
    q = _randn((B, H, D), gen, device, dt)
    cu = [0]
    for L in lengths:
        cu.append(cu[-1] + L)
    if w.layout == "packed":
        total = cu[-1]
        k = torch.full((total + pad_rows, Hkv, D), float("nan"), dtype=dt, device=device)
        v = torch.full((total + pad_rows, Hkv, D), float("nan"), dtype=dt, device=device)
        k[:total] = _randn((total, Hkv, D), gen, device, dt)
        v[:total] = _randn((total, Hkv, D), gen, device, dt)
    elif w.layout == "bhsd":
        S = max(lengths) if lengths else 0
        k = torch.full((B, Hkv, S + pad_rows, D), float("nan"), dtype=dt, device=device)
        v = torch.full((B, Hkv, S + pad_rows, D), float("nan"), dtype=dt, device=device)
        kd = _randn((B, Hkv, S, D), gen, device, dt)
        vd = _randn((B, Hkv, S, D), gen, device, dt)
        for b, L in enumerate(lengths):
            k[b, :, :L] = kd[b, :, :L]
            v[b, :, :L] = vd[b, :, :L]
        del kd, vd
    else:
        raise ValueError(f"unknown layout {w.layout!r}")
    cu_t = torch.tensor(cu, dtype=torch.int32, device=device)
    return Inputs(w, q, k, v, cu_t, lengths)


def with_(w: Workload, **kw) -> Workload:
    return replace(w, **kw)
