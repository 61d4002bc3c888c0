"""Seeded synthetic workloads for the attention forward.

This module only draws random numbers and fixes shapes. It holds none of the
attention arithmetic, so both the fp64 oracle (through the tests) and the HIP
path (through the binding) can take their inputs from here without sharing any
part of the computation.

The five workloads restate the shapes that the pages measure or discuss:

* ``tiny``   -- dense causal GQA, B=1 H=4 Hkv=1 T=128 d=64, fp32 inputs.
* ``gqa``    -- dense causal GQA prefill, B=2 H=32 Hkv=8 T=4096 d=128, bf16.
* ``mla``    -- MLA-shaped causal prefill (DeepSeek-V2-Lite-like, the q/k
  concatenation of a 128-wide no-rope part and a 64-wide rope part that the
  pith-train page, "Issues resolved" item 2, moves into the model), B=4 H=16
  Hkv=16 T=4096 d_qk=192 d_v=128, bf16.
* ``mqa512`` -- MQA with d=512 and per-head attention sinks, the DeepSeek-V4
  prefill layer shape of the ArcFlash page ("Numbers, labelled": B=1 H=64
  D=512 T=1400), bf16, sinks fp32.
* ``sparse`` -- sparse top-k MLA-style forward: 13312 queries x 64 heads x
  2176 gathered rows with d_qk=512, the FlashMLA shape of the TensorRT-LLM
  page ("Description"), over one shared pool of 65536 rows, bf16.

One more workload measures the split-KV forward (a "next" step beyond the
five): ``decode512`` -- one new token per sequence (Tq=1) of the MQA d=512
layer with sinks (the absorbed-MQA decode the ArcFlash page discusses at
t_q = 1), B=8 sequences, a 32768-token cache, bf16; seed 6, same recipe.
And one measures the sliding-window forward: ``swa1024`` -- the GQA layer of
``gqa`` at 8192 tokens where each query also sees the 1024 keys before its
own (causal, window_left = 1024), seed 7.

Generation recipe (fixed so that every consumer sees identical bits):
``torch.Generator('cpu').manual_seed(seed)`` with seed = workload number (1..5);
draw order q, k, v, sinks, each ``torch.randn(shape, dtype=float32)``; cast to
bf16 (round to nearest even) for the bf16 workloads. Sparse indices come from
``numpy.random.default_rng(seed)``, one ``choice(N, topk, replace=False)`` per
query, in query order, as int32 and unsorted. The backward's output gradient
dL/dO comes from a generator of its own seeded with 1000 + seed (``make_dout``).
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class DenseSpec:
    name: str
    seed: int
    B: int
    H: int
    Hkv: int
    Tq: int
    Tk: int
    d_qk: int
    d_v: int
    dtype: str          # "bf16" or "f32"
    causal: bool
    sinks: bool
    window: tuple = (-1, -1)  # sliding window (left, right) keys around the diagonal; -1: unbounded

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d_qk))

    @property
    def kind(self) -> str:
        return "dense"



@dataclasses.dataclass(frozen=True)
class SparseSpec:
    name: str
    seed: int
    Sq: int
    Hq: int
    N: int
    d_qk: int
    d_v: int
    topk: int
    sinks: bool = False

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d_qk))

    @property
    def kind(self) -> str:
        return "sparse"

    @property
    def dtype(self) -> str:
        return "bf16"



WORKLOADS = {
    1: DenseSpec("tiny", 1, B=1, H=4, Hkv=1, Tq=128, Tk=128, d_qk=64, d_v=64,
                 dtype="f32", causal=True, sinks=False),
    2: DenseSpec("gqa", 2, B=2, H=32, Hkv=8, Tq=4096, Tk=4096, d_qk=128, d_v=128,
                 dtype="bf16", causal=True, sinks=False),
    3: DenseSpec("mla", 3, B=4, H=16, Hkv=16, Tq=4096, Tk=4096, d_qk=192, d_v=128,
                 dtype="bf16", causal=True, sinks=False),
    4: DenseSpec("mqa512", 4, B=1, H=64, Hkv=1, Tq=1400, Tk=1400, d_qk=512, d_v=512,
                 dtype="bf16", causal=True, sinks=True),
    5: SparseSpec("sparse", 5, Sq=13312, Hq=64, N=65536, d_qk=512, d_v=512, topk=2176),
}

# measured beyond the five (split-KV decode)
NEXT_WORKLOADS = {
    6: DenseSpec("decode512", 6, B=8, H=64, Hkv=1, Tq=1, Tk=32768, d_qk=512, d_v=512,
                 dtype="bf16", causal=True, sinks=True),
    7: DenseSpec("swa1024", 7, B=2, H=32, Hkv=8, Tq=8192, Tk=8192, d_qk=128, d_v=128,
                 dtype="bf16", causal=True, sinks=False, window=(1024, -1)),
}


def spec(n: int):
    return WORKLOADS[n] if n in WORKLOADS else NEXT_WORKLOADS[n]


def _torch_dtype(name: str):
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def make_dense(s: DenseSpec, *, seed: Optional[int] = None) -> dict:
    """CPU tensors q [B,H,Tq,d_qk], k [B,Hkv,Tk,d_qk], v [B,Hkv,Tk,d_v], sinks [H] or None."""
    g = torch.Generator("cpu").manual_seed(s.seed if seed is None else seed)
    dt = _torch_dtype(s.dtype)
    q = torch.randn((s.B, s.H, s.Tq, s.d_qk), generator=g, dtype=torch.float32).to(dt)
    k = torch.randn((s.B, s.Hkv, s.Tk, s.d_qk), generator=g, dtype=torch.float32).to(dt)
    v = torch.randn((s.B, s.Hkv, s.Tk, s.d_v), generator=g, dtype=torch.float32).to(dt)
    sinks = None
    if s.sinks:
        sinks = torch.randn((s.H,), generator=g, dtype=torch.float32)
    return {"q": q, "k": k, "v": v, "sinks": sinks}


def make_dout(s: DenseSpec, *, seed: Optional[int] = None) -> torch.Tensor:
    """The output gradient dL/dO [B,H,Tq,d_v] for the backward: its own generator,
    seeded with 1000 + the workload's seed, one ``randn`` in fp32 cast to the
    workload's dtype (a random linear functional of the output)."""
    g = torch.Generator("cpu").manual_seed(1000 + (s.seed if seed is None else seed))
    return torch.randn((s.B, s.H, s.Tq, s.d_v), generator=g, dtype=torch.float32).to(_torch_dtype(s.dtype))


def randn_dout(B, H, Tq, d_v, *, dtype="bf16", seed=0) -> torch.Tensor:
    """make_dout for ad-hoc shapes."""
    return make_dout(DenseSpec("adhoc", seed, B, H, 1, Tq, 1, 1, d_v, dtype, True, False))


# ---------------------------------------------------------------------------
# Quantized K/V caches in llama.cpp's block formats (ggml's block_q8_0 and
# block_q4_0): blocks of 32 consecutive values along the head dimension,
# each stored as an fp16 scale followed by the codes. These functions only
# produce cache bytes from seeded tensors (input generation); what the bytes
# mean is decoded independently by the oracle and by the kernels.
#   q8_0: 34 bytes = fp16 d, 32 x int8 q           (value = d * q)
#   q4_0: 18 bytes = fp16 d, 16 bytes of nibbles   (byte i: element i in the
#         low nibble, element i + 16 in the high nibble; value = d * (n - 8))
# ---------------------------------------------------------------------------
QK = 32
BLOCK_BYTES = {"q8_0": 34, "q4_0": 18}


def quantize_rows(x: torch.Tensor, fmt: str) -> torch.Tensor:
    """x [..., d] float -> uint8 [..., d/32 * block bytes] in the given block format
    (round-to-nearest codes; the scale is max|x| / 127 for q8_0 and -max/8 over the
    signed maximum for q4_0, as llama.cpp's reference quantizers choose them)."""
    a = x.detach().to(torch.float32).cpu().numpy()
    lead, d = a.shape[:-1], a.shape[-1]
    assert d % QK == 0
    blk = a.reshape(-1, d // QK, QK)
    n = blk.shape[0] * blk.shape[1]
    flat = blk.reshape(n, QK)
    out = np.zeros((n, BLOCK_BYTES[fmt]), dtype=np.uint8)
    if fmt == "q8_0":
        amax = np.abs(flat).max(axis=1)
        dsc = (amax / 127.0).astype(np.float16)
        inv = np.where(dsc.astype(np.float32) > 0, 1.0 / dsc.astype(np.float32), 0.0)
        q = np.clip(np.rint(flat * inv[:, None]), -127, 127).astype(np.int8)
        out[:, 0:2] = dsc.view(np.uint8).reshape(n, 2)
        out[:, 2:] = q.view(np.uint8)
    elif fmt == "q4_0":
        idx = np.abs(flat).argmax(axis=1)
        mx = flat[np.arange(n), idx]
        dsc = (mx / -8.0).astype(np.float16)
        inv = np.where(dsc.astype(np.float32) != 0, 1.0 / dsc.astype(np.float32), 0.0)
        q = np.clip(np.floor(flat * inv[:, None] + 8.5), 0, 15).astype(np.uint8)
        out[:, 0:2] = dsc.view(np.uint8).reshape(n, 2)
        out[:, 2:] = q[:, :16] | (q[:, 16:] << 4)
    else:
        raise ValueError(fmt)
    return torch.from_numpy(out.reshape(*lead, (d // QK) * BLOCK_BYTES[fmt]))


def make_quant_kv(B, H, Hkv, Tq, Tk, d, fmt, *, seed=0, sinks=False) -> dict:
    """Seeded decode inputs with a quantized cache: q bf16 [B,H,Tq,d] and k, v as
    uint8 [B,Hkv,Tk,row bytes] in ``fmt`` (the same recipe as the dense
    workloads draws q, k, v, sinks in that order; k and v are then quantized)."""
    s = DenseSpec("adhoc", seed, B, H, Hkv, Tq, Tk, d, d, "f32", True, sinks)
    inp = make_dense(s)
    return {"q": inp["q"].to(torch.bfloat16), "k": quantize_rows(inp["k"], fmt),
            "v": quantize_rows(inp["v"], fmt), "sinks": inp["sinks"], "fmt": fmt}


# Multi-sequence decode over a q8_0 cache: 4 sequences decoding 4 tokens each
# (the llama.cpp page's case: 3 to 16 tokens per ubatch over 4 streams, head
# size 128), GQA 32/8 heads, a 16384-token cache; seed 8.
QUANT_DECODE = {"name": "qdecode", "B": 4, "H": 32, "Hkv": 8, "Tq": 4, "Tk": 16384, "d": 128, "fmt": "q8_0",
                "seed": 8}


# A packed prefill batch: the gqa layer (H32/Hkv8, d128, causal) over 8
# sequences whose lengths are drawn uniformly from [64, 4096]
# (numpy default_rng(seed)), queries = keys per sequence; seed 9.
VARLEN_PREFILL = {"name": "varlen", "n_seqs": 8, "min_len": 64, "max_len": 4096, "H": 32, "Hkv": 8, "d": 128,
                  "seed": 9}


def varlen_lengths(n_seqs: int, min_len: int, max_len: int, seed: int) -> np.ndarray:
    return np.random.default_rng(seed).integers(min_len, max_len + 1, size=n_seqs).astype(np.int64)


def make_varlen(s: dict = VARLEN_PREFILL) -> dict:
    """Packed CPU tensors q [total, H, d], k, v [total, Hkv, d] (bf16, drawn in that
    order from torch.Generator(seed), N(0,1)), the lengths and cu_seqlens int32 [n + 1]."""
    lens = varlen_lengths(s["n_seqs"], s["min_len"], s["max_len"], s["seed"])
    total = int(lens.sum())
    g = torch.Generator("cpu").manual_seed(s["seed"])
    q = torch.randn((total, s["H"], s["d"]), generator=g, dtype=torch.float32).to(torch.bfloat16)
    k = torch.randn((total, s["Hkv"], s["d"]), generator=g, dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn((total, s["Hkv"], s["d"]), generator=g, dtype=torch.float32).to(torch.bfloat16)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return {"q": q, "k": k, "v": v, "lens": lens, "cu": cu}


# fp8 pool rows for the sparse decode: OCP e4m3 (1 sign, 4 exponent bits with
# bias 7, 3 mantissa bits; largest finite 448) with one fp32 scale per
# 128-column block of a row, scale = max|x| / 448 of the block, codes rounded
# to nearest by torch's float8_e4m3fn conversion. Only the bytes and scales are
# produced here; the oracle and the kernels decode them independently.
FP8_BLOCK = 128
FP8_MAX = 448.0


def quantize_fp8_rows(x: torch.Tensor):
    """x [N, d] float -> (codes uint8 [N, d], scales fp32 [N, d / 128])."""
    a = x.detach().to(torch.float32).cpu()
    N, d = a.shape
    assert d % FP8_BLOCK == 0
    blk = a.reshape(N, d // FP8_BLOCK, FP8_BLOCK)
    sc = blk.abs().amax(dim=-1) / FP8_MAX
    sc = torch.where(sc > 0, sc, torch.ones_like(sc))
    codes = (blk / sc[..., None]).to(torch.float8_e4m3fn).view(torch.uint8).reshape(N, d)
    return codes.contiguous(), sc.contiguous()


# The sparse decode over an fp8 pool: 128 decoding queries (one token each of
# 128 sequences) x 64 heads, top-k 2048 of a 65536-row pool, d 512; seed 10.
SPARSE_FP8_DECODE = {"name": "fp8decode", "Sq": 128, "Hq": 64, "N": 65536, "d": 512, "topk": 2048, "seed": 10}


def make_sparse_fp8(Sq: int, Hq: int, N: int, d: int, topk: int, *, seed: int = 0, sinks: bool = False) -> dict:
    """q [Sq,Hq,d] bf16, the pool quantized from N(0,1) rows (codes, scales), indices as
    the sparse recipe draws them, sinks [Hq] or None; drawn in the order q, pool, sinks."""
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn((Sq, Hq, d), generator=g, dtype=torch.float32).to(torch.bfloat16)
    pool = torch.randn((N, d), generator=g, dtype=torch.float32)
    sk = torch.randn((Hq,), generator=g, dtype=torch.float32) if sinks else None
    codes, scales = quantize_fp8_rows(pool)
    idx = torch.from_numpy(make_indices(Sq, N, topk, seed))
    return {"q": q, "codes": codes, "scales": scales, "idx": idx, "sinks": sk}


def make_indices(Sq: int, N: int, topk: int, seed: int) -> np.ndarray:
    """[Sq, topk] int32, each row topk distinct values of [0, N), unsorted."""
    rng = np.random.default_rng(seed)
    out = np.empty((Sq, topk), dtype=np.int32)
    for s in range(Sq):
        out[s] = rng.choice(N, topk, replace=False)
    return out


def make_sparse(s: SparseSpec, *, seed: Optional[int] = None) -> dict:
    """CPU tensors q [Sq,Hq,d_qk], kv [N,d_qk] (V = kv[:, :d_v]), idx [Sq,topk] int32."""
    sd = s.seed if seed is None else seed
    g = torch.Generator("cpu").manual_seed(sd)
    q = torch.randn((s.Sq, s.Hq, s.d_qk), generator=g, dtype=torch.float32).to(torch.bfloat16)
    kv = torch.randn((s.N, s.d_qk), generator=g, dtype=torch.float32).to(torch.bfloat16)
    sinks = None
    if s.sinks:
        sinks = torch.randn((s.Hq,), generator=g, dtype=torch.float32)
    idx = torch.from_numpy(make_indices(s.Sq, s.N, s.topk, sd))
    return {"q": q, "kv": kv, "idx": idx, "sinks": sinks}


def make_sparse_dout(s: SparseSpec, *, seed: Optional[int] = None) -> torch.Tensor:
    """dL/dO [Sq,Hq,d_v] for the sparse backward: its own generator seeded with
    1000 + the workload's seed, one ``randn`` in fp32 cast to bf16."""
    g = torch.Generator("cpu").manual_seed(1000 + (s.seed if seed is None else seed))
    return torch.randn((s.Sq, s.Hq, s.d_v), generator=g, dtype=torch.float32).to(torch.bfloat16)


def make_keep(B: int, H: int, Tq: int, Tk: int, p_drop: float, *, seed: int = 0) -> torch.Tensor:
    """A dropout keep mask [B,H,Tq,Tk] bool: each entry kept with probability
    1 - p_drop, drawn by numpy default_rng(3000 + seed)."""
    rng = np.random.default_rng(3000 + seed)
    return torch.from_numpy(rng.random((B, H, Tq, Tk)) >= p_drop)


def pack_keep(keep: torch.Tensor) -> torch.Tensor:
    """Bit-pack a keep mask [..., Tk] into int32 words [..., ceil(Tk/32)]: bit i of
    word w is entry 32 w + i (the layout the library reads)."""
    Tk = keep.shape[-1]
    nw = (Tk + 31) // 32
    k = np.zeros(keep.shape[:-1] + (nw * 32,), dtype=np.uint64)
    k[..., :Tk] = keep.numpy().astype(np.uint64)
    k = k.reshape(keep.shape[:-1] + (nw, 32))
    words = (k << np.arange(32, dtype=np.uint64)).sum(axis=-1).astype(np.uint32)
    return torch.from_numpy(words.view(np.int32))


def make(n: int) -> dict:
    s = spec(n)
    return make_dense(s) if s.kind == "dense" else make_sparse(s)


def sha256(t: torch.Tensor) -> str:
    """Digest of a tensor's bytes, for reproducibility records."""
    a = t.contiguous()
    if a.dtype == torch.bfloat16:
        a = a.view(torch.int16)
    return hashlib.sha256(a.numpy().tobytes()).hexdigest()


def randn_dense(B, H, Hkv, Tq, Tk, d_qk, d_v, *, dtype="bf16", sinks=False, seed=0):
    """Ad-hoc dense inputs for sweeps and edge cases (same recipe, any shape)."""
    s = DenseSpec("adhoc", seed, B, H, Hkv, Tq, Tk, d_qk, d_v, dtype, True, sinks)
    return make_dense(s)


def randn_sparse(Sq, Hq, N, d_qk, topk, *, seed=0, sinks=False):
    s = SparseSpec("adhoc", seed, Sq, Hq, N, d_qk, d_qk, topk, sinks)
    return make_sparse(s)


# ---------------------------------------------------------------------------
# Wide-dynamic-range inputs. With N(0,1) rows at scale 1/sqrt(d) a row's
# largest score is reached in its first key blocks, so an online softmax
# never has to move its running maximum later in the row. These variants
# reshape the same seeded draws so that it must:
#
#   "qx16"   -- q multiplied by 16 (exact in bf16): scores ~ N(0, 256);
#   "rising" -- q multiplied by 4 and key j by 1 + 7 j / n, so each row's
#               maximum climbs along the keys. Sparse pools (whose rows are
#               the values too) rise additively instead: pool row r gains
#               0.5 r / N in each coordinate and q gains 7, which lifts the
#               score of row r by about 80 r / N while |v| stays below 3;
#   "jump"   -- every query row gains +1 in each coordinate and one late key
#               (pool row) becomes (80 / sqrt(d)) in each coordinate, so a row
#               that sees it scores it about 80 (natural units) above the rest.
#
# The value rows are halved in every mode. Such scores make the softmax
# peaky, so an output row nearly copies one value row; N(0,1) value rows
# reach |v| > 4, where one bf16 rounding of the output alone errs by up to
# 2^-6 (half a unit in the last place of [4, 8)) and the bf16 rounding of
# the probabilities adds up to 2^-9 |v|: together above the 2e-2 bar, for
# any correct kernel. With |v| < 4 the same two roundings stay below it. For
# the one-pool sparse inputs (values = the pool rows) the pool is halved
# and q doubled, so the scores are those of the unhalved pool.
#
# They only scale or overwrite input values; the attention itself is
# computed by the oracle and by the kernels.
# ---------------------------------------------------------------------------
WIDE_MODES = ("qx16", "rising", "jump")


def jump_key(n: int) -> int:
    """Position of the overwritten key in the "jump" mode: late, but not in the last block."""
    return max(0, n - 1 - n // 7)


def _key_ramp(n: int) -> torch.Tensor:
    return 1.0 + 7.0 * torch.arange(n, dtype=torch.float32) / max(n, 1)


def widen_dense(B, H, Hkv, Tq, Tk, d_qk, d_v, mode, *, dtype="bf16", sinks=False, seed=0) -> dict:
    """Dense inputs of the usual recipe (fp32 draws), reshaped by ``mode`` before the cast."""
    s = DenseSpec("adhoc", seed, B, H, Hkv, Tq, Tk, d_qk, d_v, "f32", True, sinks)
    inp = make_dense(s)
    q, k = inp["q"], inp["k"]
    if mode == "qx16":
        q = q * 16.0
    elif mode == "rising":
        q = q * 4.0
        k = k * _key_ramp(Tk)[None, None, :, None]
    elif mode == "jump":
        q = q + 1.0
        if Tk > 0:
            k = k.clone()
            k[:, :, jump_key(Tk), :] = 80.0 / float(np.sqrt(d_qk))
    else:
        raise ValueError(mode)
    dt = _torch_dtype(dtype)
    return {"q": q.to(dt), "k": k.to(dt), "v": (inp["v"] * 0.5).to(dt), "sinks": inp["sinks"]}


def widen_sparse(Sq, Hq, N, d_qk, topk, mode, *, sinks=False, seed=0) -> dict:
    """Sparse inputs: q [Sq,Hq,d], pool [N,d] (bf16), idx [Sq,topk] int32.

    "rising": pool row r gains 0.5 r / N in each coordinate, q gains 7, and
    each index list is sorted ascending, so the gathered blocks come in order
    of growing score.
    "jump": the last pool row is the large row and sits in every list at
    position ``jump_key(topk)`` (the other indices are drawn from [0, N-1)).
    "qx16": q multiplied by 16, indices as drawn."""
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn((Sq, Hq, d_qk), generator=g, dtype=torch.float32)
    kv = torch.randn((N, d_qk), generator=g, dtype=torch.float32)
    sk = torch.randn((Hq,), generator=g, dtype=torch.float32) if sinks else None
    if mode == "jump":
        idx = make_indices(Sq, N - 1, topk, seed)
        idx[:, jump_key(topk)] = N - 1
        q = q + 1.0
        kv[N - 1, :] = 80.0 / float(np.sqrt(d_qk))
    else:
        idx = make_indices(Sq, N, topk, seed)
        if mode == "rising":
            q = q + 3.5
            kv = kv + (torch.arange(N, dtype=torch.float32) / N)[:, None]
            idx = np.sort(idx, axis=1)
        elif mode == "qx16":
            q = q * 16.0
        else:
            raise ValueError(mode)
    return {"q": (q * 2.0).to(torch.bfloat16), "kv": (kv * 0.5).to(torch.bfloat16),
            "idx": torch.from_numpy(idx.astype(np.int32)), "sinks": sk}


def widen_quant_kv(B, H, Hkv, Tq, Tk, d, fmt, mode, *, sinks=False, seed=0) -> dict:
    """make_quant_kv with the dense reshaping of ``mode`` applied before quantizing."""
    inp = widen_dense(B, H, Hkv, Tq, Tk, d, d, mode, dtype="f32", sinks=sinks, seed=seed)
    return {"q": inp["q"].to(torch.bfloat16), "k": quantize_rows(inp["k"], fmt), "v": quantize_rows(inp["v"], fmt),
            "sinks": inp["sinks"], "fmt": fmt}


def widen_sparse_fp8(Sq, Hq, N, d, topk, mode, *, sinks=False, seed=0) -> dict:
    """make_sparse_fp8 with the sparse reshaping of ``mode`` applied before quantizing the pool."""
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn((Sq, Hq, d), generator=g, dtype=torch.float32)
    pool = torch.randn((N, d), generator=g, dtype=torch.float32)
    sk = torch.randn((Hq,), generator=g, dtype=torch.float32) if sinks else None
    if mode == "jump":
        idx = make_indices(Sq, N - 1, topk, seed)
        idx[:, jump_key(topk)] = N - 1
        q = q + 1.0
        pool[N - 1, :] = 80.0 / float(np.sqrt(d))
    elif mode == "rising":
        idx = np.sort(make_indices(Sq, N, topk, seed), axis=1)
        q = q + 3.5
        pool = pool + (torch.arange(N, dtype=torch.float32) / N)[:, None]
    elif mode == "qx16":
        idx = make_indices(Sq, N, topk, seed)
        q = q * 16.0
    else:
        raise ValueError(mode)
    codes, scales = quantize_fp8_rows(pool * 0.5)
    return {"q": (q * 2.0).to(torch.bfloat16), "codes": codes, "scales": scales,
            "idx": torch.from_numpy(idx.astype(np.int32)), "sinks": sk}
