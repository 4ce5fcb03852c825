"""Seeded synthetic workloads for chunked causal attention.

This module only draws inputs. It holds none of the attention arithmetic and
imports neither the oracle nor the HIP library, so both sides can consume the
same values.

The shapes are those of attention layers in the long-context fine-tuning runs
described on the pages: an 8B model at 16K tokens with chunk-wise optimization
(SeCO/SpaCO review, "Referee Report" summary) and Qwen3 4B-32B layers under
StreamBP (StreamBP review, "What carries the argument" and the skeptic's
concrete test: a 4B layer at T=8192 with partition size 500). No text or
weights are used; activations are i.i.d. Gaussian draws.

Draw recipe (one ``numpy.random.default_rng(seed)`` PCG64 stream per workload):
  1. Q, K, V, dO in that order, each ``standard_normal`` in float64, C order,
     shape [B, H, T, d] (H = Hq for Q and dO, Hkv for K and V), times 1/sqrt(d).
  2. Only when the workload asks for a key spike: Z [B, Hkv, T, rank] then
     W [B, Hkv, rank, d], both standard normal; K += amplitude * Z @ W / sqrt(rank).
  3. bf16 workloads round each float64 value to float32 and then to bfloat16,
     both round-to-nearest-even. Both sides receive exactly those values.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seq_len: int
    chunk: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str                 # "f32" or "bf16": storage type of q, k, v, o, dO
    seed: int
    softmax_scale: float = 1.0
    spike_rank: int = 0
    spike_amp: float = 0.0
    sparse_t: int = 0          # >0: backward over t of the k chunks only
    select_seed: int = 0

    @property
    def n_chunks(self) -> int:
        return -(-self.seq_len // self.chunk)

    def chunk_bounds(self, i: int):
        """(start, length) of chunk i, 0-based; the last chunk may be short."""
        s = i * self.chunk
        return s, min(self.chunk, self.seq_len - s)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 512, 128, 4, 4, 64, "f32", seed=0),
    "4b_layer": Workload("4b_layer", 1, 8192, 500, 32, 8, 128, "bf16", seed=1),
    "8b_layer": Workload("8b_layer", 1, 16384, 1024, 32, 8, 128, "bf16", seed=2,
                         spike_rank=4, spike_amp=3.0),
    "32b_layer": Workload("32b_layer", 1, 32768, 2048, 64, 8, 128, "bf16", seed=3),
    "sparse_64k": Workload("sparse_64k", 1, 65536, 1024, 32, 8, 128, "bf16", seed=4,
                           sparse_t=8, select_seed=0),
}


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> float32 (RNE) -> bfloat16 (RNE); returns the raw uint16 bits."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    # round half to even on the 16 dropped bits; inputs here are finite
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@dataclasses.dataclass
class Inputs:
    """Host copies of one workload's tensors.

    ``f64`` holds exactly the values the device receives, widened to float64.
    ``raw`` holds the storage form: float32 arrays, or uint16 bfloat16 bits.
    """
    wl: Workload
    f64: dict
    raw: dict


def _draw(rng, shape, scale):
    return rng.standard_normal(size=shape) * scale


def make_inputs(wl: Workload, seq_len: Optional[int] = None, keep_f64: bool = True) -> Inputs:
    """Draw Q, K, V, dO for ``wl`` (optionally at a different sequence length)."""
    T = wl.seq_len if seq_len is None else seq_len
    B, Hq, Hkv, d = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    rng = np.random.default_rng(wl.seed)
    s = 1.0 / math.sqrt(d)
    arrays = {
        "q": _draw(rng, (B, Hq, T, d), s),
        "k": _draw(rng, (B, Hkv, T, d), s),
        "v": _draw(rng, (B, Hkv, T, d), s),
        "do": _draw(rng, (B, Hq, T, d), s),
    }
    if wl.spike_rank > 0:
        r = wl.spike_rank
        z = rng.standard_normal(size=(B, Hkv, T, r))
        w = rng.standard_normal(size=(B, Hkv, r, d))
        arrays["k"] = arrays["k"] + wl.spike_amp * (z @ w) / math.sqrt(r)
    raw, f64 = {}, {}
    for name, a in arrays.items():
        if wl.dtype == "bf16":
            bits = round_to_bf16_bits(a)
            raw[name] = bits
            if keep_f64:
                f64[name] = bf16_bits_to_f64(bits)
        else:
            f32 = a.astype(np.float32)
            raw[name] = f32
            if keep_f64:
                f64[name] = f32.astype(np.float64)
        arrays[name] = None
    return Inputs(wl, f64, raw)


@dataclasses.dataclass(frozen=True)
class LayerWorkload:
    """An attention layer with its QKV projections: layer input H_in [B, T, d_model],
    weights W_q [d_model, Hq*d], W_k/W_v [d_model, Hkv*d], incoming gradient dO."""
    name: str
    batch: int
    seq_len: int
    chunk: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str
    seed: int

    @property
    def n_chunks(self) -> int:
        return -(-self.seq_len // self.chunk)

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


LAYER_WORKLOADS = {
    # LLaMA3-8B attention layer: d_model 4096, 32 query / 8 kv heads of 128
    "8b_attn_layer": LayerWorkload("8b_attn_layer", 1, 16384, 1024, 4096, 32, 8, 128, "bf16", 7),
}


def make_layer_inputs(wl: LayerWorkload, seq_len: Optional[int] = None, keep_f64: bool = True) -> Inputs:
    """Draw H_in ~ N(0, 1), weights ~ N(0, 1/d_model) (so Q, K, V entries are ~N(0, 1)),
    and dO ~ N(0, 1/d), rounded to the storage type like make_inputs."""
    T = wl.seq_len if seq_len is None else seq_len
    B, Hq, Hkv, d, dm = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.d_model
    rng = np.random.default_rng(wl.seed)
    ws = 1.0 / math.sqrt(dm)
    arrays = {
        "h": _draw(rng, (B, T, dm), 1.0),
        "wq": _draw(rng, (dm, Hq * d), ws),
        "wk": _draw(rng, (dm, Hkv * d), ws),
        "wv": _draw(rng, (dm, Hkv * d), ws),
        "do": _draw(rng, (B, Hq, T, d), 1.0 / math.sqrt(d)),
    }
    raw, f64 = {}, {}
    for name, a in arrays.items():
        if wl.dtype == "bf16":
            bits = round_to_bf16_bits(a)
            raw[name] = bits
            if keep_f64:
                f64[name] = bf16_bits_to_f64(bits)
        else:
            f32 = a.astype(np.float32)
            raw[name] = f32
            if keep_f64:
                f64[name] = f32.astype(np.float64)
        arrays[name] = None
    return Inputs(wl, f64, raw)


def to_torch(raw: np.ndarray, device="cpu"):
    """Storage array -> torch tensor (bfloat16 for uint16 bits, float32 otherwise)."""
    import torch
    if raw.dtype == np.uint16:
        t = torch.from_numpy(raw.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(raw)
    return t.to(device)


@dataclasses.dataclass(frozen=True)
class StackWorkload:
    """A stack of attention layers with residual connections (d_model = Hq * d) for
    SpaCO's relayed backward: input H_0 [B, T, d_model], per-layer W_q/W_k/W_v, and
    the loss gradient dy = dJ/dH_L. t of the k chunks are drawn per step; the
    relayed cache gradient is multiplied by min(k/t, relay_cap)."""
    name: str
    batch: int
    seq_len: int
    chunk: int
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str
    t: int
    relay_cap: Optional[float]
    seed: int

    @property
    def d_model(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def n_chunks(self) -> int:
        return -(-self.seq_len // self.chunk)

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def relay_factor(self) -> float:
        g = self.n_chunks / self.t
        return g if self.relay_cap is None else min(g, self.relay_cap)


STACK_WORKLOADS = {
    # four LLaMA3-8B-shaped attention layers at 16K tokens, t = 4 of k = 16
    # chunks, the relay factor k/t = 4 capped at 2 as the deployed method does
    "8b_stack4_spaco": StackWorkload("8b_stack4_spaco", 1, 16384, 1024, 4, 32, 8, 128, "bf16", 4, 2.0, 11),
}


def make_stack_inputs(wl: StackWorkload, seq_len: Optional[int] = None, keep_f64: bool = True) -> Inputs:
    """Draw H_0 ~ N(0, 1), weights ~ N(0, 1/d_model) per layer, dy ~ N(0, 1), rounded to
    the storage type like make_inputs (dy stays float32)."""
    T = wl.seq_len if seq_len is None else seq_len
    B, Hq, Hkv, d, dm = wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.d_model
    rng = np.random.default_rng(wl.seed)
    ws = 1.0 / math.sqrt(dm)
    arrays = {"h0": _draw(rng, (B, T, dm), 1.0)}
    for l in range(wl.n_layers):
        arrays[f"wq{l}"] = _draw(rng, (dm, Hq * d), ws)
        arrays[f"wk{l}"] = _draw(rng, (dm, Hkv * d), ws)
        arrays[f"wv{l}"] = _draw(rng, (dm, Hkv * d), ws)
    arrays["dy"] = _draw(rng, (B, T, dm), 1.0)
    raw, f64 = {}, {}
    for name in list(arrays):
        a = arrays[name]
        if wl.dtype == "bf16" and name != "dy":
            bits = round_to_bf16_bits(a)
            raw[name] = bits
            if keep_f64:
                f64[name] = bf16_bits_to_f64(bits)
        else:
            f32 = a.astype(np.float32)
            raw[name] = f32
            if keep_f64:
                f64[name] = f32.astype(np.float64)
        arrays[name] = None
    return Inputs(wl, f64, raw)


@dataclasses.dataclass(frozen=True)
class HeadWorkload:
    """The language-model head under SFT: final hidden states H [B, T, d_model], the
    head W [vocab, d_model], target labels (-1 on the first `prompt` positions, the
    prompt, which carries no loss), streamed in partitions of ps positions."""
    name: str
    batch: int
    seq_len: int
    d_model: int
    vocab: int
    ps: int
    prompt: int
    dtype: str
    seed: int
    dw_group: int = 1


HEAD_WORKLOADS = {
    # LLaMA3-8B head (vocab 128256) on 16K positions, ps_head = 100; the weight
    # gradient is added once per 16 partitions (1600 positions)
    "8b_head_sft": HeadWorkload("8b_head_sft", 1, 16384, 4096, 128256, 100, 1024, "bf16", 19, 16),
}


def make_head_inputs(wl: HeadWorkload, seq_len: Optional[int] = None, keep_f64: bool = True) -> Inputs:
    """Draw H ~ N(0, 1), W ~ N(0, 1/d_model) (logits ~N(0, 1)), labels uniform over
    the vocabulary, -1 on the prompt positions; H and W rounded like make_inputs."""
    T = wl.seq_len if seq_len is None else seq_len
    rng = np.random.default_rng(wl.seed)
    arrays = {"h": _draw(rng, (wl.batch, T, wl.d_model), 1.0),
              "w": _draw(rng, (wl.vocab, wl.d_model), 1.0 / math.sqrt(wl.d_model))}
    labels = rng.integers(0, wl.vocab, size=(wl.batch, T)).astype(np.int32)
    labels[:, :min(wl.prompt, T)] = -1
    raw, f64 = {"labels": labels}, {"labels": labels}
    for name in list(arrays):
        a = arrays[name]
        if wl.dtype == "bf16":
            bits = round_to_bf16_bits(a)
            raw[name] = bits
            if keep_f64:
                f64[name] = bf16_bits_to_f64(bits)
        else:
            f32 = a.astype(np.float32)
            raw[name] = f32
            if keep_f64:
                f64[name] = f32.astype(np.float64)
        arrays[name] = None
    return Inputs(wl, f64, raw)
