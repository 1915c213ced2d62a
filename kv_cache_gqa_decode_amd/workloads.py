"""Seeded synthetic decode workloads, shared by the tests, the smoke check and
the benchmark.

This module only draws random numbers and lays them out; it contains no part
of the decode computation (no rotation, no attention, no rounding beyond the
cast of the drawn values to the storage dtype), so the GPU path and the CPU
oracle can both consume its output without sharing any of the method.

Recipe (every array is a pure function of the workload name, n_kv_heads and
the overrides; see ``Spec``):

* ``rng = np.random.default_rng([cfg_id, n_kv_heads, stream])``; the streams
  are 0 (lengths), 1 (q), 2 (k_new), 3 (v_new), 4 (block permutation) and
  ``1000 + b`` (the cached history of sequence b, K then V).
* Values ~ N(0, 1) * value_scale drawn in float32, then cast to the storage
  dtype (bf16 round-to-nearest-even through torch's cast).  q is multiplied by
  ``q_gain`` before the cast (the "peaked" variants use 32).
* Sequence b holds ``L_b = positions[b] + 1`` tokens after the append: the
  history occupies slots 0 .. L_b - 2, the new token goes to slot
  ``positions[b] = L_b - 1``.
* Every slot that the attention must not read -- the append slot before the
  append, all slots >= L_b, every pool block no table row references, and the
  tail of each sequence's last block -- holds NaN when ``poison`` is set
  (zero otherwise), so a read outside the valid range shows up in the output.
* Paged pools: a seeded permutation of all physical blocks, sequence b owning
  ``perm[b * max_blocks_per_seq : (b + 1) * max_blocks_per_seq]``.
* Steps with T new tokens per sequence (``make_window``): the history of
  L_b - T tokens as above, the new tokens from streams 6 (q), 7 (k_new) and 8
  (v_new), ``positions[b] = L_b - T``.
* INT8 caches (dtype ``"i8"``): q, k_new and v_new as for bf16; the cached
  history is drawn directly as codes, N(0, 40^2) clipped to [-127, 127] and
  cast (truncating) to int8, i.e. data whose per-head absolute maximum sits
  near 3.2 standard deviations; the per-head scales (stream 5) are
  ``value_scale / 40 * U[0.75, 1.25]`` for K, then for V, in float32, so
  dequantised values have about the spread of the bf16 workloads.  Poisoned
  slots hold code 127.  Tokens are grouped by 16, each group holding per KV
  head its 16 K rows and its V block transposed: K ``[B, S_max/16, G, 16, D]``
  or ``[num_blocks, G, 16, D]``, V ``[B, S_max/16, G, D, 16]`` or
  ``[num_blocks, G, D, 16]``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

BF16_NAN = np.uint16(0x7FC0)


@dataclasses.dataclass
class Spec:
    name: str
    cfg_id: int
    dtype: str                  # "f32" | "bf16" | "i8" (bf16 inputs, INT8 cache)
    batch: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    len_lo: int                 # L_b drawn uniformly from [len_lo, len_hi]
    len_hi: int
    max_seq_len: int            # contiguous S_max (ignored when paged)
    value_scale: float = 1.0
    block_size: int = 0         # 0 = contiguous, 16 = paged
    num_blocks: int = 0
    max_blocks_per_seq: int = 0
    q_gain: float = 1.0
    poison: bool = True
    rope_base: float = 10000.0

    @property
    def n_rep(self) -> int:
        return self.n_heads // self.n_kv_heads

    @property
    def elem_bytes(self) -> int:
        """Bytes per cached K or V element."""
        return {"f32": 4, "bf16": 2, "i8": 1}[self.dtype]

    @property
    def input_dtype(self) -> str:
        """dtype of q, k_new and v_new."""
        return "bf16" if self.dtype == "i8" else self.dtype

    def replace(self, **kw) -> "Spec":
        return dataclasses.replace(self, **kw)


def spec(name: str, n_kv_heads: Optional[int] = None, **overrides) -> Spec:
    """The five workloads, by name.

    c1  fp32 B1 H8 G2 D64, 255 cached + 1 new token, S_max 256, N(0,1)
    c2  bf16 B1 H32 G8 D128, context 1024, N(0,1)/sqrt(128)
    c3  bf16 B64 H32 G8 D128, contexts U[512, 8192], padded S_max 8192
    c4  bf16 paged (16-token blocks, 65536-block pool), B32 H32 G8 D128,
        contexts U[1024, 32768], tables from a seeded block permutation
    c5  bf16 B1 H32 D128, context 131072, G in {32, 8, 1}
    """
    s128 = 1.0 / math.sqrt(128.0)
    table = {
        "c1": Spec("c1", 1, "f32", 1, 8, 2, 64, 256, 256, 256, 1.0),
        "c2": Spec("c2", 2, "bf16", 1, 32, 8, 128, 1024, 1024, 1024, s128),
        "c3": Spec("c3", 3, "bf16", 64, 32, 8, 128, 512, 8192, 8192, s128),
        "c4": Spec("c4", 4, "bf16", 32, 32, 8, 128, 1024, 32768, 32768, s128,
                   block_size=16, num_blocks=65536, max_blocks_per_seq=2048),
        "c5": Spec("c5", 5, "bf16", 1, 32, 8, 128, 131072, 131072, 131072, s128),
    }
    s = table[name]
    if n_kv_heads is not None:
        s = s.replace(n_kv_heads=n_kv_heads)
    if overrides:
        s = s.replace(**overrides)
    if s.block_size:
        s = s.replace(max_seq_len=s.max_blocks_per_seq * s.block_size)
    return s


@dataclasses.dataclass
class Problem:
    spec: Spec
    q: np.ndarray               # [B, H, D] storage dtype
    k_new: np.ndarray           # [B, G, D]
    v_new: np.ndarray           # [B, G, D]
    k_cache: np.ndarray         # [B, S_max, G, D] or [NB, 16, G, D]
    v_cache: np.ndarray
    positions: np.ndarray       # [B] int32
    seq_lens: np.ndarray        # [B] int32 = positions + 1
    block_table: Optional[np.ndarray]  # [B, max_blocks_per_seq] int32
    k_scale: Optional[np.ndarray] = None   # INT8 caches: [G] float32
    v_scale: Optional[np.ndarray] = None
    n_query: int = 1                       # new tokens per sequence (make_window)
    window: int = 0                        # mixed precision (make_mixed): ring rows W
    k_recent: Optional[np.ndarray] = None  # [B, W, G, D] bf16 bits, token p in row p mod W
    v_recent: Optional[np.ndarray] = None

    @property
    def max_len(self) -> int:
        return int(self.seq_lens.max()) if self.seq_lens.size else 0


def _rng(s: Spec, stream: int) -> np.random.Generator:
    return np.random.default_rng([s.cfg_id, s.n_kv_heads, stream])


def _to_storage(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _fill_value(s: Spec):
    if s.dtype == "f32":
        return np.float32(np.nan) if s.poison else np.float32(0)
    if s.dtype == "i8":
        return np.int8(127) if s.poison else np.int8(0)
    return BF16_NAN if s.poison else np.uint16(0)


I8_CODE_STD = 40.0


def _codes(rng: np.random.Generator, shape) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32) * np.float32(I8_CODE_STD)
    return np.clip(x, -127, 127).astype(np.int8)


def draw_scales(s: Spec):
    """Per-KV-head scales of an INT8 cache: (k_scale, v_scale), [G] float32 each."""
    rng = _rng(s, 5)
    base = s.value_scale / I8_CODE_STD
    k = (base * rng.uniform(0.75, 1.25, s.n_kv_heads)).astype(np.float32)
    v = (base * rng.uniform(0.75, 1.25, s.n_kv_heads)).astype(np.float32)
    return k, v


def group_rows(x: np.ndarray) -> np.ndarray:
    """[n * 16, G, D] -> [n, G, 16, D]: K rows regrouped into the INT8 layout."""
    n16, G, D = x.shape
    return np.ascontiguousarray(x.reshape(n16 // 16, 16, G, D).transpose(0, 2, 1, 3))


def group_transpose(x: np.ndarray) -> np.ndarray:
    """[n * 16, G, D] -> [n, G, D, 16]: V rows regrouped into the INT8 layout."""
    n16, G, D = x.shape
    return np.ascontiguousarray(x.reshape(n16 // 16, 16, G, D).transpose(0, 2, 3, 1))


def draw_lengths(s: Spec) -> np.ndarray:
    rng = _rng(s, 0)
    return rng.integers(s.len_lo, s.len_hi, size=s.batch, endpoint=True).astype(np.int32)


def draw_history(s: Spec, b: int, n_tokens: int):
    """Cached (already rotated) K and V of sequence b: two [n, G, D] arrays."""
    rng = _rng(s, 1000 + b)
    shape = (n_tokens, s.n_kv_heads, s.head_dim)
    if s.dtype == "i8":
        k = _codes(rng, shape)
        return k, _codes(rng, shape)
    k = rng.standard_normal(shape, dtype=np.float32) * np.float32(s.value_scale)
    v = rng.standard_normal(shape, dtype=np.float32) * np.float32(s.value_scale)
    return _to_storage(k, s.dtype), _to_storage(v, s.dtype)


def make_problem(s: Spec, lengths: Optional[np.ndarray] = None) -> Problem:
    """Draw every input of one decode step of workload ``s``."""
    B, H, G, D = s.batch, s.n_heads, s.n_kv_heads, s.head_dim
    L = draw_lengths(s) if lengths is None else np.asarray(lengths, np.int32).copy()
    if L.shape != (B,):
        raise ValueError("lengths must have shape [batch]")
    if (L < 1).any() or (L > s.max_seq_len).any():
        raise ValueError("every length must lie in [1, max_seq_len]")
    sc = np.float32(s.value_scale)
    q = _rng(s, 1).standard_normal((B, H, D), dtype=np.float32) * sc * np.float32(s.q_gain)
    k_new = _rng(s, 2).standard_normal((B, G, D), dtype=np.float32) * sc
    v_new = _rng(s, 3).standard_normal((B, G, D), dtype=np.float32) * sc
    store = {"f32": np.float32, "bf16": np.uint16, "i8": np.int8}[s.dtype]
    i8 = s.dtype == "i8"
    if i8 and (s.max_seq_len % 16 or s.block_size % 16):
        raise ValueError("INT8 caches group tokens by 16")
    fill = _fill_value(s)
    table = None
    if s.block_size:
        bs = s.block_size
        if B * s.max_blocks_per_seq > s.num_blocks:
            raise ValueError("pool too small for disjoint tables")
        perm = _rng(s, 4).permutation(s.num_blocks).astype(np.int32)
        table = np.ascontiguousarray(
            perm[: B * s.max_blocks_per_seq].reshape(B, s.max_blocks_per_seq))
        m = bs // 16
        gk = (G, 16, D) if m == 1 else (m, G, 16, D)
        gv = (G, D, 16) if m == 1 else (m, G, D, 16)
        k_cache = np.full((s.num_blocks, *gk) if i8 else (s.num_blocks, bs, G, D), fill,
                          dtype=store)
        v_cache = np.full((s.num_blocks, *gv) if i8 else (s.num_blocks, bs, G, D), fill,
                          dtype=store)
        for b in range(B):
            n_hist = int(L[b]) - 1
            if n_hist == 0:
                continue
            kh, vh = draw_history(s, b, n_hist)
            nblk = -(-n_hist // bs)
            pad = nblk * bs - n_hist
            if pad:
                kh = np.concatenate([kh, np.full((pad, G, D), fill, store)])
                vh = np.concatenate([vh, np.full((pad, G, D), fill, store)])
            ids = table[b, :nblk]
            if i8:
                k_cache[ids] = group_rows(kh).reshape(nblk, *gk)
                v_cache[ids] = group_transpose(vh).reshape(nblk, *gv)
            else:
                k_cache[ids] = kh.reshape(nblk, bs, G, D)
                v_cache[ids] = vh.reshape(nblk, bs, G, D)
    else:
        S = s.max_seq_len
        k_cache = np.full((B, S // 16, G, 16, D) if i8 else (B, S, G, D), fill, dtype=store)
        v_cache = np.full((B, S // 16, G, D, 16) if i8 else (B, S, G, D), fill, dtype=store)
        for b in range(B):
            n_hist = int(L[b]) - 1
            if n_hist:
                kh, vh = draw_history(s, b, n_hist)
                if i8:
                    nblk = -(-n_hist // 16)
                    pad = nblk * 16 - n_hist
                    if pad:
                        kh = np.concatenate([kh, np.full((pad, G, D), fill, store)])
                        vh = np.concatenate([vh, np.full((pad, G, D), fill, store)])
                    k_cache[b, :nblk] = group_rows(kh)
                    v_cache[b, :nblk] = group_transpose(vh)
                else:
                    k_cache[b, :n_hist] = kh
                    v_cache[b, :n_hist] = vh
    k_scale, v_scale = draw_scales(s) if i8 else (None, None)
    idt = s.input_dtype
    return Problem(spec=s, q=_to_storage(q, idt), k_new=_to_storage(k_new, idt),
                   v_new=_to_storage(v_new, idt), k_cache=k_cache, v_cache=v_cache,
                   positions=(L - 1).astype(np.int32), seq_lens=L.astype(np.int32),
                   block_table=table, k_scale=k_scale, v_scale=v_scale)


def make_window(s: Spec, n_query: int, lengths: Optional[np.ndarray] = None) -> Problem:
    """A step with ``n_query`` = T new tokens per sequence (the verification
    pass of speculative decoding).  Sequence b holds L_b tokens after the
    step (``lengths``, default the spec's draw clipped to at least T): the
    history of L_b - T tokens is drawn exactly as by ``make_problem``, the T
    new tokens go to slots ``positions[b] = L_b - T`` .. L_b - 1 (poisoned
    before the append), and q [B, T, H, D], k_new / v_new [B, T, G, D] come
    from streams 6, 7 and 8 with the distributions of streams 1, 2 and 3."""
    T = int(n_query)
    if T < 1:
        raise ValueError("n_query must be >= 1")
    L = draw_lengths(s) if lengths is None else np.asarray(lengths, np.int32).copy()
    L = np.maximum(L, T).astype(np.int32)
    if (L > s.max_seq_len).any():
        raise ValueError("every length must lie in [n_query, max_seq_len]")
    p = make_problem(s, lengths=L - T + 1)
    B, H, G, D = s.batch, s.n_heads, s.n_kv_heads, s.head_dim
    sc = np.float32(s.value_scale)
    q = _rng(s, 6).standard_normal((B, T, H, D), dtype=np.float32) * sc * np.float32(s.q_gain)
    k_new = _rng(s, 7).standard_normal((B, T, G, D), dtype=np.float32) * sc
    v_new = _rng(s, 8).standard_normal((B, T, G, D), dtype=np.float32) * sc
    idt = s.input_dtype
    return dataclasses.replace(p, q=_to_storage(q, idt), k_new=_to_storage(k_new, idt),
                               v_new=_to_storage(v_new, idt), positions=(L - T).astype(np.int32),
                               seq_lens=L, n_query=T)


def _i8_slot(p: Problem, b: int, pos: int):
    """Index tuples of token pos of sequence b in an INT8 K and V cache."""
    s = p.spec
    if s.block_size:
        blk = int(p.block_table[b, pos // s.block_size])
        r = pos % s.block_size
        if s.block_size == 16:
            return (blk, slice(None), r % 16), (blk, slice(None), slice(None), r % 16)
        return ((blk, r // 16, slice(None), r % 16),
                (blk, r // 16, slice(None), slice(None), r % 16))
    return (b, pos // 16, slice(None), pos % 16), (b, pos // 16, slice(None), slice(None), pos % 16)


def make_mixed(s: Spec, window: int, lengths: Optional[np.ndarray] = None) -> Problem:
    """A decode step on a mixed-precision cache: the ``window`` = W newest
    cached tokens of a sequence in bf16 rings (token p in row p mod W), the
    older ones in the INT8 cache of ``s`` (dtype "i8").  Before the step
    sequence b holds P = L_b - 1 tokens: the INT8 cache has codes (drawn as
    by ``make_problem``) for positions [0, P - W), and the rings hold the
    tokens [max(0, P - W), P), drawn from stream 2000 + b with the bf16
    distribution (N(0, 1) * value_scale).  Every INT8 slot from P - W on and
    every ring row past P (a short sequence) is poisoned."""
    if s.dtype != "i8":
        raise ValueError("the history of a mixed cache is INT8")
    W = int(window)
    if W < 1:
        raise ValueError("window must be >= 1")
    p = make_problem(s, lengths=lengths)
    B, G, D = s.batch, s.n_kv_heads, s.head_dim
    fill = _fill_value(s)
    kr = np.full((B, W, G, D), BF16_NAN if s.poison else np.uint16(0), np.uint16)
    vr = kr.copy()
    k_cache, v_cache = p.k_cache, p.v_cache
    for b in range(B):
        P = int(p.positions[b])
        lo = max(0, P - W)
        for pos in range(lo, P):                     # in the ring, not in the INT8 cache
            ki, vi = _i8_slot(p, b, pos)
            k_cache[ki] = fill
            v_cache[vi] = fill
        if P > lo:
            rng = _rng(s, 2000 + b)
            shape = (P - lo, G, D)
            kh = rng.standard_normal(shape, dtype=np.float32) * np.float32(s.value_scale)
            vh = rng.standard_normal(shape, dtype=np.float32) * np.float32(s.value_scale)
            rows = np.arange(lo, P) % W
            kr[b, rows] = _to_storage(kh, "bf16")
            vr[b, rows] = _to_storage(vh, "bf16")
    return dataclasses.replace(p, window=W, k_recent=kr, v_recent=vr)


def as_torch(a: np.ndarray, device=None):
    """A torch tensor holding the same bits (uint16 arrays become bfloat16)."""
    import torch
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    return t.to(device) if device is not None else t


def from_torch(t) -> np.ndarray:
    """Host numpy copy with the same bits (bfloat16 becomes uint16)."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()
