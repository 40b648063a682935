"""Seeded synthetic inputs for the HSTU attention layer.

This module is shared by the oracle tests, the GPU parity tests and the
benchmark. It draws random numbers and lays them out; it performs none of the
attention arithmetic. Every array it returns is a NumPy array on the host.

Shapes and distributions follow the workloads described for HSTU serving and
training in "HSTU Generative Recommenders: Deploy on GPU Cloud" (section "HSTU
in Plain Terms", sequence length 8,192) and "Deploying an HSTU Generative
Recommender with NVIDIA Dynamo-Triton" (batch 8, sequences up to 8,320 tokens):

* jagged user sequences packed back to back, ``seq_offsets[B+1]`` (int32);
* strictly increasing per-user timestamps in integer seconds, starting at
  1,700,000,000 with gaps ``ceil(Exp(mean 60 s))`` (at least 1 s);
* Q, K, V, U ~ N(0, 1); bias tables ~ N(0, 0.02) read as a variance
  (standard deviation sqrt(0.02));
* for the full layer, X ~ N(0, 1) and weights ~ N(0, 1/1024) (variance).

Draw order inside one generator: lengths, timestamp gaps, Q, K, V, U, tables
(the layer case draws X, W1, W2 in place of Q, K, V, U).

bf16 workloads are rounded to bf16 (round to nearest even) here, so that the
values handed to the GPU and to the fp64 oracle are the same numbers.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

TS_START = 1_700_000_000
TS_GAP_MEAN = 60.0
TABLE_VAR = 0.02


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32.

    NaN and infinity do not occur in generated data and are not handled.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    bits = (bits + 0x7FFF + lsb) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32)


def _normal(rng, shape, dtype_name, std=1.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x = (x * np.float32(std)).astype(np.float32)
    if dtype_name == "bf16":
        x = round_to_bf16(x)
    return x


def _timestamps(rng, lengths):
    """Per-user strictly increasing int64 timestamps, packed like the tokens."""
    total = int(np.sum(lengths))
    gaps = np.ceil(rng.exponential(TS_GAP_MEAN, size=total)).astype(np.int64)
    gaps = np.maximum(gaps, 1)
    ts = np.empty(total, dtype=np.int64)
    off = 0
    for n in lengths:
        n = int(n)
        if n:
            g = gaps[off:off + n].copy()
            g[0] = 0
            ts[off:off + n] = TS_START + np.cumsum(g)
        off += n
    return ts


def offsets_from_lengths(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    off = np.zeros(len(lengths) + 1, dtype=np.int64)
    off[1:] = np.cumsum(lengths)
    return off.astype(np.int32)


@dataclasses.dataclass
class Tables:
    pos: Optional[np.ndarray]   # float32 [n_pos] or None
    time: Optional[np.ndarray]  # float32 [n_time] or None


def _tables(rng, n_pos, n_time):
    std = float(np.sqrt(TABLE_VAR))
    pos = (rng.standard_normal(n_pos, dtype=np.float32) * np.float32(std)).astype(np.float32) if n_pos else None
    tim = (rng.standard_normal(n_time, dtype=np.float32) * np.float32(std)).astype(np.float32) if n_time else None
    return Tables(pos, tim)


@dataclasses.dataclass
class JaggedInputs:
    """Packed jagged inputs for the full (causal) path."""
    name: str
    dtype: str                 # "f32" or "bf16"
    num_heads: int
    head_dim: int
    lengths: np.ndarray        # int64 [B]
    seq_offsets: np.ndarray    # int32 [B+1]
    ts: np.ndarray             # int64 [T]
    q: np.ndarray              # float32 [T, H, d]
    k: np.ndarray
    v: np.ndarray
    u: np.ndarray              # float32 [T, H*d]
    tables: Tables

    @property
    def batch(self):
        return len(self.lengths)

    @property
    def total(self):
        return int(self.seq_offsets[-1])

    @property
    def max_len(self):
        return int(self.lengths.max()) if len(self.lengths) else 0


def jagged(name, seed, lengths, num_heads, head_dim, dtype, n_pos, n_time) -> JaggedInputs:
    """Generic jagged workload with the draw order stated in the module doc."""
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, dtype=np.int64)
    return _jagged_from_rng(name, rng, lengths, num_heads, head_dim, dtype, n_pos, n_time)


def _jagged_from_rng(name, rng, lengths, H, d, dtype, n_pos, n_time):
    ts = _timestamps(rng, lengths)
    T = int(lengths.sum())
    q = _normal(rng, (T, H, d), dtype)
    k = _normal(rng, (T, H, d), dtype)
    v = _normal(rng, (T, H, d), dtype)
    u = _normal(rng, (T, H * d), dtype)
    tables = _tables(rng, n_pos, n_time)
    return JaggedInputs(name, dtype, H, d, lengths, offsets_from_lengths(lengths), ts, q, k, v, u, tables)


def tiny_fp32(seed: int = 1) -> JaggedInputs:
    """Two jagged sequences {37, 100}, 2 heads of 32, fp32, 64 position buckets."""
    return jagged("tiny_fp32_B2_L37-100_H2_d32", seed, [37, 100], 2, 32, "f32", 64, 0)


def training_shape(seed: int = 2) -> JaggedInputs:
    """Batch 32, lengths uniform in [64, 1024], 4 heads of 128, bf16, pos 128 + time 128."""
    rng = np.random.default_rng(seed)
    lengths = rng.integers(64, 1024, size=32, endpoint=True).astype(np.int64)
    return _jagged_from_rng("jagged_train_B32_L64-1024_H4_d128_bf16", rng, lengths, 4, 128, "bf16", 128, 128)


def long_seq(seed: int = 6, batch: int = 8, seq_len: int = 8192) -> JaggedInputs:
    """Batch 8 sequences of 8,192 tokens, 4 heads of 128, bf16, pos 128 + time 128."""
    rng = np.random.default_rng(seed)
    lengths = np.full(batch, seq_len, dtype=np.int64)
    return _jagged_from_rng(f"causal_B{batch}_L{seq_len}_H4_d128_bf16", rng, lengths, 4, 128, "bf16", 128, 128)


def time_bucket_edges(seed: int = 91) -> JaggedInputs:
    """Edge case for the time buckets: users of 300, 200 and 257 tokens one
    second apart, so |dt| equals the distance and every bucket's lower edge
    |dt| = 2^b - 1 occurs in every row that reaches it; 2 heads of 64, bf16,
    4 position buckets (constant beyond distance 3), 16 time buckets, the
    time table scaled by 16 so that a pair in the wrong bucket moves the
    output well past the bf16 bar."""
    inp = jagged("time_bucket_edges", seed, [300, 200, 257], 2, 64, "bf16", 4, 16)
    off = inp.seq_offsets
    for b in range(len(off) - 1):
        inp.ts[off[b]:off[b + 1]] = TS_START + np.arange(off[b + 1] - off[b], dtype=np.int64)
    inp.tables.time = (inp.tables.time * 16).astype(np.float32)
    return inp


@dataclasses.dataclass
class CachedInputs:
    """KV-cache delta workload: per user a cached prefix and some new tokens.

    ``hist`` holds every user's full history (prefix then new tokens) packed
    like a jagged batch; the new tokens are the last ``new_lens[b]`` of each.
    ``page_ids`` lists, per user, the pool pages that hold its history in
    order (64 tokens per page), drawn as a seeded permutation of the pool.
    """
    name: str
    dtype: str
    num_heads: int
    head_dim: int
    hist: JaggedInputs
    cache_lens: np.ndarray      # int32 [B] prefix length before this step
    new_lens: np.ndarray        # int32 [B]
    page_size: int
    num_pages: int
    max_pages_per_seq: int
    page_table: np.ndarray      # int32 [B, max_pages_per_seq], -1 = unused

    @property
    def batch(self):
        return len(self.cache_lens)

    def new_offsets(self):
        return offsets_from_lengths(self.new_lens)

    def prefix_offsets(self):
        return offsets_from_lengths(self.cache_lens)

    def split(self):
        """Packed (prefix rows, new rows) index arrays into ``hist``."""
        off = self.hist.seq_offsets
        pre, new = [], []
        for b in range(self.batch):
            s = int(off[b])
            c = int(self.cache_lens[b])
            m = int(self.new_lens[b])
            pre.append(np.arange(s, s + c))
            new.append(np.arange(s + c, s + c + m))
        cat = lambda xs: np.concatenate(xs) if xs else np.zeros(0, np.int64)
        return cat(pre).astype(np.int64), cat(new).astype(np.int64)


def cached(name, seed, cache_lens, new_lens, H=4, d=128, dtype="bf16", n_pos=128, n_time=128,
           page_size=64, spare_pages=16) -> CachedInputs:
    rng = np.random.default_rng(seed)
    cache_lens = np.asarray(cache_lens, dtype=np.int64)
    new_lens = np.asarray(new_lens, dtype=np.int64)
    hist = _jagged_from_rng(name + "_hist", rng, cache_lens + new_lens, H, d, dtype, n_pos, n_time)
    pages_per = [(int(c + m) + page_size - 1) // page_size for c, m in zip(cache_lens, new_lens)]
    max_pages = max([1] + pages_per)
    num_pages = int(sum(pages_per)) + spare_pages
    perm = rng.permutation(num_pages).astype(np.int32)
    table = np.full((len(cache_lens), max_pages), -1, dtype=np.int32)
    p = 0
    for b, n in enumerate(pages_per):
        table[b, :n] = perm[p:p + n]
        p += n
    return CachedInputs(name, dtype, H, d, hist, cache_lens.astype(np.int32), new_lens.astype(np.int32),
                        page_size, num_pages, max_pages, table)


def kv_cache_delta(seed: int = 3) -> CachedInputs:
    """Batch 8, 8,192 cached tokens per user in 64-token pages, 128 new tokens each, 4 x 128, bf16."""
    return cached("kv_delta_B8_C8192_M128_H4_d128_bf16", seed, [8192] * 8, [128] * 8)


@dataclasses.dataclass
class CandidateInputs:
    """M-FALCON workload: per user a history followed by candidate tokens.

    Token rows of user b are ``[history (hist_lens[b]) | candidates (num_candidates[b])]``.
    Every candidate of a user carries the request timestamp.
    """
    name: str
    inputs: JaggedInputs
    hist_lens: np.ndarray        # int32 [B]
    num_candidates: np.ndarray   # int32 [B]

    def split(self):
        """Packed (history rows, candidate rows) index arrays into ``inputs``."""
        off = self.inputs.seq_offsets
        hist, cand = [], []
        for b in range(len(self.hist_lens)):
            s = int(off[b])
            n, m = int(self.hist_lens[b]), int(self.num_candidates[b])
            hist.append(np.arange(s, s + n))
            cand.append(np.arange(s + n, s + n + m))
        cat = lambda xs: np.concatenate(xs) if xs else np.zeros(0, np.int64)
        return cat(hist).astype(np.int64), cat(cand).astype(np.int64)

    def history_pages(self, seed: int, page_size: int = 64, spare_pages: int = 16):
        """A page pool for the histories: (num_pages, page_table [B, max_pages]),
        pages drawn as a seeded permutation of the pool, -1 = unused."""
        rng = np.random.default_rng(seed)
        pages_per = [(int(n) + page_size - 1) // page_size for n in self.hist_lens]
        max_pages = max([1] + pages_per)
        num_pages = int(sum(pages_per)) + spare_pages
        perm = rng.permutation(num_pages).astype(np.int32)
        table = np.full((len(self.hist_lens), max_pages), -1, dtype=np.int32)
        p = 0
        for b, n in enumerate(pages_per):
            table[b, :n] = perm[p:p + n]
            p += n
        return num_pages, table


def candidates(name, seed, hist_lens, cand_lens, H=4, d=128, dtype="bf16", n_pos=128, n_time=128):
    rng = np.random.default_rng(seed)
    hist_lens = np.asarray(hist_lens, dtype=np.int64)
    cand_lens = np.asarray(cand_lens, dtype=np.int64)
    lengths = hist_lens + cand_lens
    hist_ts = _timestamps(rng, hist_lens)
    req_gap = np.maximum(np.ceil(rng.exponential(TS_GAP_MEAN, size=len(lengths))).astype(np.int64), 1)
    T = int(lengths.sum())
    ts = np.empty(T, dtype=np.int64)
    o, ho = 0, 0
    for b in range(len(lengths)):
        n, m = int(hist_lens[b]), int(cand_lens[b])
        ts[o:o + n] = hist_ts[ho:ho + n]
        last = hist_ts[ho + n - 1] if n else TS_START
        ts[o + n:o + n + m] = last + req_gap[b]
        o += n + m
        ho += n
    q = _normal(rng, (T, H, d), dtype)
    k = _normal(rng, (T, H, d), dtype)
    v = _normal(rng, (T, H, d), dtype)
    u = _normal(rng, (T, H * d), dtype)
    tables = _tables(rng, n_pos, n_time)
    inp = JaggedInputs(name, dtype, H, d, lengths, offsets_from_lengths(lengths), ts, q, k, v, u, tables)
    return CandidateInputs(name, inp, hist_lens.astype(np.int32), cand_lens.astype(np.int32))


def mfalcon_scoring(seed: int = 4) -> CandidateInputs:
    """Batch 4 users, 4,096 history tokens + 1,024 candidates each, 4 x 128, bf16."""
    return candidates("mfalcon_B4_N4096_C1024_H4_d128_bf16", seed, [4096] * 4, [1024] * 4)


@dataclasses.dataclass
class LayerInputs:
    """Full HSTU layer: X [T, D] with f1 weight [D, 4D] and f2 weight [D, D]."""
    name: str
    lengths: np.ndarray
    seq_offsets: np.ndarray
    ts: np.ndarray
    x: np.ndarray      # float32 (bf16 values) [T, D]
    w1: np.ndarray     # [D, 4D]
    w2: np.ndarray     # [D, D]
    num_heads: int
    head_dim: int
    tables: Tables

    @property
    def total(self):
        return int(self.seq_offsets[-1])

    @property
    def max_len(self):
        return int(self.lengths.max()) if len(self.lengths) else 0


def full_layer(seed: int = 5, batch: int = 16, embed: int = 1024, num_heads: int = 8, head_dim: int = 128,
               median_len: float = 2048.0, sigma: float = 1.0, max_len: int = 8192,
               lengths=None) -> LayerInputs:
    """Batch 16, lengths lognormal(median 2048, sigma 1) capped at 8,192, D=1024, 8 x 128, bf16."""
    rng = np.random.default_rng(seed)
    if lengths is None:
        raw = rng.lognormal(np.log(median_len), sigma, size=batch)
        lengths = np.minimum(max_len, np.maximum(1, np.rint(raw))).astype(np.int64)
    else:
        lengths = np.asarray(lengths, dtype=np.int64)
    ts = _timestamps(rng, lengths)
    T = int(lengths.sum())
    x = _normal(rng, (T, embed), "bf16")
    w1 = _normal(rng, (embed, 4 * num_heads * head_dim), "bf16", std=float(np.sqrt(1.0 / embed)))
    w2 = _normal(rng, (num_heads * head_dim, embed), "bf16", std=float(np.sqrt(1.0 / embed)))
    tables = _tables(rng, 128, 128)
    return LayerInputs(f"layer_B{batch}_D{embed}_H{num_heads}_d{head_dim}_bf16", lengths,
                       offsets_from_lengths(lengths), ts, x, w1, w2, num_heads, head_dim, tables)


def upstream_grad(seed: int, shape, dtype: str = "bf16") -> np.ndarray:
    """Gradient of a training loss with respect to the layer output, N(0, 1) (seeded)."""
    return _normal(np.random.default_rng(seed), tuple(shape), dtype)


def affine_terms(seed: int, width: int):
    """LayerNorm affine terms: weight ~ N(1, 0.1^2), bias ~ N(0, 0.1^2), fp32."""
    rng = np.random.default_rng(seed)
    w = (1.0 + 0.1 * rng.standard_normal(width, dtype=np.float32)).astype(np.float32)
    b = (0.1 * rng.standard_normal(width, dtype=np.float32)).astype(np.float32)
    return w, b


def dense_operands(seed: int, M: int, N: int, K: int):
    """Operands of a dense product: A ~ N(0, 1) [M, K] and B ~ N(0, 1/K) [K, N], bf16 values."""
    rng = np.random.default_rng(seed)
    return _normal(rng, (M, K), "bf16"), _normal(rng, (K, N), "bf16", std=float(np.sqrt(1.0 / K)))
