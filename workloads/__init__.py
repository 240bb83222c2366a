"""Seeded synthetic inputs for the paged-KV attention path.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark. It holds no attention, softmax, allocator, block-table or cache-write
arithmetic: only random draws, the rounding of those draws to the storage dtype,
and the shape recipes (lengths, pool sizes, initial free-list orders, and the
list of alloc/free *requests* that fragments a pool). Block ids are never chosen
here; an allocator replays the request list.

Shapes and orders come from NumPy PCG64 generators keyed by integer SeedSequences.
Q/K/V values come from a counter-based hash so that any element can be produced
independently, on the CPU (here) or on the GPU (workloads/gen.hip), bit for bit:

  key(seed, stream, seq) = mix(seed * 2^32 + stream * 2^24 + seq)
  h_n = mix(key + (n + 1) * 0x9E3779B97F4A7C15)          (SplitMix64: Steele, Lea
                                                         and Flood, OOPSLA 2014)
  element e of a (seq, stream) lives in h_{e//3}, bits 18*(e%3) .. +17, as three
  6-bit fields a, b, c; value = sigma * (2(a+b+c) - 189) / 64.

mix is the SplitMix64 finaliser. The value is the Irwin-Hall(3) approximation of
N(0, sigma^2): mean 0, variance (4095/4096) sigma^2, support |x| <= 2.953 sigma, and
every value (an odd multiple of sigma/64 below 189 sigma/64) is exact in bfloat16.
Element index e = (position * heads + head) * head_dim + dim.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Tuple

import numpy as np

# dtype names used throughout: "f32", "bf16", "fp8" (OCP E4M3 cache only)

_STREAM_LENGTHS = 11
_STREAM_POOL = 12
_STREAM_HISTORY = 13
_STREAM_Q = 20
_STREAM_K = 21
_STREAM_V = 22
STREAMS = {"q": _STREAM_Q, "k": _STREAM_K, "v": _STREAM_V}
_STREAM_TRACE = 30
_STREAM_ARRIVALS = 31
_STREAM_PROMPTS = 32
_STREAM_OUTPUTS = 33
_STREAM_LAYER_BASE = 40     # per-layer q/k/v streams: 40 + 3 * layer + (0, 1, 2)
_STREAM_GROUPS = 34         # prefix traces: group of each request
_STREAM_SHARED = 35         #   lengths of the groups' shared prompts
_STREAM_UNIQUE = 36         #   lengths of the requests' own prompt parts
_STREAM_TOKENS = 37         #   token ids
_STREAM_PRIORITY = 38       # priority class of each request
_STREAM_OUT_LOGN = 39       # lognormal output lengths (output-length variants)
GROUP_OWNER = 1 << 23       # value/token streams of group g are owned by GROUP_OWNER + g


def rng_for(*key: int) -> np.random.Generator:
    """A PCG64 generator for the integer key (seed, stream, index...)."""
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_MIX1 = np.uint64(0xBF58476D1CE4E5B9)
_MIX2 = np.uint64(0x94D049BB133111EB)
_MASK64 = (1 << 64) - 1
_CHUNK = 1 << 16


def _mix_int(z: int) -> int:
    """SplitMix64 finaliser on a Python int (mod 2^64)."""
    z &= _MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
    return z ^ (z >> 31)


def hash_key(seed: int, stream: int, seq: int) -> int:
    """64-bit key of one (seed, stream, sequence) value stream."""
    if not (0 <= seq < (1 << 24) and 0 <= stream < 256 and 0 <= seed < (1 << 31)):
        raise ValueError("key field out of range")
    return _mix_int((seed << 32) + (stream << 24) + seq)


def _hash_at(key: int, e: np.ndarray, sigma: float) -> np.ndarray:
    """Values of the elements with flat indices e (uint64 array) of stream `key`."""
    k = np.uint64(key)
    n = e // np.uint64(3)
    j = (e - n * np.uint64(3)) * np.uint64(18)
    z = (n + np.uint64(1)) * _GAMMA
    z += k
    z ^= z >> np.uint64(30)
    z *= _MIX1
    z ^= z >> np.uint64(27)
    z *= _MIX2
    z ^= z >> np.uint64(31)
    f = ((z >> j) & np.uint64(0x3FFFF)).astype(np.uint32)
    tot = (f & np.uint32(63)) + ((f >> np.uint32(6)) & np.uint32(63)) + (f >> np.uint32(12))
    v = tot.astype(np.float32) * np.float32(2.0 / 64.0) - np.float32(189.0 / 64.0)
    if np.float32(sigma) != np.float32(1.0):
        v *= np.float32(sigma)
    return v


def hash_values_strided(key: int, starts: np.ndarray, width: int, sigma: float = 1.0) -> np.ndarray:
    """Values of the runs [starts[i], starts[i]+width) of stream `key`, as [len(starts)][width]."""
    starts = np.asarray(starts, dtype=np.uint64)
    out = np.empty((len(starts), width), np.float32)
    rows = max(1, _CHUNK // max(width, 1))
    cols = np.arange(width, dtype=np.uint64)[None, :]
    for i in range(0, len(starts), rows):
        e = starts[i:i + rows, None] + cols
        out[i:i + rows] = _hash_at(key, e, sigma)
    return out


def hash_values(key: int, e0: int, e1: int, sigma: float = 1.0) -> np.ndarray:
    """float32 values of elements e0 .. e1-1 of the stream `key` (see module doc)."""
    if e1 <= e0:
        return np.zeros(0, np.float32)
    n0, n1 = e0 // 3, (e1 - 1) // 3 + 1
    res = np.empty(3 * (n1 - n0), np.float32)
    z = np.empty(_CHUNK, np.uint64)
    t = np.empty(_CHUNK, np.uint64)
    f = np.empty((_CHUNK, 3), np.uint32)
    acc = np.empty((_CHUNK, 3), np.uint32)
    tmp = np.empty((_CHUNK, 3), np.uint32)
    ones = np.arange(1, _CHUNK + 1, dtype=np.uint64)
    k = np.uint64(key)
    sig = np.float32(sigma)
    # every buffer is reused across chunks (a fresh temporary per chunk costs page faults)
    for c0 in range(n0, n1, _CHUNK):
        m = min(_CHUNK, n1 - c0)
        zz, tt = z[:m], t[:m]
        np.add(ones[:m], np.uint64(c0), out=zz)
        np.multiply(zz, _GAMMA, out=zz)
        np.add(zz, k, out=zz)
        np.right_shift(zz, np.uint64(30), out=tt)
        np.bitwise_xor(zz, tt, out=zz)
        np.multiply(zz, _MIX1, out=zz)
        np.right_shift(zz, np.uint64(27), out=tt)
        np.bitwise_xor(zz, tt, out=zz)
        np.multiply(zz, _MIX2, out=zz)
        np.right_shift(zz, np.uint64(31), out=tt)
        np.bitwise_xor(zz, tt, out=zz)
        ff, aa, tm = f[:m], acc[:m], tmp[:m]
        for j in range(3):
            np.right_shift(zz, np.uint64(18 * j), out=tt)
            np.bitwise_and(tt, np.uint64(0x3FFFF), out=tt)
            ff[:, j] = tt
        np.bitwise_and(ff, np.uint32(63), out=aa)
        np.right_shift(ff, np.uint32(6), out=ff)
        np.bitwise_and(ff, np.uint32(63), out=tm)
        aa += tm
        np.right_shift(ff, np.uint32(6), out=ff)
        aa += ff
        o = res[3 * (c0 - n0): 3 * (c0 - n0 + m)].reshape(m, 3)
        o[:] = aa
        o *= np.float32(2.0 / 64.0)
        o -= np.float32(189.0 / 64.0)
        if sig != np.float32(1.0):
            o *= sig
    return res[e0 - 3 * n0: e1 - 3 * n0]


# ----------------------------------------------------------------------------
# storage rounding of draws (input preparation, not part of the method)
# ----------------------------------------------------------------------------

def bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 bit patterns, nearest-even; NaN kept quiet."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    if np.any(nan):
        r = np.where(nan, ((u >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16), r)
    return r


def bf16_to_f32(bits) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def as_storage(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Float32 draws -> storage array: float32 for "f32", uint16 bits for "bf16"."""
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits(x32)
    raise ValueError(f"unsupported storage dtype {dtype!r}")


def storage_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of an f32 array or bf16 bit array."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_to_f32(a).astype(np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# workload recipes
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class Workload:
    """One attention step over a paged KV cache, described by shapes and seeds.

    seq_lens[s] counts the tokens of sequence s in the cache *after* this step's
    new tokens are written; q_lens[s] is the number of new (query) tokens, which
    occupy positions seq_lens[s]-q_lens[s] .. seq_lens[s]-1.
    """

    name: str
    seed: int
    dtype: str                 # query / new K,V / output dtype: "f32" or "bf16"
    cache_dtype: str           # "f32", "bf16" or "fp8"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    seq_lens: np.ndarray       # int32 [B]
    q_lens: np.ndarray         # int32 [B]
    num_blocks: int
    free_order: np.ndarray     # int32 [num_blocks], initial free list (popped from the end)
    history: List[Tuple] = dataclasses.field(default_factory=list)
    partition_size: int = 0    # split-context partition length in tokens (0 = none)
    sigma: float = 1.0         # value scale: 1.0 or 0.5 keep every value exact in bf16
    scale: Optional[float] = None  # softmax scale; None = 1/sqrt(head_dim)
    k_scale: float = 1.0
    v_scale: float = 1.0
    # per-KV-head factors of the E4M3 scales (float32 [num_kv_heads]) or None
    k_head_scales: Optional[np.ndarray] = None
    v_head_scales: Optional[np.ndarray] = None

    @property
    def num_seqs(self) -> int:
        return int(len(self.seq_lens))

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def softmax_scale(self) -> float:
        return float(self.scale) if self.scale is not None else 1.0 / float(np.sqrt(self.head_dim))

    @property
    def total_q(self) -> int:
        return int(self.q_lens.sum())

    @property
    def is_decode(self) -> bool:
        return bool(np.all(self.q_lens == 1))

    def blocks_needed(self) -> np.ndarray:
        """ceil(seq_len / block_size) per sequence (used to size pools)."""
        return (self.seq_lens.astype(np.int64) + self.block_size - 1) // self.block_size

    def max_blocks_per_seq(self) -> int:
        return int(self.blocks_needed().max()) if self.num_seqs else 0

    # -- values -----------------------------------------------------------
    def _draw(self, stream: int, s: int, pos0: int, pos1: int, heads: int) -> np.ndarray:
        key = hash_key(self.seed, stream, s)
        e0 = pos0 * heads * self.head_dim
        e1 = pos1 * heads * self.head_dim
        x = hash_values(key, e0, e1, self.sigma)
        return x.reshape(pos1 - pos0, heads, self.head_dim)

    def kv_f32(self, s: int) -> Tuple[np.ndarray, np.ndarray]:
        """Float32 draws of K and V for positions 0..seq_lens[s]-1 of sequence s."""
        L = int(self.seq_lens[s])
        return (self._draw(_STREAM_K, s, 0, L, self.num_kv_heads),
                self._draw(_STREAM_V, s, 0, L, self.num_kv_heads))

    def value_key(self, which: str, s: int) -> int:
        """Hash key of sequence s's "q", "k" or "v" value stream."""
        return hash_key(self.seed, STREAMS[which], s)

    def kv_head_f32(self, s: int, g: int) -> Tuple[np.ndarray, np.ndarray]:
        """Float32 K and V of KV head g of sequence s, [seq_len][head_dim] each."""
        L = int(self.seq_lens[s])
        starts = (np.arange(L, dtype=np.int64) * self.num_kv_heads + g) * self.head_dim
        return (hash_values_strided(hash_key(self.seed, _STREAM_K, s), starts, self.head_dim, self.sigma),
                hash_values_strided(hash_key(self.seed, _STREAM_V, s), starts, self.head_dim, self.sigma))

    def kv(self, s: int) -> Tuple[np.ndarray, np.ndarray]:
        """K and V of sequence s in the step's input dtype (float32 or bf16 bits)."""
        k, v = self.kv_f32(s)
        return as_storage(k, self.dtype), as_storage(v, self.dtype)

    def q(self, s: int) -> np.ndarray:
        """Queries of sequence s, [q_lens[s], Hq, d], in the input dtype."""
        L, q = int(self.seq_lens[s]), int(self.q_lens[s])
        x = self._draw(_STREAM_Q, s, L - q, L, self.num_q_heads)
        return as_storage(x, self.dtype)

    def q_all(self) -> np.ndarray:
        parts = [self.q(s) for s in range(self.num_seqs)]
        if not parts:
            shape = (0, self.num_q_heads, self.head_dim)
            return np.zeros(shape, np.float32 if self.dtype == "f32" else np.uint16)
        return np.concatenate(parts, axis=0)

    def cu_q(self) -> np.ndarray:
        cu = np.zeros(self.num_seqs + 1, np.int32)
        np.cumsum(self.q_lens, out=cu[1:])
        return cu


def _permutation(seed: int, n: int) -> np.ndarray:
    return rng_for(seed, _STREAM_POOL).permutation(n).astype(np.int32)


def _pool_1p2(need_blocks: np.ndarray) -> int:
    return int(np.ceil(1.2 * float(need_blocks.sum())))


def config1() -> Workload:
    """Tiny fp32 decode: 4 sequences of context 17/14/13/14 (the four prompt lengths
    of the tiny-vllm queue), 32 query / 8 KV heads, head_dim 64, blocks of 16,
    a 64-block pool whose free list is a seeded permutation."""
    seed = 1
    L = np.array([17, 14, 13, 14], np.int32)
    return Workload("cfg1_tiny_decode_f32", seed, "f32", "f32", 32, 8, 64, 16,
                    L, np.ones(4, np.int32), 64, _permutation(seed, 64))


def config2() -> Workload:
    """Mixed continuous-batching step, bf16: 48 decode rows (context U{16..2048})
    and 4 prefill chunks of 512 new tokens after 0/512/1024/1536 cached tokens
    (the four chunks of a 2048-token prompt); 32/8 heads, d=128, blocks of 16.
    The pool is 1.5x the need and is fragmented by 2000 seeded alloc/free
    requests from dummy owners that stay live."""
    seed = 2
    g = rng_for(seed, _STREAM_LENGTHS)
    dec = g.integers(16, 2048, size=48, endpoint=True).astype(np.int32)
    c0 = np.array([0, 512, 1024, 1536], np.int32)
    L = np.concatenate([dec, c0 + 512]).astype(np.int32)
    q = np.concatenate([np.ones(48, np.int32), np.full(4, 512, np.int32)])
    w = Workload("cfg2_mixed_step_bf16", seed, "bf16", "bf16", 32, 8, 128, 16,
                 L, q, 0, np.zeros(0, np.int32))
    need = int(w.blocks_needed().sum())
    w.num_blocks = int(np.ceil(1.5 * need))
    w.free_order = np.arange(w.num_blocks, dtype=np.int32)
    w.history = alloc_free_history(seed, w.num_blocks, w.num_blocks - need, 2000)
    return w


def config3() -> Workload:
    """Large bf16 decode batch: 256 sequences, context lognormal with median 1024
    (sigma 1.0 in natural log), capped at 8192; 32/8 heads, d=128, blocks of 16;
    pool 1.2x the total blocks with a shuffled free list."""
    seed = 3
    g = rng_for(seed, _STREAM_LENGTHS)
    L = np.clip(np.rint(g.lognormal(np.log(1024.0), 1.0, size=256)), 1, 8192).astype(np.int32)
    w = Workload("cfg3_large_decode_bf16", seed, "bf16", "bf16", 32, 8, 128, 16,
                 L, np.ones(256, np.int32), 0, np.zeros(0, np.int32), partition_size=512)
    w.num_blocks = _pool_1p2(w.blocks_needed())
    w.free_order = _permutation(seed, w.num_blocks)
    return w


def config4() -> Workload:
    """Long-context bf16 decode with split context: 16 sequences of U{32k..128k}
    tokens, 64/8 heads, d=128, blocks of 32, 512-token partitions; values N(0, 0.5)."""
    seed = 4
    g = rng_for(seed, _STREAM_LENGTHS)
    L = g.integers(32768, 131072, size=16, endpoint=True).astype(np.int32)
    w = Workload("cfg4_long_context_bf16", seed, "bf16", "bf16", 64, 8, 128, 32,
                 L, np.ones(16, np.int32), 0, np.zeros(0, np.int32),
                 partition_size=512, sigma=0.5)
    w.num_blocks = _pool_1p2(w.blocks_needed())
    w.free_order = _permutation(seed, w.num_blocks)
    return w


def alloc_free_history(seed: int, pool_blocks: int, final_budget: int, n_ops: int) -> List[Tuple]:
    """A seeded list of pool requests from dummy owners: ("alloc", owner, n) with
    n in 1..64, or ("free", owner). Only counts are tracked here (never block ids).
    During the first n_ops requests the dummies may hold the whole pool, which
    churns the free list; then random dummies are freed until they hold at most
    `final_budget` blocks, and the rest stay live as holes."""
    g = rng_for(seed, _STREAM_HISTORY)
    ops: List[Tuple] = []
    live: List[Tuple[int, int]] = []   # (owner, n)
    held = 0
    next_owner = 0
    for _ in range(n_ops):
        want_alloc = (not live) or g.random() < 0.55
        if want_alloc:
            n = int(g.integers(1, 64, endpoint=True))
            if held + n <= pool_blocks:
                ops.append(("alloc", next_owner, n))
                live.append((next_owner, n))
                held += n
                next_owner += 1
                continue
            if not live:
                continue
        i = int(g.integers(0, len(live)))
        owner, n = live.pop(i)
        ops.append(("free", owner))
        held -= n
    while held > final_budget:
        i = int(g.integers(0, len(live)))
        owner, n = live.pop(i)
        ops.append(("free", owner))
        held -= n
    return ops


def small_decode(seed: int, seq_lens, num_q_heads=8, num_kv_heads=2, head_dim=64,
                 block_size=16, dtype="f32", cache_dtype=None, pool_extra=7,
                 sigma=1.0, partition_size=0) -> Workload:
    """A small decode step with a seeded permuted pool (test helper)."""
    L = np.asarray(seq_lens, np.int32)
    w = Workload(f"small_decode_{seed}", seed, dtype, cache_dtype or dtype, num_q_heads,
                 num_kv_heads, head_dim, block_size, L, np.ones(len(L), np.int32), 0,
                 np.zeros(0, np.int32), sigma=sigma, partition_size=partition_size)
    w.num_blocks = int(w.blocks_needed().sum()) + pool_extra
    w.free_order = _permutation(seed, w.num_blocks)
    return w


def small_varlen(seed: int, seq_lens, q_lens, num_q_heads=8, num_kv_heads=2, head_dim=64,
                 block_size=16, dtype="bf16", cache_dtype=None, pool_extra=5) -> Workload:
    """A small mixed step (decode rows and prefill chunks) with a permuted pool."""
    L = np.asarray(seq_lens, np.int32)
    q = np.asarray(q_lens, np.int32)
    w = Workload(f"small_varlen_{seed}", seed, dtype, cache_dtype or dtype, num_q_heads,
                 num_kv_heads, head_dim, block_size, L, q, 0, np.zeros(0, np.int32))
    w.num_blocks = int(w.blocks_needed().sum()) + pool_extra
    w.free_order = _permutation(seed, w.num_blocks)
    return w


@dataclasses.dataclass
class Trace:
    """A request trace for the continuous-batching replay: request r arrives at step
    arrival[r] with a prompt of prompt[r] tokens and stops after max_tokens[r] outputs.
    Q/K/V of (request, layer, position) are counter-hash values, so a recompute after a
    preemption writes the same bytes."""
    name: str
    seed: int
    arrival: np.ndarray
    prompt: np.ndarray
    max_tokens: np.ndarray
    num_blocks: int
    free_order: np.ndarray
    block_size: int = 16
    max_running: int = 128
    num_layers: int = 16
    num_q_heads: int = 32
    num_kv_heads: int = 8
    head_dim: int = 64
    dtype: str = "bf16"
    cache_dtype: str = "bf16"
    sigma: float = 1.0
    k_scale: float = 1.0
    v_scale: float = 1.0
    # prefix traces: request r's first prefix_len[r] prompt tokens are the system prompt of
    # group prefix_group[r] (-1: none), identical across the group, so their K/V are too
    prefix_group: Optional[np.ndarray] = None
    prefix_len: Optional[np.ndarray] = None

    @property
    def num_requests(self) -> int:
        return len(self.arrival)

    def owner_segments(self, req: int, pos0: int, pos1: int):
        """[(owner, lo, hi)] covering positions pos0..pos1-1 of request req: positions in its
        group's shared prompt belong to the group's streams, the rest to the request's."""
        S, g = 0, -1
        if self.prefix_group is not None and self.prefix_group[req] >= 0:
            S, g = int(self.prefix_len[req]), int(self.prefix_group[req])
        segs = []
        if pos0 < min(S, pos1):
            segs.append((GROUP_OWNER + g, pos0, min(S, pos1)))
        if max(pos0, S) < pos1:
            segs.append((req, max(pos0, S), pos1))
        return segs

    def prompt_tokens(self, req: int) -> np.ndarray:
        """Token ids of request req's prompt (int32 [prompt]): hashed from (owner, position)."""
        out = np.empty(int(self.prompt[req]), np.int32)
        for owner, lo, hi in self.owner_segments(req, 0, int(self.prompt[req])):
            z = (np.arange(lo, hi, dtype=np.uint64) + np.uint64(1)) * _GAMMA + np.uint64(hash_key(self.seed, _STREAM_TOKENS, owner))
            z = (z ^ (z >> np.uint64(30))) * _MIX1
            z = (z ^ (z >> np.uint64(27))) * _MIX2
            out[lo:hi] = ((z ^ (z >> np.uint64(31))) >> np.uint64(33)).astype(np.int32)
        return out

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def softmax_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))

    def value_key(self, which: str, layer: int, req: int) -> int:
        return hash_key(self.seed, _STREAM_LAYER_BASE + 3 * layer + "qkv".index(which), req)

    def rows_f32(self, which: str, layer: int, req: int, pos0: int, pos1: int) -> np.ndarray:
        """Values of positions pos0..pos1-1 of a request in one layer: [n][heads][d] float32."""
        heads = self.num_q_heads if which == "q" else self.num_kv_heads
        per = heads * self.head_dim
        parts = [hash_values(self.value_key(which, layer, owner), lo * per, hi * per, self.sigma)
                 for owner, lo, hi in self.owner_segments(req, pos0, pos1)]
        v = np.concatenate(parts) if parts else np.zeros(0, np.float32)
        return v.reshape(pos1 - pos0, heads, self.head_dim)


def config5(cache_dtype: str = "bf16") -> Trace:
    """Continuous-batching trace: 2000 requests, Poisson arrivals of one per step on
    average (arrival step = floor of the summed Exp(1) gaps), prompts lognormal with
    median 512 (sigma 1) capped at 4096, outputs Geometric(1/256) capped at 4096; at most
    128 running; blocks of 16 in a 4096-block pool (shuffled ids) that forces
    preemption; 16 layers, 32/8 heads, d=64; bf16 values, bf16 or E4M3 cache."""
    seed, n = 5, 2000
    arrival = np.floor(np.cumsum(rng_for(seed, _STREAM_ARRIVALS).exponential(1.0, size=n))).astype(np.int32)
    prompt = np.clip(np.rint(rng_for(seed, _STREAM_PROMPTS).lognormal(np.log(512.0), 1.0, size=n)),
                     1, 4096).astype(np.int32)
    max_tokens = np.minimum(rng_for(seed, _STREAM_OUTPUTS).geometric(1.0 / 256.0, size=n), 4096).astype(np.int32)
    return Trace(f"cfg5_trace_{cache_dtype}", seed, arrival, prompt, max_tokens, 4096, _permutation(seed, 4096),
                 cache_dtype=cache_dtype)


def config5_outputs(kind: str, cache_dtype: str = "bf16") -> Trace:
    """Config 5 with another output-length distribution (same arrivals, prompts, pool):
    "constant" (every request 256 outputs), "geometric" (config 5: Geometric(1/256)),
    "lognormal" (median 128, sigma 1.5, capped at 4096: a long tail)."""
    base = config5(cache_dtype)
    n = base.num_requests
    if kind == "geometric":
        return base
    if kind == "constant":
        out = np.full(n, 256, np.int32)
    elif kind == "lognormal":
        out = np.clip(np.rint(rng_for(base.seed, _STREAM_OUT_LOGN).lognormal(np.log(128.0), 1.5, size=n)),
                      1, 4096).astype(np.int32)
    else:
        raise ValueError(kind)
    return dataclasses.replace(base, name=f"cfg5_{kind}_outputs_{cache_dtype}", max_tokens=out)


def config5_prefix(cache_dtype: str = "bf16") -> Trace:
    """Config 5 with shared system prompts (prefix caching): the same arrivals and output
    lengths; each request belongs to one of 16 groups (uniform), and its prompt is the
    group's system prompt (lognormal, median 512, sigma 0.5, 64..2048 tokens) followed by
    its own part (lognormal, median 128, sigma 1, 1..2048 tokens), capped at 4096."""
    seed, n, G = 5, 2000, 16
    base = config5(cache_dtype)
    group = rng_for(seed, _STREAM_GROUPS).integers(0, G, size=n).astype(np.int32)
    shared = np.clip(np.rint(rng_for(seed, _STREAM_SHARED).lognormal(np.log(512.0), 0.5, size=G)), 64, 2048)
    own = np.clip(np.rint(rng_for(seed, _STREAM_UNIQUE).lognormal(np.log(128.0), 1.0, size=n)), 1, 2048)
    plen = shared.astype(np.int32)[group]
    prompt = np.minimum(plen + own.astype(np.int32), 4096).astype(np.int32)
    return dataclasses.replace(base, name=f"cfg5p_prefix_trace_{cache_dtype}", prompt=prompt, prefix_group=group,
                               prefix_len=np.minimum(plen, prompt - 1).astype(np.int32))


def priority_classes(tr: Trace, premium: float = 0.25) -> np.ndarray:
    """Priority class per request for the priority-admission variant: 0 (premium) with
    probability `premium`, else 1 (bulk); a seeded draw of its own."""
    u = rng_for(tr.seed, _STREAM_PRIORITY).random(tr.num_requests)
    return np.where(u < premium, 0, 1).astype(np.int32)


def small_trace(seed: int, n: int, num_blocks: int, block_size: int = 4, max_running: int = 8,
                prompt_max: int = 40, out_max: int = 30, rate: float = 1.0, groups: int = 0) -> Trace:
    """A small seeded trace for tests (same generation rules, small sizes); groups > 0
    gives every request a shared prompt of one of that many groups (prefix traces).
    Output counts are cut so that every request fits the pool on its own."""
    arrival = np.floor(np.cumsum(rng_for(seed, _STREAM_ARRIVALS).exponential(1.0 / rate, size=n))).astype(np.int32)
    prompt = rng_for(seed, _STREAM_PROMPTS).integers(1, prompt_max, size=n, endpoint=True).astype(np.int32)
    max_tokens = rng_for(seed, _STREAM_OUTPUTS).integers(1, out_max, size=n, endpoint=True).astype(np.int32)
    tr = Trace(f"small_trace_{seed}", seed, arrival, prompt, max_tokens, num_blocks,
               _permutation(seed, num_blocks), block_size=block_size, max_running=max_running,
               num_layers=2, num_q_heads=8, num_kv_heads=2, head_dim=64)
    if groups > 0:
        group = rng_for(seed, _STREAM_GROUPS).integers(0, groups, size=n).astype(np.int32)
        shared = rng_for(seed, _STREAM_SHARED).integers(1, prompt_max, size=groups, endpoint=True).astype(np.int32)
        own = rng_for(seed, _STREAM_UNIQUE).integers(1, max(2, prompt_max // 2), size=n, endpoint=True).astype(np.int32)
        plen = shared[group]
        tr.prompt = (plen + own).astype(np.int32)
        tr.prefix_group, tr.prefix_len = group, plen.astype(np.int32)
        tr.name = f"small_prefix_trace_{seed}"
    # every request must fit the pool on its own (prompt + max_tokens - 1 tokens)
    tr.max_tokens = np.clip(num_blocks * block_size + 1 - tr.prompt, 1, tr.max_tokens).astype(np.int32)
    tr.prompt = np.minimum(tr.prompt, num_blocks * block_size).astype(np.int32)
    if tr.prefix_len is not None:
        tr.prefix_len = np.minimum(tr.prefix_len, tr.prompt).astype(np.int32)
    return tr


CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4}


def config(n: int) -> Workload:
    return CONFIGS[n]()
