"""ctypes binding of libpkv (argument marshalling only).

Every compute step runs in libpkv's HIP kernels or its C++ host code; this module
only converts torch tensors / numpy arrays to pointers and sizes, and raises on a
non-zero status. It fails loudly when libpkv.so has not been built.
"""
from __future__ import annotations

import ctypes as C
import os
import re
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpkv.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "pkv.h")

PKV_OK, PKV_ERR_INVALID, PKV_ERR_OUT_OF_BLOCKS, PKV_ERR_HIP, PKV_ERR_UNSUPPORTED = 0, -1, -2, -3, -4
F32, BF16, FP8 = 0, 1, 2
DTYPE_CODES = {"f32": F32, "bf16": BF16, "fp8": FP8}


class PkvError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libpkv status {status}: {msg}")
        self.status = status


class OutOfBlocks(PkvError):
    pass


_lib = None

i32, i64, f32, vp, sz = C.c_int32, C.c_int64, C.c_float, C.c_void_p, C.c_size_t
P_i32 = C.POINTER(C.c_int32)
P_i64 = C.POINTER(C.c_int64)


class PkvLayers(C.Structure):
    """struct pkv_layers: layer count and the strides between layers (bytes; lse in floats)."""
    _fields_ = [("num_layers", C.c_int32), ("in_bytes", C.c_int64), ("out_bytes", C.c_int64),
                ("cache_bytes", C.c_int64), ("lse_floats", C.c_int64)]


_SIGS = {
    "pkv_version": (C.c_char_p, []),
    "pkv_last_error": (C.c_char_p, []),
    "pkv_alloc_pool": (C.c_int, [i32, i32, i32, i32, i32, vp, C.POINTER(vp), P_i64]),
    "pkv_destroy_pool": (None, [vp]),
    "pkv_pool_alloc": (C.c_int, [vp, i32, vp]),
    "pkv_pool_free": (C.c_int, [vp, vp, i32]),
    "pkv_pool_stats": (C.c_int, [vp, P_i32, P_i32]),
    "pkv_pool_free_list": (C.c_int, [vp, vp, i32, P_i32]),
    "pkv_seq_reserve": (C.c_int, [vp, i64, i32]),
    "pkv_seq_release": (C.c_int, [vp, i64]),
    "pkv_seq_table": (C.c_int, [vp, i64, vp, i32, P_i32]),
    "pkv_build_block_table": (C.c_int, [vp, i32, vp, vp, vp, i32, vp, vp, vp]),
    "pkv_kv_cache_write": (C.c_int, [vp, vp, i32, i32, i32, i32, vp, vp, i32, i32, i32, vp, f32, f32, vp, vp, vp]),
    "pkv_kv_cache_write_layers": (C.c_int, [vp, vp, i32, i32, i32, i32, vp, vp, i32, i32, i32, vp, f32, f32, vp,
                                            vp, vp, vp]),
    "pkv_decode_workspace_bytes": (sz, [i32, i32, i32, i32, i32]),
    "pkv_decode_set_profile_event": (None, [vp]),
    "pkv_paged_attention_decode": (C.c_int, [vp, vp, i32, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32,
                                             i32, i32, f32, f32, f32, vp, vp, i32, vp, sz, vp, vp, i32, vp]),
    "pkv_build_decode_work": (C.c_int, [i32, vp, i32, vp, i32, P_i32]),
    "pkv_build_varlen_work": (C.c_int, [i32, vp, vp, i32, i32, vp, i32, P_i32]),
    "pkv_build_decode_split": (C.c_int, [i32, vp, i32, i32, i32, vp, i32, P_i32, P_i32]),
    "pkv_paged_attention_prefill_chunks": (C.c_int, [vp, vp, i32, vp, vp, i32, vp, vp, vp, i32, i32, i32, i32, i32,
                                                     i32, i32, i32, i32, f32, f32, f32, vp, vp, vp, i32, vp, i32,
                                                     i32, vp, i64, vp, vp]),
    "pkv_paged_attention_prefill_chunks_layers": (C.c_int, [vp, vp, i32, vp, vp, i32, vp, vp, vp, i32, i32, i32, i32,
                                                            i32, i32, i32, i32, i32, f32, f32, f32, vp, vp, vp, i32,
                                                            vp, i32, i32, vp, i64, vp, vp, vp]),
    "pkv_build_chunk_work": (C.c_int, [i32, vp, vp, i32, i32, i32, i32, vp, i32, P_i32, vp, i32, P_i32, P_i32]),
    "pkv_chunk_slots": (C.c_int, [i32, i32, i32, P_i32]),
    "pkv_build_mixed_step": (C.c_int, [i32, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, P_i32, vp, i32, P_i32,
                                       P_i32, vp, i32, P_i32, vp, i32, P_i32, P_i32]),
    "pkv_chunk_workspace_bytes": (i64, [i32, i32]),
    "pkv_swap_workspace_bytes": (i64, [i32, i32, i64]),
    "pkv_swap_out": (C.c_int, [vp, vp, i32, i32, i64, vp, vp, i32, vp, i32, vp, i64, vp, vp]),
    "pkv_swap_in": (C.c_int, [vp, vp, i32, i32, i64, vp, vp, i32, vp, i32, vp, i64, vp]),
    "pkv_sched_create": (C.c_int, [vp, i32, C.POINTER(vp)]),
    "pkv_sched_destroy": (None, [vp]),
    "pkv_sched_add_requests": (C.c_int, [vp, i32, vp, vp, vp, vp]),
    "pkv_sched_schedule": (C.c_int, [vp, P_i32, P_i32, P_i32]),
    "pkv_sched_plan": (C.c_int, [vp, i32, vp, vp, vp, vp, vp, vp, vp]),
    "pkv_sched_update": (C.c_int, [vp]),
    "pkv_sched_counters": (C.c_int, [vp, vp]),
    "pkv_sched_set_admission_check": (C.c_int, [vp, i32]),
    "pkv_sched_enable_prefix_cache": (C.c_int, [vp]),
    "pkv_sched_set_prompt_tokens": (C.c_int, [vp, i64, vp, i32]),
    "pkv_sched_set_token_budget": (C.c_int, [vp, i32, i32]),
    "pkv_sched_enable_swap": (C.c_int, [vp, i32]),
    "pkv_sched_set_victim_policy": (C.c_int, [vp, i32]),
    "pkv_sched_set_static_batching": (C.c_int, [vp, i32]),
    "pkv_sched_set_priorities": (C.c_int, [vp, i32, vp, vp]),
    "pkv_sched_swap_pairs": (C.c_int, [vp, P_i32, P_i32, vp, vp]),
    "pkv_sched_swap_counters": (C.c_int, [vp, vp]),
    "pkv_seq_share": (C.c_int, [vp, i64, vp, i32]),
    "pkv_block_refs": (C.c_int, [vp, vp, i32]),
    "pkv_decode_split_slots": (C.c_int, [i32, i32, i32, i32, P_i32]),
    "pkv_decode_split_workspace_bytes": (sz, [i32, i32, i32, i32]),
    "pkv_paged_attention_decode_split": (C.c_int, [vp, vp, i32, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32,
                                                   i32, i32, f32, f32, f32, vp, vp, vp, i32, vp, i32, vp, i32, i32,
                                                   i32, vp, sz, vp, vp]),
    "pkv_paged_attention_decode_split_layers": (C.c_int, [vp, vp, i32, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32,
                                                          i32, i32, i32, f32, f32, f32, vp, vp, vp, i32, vp, i32, vp,
                                                          i32, i32, i32, vp, sz, vp, vp, vp]),
    "pkv_decode_split_noalloc_max_bytes": (sz, []),
    "pkv_paged_attention_decode_split_noalloc": (C.c_int, [vp, vp, i32, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32,
                                                           i32, i32, i32, f32, f32, f32, vp, vp, vp, i32, vp, i32, vp,
                                                           i32, i32, i32, vp, vp]),
    "pkv_paged_attention_prefill_varlen": (C.c_int, [vp, vp, i32, vp, vp, i32, vp, vp, vp, i32, i32, i32, i32, i32,
                                                     i32, i32, i32, i32, f32, f32, f32, vp, vp, vp, i32, vp, vp]),
    "pkv_mixed_decode_slots": (C.c_int, [i32, vp, vp, i32, i32, i32, i32, i32, i32, P_i32]),
    "pkv_paged_attention_mixed": (C.c_int, [vp, vp, i32, vp, vp, i32, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                            i32, i32, f32, f32, f32, vp, vp, vp, i32, vp, i32, i32, i32, vp, sz, vp,
                                            i32, vp, i32, i32, vp, i64, vp, vp]),
    "pkv_paged_attention_mixed_layers": (C.c_int, [vp, vp, i32, vp, vp, i32, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                                   i32, i32, i32, f32, f32, f32, vp, vp, vp, i32, vp, i32, i32, i32,
                                                   vp, sz, vp, i32, vp, i32, i32, vp, i64, vp, vp, vp]),
}


class StepPlan:
    """Host arrays of one scheduled step (rows in running order)."""

    def __init__(self, step, ids, stages, q_lens, seq_lens, block_tables, cu_seqlens_q, slot_mapping):
        self.step, self.ids, self.stages, self.q_lens, self.seq_lens = step, ids, stages, q_lens, seq_lens
        self.block_tables, self.cu_seqlens_q, self.slot_mapping = block_tables, cu_seqlens_q, slot_mapping


class Scheduler:
    """pkv_sched handle: the continuous-batching step over a Pool (which it must not outlive)."""

    COUNTERS = ("step", "free", "running", "waiting", "preempted", "finished", "requests", "cached_tokens")

    def __init__(self, pool: Pool, max_running: int):
        self.pool = pool                        # keeps the pool alive
        h = vp()
        check(lib().pkv_sched_create(pool.handle, max_running, C.byref(h)))
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.pkv_sched_destroy(h)
            self._h = None

    def add_requests(self, ids, arrival, prompt, max_tokens) -> None:
        a = [np.ascontiguousarray(x, dtype=t) for x, t in
             ((ids, np.int64), (arrival, np.int32), (prompt, np.int32), (max_tokens, np.int32))]
        check(lib().pkv_sched_add_requests(self._h, len(a[0]), *[_np_ptr(x) for x in a]))

    def schedule(self):
        n, q, mb = i32(), i32(), i32()
        check(lib().pkv_sched_schedule(self._h, C.byref(n), C.byref(q), C.byref(mb)))
        return int(n.value), int(q.value), int(mb.value)

    def plan(self, num_rows: int, total_q: int, table_width: int) -> StepPlan:
        ids = np.zeros(num_rows, np.int64)
        st = np.zeros(num_rows, np.int32)
        ql = np.zeros(num_rows, np.int32)
        sl = np.zeros(num_rows, np.int32)
        bt = np.zeros((num_rows, table_width), np.int32)
        cu = np.zeros(num_rows + 1, np.int32)
        slots = np.zeros(total_q, np.int64)
        check(lib().pkv_sched_plan(self._h, table_width, _np_ptr(ids), _np_ptr(st), _np_ptr(ql), _np_ptr(sl),
                                   _np_ptr(bt), _np_ptr(cu), _np_ptr(slots)))
        return StepPlan(self.counters()["step"], ids, st, ql, sl, bt, cu, slots)

    def update(self) -> None:
        check(lib().pkv_sched_update(self._h))

    def set_admission_check(self, enabled: bool) -> None:
        """False: admit without checking for free blocks (the Break-It sabotage); schedule()
        then raises OutOfBlocks at the step whose admission does not fit."""
        check(lib().pkv_sched_set_admission_check(self._h, int(bool(enabled))))

    def enable_prefix_cache(self, prompt_tokens=None) -> None:
        """Prefix caching on (before the first step); prompt_tokens: {id: token ids} or a
        sequence indexed like the ids added so far."""
        check(lib().pkv_sched_enable_prefix_cache(self._h))
        items = prompt_tokens.items() if isinstance(prompt_tokens, dict) else enumerate(prompt_tokens or [])
        for rid, tok in items:
            t = np.ascontiguousarray(tok, dtype=np.int32)
            check(lib().pkv_sched_set_prompt_tokens(self._h, int(rid), _np_ptr(t), len(t)))

    def set_token_budget(self, max_batched_tokens: int, chunk_tokens: int = 0) -> None:
        """Chunked prefill: at most max_batched_tokens new tokens per step, prefills cut into
        chunks of at most chunk_tokens (0: no limit); before the first step."""
        check(lib().pkv_sched_set_token_budget(self._h, int(max_batched_tokens), int(chunk_tokens)))

    VICTIMS = {"self": 0, "lifo": 1, "fewest": 2}

    def set_victim_policy(self, policy: str) -> None:
        """"self" (default), "lifo" or "fewest" (before the first step)."""
        if policy not in self.VICTIMS:
            raise ValueError(f"unknown victim policy {policy!r}")
        check(lib().pkv_sched_set_victim_policy(self._h, self.VICTIMS[policy]))

    def set_static_batching(self, enabled: bool = True) -> None:
        """Admit only when nothing runs (static batching, the baseline); before the first step."""
        check(lib().pkv_sched_set_static_batching(self._h, int(bool(enabled))))

    def set_priorities(self, ids, classes) -> None:
        """Priority classes (0 most important) of the given request ids (before the first step)."""
        i = np.ascontiguousarray(ids, dtype=np.int64)
        c = np.ascontiguousarray(classes, dtype=np.int32)
        if i.shape != c.shape:
            raise ValueError("one class per id")
        check(lib().pkv_sched_set_priorities(self._h, len(i), _np_ptr(i), _np_ptr(c)))

    def enable_swap(self, host_blocks: int) -> None:
        """Preemption by swap into a host space of host_blocks blocks (before the first step)."""
        check(lib().pkv_sched_enable_swap(self._h, int(host_blocks)))

    def swap_pairs(self):
        """(swap-outs of the last update [n][2] (device, host), swap-ins of the last schedule
        [m][2] (host, device)) as int32 arrays."""
        n, m = i32(), i32()
        check(lib().pkv_sched_swap_pairs(self._h, C.byref(n), C.byref(m), None, None))
        out = np.zeros((n.value, 2), np.int32)
        inn = np.zeros((m.value, 2), np.int32)
        check(lib().pkv_sched_swap_pairs(self._h, C.byref(n), C.byref(m), _np_ptr(out), _np_ptr(inn)))
        return out, inn

    def swap_counters(self) -> dict:
        out = np.zeros(4, np.int64)
        check(lib().pkv_sched_swap_counters(self._h, _np_ptr(out)))
        return dict(zip(("swapped_out", "blocks_out", "blocks_in", "host_free"), (int(x) for x in out)))

    def counters(self) -> dict:
        out = np.zeros(8, np.int64)
        check(lib().pkv_sched_counters(self._h, _np_ptr(out)))
        return dict(zip(self.COUNTERS, (int(x) for x in out)))


def header_functions() -> list:
    """Names of the functions declared in include/pkv.h."""
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", txt)))


def lib():
    """Load libpkv.so (once); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m paged_kv_cache_42_amd.build`")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def last_error() -> str:
    return lib().pkv_last_error().decode()


def check(status: int) -> None:
    if status != PKV_OK:
        msg = last_error()
        if status == PKV_ERR_OUT_OF_BLOCKS:
            raise OutOfBlocks(status, msg)
        raise PkvError(status, msg)


def _np_ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(vp)


# ----------------------------------------------------------------------------
# host pool
# ----------------------------------------------------------------------------

class Pool:
    """pkv_pool handle: block pool + per-sequence tables (host state)."""

    def __init__(self, num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int,
                 cache_dtype: str = "bf16", free_order: Optional[Sequence[int]] = None):
        self.block_size = int(block_size)
        self.num_blocks = int(num_blocks)
        h = vp()
        pb = i64()
        order = None if free_order is None else np.ascontiguousarray(free_order, dtype=np.int32)
        check(lib().pkv_alloc_pool(num_blocks, block_size, num_kv_heads, head_dim,
                                   DTYPE_CODES[cache_dtype], _np_ptr(order), C.byref(h), C.byref(pb)))
        self._h = h
        self.plane_bytes = int(pb.value)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.pkv_destroy_pool(h)
            self._h = None

    @property
    def handle(self):
        return self._h

    def alloc(self, n: int) -> list:
        out = np.zeros(max(n, 1), np.int32)
        check(lib().pkv_pool_alloc(self._h, n, _np_ptr(out)))
        return out[:n].tolist()

    def free(self, ids: Sequence[int]) -> None:
        a = np.ascontiguousarray(ids, dtype=np.int32)
        check(lib().pkv_pool_free(self._h, _np_ptr(a), len(a)))

    def stats(self):
        f, s = i32(), i32()
        check(lib().pkv_pool_stats(self._h, C.byref(f), C.byref(s)))
        return int(f.value), int(s.value)

    def free_list(self) -> list:
        n = i32()
        out = np.zeros(max(self.num_blocks, 1), np.int32)
        check(lib().pkv_pool_free_list(self._h, _np_ptr(out), len(out), C.byref(n)))
        return out[: n.value].tolist()

    def seq_reserve(self, seq_id: int, total_tokens: int) -> None:
        check(lib().pkv_seq_reserve(self._h, int(seq_id), int(total_tokens)))

    def seq_release(self, seq_id: int) -> None:
        check(lib().pkv_seq_release(self._h, int(seq_id)))

    def seq_share(self, seq_id: int, blocks) -> None:
        b = np.ascontiguousarray(blocks, dtype=np.int32)
        check(lib().pkv_seq_share(self._h, int(seq_id), _np_ptr(b), len(b)))

    def block_refs(self) -> np.ndarray:
        out = np.zeros(max(self.num_blocks, 1), np.int32)
        check(lib().pkv_block_refs(self._h, _np_ptr(out), len(out)))
        return out[:self.num_blocks]

    def seq_table(self, seq_id: int) -> list:
        n = i32()
        out = np.zeros(max(self.num_blocks, 1), np.int32)
        check(lib().pkv_seq_table(self._h, int(seq_id), _np_ptr(out), len(out), C.byref(n)))
        return out[: n.value].tolist()

    def build_block_table(self, seq_ids, q_lens, seq_lens, table_width: int):
        """Returns numpy (block_tables [B][W] int32, cu_seqlens_q [B+1] int32, slot_mapping int64)."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        q = np.ascontiguousarray(q_lens, dtype=np.int32)
        L = np.ascontiguousarray(seq_lens, dtype=np.int32)
        B = len(ids)
        bt = np.zeros((B, table_width), np.int32)
        cu = np.zeros(B + 1, np.int32)
        slots = np.zeros(max(int(q.sum()) if B else 0, 1), np.int64)
        check(lib().pkv_build_block_table(self._h, B, _np_ptr(ids), _np_ptr(q), _np_ptr(L), table_width,
                                          _np_ptr(bt), _np_ptr(cu), _np_ptr(slots)))
        return bt, cu, slots[: int(cu[-1])]


# ----------------------------------------------------------------------------
# device entry points (torch tensors supply memory and the stream)
# ----------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return vp(stream.cuda_stream)


def tensor_dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype in (torch.uint8, getattr(torch, "float8_e4m3fn", None)):
        return FP8
    raise ValueError(f"unsupported tensor dtype {t.dtype}")


def _require_cuda_contig(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("device tensor expected (libpkv computes on the GPU only)")
        if not t.is_contiguous():
            raise ValueError("contiguous tensor expected")


def _check_plane(k_cache, v_cache, block_size, Hkv, d):
    if k_cache.dim() != 4 or tuple(k_cache.shape[1:]) != (block_size, Hkv, d):
        raise ValueError(f"cache plane must be [num_blocks][{block_size}][{Hkv}][{d}], got {tuple(k_cache.shape)}")
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("K and V planes must have the same shape and dtype")


def _layer_stride(t, num_layers: int, what: str) -> int:
    """Byte stride between the layers of a layer-batched tensor t [L][...]: each layer
    contiguous on the device, layers apart by a non-negative stride that does not overlap."""
    if t.dim() < 2 or t.shape[0] != num_layers:
        raise ValueError(f"{what} must have a leading layer axis of {num_layers}")
    if not t.is_cuda or not t[0].is_contiguous():
        raise ValueError(f"{what}: each layer must be a contiguous device tensor")
    st = t.stride(0) if num_layers > 1 else t[0].numel()
    if st < t[0].numel():
        raise ValueError(f"{what}: layers overlap")
    return st * t.element_size()


def _layers_arg(num_layers: int, in_bytes: int = 0, out_bytes: int = 0, cache_bytes: int = 0, lse_floats: int = 0):
    return C.byref(PkvLayers(num_layers, in_bytes, out_bytes, cache_bytes, lse_floats))


def swap_workspace_bytes(n: int, num_layers: int, block_bytes: int) -> int:
    return int(lib().pkv_swap_workspace_bytes(int(n), int(num_layers), int(block_bytes)))


def _swap_args(k_cache, v_cache, pairs, host_space, workspace):
    torch = _torch()
    _require_cuda_contig(k_cache, v_cache, workspace)
    if k_cache.dim() != 5 or v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("caches must both be [layers][num_blocks][block_size][Hkv][d] of one dtype")
    if host_space.is_cuda or not host_space.is_contiguous() or not host_space.is_pinned():
        raise ValueError("host_space must be a contiguous pinned host tensor")
    pairs = np.ascontiguousarray(pairs, dtype=np.int32).reshape(-1, 2)
    L, nb = int(k_cache.shape[0]), int(k_cache.shape[1])
    block_bytes = k_cache[0, 0].numel() * k_cache.element_size()
    cap = host_space.numel() * host_space.element_size() // (L * 2 * block_bytes)
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return pairs, L, nb, block_bytes, cap, ws, torch


def swap_out(k_cache, v_cache, pairs, host_space, workspace, stream=None, copy_stream=None) -> None:
    """Copy device blocks to host blocks: pairs int32 [n][2] = (device block, host block);
    caches [layers][num_blocks][bs][Hkv][d]; host_space pinned, [host_blocks][layers][2][block]
    bytes; workspace device, >= swap_workspace_bytes(n, layers, block bytes). copy_stream:
    the DMA leg runs there (after the gather on stream); the workspace and host blocks stay
    busy until it is done."""
    pairs, L, nb, bb, cap, ws, _ = _swap_args(k_cache, v_cache, pairs, host_space, workspace)
    dev, host = np.ascontiguousarray(pairs[:, 0]), np.ascontiguousarray(pairs[:, 1])
    check(lib().pkv_swap_out(_dptr(k_cache), _dptr(v_cache), L, nb, bb, _np_ptr(dev), _np_ptr(host), len(pairs),
                             vp(host_space.data_ptr()), cap, _dptr(workspace), ws, _stream(stream),
                             None if copy_stream is None else vp(copy_stream.cuda_stream)))


def swap_in(k_cache, v_cache, pairs, host_space, workspace, stream=None) -> None:
    """Copy host blocks back: pairs int32 [n][2] = (host block, device block); layouts as
    swap_out."""
    pairs, L, nb, bb, cap, ws, _ = _swap_args(k_cache, v_cache, pairs, host_space, workspace)
    host, dev = np.ascontiguousarray(pairs[:, 0]), np.ascontiguousarray(pairs[:, 1])
    check(lib().pkv_swap_in(_dptr(k_cache), _dptr(v_cache), L, nb, bb, _np_ptr(host), _np_ptr(dev), len(pairs),
                            vp(host_space.data_ptr()), cap, _dptr(workspace), ws, _stream(stream)))


def _heads(k_head_scales, v_head_scales, num_kv_heads: int):
    """float32 arrays [num_kv_heads] (or None) of the per-head scale factors."""
    out = []
    for h in (k_head_scales, v_head_scales):
        if h is not None:
            h = np.ascontiguousarray(h, dtype=np.float32)
            if h.shape != (num_kv_heads,):
                raise ValueError(f"per-head scales must be [{num_kv_heads}]")
        out.append(h)
    return out


def _launch(fn, args, defer: bool):
    """Call fn(*args) now, or (defer) return a callable that makes the call: the checks and
    the argument marshalling are done either way, so a deferred call only crosses the ABI."""
    if defer:
        return lambda: check(fn(*args))
    check(fn(*args))
    return None


def kv_cache_write(k, v, k_cache, v_cache, slot_mapping, block_size: int, k_scale: float = 1.0,
                   v_scale: float = 1.0, stream=None, k_head_scales=None, v_head_scales=None, defer: bool = False):
    """k, v: [T][Hkv][d]; caches: [num_blocks][block_size][Hkv][d]; slot_mapping int64 [T];
    k_head_scales / v_head_scales: optional per-KV-head factors of the E4M3 scales. With a
    leading layer axis on every tensor but slot_mapping (k, v [L][T][Hkv][d], each layer
    contiguous, any layer stride; caches [L][num_blocks][...] contiguous) the L layers are
    written in one launch (pkv_kv_cache_write_layers). defer: return the checked call
    instead of making it."""
    torch = _torch()
    layers = None
    if k_cache.dim() == 5:
        NL = k_cache.shape[0]
        _require_cuda_contig(k_cache, v_cache)
        ks, vs = _layer_stride(k, NL, "k"), _layer_stride(v, NL, "v")
        if ks != vs:
            raise ValueError("k and v must have the same layer stride")
        if v_cache.shape != k_cache.shape:
            raise ValueError("K and V planes must have the same shape")
        layers = _layers_arg(NL, in_bytes=ks, cache_bytes=k_cache[0].numel() * k_cache.element_size())
        k, v, k_cache, v_cache = k[0], v[0], k_cache[0], v_cache[0]
    _require_cuda_contig(k, v, k_cache, v_cache, slot_mapping)
    if k.dim() != 3 or v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("k and v must both be [T][Hkv][d] of one dtype")
    T, Hkv, d = k.shape
    _check_plane(k_cache, v_cache, block_size, Hkv, d)
    if slot_mapping.dtype != torch.int64 or tuple(slot_mapping.shape) != (T,):
        raise ValueError("slot_mapping must be int64 [T]")
    kh, vh = _heads(k_head_scales, v_head_scales, Hkv)
    args = (_dptr(k), _dptr(v), tensor_dtype_code(k), T, Hkv, d, _dptr(k_cache), _dptr(v_cache),
            tensor_dtype_code(k_cache), k_cache.shape[0], block_size, _dptr(slot_mapping), k_scale, v_scale,
            _np_ptr(kh), _np_ptr(vh))
    if layers is None:
        return _launch(lib().pkv_kv_cache_write, (*args, _stream(stream)), defer)
    return _launch(lib().pkv_kv_cache_write_layers, (*args, layers, _stream(stream)), defer)


def decode_workspace_bytes(num_seqs: int, num_q_heads: int, head_dim: int, max_seq_len: int,
                           partition_size: int) -> int:
    return int(lib().pkv_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_seq_len, partition_size))


def build_decode_work(seq_lens, partition_size: int) -> np.ndarray:
    """Host decode work list: int32 [n][4] (seq, partition, partitions, end token)."""
    L = np.ascontiguousarray(seq_lens, dtype=np.int32)
    cap = int(sum(max(1, -(-int(x) // partition_size)) if partition_size > 0 else 1 for x in L)) or 1
    out = np.zeros((cap, 4), np.int32)
    n = i32()
    check(lib().pkv_build_decode_work(len(L), _np_ptr(L), partition_size, _np_ptr(out), cap, C.byref(n)))
    return out[: n.value]


def paged_attention_decode(out, q, k_cache, v_cache, block_tables, seq_lens, num_kv_heads: int,
                           block_size: int, max_seq_len: int, scale: float, k_scale: float = 1.0,
                           v_scale: float = 1.0, partition_size: int = 0, workspace=None, lse=None,
                           work=None, stream=None, k_head_scales=None, v_head_scales=None) -> None:
    """q/out: [B][Hq][d]; block_tables int32 [B][W]; seq_lens int32 [B]."""
    torch = _torch()
    _require_cuda_contig(out, q, k_cache, v_cache, block_tables, seq_lens, workspace, lse)
    if q.dim() != 3 or out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("q and out must both be [B][Hq][d] of one dtype")
    B, Hq, d = q.shape
    _check_plane(k_cache, v_cache, block_size, num_kv_heads, d)
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be int32 [B][W]")
    if seq_lens.dtype != torch.int32 or tuple(seq_lens.shape) != (B,):
        raise ValueError("seq_lens must be int32 [B]")
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq)):
        raise ValueError("lse must be float32 [B][Hq]")
    if work is not None:
        _require_cuda_contig(work)
        if work.dtype != torch.int32 or work.dim() != 2 or work.shape[1] != 4:
            raise ValueError("work must be int32 [n][4] (from build_decode_work)")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(lib().pkv_paged_attention_decode(
        _dptr(out), _dptr(q), tensor_dtype_code(q), _dptr(k_cache), _dptr(v_cache), tensor_dtype_code(k_cache),
        _dptr(block_tables), _dptr(seq_lens), block_tables.shape[1], B, Hq, num_kv_heads, d, block_size,
        k_cache.shape[0], max_seq_len, scale, k_scale, v_scale, *map(_np_ptr, _heads(k_head_scales, v_head_scales,
                                                                                   num_kv_heads)),
        partition_size, _dptr(workspace), ws_bytes,
        _dptr(lse), _dptr(work), 0 if work is None else work.shape[0], _stream(stream)))


class SplitPlan:
    """Host result of build_decode_split: plan (int32 numpy), slots, tiles per slot, max pieces."""

    def __init__(self, plan: np.ndarray, num_slots: int, tiles_per_slot: int, max_pieces: int):
        self.plan, self.num_slots, self.tiles_per_slot, self.max_pieces = plan, num_slots, tiles_per_slot, max_pieces


SPLIT_PIECE_COST_TOKENS = 22


def split_plan_len(num_seqs: int, num_slots: int) -> int:
    """Entries of a balanced split plan (int32)."""
    return 3 * int(num_seqs) + 2 * int(num_slots) + 2


def build_decode_split(seq_lens, num_slots: int, min_piece_tokens: int = 0,
                       piece_cost_tokens: int = SPLIT_PIECE_COST_TOKENS) -> SplitPlan:
    """Balanced split of the 16-token tiles of all sequences over num_slots workgroup slots
    (each slot's tiles plus piece_cost_tokens / 16 per piece equalised)."""
    L = np.ascontiguousarray(seq_lens, dtype=np.int32)
    cap = split_plan_len(len(L), num_slots)
    plan = np.zeros(cap, np.int32)
    c, mp = i32(), i32()
    check(lib().pkv_build_decode_split(len(L), _np_ptr(L), min_piece_tokens, piece_cost_tokens, num_slots,
                                       _np_ptr(plan), cap, C.byref(c), C.byref(mp)))
    return SplitPlan(plan, int(num_slots), c.value, mp.value)


def decode_split_slots(cache_dtype: int, num_kv_heads: int, head_dim: int, block_size: int) -> int:
    """Workgroup slots that fill the current device for the balanced-split decode kernel."""
    n = i32()
    check(lib().pkv_decode_split_slots(cache_dtype, num_kv_heads, head_dim, block_size, C.byref(n)))
    return n.value


def decode_split_workspace_bytes(num_slots: int, num_q_heads: int, head_dim: int, max_pieces: int) -> int:
    """Workspace bytes of a balanced-split launch over num_slots slots (from its SplitPlan)."""
    return int(lib().pkv_decode_split_workspace_bytes(num_slots, num_q_heads, head_dim, max_pieces))


def decode_split_workspace(split: SplitPlan, num_q_heads: int, head_dim: int, device="cuda", num_layers: int = 1):
    """A device workspace for a balanced-split launch of this plan over num_layers layers
    (None when the plan needs none)."""
    torch = _torch()
    nb = decode_split_workspace_bytes(split.num_slots, num_q_heads, head_dim, split.max_pieces) * num_layers
    return torch.empty(nb, dtype=torch.uint8, device=device) if nb else None


def paged_attention_decode_split(out, q, k_cache, v_cache, block_tables, seq_lens, plan_dev, split: SplitPlan,
                                 num_kv_heads: int, block_size: int, max_seq_len: int, scale: float,
                                 k_scale: float = 1.0, v_scale: float = 1.0, workspace=None, lse=None,
                                 rows=None, cu_seqlens_q=None, stream=None, k_head_scales=None,
                                 v_head_scales=None, defer: bool = False):
    """Balanced-split decode. Without rows / cu_seqlens_q: q/out [B][Hq][d], one plan row per
    sequence. rows (device int32 [n]): the batch sequences the plan covers; cu_seqlens_q
    (device int32 [B + 1]): q/out are [total_q][Hq][d] and a sequence's row is its last
    new token. plan_dev: device int32 copy of split.plan. With a leading layer axis on q,
    out, the caches and lse (each layer contiguous) the layers run in one launch of each
    kernel (pkv_paged_attention_decode_split_layers); the workspace then holds one
    plan's partials per layer. defer: return the checked call instead of making it."""
    layers = None
    if q.dim() == 4:
        NL = q.shape[0]
        layers, (out, q, k_cache, v_cache, lse) = _layered_attention(NL, out, q, k_cache, v_cache, lse)
    args = _split_args(out, q, k_cache, v_cache, block_tables, seq_lens, plan_dev, split, num_kv_heads, block_size,
                       max_seq_len, scale, k_scale, v_scale, workspace, lse, rows, cu_seqlens_q, k_head_scales,
                       v_head_scales)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if layers is None:
        return _launch(lib().pkv_paged_attention_decode_split,
                       (*args, _dptr(workspace), ws_bytes, _dptr(lse), _stream(stream)), defer)
    return _launch(lib().pkv_paged_attention_decode_split_layers,
                   (*args, _dptr(workspace), ws_bytes, _dptr(lse), layers, _stream(stream)), defer)


def _layered_attention(NL, out, q, k_cache, v_cache, lse):
    """The layer descriptor of a layer-batched attention call and its layer-0 views."""
    if k_cache.dim() != 5 or v_cache.shape != k_cache.shape or k_cache.shape[0] != NL:
        raise ValueError(f"layer-batched caches must be [{NL}][num_blocks][block_size][Hkv][d]")
    _require_cuda_contig(k_cache, v_cache)
    lse_floats = 0
    if lse is not None:
        lse_floats = _layer_stride(lse, NL, "lse") // 4
    layers = _layers_arg(NL, in_bytes=_layer_stride(q, NL, "q"), out_bytes=_layer_stride(out, NL, "out"),
                         cache_bytes=k_cache[0].numel() * k_cache.element_size(), lse_floats=lse_floats)
    return layers, (out[0], q[0], k_cache[0], v_cache[0], None if lse is None else lse[0])


def decode_split_noalloc_max_bytes() -> int:
    """Size of the library's per-device partials array used by paged_attention_decode_split_noalloc."""
    return int(lib().pkv_decode_split_noalloc_max_bytes())


def paged_attention_decode_split_noalloc(out, q, k_cache, v_cache, block_tables, seq_lens, plan_dev,
                                         split: SplitPlan, num_kv_heads: int, block_size: int, max_seq_len: int,
                                         scale: float, k_scale: float = 1.0, v_scale: float = 1.0, lse=None,
                                         rows=None, cu_seqlens_q=None, stream=None, k_head_scales=None,
                                         v_head_scales=None) -> None:
    """paged_attention_decode_split without a workspace: the partials go to the library's
    per-device array (calls on one device must not overlap)."""
    args = _split_args(out, q, k_cache, v_cache, block_tables, seq_lens, plan_dev, split, num_kv_heads, block_size,
                       max_seq_len, scale, k_scale, v_scale, None, lse, rows, cu_seqlens_q, k_head_scales,
                       v_head_scales)
    check(lib().pkv_paged_attention_decode_split_noalloc(*args, _dptr(lse), _stream(stream)))


def _split_args(out, q, k_cache, v_cache, block_tables, seq_lens, plan_dev, split, num_kv_heads, block_size,
                max_seq_len, scale, k_scale, v_scale, workspace, lse, rows, cu_seqlens_q, k_head_scales,
                v_head_scales):
    """Checks and the leading arguments (out .. max_pieces) of the balanced-split calls."""
    torch = _torch()
    _require_cuda_contig(out, q, k_cache, v_cache, block_tables, seq_lens, plan_dev, workspace, lse, rows,
                         cu_seqlens_q)
    if q.dim() != 3 or out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("q and out must both be [rows][Hq][d] of one dtype")
    T, Hq, d = q.shape
    B = seq_lens.shape[0] if seq_lens.dim() == 1 else -1
    _check_plane(k_cache, v_cache, block_size, num_kv_heads, d)
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be int32 [B][W]")
    if seq_lens.dtype != torch.int32 or B < 0:
        raise ValueError("seq_lens must be int32 [B]")
    n = B if rows is None else rows.shape[0]
    if rows is not None and (rows.dtype != torch.int32 or rows.dim() != 1):
        raise ValueError("rows must be int32 [n]")
    if cu_seqlens_q is None and T != B:
        raise ValueError("q must be [B][Hq][d] without cu_seqlens_q")
    if cu_seqlens_q is not None and (cu_seqlens_q.dtype != torch.int32 or tuple(cu_seqlens_q.shape) != (B + 1,)):
        raise ValueError("cu_seqlens_q must be int32 [B + 1]")
    if plan_dev.dtype != torch.int32 or tuple(plan_dev.shape) != (split_plan_len(n, split.num_slots),):
        raise ValueError("plan must be int32 [3 rows + 2 num_slots + 2] (from build_decode_split)")
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (T, Hq)):
        raise ValueError("lse must be float32 [rows][Hq]")
    return (_dptr(out), _dptr(q), tensor_dtype_code(q), _dptr(k_cache), _dptr(v_cache), tensor_dtype_code(k_cache),
            _dptr(block_tables), _dptr(seq_lens), block_tables.shape[1], B, Hq, num_kv_heads, d, block_size,
            k_cache.shape[0], max_seq_len, scale, k_scale, v_scale,
            *map(_np_ptr, _heads(k_head_scales, v_head_scales, num_kv_heads)), _dptr(rows), n,
            _dptr(cu_seqlens_q), T, _dptr(plan_dev), split.num_slots, split.tiles_per_slot, split.max_pieces)


def decode_set_profile_event(event) -> None:
    """Record torch.cuda.Event `event` after the decode partition pass (None: off)."""
    if event is None:
        lib().pkv_decode_set_profile_event(None)
        return
    lib().pkv_decode_set_profile_event(vp(event.cuda_event))


def build_varlen_work(q_lens, seq_lens, num_kv_heads: int, group: int) -> np.ndarray:
    """Host varlen work list: int32 [n][4] (seq, kind<<24 | head or group, first token, keys)."""
    q = np.ascontiguousarray(q_lens, dtype=np.int32)
    L = np.ascontiguousarray(seq_lens, dtype=np.int32)
    qb = max(1, 128 // max(group, 1))
    cap = int(sum((-(-int(x) // qb)) * num_kv_heads if x > 1 else (num_kv_heads if x == 1 else 0)
                  for x in q)) or 1
    out = np.zeros((cap, 4), np.int32)
    n = i32()
    check(lib().pkv_build_varlen_work(len(q), _np_ptr(q), _np_ptr(L), num_kv_heads, group, _np_ptr(out), cap,
                                      C.byref(n)))
    return out[: n.value]


class ChunkPlan:
    """Host result of build_chunk_work: items int32 [n][8], merges int32 [m][4], workspace slots."""

    def __init__(self, items: np.ndarray, merges: np.ndarray, num_partials: int):
        self.items, self.merges, self.num_partials = items, merges, num_partials

    def to_device(self, head_dim: int, device="cuda", num_layers: int = 1):
        """(work, merges or None, workspace or None) as device tensors for
        paged_attention_prefill_chunks (the workspace sized for num_layers layers); None
        when there are no items."""
        torch = _torch()
        if len(self.items) == 0:
            return None
        work = torch.from_numpy(self.items).to(device)
        merges = torch.from_numpy(self.merges).to(device) if len(self.merges) else None
        nb = chunk_workspace_bytes(self.num_partials, head_dim) * num_layers
        ws = torch.empty(nb, dtype=torch.uint8, device=device) if nb else None
        return work, merges, ws


def build_chunk_work(q_lens, seq_lens, num_kv_heads: int, group: int, num_slots: int = 0,
                     min_piece_tiles: int = 0) -> ChunkPlan:
    """Row blocks of the sequences with two or more new tokens; blocks longer than the
    even share of num_slots are cut along the keys (num_slots <= 0: never)."""
    q = np.ascontiguousarray(q_lens, dtype=np.int32)
    L = np.ascontiguousarray(seq_lens, dtype=np.int32)
    n, m, p = i32(), i32(), i32()
    cap, mcap = 64, 16
    while True:
        items = np.zeros((cap, 8), np.int32)
        merges = np.zeros((mcap, 4), np.int32)
        st = lib().pkv_build_chunk_work(len(q), _np_ptr(q), _np_ptr(L), num_kv_heads, group, num_slots,
                                        min_piece_tiles, _np_ptr(items), cap, C.byref(n), _np_ptr(merges), mcap,
                                        C.byref(m), C.byref(p))
        if st == PKV_OK:
            return ChunkPlan(items[:n.value].copy(), merges[:m.value].copy(), p.value)
        if st != PKV_ERR_INVALID or (n.value <= cap and m.value <= mcap):
            check(st)
        cap, mcap = max(cap, n.value), max(mcap, m.value)


def chunk_slots(cache_dtype: int, head_dim: int, block_size: int) -> int:
    """Chunk-kernel workgroups resident on the current device at once."""
    out = i32()
    check(lib().pkv_chunk_slots(cache_dtype, head_dim, block_size, C.byref(out)))
    return out.value


def chunk_workspace_bytes(num_partials: int, head_dim: int) -> int:
    return int(lib().pkv_chunk_workspace_bytes(num_partials, head_dim))


class MixedPlan:
    """Host plan of a mixed step: decode rows (batch indices) with their balanced split
    plan, and the chunk work of the other rows."""

    def __init__(self, decode_rows, split, chunks):
        self.decode_rows, self.split, self.chunks = decode_rows, split, chunks

    def to_device(self, head_dim: int, num_q_heads: int, device="cuda", num_layers: int = 1):
        """The device arrays of paged_attention_mixed: (rows, split plan, split workspace)
        (None when there is no decode row) and ChunkPlan.to_device (None when no chunk),
        workspaces sized for num_layers layers."""
        torch = _torch()
        dec = None
        if self.split is not None:
            dec = (torch.from_numpy(self.decode_rows).to(device), torch.from_numpy(self.split.plan).to(device),
                   decode_split_workspace(self.split, num_q_heads, head_dim, device, num_layers))
        return dec, self.chunks.to_device(head_dim, device, num_layers)


def build_mixed_step(q_lens, seq_lens, num_kv_heads: int, group: int, num_slots: int,
                     min_piece_tokens: int = 0, chunk_slots: int = 0, min_piece_tiles: int = 0,
                     piece_cost_tokens: int = SPLIT_PIECE_COST_TOKENS) -> MixedPlan:
    """libpkv's mixed-step plan: sequences with exactly one new token go to a balanced
    split plan over num_slots (rows in batch order), those with more to the chunk work list
    (cut along the keys over chunk_slots resident workgroups, 0: uncut)."""
    q = np.ascontiguousarray(q_lens, dtype=np.int32)
    L = np.ascontiguousarray(seq_lens, dtype=np.int32)
    B = len(q)
    dec = np.zeros(max(B, 1), np.int32)
    plan = np.zeros(split_plan_len(B, num_slots), np.int32)
    nd, c, mp = i32(), i32(), i32()
    n, m, p = i32(), i32(), i32()
    cap, mcap = 64, 16
    while True:
        items = np.zeros((cap, 8), np.int32)
        merges = np.zeros((mcap, 4), np.int32)
        st = lib().pkv_build_mixed_step(B, _np_ptr(q), _np_ptr(L), num_kv_heads, group, num_slots, min_piece_tokens,
                                        piece_cost_tokens, chunk_slots, min_piece_tiles, _np_ptr(dec), C.byref(nd),
                                        _np_ptr(plan), len(plan), C.byref(c), C.byref(mp), _np_ptr(items), cap,
                                        C.byref(n), _np_ptr(merges), mcap, C.byref(m), C.byref(p))
        if st == PKV_OK:
            break
        if st != PKV_ERR_INVALID or (n.value <= cap and m.value <= mcap):
            check(st)
        cap, mcap = max(cap, n.value), max(mcap, m.value)
    k = nd.value
    split = SplitPlan(plan[:split_plan_len(k, num_slots)].copy(), int(num_slots), c.value, mp.value) if k else None
    chunks = ChunkPlan(items[:n.value].copy(), merges[:m.value].copy(), p.value)
    return MixedPlan(dec[:k].copy(), split, chunks)


def mixed_decode_slots(q_lens, seq_lens, cache_dtype: int, num_kv_heads: int, group: int, head_dim: int,
                       block_size: int, num_layers: int = 1) -> int:
    """Decode slots per layer for paged_attention_mixed's one launch: the slots that let
    the decode rows finish with the chunk items running beside them (the layers' share of
    the device when the step has one kind of row only, or when the shape runs as two
    launches)."""
    q = np.ascontiguousarray(q_lens, dtype=np.int32)
    L = np.ascontiguousarray(seq_lens, dtype=np.int32)
    n = i32()
    check(lib().pkv_mixed_decode_slots(len(q), _np_ptr(q), _np_ptr(L), cache_dtype, num_kv_heads, group, head_dim,
                                       block_size, num_layers, C.byref(n)))
    return n.value


def paged_attention_mixed(out, q, k_cache, v_cache, block_tables, seq_lens, cu_seqlens_q, plan: MixedPlan, dev,
                          num_kv_heads: int, block_size: int, max_seq_len: int, scale: float, k_scale: float = 1.0,
                          v_scale: float = 1.0, lse=None, stream=None, k_head_scales=None, v_head_scales=None,
                          defer: bool = False):
    """The attention of a mixed step (decode rows and prefill chunks) as one launch plus
    the merges. plan: build_mixed_step's result (for one launch, over mixed_decode_slots
    decode slots); dev: plan.to_device(head_dim, num_q_heads); q/out [total_q][Hq][d],
    cu_seqlens_q int32 [B + 1]; the rest as for paged_attention_prefill_chunks. With a
    leading layer axis on q, out, the caches and lse (each layer contiguous) the layers run
    in the same launch (pkv_paged_attention_mixed_layers; dev from
    plan.to_device(..., num_layers=NL))."""
    torch = _torch()
    ddev, cdev = dev
    layers = None
    if q.dim() == 4:
        layers, (out, q, k_cache, v_cache, lse) = _layered_attention(q.shape[0], out, q, k_cache, v_cache, lse)
    _require_cuda_contig(out, q, k_cache, v_cache, block_tables, seq_lens, cu_seqlens_q, lse)
    if q.dim() != 3 or out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("q and out must both be [total_q][Hq][d] of one dtype")
    T, Hq, d = q.shape
    _check_plane(k_cache, v_cache, block_size, num_kv_heads, d)
    B = seq_lens.shape[0]
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be int32 [B][W]")
    if seq_lens.dtype != torch.int32 or cu_seqlens_q.dtype != torch.int32 or tuple(cu_seqlens_q.shape) != (B + 1,):
        raise ValueError("seq_lens int32 [B] and cu_seqlens_q int32 [B+1] expected")
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (T, Hq)):
        raise ValueError("lse must be float32 [total_q][Hq]")
    rows = plan_d = sws = None
    n_rows, slots, tps, mp, sws_bytes = 0, 1, 0, 0, 0
    if ddev is not None:
        rows, plan_d, sws = ddev
        _require_cuda_contig(rows, plan_d, sws)
        if rows.dtype != torch.int32 or plan_d.dtype != torch.int32 or \
                tuple(plan_d.shape) != (split_plan_len(rows.shape[0], plan.split.num_slots),):
            raise ValueError("decode rows / split plan do not match the mixed plan")
        n_rows, slots, tps, mp = rows.shape[0], plan.split.num_slots, plan.split.tiles_per_slot, plan.split.max_pieces
        sws_bytes = 0 if sws is None else sws.numel() * sws.element_size()
    work = merges = cws = None
    n_work = n_merges = 0
    if cdev is not None:
        work, merges, cws = cdev
        _require_cuda_contig(work, merges, cws)
        if work.dtype != torch.int32 or work.dim() != 2 or work.shape[1] != 8:
            raise ValueError("work must be int32 [n][8] (from build_mixed_step)")
        n_work = work.shape[0]
        n_merges = 0 if merges is None else merges.shape[0]
    cws_bytes = 0 if cws is None else cws.numel() * cws.element_size()
    args = (_dptr(out), _dptr(q), tensor_dtype_code(q), _dptr(k_cache), _dptr(v_cache), tensor_dtype_code(k_cache),
            _dptr(block_tables), _dptr(seq_lens), _dptr(cu_seqlens_q), block_tables.shape[1], B, T, Hq, num_kv_heads,
            d, block_size, k_cache.shape[0], max_seq_len, scale, k_scale, v_scale,
            *map(_np_ptr, _heads(k_head_scales, v_head_scales, num_kv_heads)), _dptr(rows), n_rows, _dptr(plan_d),
            slots, tps, mp, _dptr(sws), sws_bytes, _dptr(work), n_work, _dptr(merges), n_merges,
            plan.chunks.num_partials, _dptr(cws), cws_bytes, _dptr(lse))
    if layers is None:
        return _launch(lib().pkv_paged_attention_mixed, (*args, _stream(stream)), defer)
    return _launch(lib().pkv_paged_attention_mixed_layers, (*args, layers, _stream(stream)), defer)


def paged_attention_prefill_varlen(out, q, k_cache, v_cache, block_tables, seq_lens, cu_seqlens_q, work,
                                   num_kv_heads: int, block_size: int, max_seq_len: int, scale: float,
                                   k_scale: float = 1.0, v_scale: float = 1.0, lse=None, stream=None,
                                   k_head_scales=None, v_head_scales=None) -> None:
    """q/out: [total_q][Hq][d] bf16; cu_seqlens_q int32 [B+1]; work int32 [n][4] (device)."""
    torch = _torch()
    _require_cuda_contig(out, q, k_cache, v_cache, block_tables, seq_lens, cu_seqlens_q, work, lse)
    if q.dim() != 3 or out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("q and out must both be [total_q][Hq][d] of one dtype")
    T, Hq, d = q.shape
    _check_plane(k_cache, v_cache, block_size, num_kv_heads, d)
    B = seq_lens.shape[0]
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be int32 [B][W]")
    if seq_lens.dtype != torch.int32 or cu_seqlens_q.dtype != torch.int32 or tuple(cu_seqlens_q.shape) != (B + 1,):
        raise ValueError("seq_lens int32 [B] and cu_seqlens_q int32 [B+1] expected")
    if work.dtype != torch.int32 or work.dim() != 2 or work.shape[1] != 4:
        raise ValueError("work must be int32 [n][4] (from build_varlen_work)")
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (T, Hq)):
        raise ValueError("lse must be float32 [total_q][Hq]")
    check(lib().pkv_paged_attention_prefill_varlen(
        _dptr(out), _dptr(q), tensor_dtype_code(q), _dptr(k_cache), _dptr(v_cache), tensor_dtype_code(k_cache),
        _dptr(block_tables), _dptr(seq_lens), _dptr(cu_seqlens_q), block_tables.shape[1], B, T, Hq, num_kv_heads, d,
        block_size, k_cache.shape[0], max_seq_len, scale, k_scale, v_scale,
        *map(_np_ptr, _heads(k_head_scales, v_head_scales, num_kv_heads)), _dptr(work), work.shape[0], _dptr(lse),
        _stream(stream)))


def paged_attention_prefill_chunks(out, q, k_cache, v_cache, block_tables, seq_lens, cu_seqlens_q, work,
                                   merges, num_partials: int, workspace, num_kv_heads: int, block_size: int,
                                   max_seq_len: int, scale: float, k_scale: float = 1.0, v_scale: float = 1.0,
                                   lse=None, stream=None, k_head_scales=None, v_head_scales=None,
                                   defer: bool = False):
    """Rows of the sequences with two or more new tokens. work: device int32 [n][8] and
    merges: device int32 [m][4] (or None) from build_chunk_work, num_partials its slots,
    workspace: device tensor of at least chunk_workspace_bytes (None when no slots); the
    rest as for paged_attention_prefill_varlen. With a leading layer axis on q, out, the
    caches and lse (each layer contiguous) the layers run in one launch of each kernel
    (pkv_paged_attention_prefill_chunks_layers); the workspace then holds the partials of
    every layer. defer: return the checked call instead of making it."""
    torch = _torch()
    layers = None
    if q.dim() == 4:
        layers, (out, q, k_cache, v_cache, lse) = _layered_attention(q.shape[0], out, q, k_cache, v_cache, lse)
    _require_cuda_contig(out, q, k_cache, v_cache, block_tables, seq_lens, cu_seqlens_q, work, merges, workspace, lse)
    if q.dim() != 3 or out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("q and out must both be [total_q][Hq][d] of one dtype")
    T, Hq, d = q.shape
    _check_plane(k_cache, v_cache, block_size, num_kv_heads, d)
    B = seq_lens.shape[0]
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be int32 [B][W]")
    if seq_lens.dtype != torch.int32 or cu_seqlens_q.dtype != torch.int32 or tuple(cu_seqlens_q.shape) != (B + 1,):
        raise ValueError("seq_lens int32 [B] and cu_seqlens_q int32 [B+1] expected")
    if work.dtype != torch.int32 or work.dim() != 2 or work.shape[1] != 8:
        raise ValueError("work must be int32 [n][8] (from build_chunk_work)")
    nm = 0
    if merges is not None:
        if merges.dtype != torch.int32 or merges.dim() != 2 or merges.shape[1] != 4:
            raise ValueError("merges must be int32 [m][4] (from build_chunk_work)")
        nm = merges.shape[0]
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (T, Hq)):
        raise ValueError("lse must be float32 [total_q][Hq]")
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = (_dptr(out), _dptr(q), tensor_dtype_code(q), _dptr(k_cache), _dptr(v_cache), tensor_dtype_code(k_cache),
            _dptr(block_tables), _dptr(seq_lens), _dptr(cu_seqlens_q), block_tables.shape[1], B, T, Hq, num_kv_heads,
            d, block_size, k_cache.shape[0], max_seq_len, scale, k_scale, v_scale,
            *map(_np_ptr, _heads(k_head_scales, v_head_scales, num_kv_heads)), _dptr(work), work.shape[0],
            _dptr(merges), nm, num_partials, _dptr(workspace), wsb, _dptr(lse))
    if layers is None:
        return _launch(lib().pkv_paged_attention_prefill_chunks, (*args, _stream(stream)), defer)
    return _launch(lib().pkv_paged_attention_prefill_chunks_layers, (*args, layers, _stream(stream)), defer)
