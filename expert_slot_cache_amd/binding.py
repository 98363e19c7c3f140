"""ctypes binding of libmoe_pool.so (the C ABI declared in include/moe_pool.h).

Argument marshalling only: every step of the path runs in the library.  Torch
tensors are accepted for convenience and passed as raw device pointers; the
compute stream is a hipStream_t (torch's current stream by default).  The
library must have been built (``python -m expert_slot_cache_amd.build``); a
missing library raises, there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_pool.so")

OK, EINVAL, ENOMEM, EHIP, ERANGE, ESTATE = 0, -1, -2, -3, -4, -5
W_F32, W_BF16, W_INT4_G128 = 0, 1, 2
A_F32, A_BF16 = 0, 1
RULE_DISTINCT, RULE_STATIC = 0, 1
COPY_KERNEL, COPY_DMA = 0, 1
PATH_POOL, PATH_FALLBACK = 0, 1

WTYPES = {"f32": W_F32, "bf16": W_BF16, "int4": W_INT4_G128}
ATYPES = {"f32": A_F32, "bf16": A_BF16}
RULES = {"distinct": RULE_DISTINCT, "static": RULE_STATIC}
COPY_ENGINES = {"dma": COPY_DMA, "kernel": COPY_KERNEL}
POLICY_HOST, POLICY_DEVICE = 0, 1
POLICIES = {"host": POLICY_HOST, "device": POLICY_DEVICE}
EVICT_LRU, EVICT_FIFO, EVICT_LFU, EVICT_SLRU, EVICT_DECAY = 0, 1, 2, 3, 4
EVICTS = {"lru": EVICT_LRU, "fifo": EVICT_FIFO, "lfu": EVICT_LFU, "slru": EVICT_SLRU, "decay": EVICT_DECAY}
PREFETCH_AFTER = {"layer": 0, "queued": 1, "previous": 2}


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[{status}] {msg}")
        self.status = status


class ExpertRangeError(MoeError):
    pass


class StateError(MoeError):
    pass


class Config(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("n_experts", C.c_int32), ("top_k", C.c_int32),
                ("hidden", C.c_int32), ("inter", C.c_int32), ("n_slots", C.c_int32),
                ("wtype", C.c_int32), ("atype", C.c_int32), ("rule", C.c_int32),
                ("resident", C.c_int32), ("max_tokens", C.c_int32), ("n_copy_streams", C.c_int32),
                ("copy_chunk_bytes", C.c_size_t), ("hbm_budget_bytes", C.c_size_t),
                ("timing", C.c_int32), ("copy_engine", C.c_int32), ("policy", C.c_int32),
                ("read_through", C.c_int32), ("evict", C.c_int32), ("prefetch_slots", C.c_int32)]


class Miss(C.Structure):
    _fields_ = [("expert", C.c_int32), ("slot", C.c_int32), ("evicted", C.c_int32)]


class Stats(C.Structure):
    _fields_ = [("steps", C.c_uint64), ("hits", C.c_uint64), ("misses", C.c_uint64),
                ("fallbacks", C.c_uint64), ("bytes_h2d", C.c_uint64), ("staged", C.c_uint64),
                ("prefetched", C.c_uint64), ("prefetch_bytes", C.c_uint64), ("moves", C.c_uint64)]


class Timing(C.Structure):
    _fields_ = [("copy_ms", C.c_double), ("copy_calls", C.c_uint64), ("copy_bytes", C.c_uint64),
                ("w13_ms", C.c_double), ("w2_ms", C.c_double), ("kernel_calls", C.c_uint64),
                ("sync_wait_ms", C.c_double)]


_P = C.c_void_p
_I32 = C.c_int32
_PI32 = C.POINTER(C.c_int32)

_SIGS = {
    "moe_strerror": (C.c_char_p, [_I32]),
    "moe_last_error": (C.c_char_p, []),
    "moe_expert_bytes": (C.c_size_t, [_I32, _I32, _I32]),
    "moe_pool_create": (_I32, [C.POINTER(Config), _P, C.POINTER(_P)]),
    "moe_pool_destroy": (None, [_P]),
    "moe_pool_load_expert": (_I32, [_P, _I32, _I32, _P, C.c_size_t]),
    "moe_pool_reset": (_I32, [_P]),
    "moe_pool_prepare": (_I32, [_P, _I32, _P, _I32, _P, C.POINTER(Miss), _I32, _PI32, _PI32]),
    "moe_pool_forward": (_I32, [_P, _I32, _P, _P, _P, _P, _I32, _P]),
    "moe_pool_step": (_I32, [_P, _I32, _P, _I32, _P, _P, _P, _P, _P, C.POINTER(Miss), _I32, _PI32,
                             _PI32]),
    "moe_pool_sync": (_I32, [_P]),
    "moe_pool_prefetch": (_I32, [_P, _I32, _P, _I32, _I32]),
    "moe_pool_last_step": (_I32, [_P, _I32, _PI32, C.POINTER(Miss), _I32, _PI32]),
    "moe_pool_get_stats": (_I32, [_P, _I32, C.POINTER(Stats)]),
    "moe_pool_get_state": (_I32, [_P, _I32, _P, _P, _P]),
    "moe_pool_read_slot": (_I32, [_P, _I32, _I32, _P, C.c_size_t]),
    "moe_pool_slot_ptr": (_I32, [_P, _I32, _I32, C.POINTER(_P)]),
    "moe_pool_store_ptr": (_I32, [_P, _I32, _I32, C.POINTER(_P)]),
    "moe_ptr_is_pinned_host": (_I32, [_P, _PI32]),
    "moe_pool_get_timing": (_I32, [_P, C.POINTER(Timing)]),
    "moe_pool_reset_timing": (_I32, [_P]),
    "moe_pool_set_timing": (_I32, [_P, _I32]),
    "moe_read_calibration": (_I32, [_P, C.c_size_t, C.c_size_t, _I32, _P, C.POINTER(C.c_double)]),
    "moe_link_calibration": (_I32, [C.c_size_t, _I32, _I32, _I32, _P, C.POINTER(C.c_double)]),
    "moe_pool_set_slots": (_I32, [_P, _I32]),
    "moe_pool_set_eviction": (_I32, [_P, _I32]),
    "moe_forward_slots": (_I32, [_I32, _I32, _I32, _I32, _I32, _P, _I32, _P, _P, _P, _P, _I32, _P, _P]),
    "moe_lru_create": (_I32, [_I32, _I32, _I32, C.POINTER(_P)]),
    "moe_lru_destroy": (None, [_P]),
    "moe_lru_step": (_I32, [_P, _P, _I32, _I32, _P, C.POINTER(Miss), _I32, _PI32, _PI32]),
    "moe_lru_get_state": (_I32, [_P, _P, _P, _P]),
    "moe_lru_get_stats": (_I32, [_P, C.POINTER(Stats)]),
}

_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m expert_slot_cache_amd.build`")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def exported_symbols():
    return sorted(_SIGS)


def _check(status: int):
    if status == OK:
        return
    msg = lib().moe_last_error().decode(errors="replace")
    if status == ERANGE:
        raise ExpertRangeError(status, msg)
    if status == ESTATE:
        raise StateError(status, msg)
    raise MoeError(status, msg)


def forward_slots(*, wtype: str, atype: str, hidden: int, inter: int, top_k: int, slots, n_slots: int,
                  slot_ids, x, topk_w, out, n_tokens: int, resid=None, stream=None):
    """moe_forward_slots: the fused MoE over caller-held slots, scratch in the library's
    static device array (no allocation)."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    _check(lib().moe_forward_slots(WTYPES[wtype], ATYPES[atype], hidden, inter, top_k, _ptr(slots), n_slots,
                                   _ptr(slot_ids), _ptr(x), _ptr(topk_w), _ptr(resid), n_tokens, _ptr(out),
                                   C.c_void_p(stream)))


def expert_bytes(wtype: str, hidden: int, inter: int) -> int:
    return int(lib().moe_expert_bytes(WTYPES[wtype], hidden, inter))


def _ptr(t) -> int:
    """Device/host address of a torch tensor, a numpy array, or an int."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _misses(buf, n):
    return [(buf[i].expert, buf[i].slot, buf[i].evicted) for i in range(n)]


class MoePool:
    """One pool object: n_layers layers of n_slots HBM slots over a pinned store."""

    def __init__(self, *, layers: int, experts: int, top_k: int, hidden: int, inter: int,
                 slots: int, wtype: str = "bf16", atype: str = "bf16", rule: str = "distinct",
                 resident: bool = False, max_tokens: int = 1, copy_streams: int = 1,
                 copy_chunk_bytes: int = 0, hbm_budget_bytes: int = 0, timing: int = 0,
                 copy_engine: str = "kernel", policy: str = "host", read_through: bool = False,
                 evict: str = "lru", prefetch_slots: int = 0, stream=None):
        self._h = None
        cfg = Config(layers, experts, top_k, hidden, inter, slots, WTYPES[wtype], ATYPES[atype],
                     RULES[rule], int(bool(resident)), max_tokens, copy_streams,
                     copy_chunk_bytes, hbm_budget_bytes, int(timing), COPY_ENGINES[copy_engine],
                     POLICIES[policy], int(bool(read_through)), EVICTS[evict], int(prefetch_slots))
        if stream is None:
            import torch
            stream = torch.cuda.current_stream().cuda_stream
        h = C.c_void_p()
        _check(lib().moe_pool_create(C.byref(cfg), C.c_void_p(stream), C.byref(h)))
        self._h = h
        self.cfg = cfg
        self.layers, self.experts, self.top_k = layers, experts, top_k
        self.hidden, self.inter, self.slots = hidden, inter, slots
        self.wtype, self.atype, self.resident = wtype, atype, resident
        self.policy = policy
        self.evict = evict
        self.read_through = bool(read_through)
        self.max_tokens = max_tokens
        self.expert_nbytes = expert_bytes(wtype, hidden, inter)
        self._miss_buf = (Miss * max(1, experts))()

    # -- lifetime ----------------------------------------------------------------
    def close(self):
        if self._h is not None and self._h.value:
            lib().moe_pool_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *a):
        self.close()

    # -- store -------------------------------------------------------------------
    def load_expert(self, layer: int, expert: int, data: np.ndarray):
        b = np.ascontiguousarray(data).view(np.uint8).ravel()
        _check(lib().moe_pool_load_expert(self._h, layer, expert, b.ctypes.data, b.size))

    def reset(self):
        _check(lib().moe_pool_reset(self._h))

    def set_slots(self, n_slots: int):
        """Slots per layer from now on (<= the count at create); the pool goes cold."""
        _check(lib().moe_pool_set_slots(self._h, n_slots))
        self.slots = n_slots

    def set_eviction(self, evict: str):
        """Eviction policy from now on ("lru", "fifo", "lfu", "slru", "decay"); the pool
        goes cold."""
        _check(lib().moe_pool_set_eviction(self._h, EVICTS[evict]))
        self.evict = evict

    # -- the step ------------------------------------------------------------------
    def prepare(self, layer: int, topk_ids, n_tokens: int, slot_ids):
        """topk_ids/slot_ids: int32 [n_tokens, top_k] on the device (tensor or address).
        Returns (path, misses) with misses a list of (expert, slot, evicted)."""
        nm, path = C.c_int32(0), C.c_int32(0)
        _check(lib().moe_pool_prepare(self._h, layer, _ptr(topk_ids), n_tokens, _ptr(slot_ids),
                                      self._miss_buf, len(self._miss_buf), C.byref(nm),
                                      C.byref(path)))
        return path.value, _misses(self._miss_buf, min(nm.value, len(self._miss_buf)))

    def prepare_raw(self, layer: int, ids_ptr: int, n_tokens: int, slot_ptr: int) -> int:
        """prepare() without building the miss list; returns the path."""
        path = C.c_int32(0)
        _check(lib().moe_pool_prepare(self._h, layer, ids_ptr, n_tokens, slot_ptr, None, 0, None,
                                      C.byref(path)))
        return path.value

    def forward(self, layer: int, x, slot_ids, topk_w, out, n_tokens: int, resid=None):
        _check(lib().moe_pool_forward(self._h, layer, _ptr(x), _ptr(slot_ids), _ptr(topk_w),
                                      _ptr(resid), n_tokens, _ptr(out)))
        return out

    def step(self, layer: int, topk_ids, n_tokens: int, slot_ids, x, topk_w, out, resid=None):
        """prepare + forward in one call; returns (path, misses)."""
        nm, path = C.c_int32(0), C.c_int32(0)
        _check(lib().moe_pool_step(self._h, layer, _ptr(topk_ids), n_tokens, _ptr(slot_ids), _ptr(x),
                                   _ptr(topk_w), _ptr(resid), _ptr(out), self._miss_buf,
                                   len(self._miss_buf), C.byref(nm), C.byref(path)))
        return path.value, _misses(self._miss_buf, min(nm.value, len(self._miss_buf)))

    def sync(self):
        _check(lib().moe_pool_sync(self._h))

    def prefetch(self, layer: int, predicted_ids, n_tokens: int, after: str = "queued"):
        """Hint: the next step of `layer` will use these ids (int32 [n_tokens, top_k] on
        the device); predicted experts the layer does not hold are copied into its
        prefetch buffer on a copy stream, starting after everything queued on the compute
        stream ("queued"), after the layer's last step ("layer") or after the previous
        prefetch ("previous")."""
        _check(lib().moe_pool_prefetch(self._h, layer, _ptr(predicted_ids), n_tokens, PREFETCH_AFTER[after]))

    def last_step(self, layer: int):
        """(path, misses) of the layer's last prepare/step (waits for it under the
        device policy)."""
        nm, path = C.c_int32(0), C.c_int32(0)
        _check(lib().moe_pool_last_step(self._h, layer, C.byref(path), self._miss_buf, len(self._miss_buf),
                                        C.byref(nm)))
        return path.value, _misses(self._miss_buf, min(nm.value, len(self._miss_buf)))

    # -- introspection ---------------------------------------------------------------
    def stats(self, layer: int = -1) -> dict:
        s = Stats()
        _check(lib().moe_pool_get_stats(self._h, layer, C.byref(s)))
        return {f: int(getattr(s, f)) for f, _ in Stats._fields_}

    def state(self, layer: int):
        m = np.empty(self.experts, np.int32)
        n = max(1, self.slots)
        o = np.empty(n, np.int32)
        l = np.empty(n, np.int32)
        _check(lib().moe_pool_get_state(self._h, layer, m.ctypes.data, o.ctypes.data, l.ctypes.data))
        k = self.slots if not self.resident else 0
        return m, o[:k], l[:k]

    def read_slot(self, layer: int, slot: int, n: int | None = None) -> np.ndarray:
        n = self.expert_nbytes if n is None else n
        buf = np.empty(n, np.uint8)
        _check(lib().moe_pool_read_slot(self._h, layer, slot, buf.ctypes.data, n))
        return buf

    def read_staging(self, rank: int, n: int | None = None) -> np.ndarray:
        return self.read_slot(0, -rank - 1, n)

    def slot_ptr(self, layer: int, slot: int) -> int:
        p = C.c_void_p()
        _check(lib().moe_pool_slot_ptr(self._h, layer, slot, C.byref(p)))
        return p.value

    def store_ptr(self, layer: int, expert: int) -> int:
        p = C.c_void_p()
        _check(lib().moe_pool_store_ptr(self._h, layer, expert, C.byref(p)))
        return p.value

    def store_view(self, layer: int, expert: int) -> np.ndarray:
        """numpy view of an expert's bytes in the pinned store (for bulk filling)."""
        addr = self.store_ptr(layer, expert)
        buf = (C.c_uint8 * self.expert_nbytes).from_address(addr)
        return np.frombuffer(buf, dtype=np.uint8)

    def timing(self) -> dict:
        t = Timing()
        _check(lib().moe_pool_get_timing(self._h, C.byref(t)))
        return {f: (float(getattr(t, f)) if "ms" in f else int(getattr(t, f)))
                for f, _ in Timing._fields_}

    def reset_timing(self):
        _check(lib().moe_pool_reset_timing(self._h))

    def set_timing(self, every: int):
        """Event-timing period from now on (0 = off, e.g. before a graph capture)."""
        _check(lib().moe_pool_set_timing(self._h, int(every)))


def read_calibration(buf, bytes_per_launch: int, reps: int = 20, stream=None) -> float:
    """Mean event-timed duration (us) of a plain streaming read of bytes_per_launch,
    rotating over the device buffer `buf` (a torch tensor)."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    us = C.c_double(0)
    _check(lib().moe_read_calibration(_ptr(buf), buf.numel() * buf.element_size(), bytes_per_launch, reps,
                                      C.c_void_p(stream), C.byref(us)))
    return us.value


def link_calibration(nbytes: int, engine: str = "kernel", reps: int = 8, streams: int = 1, stream=None) -> float:
    """Mean event-timed duration (us) of one pinned host -> HBM copy of nbytes with
    the given engine ("kernel" or "dma"), split over `streams` streams."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    us = C.c_double(0)
    _check(lib().moe_link_calibration(nbytes, reps, COPY_ENGINES[engine], streams, C.c_void_p(stream),
                                      C.byref(us)))
    return us.value


def is_pinned_host(addr: int) -> bool:
    v = C.c_int32(0)
    _check(lib().moe_ptr_is_pinned_host(addr, C.byref(v)))
    return bool(v.value)


class SlotLRU:
    """The library's slot manager on host ids (no GPU)."""

    def __init__(self, experts: int, slots: int, rule: str = "distinct"):
        self._h = None
        h = C.c_void_p()
        _check(lib().moe_lru_create(experts, slots, RULES[rule], C.byref(h)))
        self._h = h
        self.experts, self.slots = experts, slots
        self._miss_buf = (Miss * max(1, experts))()

    def close(self):
        if self._h is not None and self._h.value:
            lib().moe_lru_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def step(self, ids: np.ndarray):
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        T, K = ids.shape
        out = np.empty_like(ids)
        nm, path = C.c_int32(0), C.c_int32(0)
        _check(lib().moe_lru_step(self._h, ids.ctypes.data, T, K, out.ctypes.data, self._miss_buf,
                                  len(self._miss_buf), C.byref(nm), C.byref(path)))
        return out, path.value, _misses(self._miss_buf, min(nm.value, len(self._miss_buf)))

    def state(self):
        m = np.empty(self.experts, np.int32)
        o = np.empty(max(1, self.slots), np.int32)
        l = np.empty(max(1, self.slots), np.int32)
        _check(lib().moe_lru_get_state(self._h, m.ctypes.data, o.ctypes.data, l.ctypes.data))
        return m, o[:self.slots], l[:self.slots]

    def stats(self) -> dict:
        s = Stats()
        _check(lib().moe_lru_get_stats(self._h, C.byref(s)))
        return {f: int(getattr(s, f)) for f, _ in Stats._fields_}
