"""Python binding of libthdattn: causal + EOD-reset attention over THD-packed
sequences for one context-parallel rank, on AMD MI355X (gfx950).

This module only marshals arguments: every step of the computation runs in
the C-ABI library (host planner and HIP kernels). PyTorch supplies device
memory and the stream. All functions are keyword-only, so that a change of the
argument list cannot silently shift positional arguments.

The library must have been built in-tree (``python
packed_sequence_causal_amd/build.py`` or ``__graft_entry__.build()``); importing
this package raises if it is missing. There is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libthdattn.so")

THD_OK = 0
STATUS_NAMES = {
    -1: "THD_EINVAL", -2: "THD_ENOTDIV", -3: "THD_ERANGE", -4: "THD_EALIGN",
    -5: "THD_EMISMATCH", -6: "THD_EHIP", -7: "THD_ENOMEM", -8: "THD_EUNSUPPORTED",
}
FIELDS = {"q_global": 0, "kv_row": 1, "chunk_off": 2, "tiles": 3, "order": 4, "kvtiles": 5,
          "items": 6, "splits": 7, "doc_end": 8, "pack_rows": 9, "pack_keys": 10}
META_VERSION = 4


class ThdError(RuntimeError):
    """A negative status returned by the library, with its message."""

    def __init__(self, code: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {message}")
        self.code = code
        self.status = STATUS_NAMES.get(code, str(code))


class _Info(ctypes.Structure):
    _fields_ = [
        ("total_tokens", ctypes.c_int64), ("local_tokens", ctypes.c_int64),
        ("n_tiles", ctypes.c_int64), ("n_kvtiles", ctypes.c_int64),
        ("useful_pairs", ctypes.c_int64), ("max_kv_tiles", ctypes.c_int64),
        ("n_items", ctypes.c_int64), ("n_splits", ctypes.c_int64), ("n_part_slots", ctypes.c_int64),
        ("pad_tokens", ctypes.c_int64),
        ("concurrency", ctypes.c_int32), ("kv_split", ctypes.c_int32),
        ("n_docs", ctypes.c_int32), ("cp", ctypes.c_int32), ("rank", ctypes.c_int32),
        ("block_t", ctypes.c_int32), ("block_n", ctypes.c_int32), ("version", ctypes.c_int32),
        ("device", ctypes.c_int32), ("cache_hit", ctypes.c_int32),
        ("is_pass", ctypes.c_int32), ("item_ints", ctypes.c_int32),
        ("shard_mask", ctypes.c_uint64),
        ("n_packed_tiles", ctypes.c_int64), ("n_pack_rows", ctypes.c_int64),
        ("n_pack_keys", ctypes.c_int64), ("is_packed", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first with "
            "`python packed_sequence_causal_amd/build.py` (no fallback path exists)")
    lib = ctypes.CDLL(LIB_PATH)
    i32, i64, p = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    pi32 = ctypes.POINTER(ctypes.c_int32)
    pi64 = ctypes.POINTER(ctypes.c_int64)
    sigs = {
        "thd_last_error": (ctypes.c_char_p, []),
        "thd_plan_partition": (ctypes.c_int, [pi32, i32, i32, i32, pi64, pi64, pi32, pi32, pi32]),
        "thd_build_metadata": (ctypes.c_int, [pi32, i32, i32, i32, i32, i32, i32, i32,
                                              ctypes.POINTER(p)]),
        "thd_pad_lengths": (ctypes.c_int, [pi32, i32, i32, pi32]),
        "thd_build_metadata_padded": (ctypes.c_int, [pi32, i32, i32, i32, i32, i32, i32, i32,
                                                     ctypes.POINTER(p)]),
        "thd_build_packed_metadata": (ctypes.c_int, [pi32, i32, i32, i32, i32, i32, i32, i32, i32,
                                                     ctypes.POINTER(p)]),
        "thd_meta_info": (ctypes.c_int, [p, ctypes.POINTER(_Info)]),
        "thd_meta_copy": (ctypes.c_int, [p, i32, pi32, i64]),
        "thd_meta_release": (None, [p]),
        "thd_cache_stats": (ctypes.c_int, [pi64, pi64, pi64, pi64]),
        "thd_cache_clear": (ctypes.c_int, []),
        "thd_preferred_tiles": (ctypes.c_int, [i32, i32, i32, i32, pi32, pi32]),
        "thd_preferred_fwd_tiles": (ctypes.c_int, [pi32, i32, i32, i32, i32, i32, i32, i32, i32,
                                                   pi32, pi32]),
        "thd_fwd_concurrency": (ctypes.c_int, [i32, i32, i32, pi32]),
        "thd_attn_fwd_workspace": (ctypes.c_int, [p, i32, i32, i32, pi64]),
        "thd_attn_fwd": (ctypes.c_int, [p, p, p, p, p, p, p, i32, i32, i32, i32, ctypes.c_float, p,
                                        i64, p]),
        "thd_attn_fwd_noalloc": (ctypes.c_int, [p, p, p, p, p, p, p, i32, i32, i32, i32,
                                                ctypes.c_float, p]),
        "thd_build_pass_metadata": (ctypes.c_int, [pi32, i32, i32, i32, i32, i32, ctypes.c_uint64,
                                                   i32, ctypes.POINTER(p)]),
        "thd_build_pass_metadata_padded": (ctypes.c_int, [pi32, i32, i32, i32, i32, i32,
                                                          ctypes.c_uint64, i32,
                                                          ctypes.POINTER(p)]),
        "thd_attn_fwd_pass_state_bytes": (ctypes.c_int, [p, i32, i32, i32, pi64]),
        "thd_attn_fwd_pass": (ctypes.c_int, [p, p, p, p, p, p, p, i32, i32, i32, i32, i32,
                                             ctypes.c_float, p]),
        "thd_attn_bwd_workspace": (ctypes.c_int, [p, i32, pi64]),
        "thd_attn_bwd": (ctypes.c_int, [p, p, p, p, p, p, p, p, p, p, i32, i32, i32, i32,
                                        ctypes.c_float, p, i64, p]),
        "thd_attn_bwd_bf16kv": (ctypes.c_int, [p, p, p, p, p, p, p, p, p, p, i32, i32, i32,
                                               i32, ctypes.c_float, p, i64, p]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()
EXPORTS = ("thd_last_error", "thd_plan_partition", "thd_build_metadata", "thd_pad_lengths",
           "thd_build_metadata_padded", "thd_build_packed_metadata", "thd_meta_info",
           "thd_meta_copy", "thd_meta_release", "thd_cache_stats", "thd_cache_clear",
           "thd_preferred_tiles", "thd_preferred_fwd_tiles", "thd_fwd_concurrency",
           "thd_attn_fwd_workspace", "thd_attn_fwd", "thd_attn_fwd_noalloc",
           "thd_build_pass_metadata", "thd_build_pass_metadata_padded",
           "thd_attn_fwd_pass_state_bytes", "thd_attn_fwd_pass",
           "thd_attn_bwd_workspace", "thd_attn_bwd", "thd_attn_bwd_bf16kv")
PASS_FIRST = 1
PASS_LAST = 2


def _check(code: int):
    if code != THD_OK:
        raise ThdError(code, _lib.thd_last_error().decode(errors="replace"))


_I32 = np.dtype(np.int32)


def _lengths(seqlens) -> np.ndarray:
    if type(seqlens) is np.ndarray and seqlens.dtype == _I32 and seqlens.ndim == 1 \
            and seqlens.flags.c_contiguous:
        return seqlens   # already what the library takes: no copy, no range check needed
    arr = np.ascontiguousarray(np.asarray(seqlens).reshape(-1))
    if arr.size and not np.issubdtype(arr.dtype, np.integer):
        raise TypeError("seqlens must be integers")
    if arr.size and (arr.min() < np.iinfo(np.int32).min or arr.max() > np.iinfo(np.int32).max):
        raise ThdError(-3, "a length does not fit int32")
    return np.ascontiguousarray(arr, dtype=np.int32)


def _ptr32(arr: np.ndarray):
    return arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) if arr is not None else None


def plan_partition(*, seqlens, cp: int, rank: int) -> dict:
    """Per-rank partition maps (host numpy int32): q_global, kv_row, chunk_off."""
    lens = _lengths(seqlens)
    total, local = ctypes.c_int64(), ctypes.c_int64()
    _check(_lib.thd_plan_partition(_ptr32(lens), len(lens), cp, rank, ctypes.byref(total),
                                   ctypes.byref(local), None, None, None))
    q_global = np.empty(local.value, np.int32)
    kv_row = np.empty(total.value, np.int32)
    chunk_off = np.empty(len(lens) * 2 * cp, np.int32)
    _check(_lib.thd_plan_partition(_ptr32(lens), len(lens), cp, rank, None, None,
                                   _ptr32(q_global), _ptr32(kv_row), _ptr32(chunk_off)))
    return {"total": total.value, "local": local.value, "q_global": q_global,
            "kv_row": kv_row, "chunk_off": chunk_off}


class Meta:
    """One reference to a cached metadata object; released when dropped."""

    def __init__(self, handle):
        self._h = handle
        self._info = None   # a handle's info never changes: read it once
        self._fwd_ws = {}   # forward workspace bytes per (hq, hkv, d_v)

    @property
    def handle(self):
        return self._h

    def info(self) -> dict:
        if self._info is None:
            inf = _Info()
            _check(_lib.thd_meta_info(self._h, ctypes.byref(inf)))
            self._info = {name: getattr(inf, name) for name, _ in _Info._fields_}
        return dict(self._info)

    def _cached_info(self) -> dict:
        if self._info is None:
            self.info()
        return self._info

    def fwd_workspace_bytes(self, hq: int, hkv: int, d_v: int) -> int:
        key = (hq, hkv, d_v)
        if key not in self._fwd_ws:
            need = ctypes.c_int64()
            _check(_lib.thd_attn_fwd_workspace(self._h, hq, hkv, d_v, ctypes.byref(need)))
            self._fwd_ws[key] = need.value
        return self._fwd_ws[key]

    def field(self, name: str) -> np.ndarray:
        inf = self.info()
        n = {"q_global": inf["local_tokens"], "kv_row": inf["total_tokens"],
             "chunk_off": inf["n_docs"] * 2 * inf["cp"], "tiles": inf["n_tiles"] * 8,
             "order": inf["n_tiles"], "kvtiles": inf["n_kvtiles"] * 8,
             "items": inf["n_items"] * inf["item_ints"],
             "splits": (inf["n_tiles"] if inf["is_pass"] else inf["n_splits"]) * 4,
             "doc_end": inf["n_docs"], "pack_rows": inf["n_pack_rows"] * 4,
             "pack_keys": inf["n_pack_keys"]}[name]
        out = np.empty(n, np.int32)
        _check(_lib.thd_meta_copy(self._h, FIELDS[name], _ptr32(out), n))
        if name in ("tiles", "kvtiles"):
            out = out.reshape(-1, 8)
        if name == "items":
            out = out.reshape(-1, inf["item_ints"])
        if name in ("splits", "pack_rows"):
            out = out.reshape(-1, 4)
        return out

    def release(self):
        if self._h is not None:
            _lib.thd_meta_release(self._h)
            self._h = None

    def __del__(self):
        try:
            self.release()
        except Exception:
            pass


def pad_lengths(*, seqlens, cp: int) -> np.ndarray:
    """Padded length of each document: the least multiple of 2*cp holding it."""
    lens = _lengths(seqlens)
    out = np.empty_like(lens)
    _check(_lib.thd_pad_lengths(_ptr32(lens), len(lens), cp, _ptr32(out)))
    return out


def build_metadata(*, seqlens, cp: int, rank: int, block_t: int, block_n: int,
                   concurrency: int = 0, device: int = -1, padded: bool = False,
                   packed: bool = False) -> Meta:
    """Build or fetch cached metadata; device >= 0 also uploads it there.

    concurrency: work items of one kv head the device runs at once (0 = never
    split a tile's key range). padded: seqlens are real lengths of any size;
    each document is stored padded to pad_lengths() tokens, real tokens first
    (tensors use the padded layout; pad rows get O = 0 and LSE = +inf).
    packed: a forward-only plan whose short partial query tiles are packed
    together (thd_build_packed_metadata)."""
    lens = _lengths(seqlens)
    h = ctypes.c_void_p()
    if packed:
        _check(_lib.thd_build_packed_metadata(_ptr32(lens), len(lens), cp, rank, block_t, block_n,
                                              concurrency, int(bool(padded)), device,
                                              ctypes.byref(h)))
        return Meta(h)
    fn = _lib.thd_build_metadata_padded if padded else _lib.thd_build_metadata
    _check(fn(_ptr32(lens), len(lens), cp, rank, block_t, block_n, concurrency, device,
              ctypes.byref(h)))
    return Meta(h)


_TILES = {}


def preferred_tiles(*, hq: int, hkv: int, d_qk: int, d_v: int) -> tuple[int, int]:
    key = (hq, hkv, d_qk, d_v)
    if key not in _TILES:
        bt, bn = ctypes.c_int32(), ctypes.c_int32()
        _check(_lib.thd_preferred_tiles(hq, hkv, d_qk, d_v, ctypes.byref(bt), ctypes.byref(bn)))
        _TILES[key] = (bt.value, bn.value)
    return _TILES[key]


def cache_stats() -> dict:
    vals = [ctypes.c_int64() for _ in range(4)]
    _check(_lib.thd_cache_stats(*[ctypes.byref(v) for v in vals]))
    return dict(zip(("hits", "misses", "uploads", "entries"), (v.value for v in vals)))


def cache_clear():
    _check(_lib.thd_cache_clear())


def _torch():
    import torch
    return torch


def _stream_handle(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


_CONCURRENCY = {}


def preferred_fwd_tiles(*, seqlens, cp: int, rank: int, hq: int, hkv: int, d_qk: int, d_v: int,
                        padded: bool = False, device: int | None = None,
                        concurrency32: int | None = None) -> tuple[int, int]:
    """Forward tile sizes for this batch (thd_preferred_fwd_tiles): 32-key
    tiles when d_qk <= 128 and they compute at least 7% fewer key slots than
    64-key tiles (query tiles visit whole KV tiles up to their last row), or,
    given the device (or its 32-key concurrency), when query tiles hold at most
    32 tokens and there are enough of them that no key range is split."""
    lens = pad_lengths(seqlens=seqlens, cp=cp) if padded else _lengths(seqlens)
    if concurrency32 is None:
        concurrency32 = 0 if device is None else device_concurrency(device, hkv, 32)
    bt, bn = ctypes.c_int32(), ctypes.c_int32()
    _check(_lib.thd_preferred_fwd_tiles(_ptr32(lens), len(lens), cp, rank, hq, hkv, d_qk, d_v,
                                        concurrency32, ctypes.byref(bt), ctypes.byref(bn)))
    return bt.value, bn.value


def device_concurrency(device: int, hkv: int, block_n: int = 64) -> int:
    """Forward work items of one kv head the device runs at once (thd_fwd_concurrency)."""
    key = (device, hkv, block_n)
    if key not in _CONCURRENCY:
        c = ctypes.c_int32()
        _check(_lib.thd_fwd_concurrency(device, hkv, block_n, ctypes.byref(c)))
        _CONCURRENCY[key] = c.value
    return _CONCURRENCY[key]


def device_metadata(*, seqlens, cp: int, rank: int, hq: int, hkv: int, d_qk: int, d_v: int,
                    device: int, concurrency: int | None = None, padded: bool = False,
                    forward: bool = False, packed: bool = False) -> Meta:
    """Metadata on a device with the kernels' tile sizes. forward=True picks the
    forward's sizes for this batch (possibly 32-key tiles, which the backward
    does not take); otherwise the sizes serve both directions. packed (with
    forward=True): pack the short partial query tiles (forward only)."""
    if packed and not forward:
        raise ThdError(-1, "packed plans are forward-only: pass forward=True")
    if forward:
        bt, bn = preferred_fwd_tiles(seqlens=seqlens, cp=cp, rank=rank, hq=hq, hkv=hkv, d_qk=d_qk,
                                     d_v=d_v, padded=padded, device=device)
    else:
        bt, bn = preferred_tiles(hq=hq, hkv=hkv, d_qk=d_qk, d_v=d_v)
    if concurrency is None:
        concurrency = device_concurrency(device, hkv, bn)
    return build_metadata(seqlens=seqlens, cp=cp, rank=rank, block_t=bt, block_n=bn,
                          concurrency=concurrency, device=device, padded=padded, packed=packed)


def _scratch(device, nbytes: int, stream):
    """A device buffer of nbytes (None for 0) from torch's caching allocator,
    fresh per call: calls on different streams never share it. When the kernel
    runs on a stream other than the current one, the buffer is recorded on it,
    so the allocator does not hand it out again before that stream's work ends."""
    if nbytes <= 0:
        return None
    torch = _torch()
    buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if stream is not None and stream != torch.cuda.current_stream(device):
        buf.record_stream(stream)
    return buf


def _need(name, t, dtype, shape, dev):
    """Raise ThdError unless t is a contiguous tensor of this dtype, shape and
    device: the kernels size every load and store from the head counts and
    dims, so a mismatched tensor must be refused before the launch."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise ThdError(-1, f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise ThdError(-1, f"{name} must be {dtype}, not {t.dtype}")
    if t.device != dev:
        raise ThdError(-1, f"{name} is on {t.device}, the call runs on {dev}")
    if not t.is_contiguous():
        raise ThdError(-1, f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ThdError(-5, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _qkv_shapes(q, k, v):
    """Head counts and dims from q, k, v (checked: 3-d bf16 device tensors)."""
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dim() != 3 or t.dtype != torch.bfloat16 \
                or not t.is_cuda:
            raise ThdError(-1, f"{name} must be a 3-d bf16 device tensor")
    return q.shape[1], k.shape[1], q.shape[2], v.shape[2]


def attn_fwd(*, q, k, v, seqlens, cp: int, rank: int, softmax_scale=None, out=None, lse=None,
             out_f32=None, stream=None, meta: Meta | None = None, concurrency: int | None = None,
             padded: bool = False, packed: bool = False):
    """Forward attention for one rank. Returns (o bf16 [T_loc,Hq,dv], lse fp32 [T_loc,Hq]).

    q [T_loc, Hq, dqk], k [T, Hkv, dqk], v [T, Hkv, dv]: bf16 CUDA tensors,
    k/v already gathered rank-major. softmax_scale None lets the library use
    1/sqrt(dqk). out_f32 (optional fp32 [T_loc, Hq, dv] tensor) also receives O
    in fp32, computed with split probabilities: pass it to attn_bwd as o_f32.
    padded: seqlens are real lengths and the tensors use the padded layout
    (see build_metadata); pad rows get O = 0 and LSE = +inf. packed: pack the
    short partial query tiles of several documents into shared tiles (the same
    attention with fewer workgroups; see build_metadata).
    """
    torch = _torch()
    hq, hkv, d_qk, d_v = _qkv_shapes(q, k, v)
    dev = q.device
    if meta is None:
        meta = device_metadata(seqlens=seqlens, cp=cp, rank=rank, hq=hq, hkv=hkv, d_qk=d_qk,
                               d_v=d_v, device=dev.index, concurrency=concurrency,
                               padded=padded, forward=True, packed=packed)
    inf = meta._cached_info()
    t_loc, total = inf["local_tokens"], inf["total_tokens"]
    _need("q", q, torch.bfloat16, (t_loc, hq, d_qk), dev)
    _need("k", k, torch.bfloat16, (total, hkv, d_qk), dev)
    _need("v", v, torch.bfloat16, (total, hkv, d_v), dev)
    if out is None:
        out = torch.empty((t_loc, hq, d_v), dtype=torch.bfloat16, device=dev)
    else:
        _need("out", out, torch.bfloat16, (t_loc, hq, d_v), dev)
    if lse is None:
        lse = torch.empty((t_loc, hq), dtype=torch.float32, device=dev)
    else:
        _need("lse", lse, torch.float32, (t_loc, hq), dev)
    if out_f32 is not None:
        _need("out_f32", out_f32, torch.float32, (t_loc, hq, d_v), dev)
    need = meta.fwd_workspace_bytes(hq, hkv, d_v)
    ws = _scratch(dev, need, stream)
    scale = 0.0 if softmax_scale is None else float(softmax_scale)
    _check(_lib.thd_attn_fwd(meta.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                             out.data_ptr(), lse.data_ptr(),
                             None if out_f32 is None else out_f32.data_ptr(),
                             hq, hkv, d_qk, d_v, scale,
                             None if ws is None else ws.data_ptr(), need,
                             _stream_handle(stream, dev)))
    return out, lse


def build_pass_metadata(*, seqlens, cp: int, rank: int, block_t: int, block_n: int, shards,
                        device: int = -1, padded: bool = False) -> Meta:
    """Metadata of one forward pass over the keys of the listed source ranks'
    shards (all-gather overlap; thd_build_pass_metadata). padded: seqlens are
    real lengths and the tensors use the padded layout (as build_metadata)."""
    lens = _lengths(seqlens)
    mask = 0
    for s_ in shards:
        s_ = int(s_)
        if not 0 <= s_ < 64:
            raise ThdError(-1, "shard ranks must lie in [0, 64)")
        mask |= 1 << s_
    h = ctypes.c_void_p()
    fn = _lib.thd_build_pass_metadata_padded if padded else _lib.thd_build_pass_metadata
    _check(fn(_ptr32(lens), len(lens), cp, rank, block_t, block_n, mask, device, ctypes.byref(h)))
    return Meta(h)


def pass_state(*, meta: Meta, hq: int, hkv: int, d_v: int, device):
    """A state buffer (fp32) for the passes of one forward (thd_attn_fwd_pass_state_bytes)."""
    torch = _torch()
    state = ctypes.c_int64()
    _check(_lib.thd_attn_fwd_pass_state_bytes(meta.handle, hq, hkv, d_v, ctypes.byref(state)))
    return torch.empty(state.value // 4, dtype=torch.float32, device=device)


def attn_fwd_pass(*, q, k, v, meta: Meta, state, first: bool, last: bool, out=None, lse=None,
                  softmax_scale=None, stream=None):
    """One pass of a shard-by-shard forward (thd_attn_fwd_pass): merges the
    attention over the pass's shards into ``state``; with last=True writes and
    returns (o, lse), else returns None. The rows of k and v outside the pass's
    shards are not read."""
    torch = _torch()
    hq, hkv, d_qk, d_v = _qkv_shapes(q, k, v)
    dev = q.device
    inf = meta._cached_info()
    if not inf["is_pass"]:
        raise ThdError(-5, "metadata is not a pass plan")
    t_loc, total = inf["local_tokens"], inf["total_tokens"]
    _need("q", q, torch.bfloat16, (t_loc, hq, d_qk), dev)
    _need("k", k, torch.bfloat16, (total, hkv, d_qk), dev)
    _need("v", v, torch.bfloat16, (total, hkv, d_v), dev)
    _need("state", state, torch.float32, (t_loc * hq * (d_v + 1),), dev)
    if last:
        if out is None:
            out = torch.empty((t_loc, hq, d_v), dtype=torch.bfloat16, device=dev)
        else:
            _need("out", out, torch.bfloat16, (t_loc, hq, d_v), dev)
        if lse is None:
            lse = torch.empty((t_loc, hq), dtype=torch.float32, device=dev)
        else:
            _need("lse", lse, torch.float32, (t_loc, hq), dev)
    flags = (PASS_FIRST if first else 0) | (PASS_LAST if last else 0)
    scale = 0.0 if softmax_scale is None else float(softmax_scale)
    _check(_lib.thd_attn_fwd_pass(meta.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                  None if out is None else out.data_ptr(),
                                  None if lse is None else lse.data_ptr(), state.data_ptr(), flags,
                                  hq, hkv, d_qk, d_v, scale, _stream_handle(stream, dev)))
    return (out, lse) if last else None


def attn_fwd_noalloc(*, q, k, v, out, lse, meta: Meta, out_f32=None, softmax_scale=None,
                     stream=None):
    """thd_attn_fwd_noalloc: the forward into caller-given out and lse with
    metadata built beforehand; nothing is allocated (the split tiles' partial
    results use the library's per-device static array). Calls that overlap on
    one device race on that array."""
    torch = _torch()
    hq, hkv, d_qk, d_v = _qkv_shapes(q, k, v)
    dev = q.device
    inf = meta._cached_info()
    t_loc, total = inf["local_tokens"], inf["total_tokens"]
    _need("q", q, torch.bfloat16, (t_loc, hq, d_qk), dev)
    _need("k", k, torch.bfloat16, (total, hkv, d_qk), dev)
    _need("v", v, torch.bfloat16, (total, hkv, d_v), dev)
    _need("out", out, torch.bfloat16, (t_loc, hq, d_v), dev)
    _need("lse", lse, torch.float32, (t_loc, hq), dev)
    if out_f32 is not None:
        _need("out_f32", out_f32, torch.float32, (t_loc, hq, d_v), dev)
    scale = 0.0 if softmax_scale is None else float(softmax_scale)
    _check(_lib.thd_attn_fwd_noalloc(meta.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                     out.data_ptr(), lse.data_ptr(),
                                     None if out_f32 is None else out_f32.data_ptr(),
                                     hq, hkv, d_qk, d_v, scale, _stream_handle(stream, dev)))
    return out, lse


def attn_bwd(*, q, k, v, lse, d_o, seqlens, cp: int, rank: int, softmax_scale=None,
             o_f32=None, stream=None, meta: Meta | None = None, workspace=None,
             padded: bool = False, dkdv_dtype=None):
    """Backward for one rank. Returns (dq fp32, dk, dv); dk/dv are this rank's
    partial sums in the gathered layout (zeros for unseen keys), fp32, or bf16
    (the fp32 results rounded to nearest even; thd_attn_bwd_bf16kv) when
    dkdv_dtype is torch.bfloat16.
    lse is the forward's. o_f32 (optional) is the forward's fp32 O from
    attn_fwd(out_f32=...): D then comes from it instead of a pass over the keys.
    workspace (optional): a device tensor of at least the bytes
    thd_attn_bwd_workspace gives. padded: as for attn_fwd; the forward's
    LSE = +inf on pad rows gives them dQ = 0 and no share in dK, dV, whatever
    d_o holds there."""
    torch = _torch()
    hq, hkv, d_qk, d_v = _qkv_shapes(q, k, v)
    dev = q.device
    if meta is None or meta._cached_info()["block_n"] != preferred_tiles(
            hq=hq, hkv=hkv, d_qk=d_qk, d_v=d_v)[1]:
        # the backward kernels take the general tile sizes only
        meta = device_metadata(seqlens=seqlens, cp=cp, rank=rank, hq=hq, hkv=hkv, d_qk=d_qk,
                               d_v=d_v, device=dev.index, padded=padded)
    inf = meta._cached_info()
    t_loc, total = inf["local_tokens"], inf["total_tokens"]
    _need("q", q, torch.bfloat16, (t_loc, hq, d_qk), dev)
    _need("k", k, torch.bfloat16, (total, hkv, d_qk), dev)
    _need("v", v, torch.bfloat16, (total, hkv, d_v), dev)
    _need("lse", lse, torch.float32, (t_loc, hq), dev)
    _need("d_o", d_o, torch.bfloat16, (t_loc, hq, d_v), dev)
    if o_f32 is not None:
        _need("o_f32", o_f32, torch.float32, (t_loc, hq, d_v), dev)
    need = ctypes.c_int64()
    _check(_lib.thd_attn_bwd_workspace(meta.handle, hq, ctypes.byref(need)))
    if workspace is None:
        workspace = _scratch(dev, need.value, stream)
    elif not isinstance(workspace, torch.Tensor) or workspace.device != dev \
            or not workspace.is_contiguous():
        raise ThdError(-1, f"workspace must be a contiguous tensor on {dev}")
    ws_bytes = workspace.numel() * workspace.element_size()
    if ws_bytes < need.value:
        raise ThdError(-1, f"workspace has {ws_bytes} bytes, needs {need.value}")
    if dkdv_dtype not in (None, torch.float32, torch.bfloat16):
        raise ThdError(-1, f"dkdv_dtype must be torch.float32 or torch.bfloat16, not {dkdv_dtype}")
    kv_dtype = torch.float32 if dkdv_dtype is None else dkdv_dtype
    dq = torch.empty(q.shape, dtype=torch.float32, device=dev)
    dk = torch.empty(k.shape, dtype=kv_dtype, device=dev)
    dv = torch.empty(v.shape, dtype=kv_dtype, device=dev)
    scale = 0.0 if softmax_scale is None else float(softmax_scale)
    fn = _lib.thd_attn_bwd_bf16kv if kv_dtype == torch.bfloat16 else _lib.thd_attn_bwd
    _check(fn(meta.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), lse.data_ptr(),
              None if o_f32 is None else o_f32.data_ptr(), d_o.data_ptr(), dq.data_ptr(),
              dk.data_ptr(), dv.data_ptr(), hq, hkv, d_qk, d_v, scale, workspace.data_ptr(),
              ws_bytes, _stream_handle(stream, dev)))
    return dq, dk, dv
