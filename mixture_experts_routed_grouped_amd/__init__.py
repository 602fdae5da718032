"""Routed fused-MoE expert FFN for MI355X (gfx950): Python binding.

A thin ctypes layer over ``librmoe.so`` (declared in ``include/routed_moe.h``)
with the same entry-point names.  It only marshals arguments: torch tensors
become device pointers plus the current HIP stream, numpy arrays become host
pointers.  Every step of the routed path runs in the library's HIP kernels
or its C++ host code; if the library is missing, importing works but every
call raises ``RmoeError`` -- there is no fallback.

The submission-style entry point ``run_kernel`` keeps the argument order of
"Fused MoE GEMM 提交说明" (section 提交文件) and, like that template, caches
the fp16 hidden workspace per (device, rows, intermediate).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "librmoe.so")
# diagnostic build: the same library with the tiled kernels' phase timing
PHASE_LIB_PATH = os.path.join(_PKG, "librmoe_phase.so")

VARIANT_AUTO, VARIANT_STREAM, VARIANT_TILE = 0, 1, 2
_VARIANTS = {"auto": 0, "stream": 1, "tile": 2, 0: 0, 1: 1, 2: 2}
_VARIANT_NAMES = {VARIANT_STREAM: "stream", VARIANT_TILE: "tile"}
_HANDOVER = {"auto": 0, "local": 1, "global": 2}


class RmoeError(RuntimeError):
    pass


_lib = None

_P = ctypes.c_void_p
_I32P = ctypes.POINTER(ctypes.c_int32)
_I64, _I32 = ctypes.c_int64, ctypes.c_int32

_SIGS = {
    "rmoe_status_str": ([ctypes.c_int], ctypes.c_char_p),
    "rmoe_version": ([], ctypes.c_char_p),
    "rmoe_build_contract": ([_P, _I64, _I32, _I32, _P, _P, _P, _P, _I64, _P, _P, _P, _P], ctypes.c_int),
    "rmoe_validate_contract": ([_P, _P, _P, _P, _I32, _I32, _I64, _I64], ctypes.c_int),
    "rmoe_validate_contract_device": ([_P, _P, _P, _P, _I32, _I32, _I64, _I64, _P, _P], ctypes.c_int),
    "rmoe_workspace_bytes": ([_I64, _I64], ctypes.c_size_t),
    "rmoe_contract_sizes": ([_I64, _I32, _P, _P], ctypes.c_int),
    "rmoe_pick_variant": ([_I32, _I64, _I32, _I64], ctypes.c_int),
    "rmoe_forward_f16": ([_P] * 11 + [_I64, _I64, _I32, _I64, _I64, _I32, _P], ctypes.c_int),
    "rmoe_forward_f16_variant": ([_P] * 11 + [_I64, _I64, _I32, _I64, _I64, _I32, _I32, _P],
                                 ctypes.c_int),
    "rmoe_fused_sync_words": ([_I32], ctypes.c_size_t),
    "rmoe_forward_fused_f16": ([_P] * 12 + [_I64, _I64, _I32, _I64, _I64, _I32, _I32, _I32, _P],
                               ctypes.c_int),
    "rmoe_gate_up_f16": ([_P] * 7 + [_I64, _I64, _I32, _I64, _I64, _I32, _I32, _P], ctypes.c_int),
    "rmoe_down_f16": ([_P] * 8 + [_I64, _I64, _I32, _I64, _I64, _I32, _I32, _P], ctypes.c_int),
    "rmoe_pack_f16": ([_P] * 4 + [_I64, _I32, _I64, _P, _P, _I64, _P], ctypes.c_int),
    "rmoe_combine_f16": ([_P, _P, _I64, _I32, _I64, _P, _I64, _P], ctypes.c_int),
    "rmoe_contract_workspace_bytes": ([_I64, _I32], ctypes.c_size_t),
    "rmoe_router_f16": ([_P, _P, _I64, _I64, _I32, _I32, _P, _P, _P], ctypes.c_int),
    "rmoe_build_contract_device": ([_P, _I64, _I32, _I32, _P, _P, _P, _P, _I64, _P, _P, _P, _P, _P,
                                    _P, ctypes.c_size_t, _P], ctypes.c_int),
    "rmoe_contract_noalloc_max_words": ([], ctypes.c_size_t),
    "rmoe_build_contract_device_noalloc": ([_P, _I64, _I32, _I32, _P, _P, _P, _P, _I64, _P, _P, _P,
                                            _P, _P, _P], ctypes.c_int),
}


def lib():
    """The loaded library; raises RmoeError if it was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RmoeError(f"{LIB_PATH} is missing: build it with "
                            "`python mixture_experts_routed_grouped_amd/build_lib.py`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def use_library(path: str) -> str:
    """Load the library at ``path`` for every later call (for instance
    PHASE_LIB_PATH, the phase-timing diagnostic build); returns the path that
    was in use.  Buffers and streams stay valid across the switch."""
    global _lib, LIB_PATH
    prev = LIB_PATH
    LIB_PATH, _lib = path, None
    lib()
    return prev


def phase_cycles():
    """The phase-timing records of the last tiled launches
    (rmoe_phase_cycles; only the diagnostic library exports it): uint64
    [2 stages (gate/up, down), RMOE_PHASE_WG workgroups, 5] = prologue,
    K loop, epilogue, items, whole run, in shader-clock ticks."""
    L = lib()
    if not hasattr(L, "rmoe_phase_cycles"):
        raise RmoeError(f"{LIB_PATH} is not the phase-timing build ({PHASE_LIB_PATH})")
    fn = L.rmoe_phase_cycles
    fn.argtypes, fn.restype = [_P, ctypes.c_size_t], ctypes.c_int
    out = np.zeros((2, 1024, 5), dtype=np.uint64)
    _check(fn(_np_ptr(out), out.nbytes), "rmoe_phase_cycles")
    return out


def status_str(status: int) -> str:
    return lib().rmoe_status_str(int(status)).decode()


def _check(status: int, what: str):
    if status != 0:
        raise RmoeError(f"{what}: {status_str(status)} ({status})")


def _np_ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


# ------------------------------------------------------------- host contract
def build_contract(topk_ids, num_experts: int) -> dict:
    """Dispatch tables for a routing ``topk_ids`` [T, k] (host int32), built
    by the library's C++ contract builder.  Returns numpy int32 arrays."""
    ids = np.ascontiguousarray(np.asarray(topk_ids, dtype=np.int32))
    if ids.ndim != 2:
        raise ValueError("topk_ids must be [num_tokens, top_k]")
    T, k = ids.shape
    E = int(num_experts)
    pairs = T * k
    M_cap, Tp = contract_sizes(pairs, E)
    gs = np.zeros(E, np.int32)
    go = np.zeros(E + 1, np.int32)
    gpo = np.zeros(E + 1, np.int32)
    gidx = np.zeros(max(M_cap, 1), np.int32)
    M = np.zeros(1, np.int32)
    order = np.zeros(max(pairs, 1), np.int32)
    prow = np.zeros(max(pairs, 1), np.int32)
    cpos = np.zeros(max(pairs, 1), np.int32)
    st = lib().rmoe_build_contract(_np_ptr(ids), T, k, E, _np_ptr(gs), _np_ptr(go), _np_ptr(gpo),
                                   _np_ptr(gidx), M_cap, _np_ptr(M), _np_ptr(order), _np_ptr(prow),
                                   _np_ptr(cpos))
    _check(st, "rmoe_build_contract")
    M = int(M[0])
    return {
        "n_experts": E,
        "pairs": pairs,
        "group_sizes": gs,
        "group_offsets": go,
        "group_padded_offsets": gpo,
        "num_blocks_m": M,
        "group_idx_for_bx": gidx[:M].copy(),
        "order": order[:pairs].copy(),
        "padded_row_of_pair": prow[:pairs].copy(),
        "compact_pos_of_pair": cpos[:pairs].copy(),
        "total_padded_tokens": Tp,
    }


def validate_contract(group_sizes, group_offsets, group_padded_offsets, group_idx_for_bx,
                      num_experts, num_blocks_m, total_padded_tokens, total_valid_tokens) -> int:
    """Returns the library status (0 = the tables satisfy the contract)."""
    arrs = [np.ascontiguousarray(np.asarray(a, dtype=np.int32)) for a in
            (group_sizes, group_offsets, group_padded_offsets, group_idx_for_bx)]
    return int(lib().rmoe_validate_contract(*[_np_ptr(a) for a in arrs], int(num_experts),
                                            int(num_blocks_m), int(total_padded_tokens),
                                            int(total_valid_tokens)))


def validate_contract_device(group_sizes, group_offsets, group_padded_offsets, group_idx_for_bx,
                             total_padded_tokens, total_valid_tokens, violations=None, stream=None):
    """Enqueue the contract check on device tables (rmoe_validate_contract_device);
    returns the device int32 tensor [1] that receives the violation count
    (0: valid).  Rules on sizes alone raise RmoeError at once."""
    torch = _torch()
    i32 = torch.int32
    E = group_sizes.numel()
    if violations is None:
        violations = torch.empty(1, dtype=i32, device=group_sizes.device)
    st = lib().rmoe_validate_contract_device(
        _dev(group_sizes, i32, "group_sizes"), _dev(group_offsets, i32, "group_offsets"),
        _dev(group_padded_offsets, i32, "group_padded_offsets"),
        _dev(group_idx_for_bx, i32, "group_idx_for_bx"), E, group_idx_for_bx.numel(),
        int(total_padded_tokens), int(total_valid_tokens), _dev(violations, i32, "violations"),
        _stream(group_sizes, stream))
    _check(st, "rmoe_validate_contract_device")
    return violations


def workspace_bytes(total_padded_tokens: int, intermediate: int) -> int:
    return int(lib().rmoe_workspace_bytes(int(total_padded_tokens), int(intermediate)))


def contract_sizes(num_pairs: int, num_experts: int) -> tuple[int, int]:
    """(num_blocks_m, total_padded_tokens) of the contract for a batch, from
    the library (rmoe_contract_sizes)."""
    m = ctypes.c_int32(0)
    tp = ctypes.c_int64(0)
    _check(lib().rmoe_contract_sizes(int(num_pairs), int(num_experts), ctypes.byref(m),
                                     ctypes.byref(tp)), "rmoe_contract_sizes")
    return int(m.value), int(tp.value)


def pick_variant(num_pairs: int, num_experts: int, variant="auto", max_group_rows: int = -1) -> str:
    """The kernel family ("stream" or "tile") for a batch (rmoe_pick_variant).
    With the default max_group_rows=-1 it is the choice every forward and
    stage entry makes under AUTO; with the largest group size (host tables)
    it also weighs the skew."""
    v = int(lib().rmoe_pick_variant(_VARIANTS[variant], int(num_pairs), int(num_experts),
                                    int(max_group_rows)))
    _check(min(v, 0), "rmoe_pick_variant")
    return _VARIANT_NAMES[v]


# ------------------------------------------------------------- device calls
def _torch():
    import torch
    return torch


def _dev(t, dtype, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live in GPU memory")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(t, stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(int(stream.cuda_stream if hasattr(stream, "cuda_stream") else stream))


def forward(stacked_expert_tokens, gate_w, up_w, down_w, routed_expert_weights, group_sizes,
            group_offsets, group_padded_offsets, group_idx_for_bx, workspace, out,
            variant="auto", stream=None):
    """Enqueue the fused expert FFN (gate/up then down) on ``stream`` (default:
    the current stream).  Shapes: tokens [Tp, H], gate/up [E, I, H], down
    [E, H, I] fp16; routed weights [pairs] fp32; tables int32; workspace
    [Tp, I] and out [Tp, H] fp16.  Asynchronous; writes only valid rows."""
    torch = _torch()
    x = stacked_expert_tokens
    E, I, H = gate_w.shape
    Tp = x.shape[0]
    if x.dim() != 2 or x.shape[1] != H or tuple(up_w.shape) != (E, I, H) or \
            tuple(down_w.shape) != (E, H, I):
        raise ValueError("inconsistent shapes")
    if tuple(workspace.shape) != (Tp, I) or tuple(out.shape) != (Tp, H):
        raise ValueError("workspace must be [Tp, I] and out [Tp, H]")
    if group_sizes.numel() != E or group_offsets.numel() != E + 1 or \
            group_padded_offsets.numel() != E + 1:
        raise ValueError("group tables must have E, E+1, E+1 entries")
    pairs = routed_expert_weights.numel()
    M = group_idx_for_bx.numel()
    f16, i32 = torch.float16, torch.int32
    st = lib().rmoe_forward_f16_variant(
        _dev(x, f16, "stacked_expert_tokens"), _dev(gate_w, f16, "gate_w"),
        _dev(up_w, f16, "up_w"), _dev(down_w, f16, "down_w"),
        _dev(routed_expert_weights, torch.float32, "routed_expert_weights"),
        _dev(group_sizes, i32, "group_sizes"), _dev(group_offsets, i32, "group_offsets"),
        _dev(group_padded_offsets, i32, "group_padded_offsets"),
        _dev(group_idx_for_bx, i32, "group_idx_for_bx"), _dev(workspace, f16, "workspace"),
        _dev(out, f16, "out"), H, I, E, Tp, pairs, M, _VARIANTS[variant], _stream(x, stream))
    _check(st, "rmoe_forward_f16")


FUSED_SYNC_ERROR = 9  # RMOE_FUSED_SYNC_ERROR: sticky count of skipped tiles
_SYNC = {}


def fused_sync_words(num_blocks_m: int) -> int:
    return int(lib().rmoe_fused_sync_words(int(num_blocks_m)))


def fused_sync(device, num_blocks_m: int, stream=None):
    """A zeroed int32 sync buffer for forward_fused, cached per (device, size,
    stream): calls on one stream run one after another and may share it,
    calls on different streams get different buffers.  The kernel leaves it
    zero after each completed call, except the sticky error word."""
    torch = _torch()
    device = torch.device(device)
    if stream is None:
        stream = torch.cuda.current_stream(device)
    handle = int(stream.cuda_stream if hasattr(stream, "cuda_stream") else stream)
    key = (device.index or 0, fused_sync_words(num_blocks_m), handle)
    buf = _SYNC.get(key)
    if buf is None:
        buf = torch.zeros(key[1], dtype=torch.int32, device=device)
        _SYNC[key] = buf
    return buf


def fused_sync_errors(sync, clear: bool = True) -> int:
    """Tiles the single-launch forwards on ``sync`` skipped because a wait
    for hidden rows timed out (their out rows are then unwritten); 0 in
    normal operation.  Waits for the device (it reads the word back), so
    call it when a result is about to be used; ``clear`` resets the count."""
    torch = _torch()
    torch.cuda.synchronize(sync.device)
    n = int(sync[FUSED_SYNC_ERROR].item())
    if clear and n:
        sync[FUSED_SYNC_ERROR] = 0
        torch.cuda.synchronize(sync.device)
    return n


def forward_fused(stacked_expert_tokens, gate_w, up_w, down_w, routed_expert_weights, group_sizes,
                  group_offsets, group_padded_offsets, group_idx_for_bx, workspace, out, sync=None,
                  max_wait_us=0, handover="auto", stream=None):
    """Both stages in one launch (rmoe_forward_fused_f16): same arguments and
    results as forward(..., variant="tile"); ``sync`` is the int32 queue
    state (default: a zeroed buffer cached per device, size and stream;
    calls sharing one must not overlap in time); ``max_wait_us`` bounds a
    down tile's wait for its hidden rows (0: the library's default).  A wait
    that times out skips its tile and counts it in the sync buffer's error
    word: check it with ``fused_sync_errors(sync)`` before using ``out``.
    ``handover``: "local" (each pair's hidden rows stay in one XCD's L2),
    "global" (handed over through memory) or "auto" (the library's choice)."""
    torch = _torch()
    x = stacked_expert_tokens
    E, I, H = gate_w.shape
    Tp = x.shape[0]
    if x.dim() != 2 or x.shape[1] != H or tuple(up_w.shape) != (E, I, H) or \
            tuple(down_w.shape) != (E, H, I):
        raise ValueError("inconsistent shapes")
    if tuple(workspace.shape) != (Tp, I) or tuple(out.shape) != (Tp, H):
        raise ValueError("workspace must be [Tp, I] and out [Tp, H]")
    if group_sizes.numel() != E or group_offsets.numel() != E + 1 or \
            group_padded_offsets.numel() != E + 1:
        raise ValueError("group tables must have E, E+1, E+1 entries")
    M = group_idx_for_bx.numel()
    if sync is None:
        sync = fused_sync(x.device, M, stream)
    if sync.numel() < fused_sync_words(M):
        raise ValueError("sync buffer too small")
    f16, i32 = torch.float16, torch.int32
    st = lib().rmoe_forward_fused_f16(
        _dev(x, f16, "stacked_expert_tokens"), _dev(gate_w, f16, "gate_w"),
        _dev(up_w, f16, "up_w"), _dev(down_w, f16, "down_w"),
        _dev(routed_expert_weights, torch.float32, "routed_expert_weights"),
        _dev(group_sizes, i32, "group_sizes"), _dev(group_offsets, i32, "group_offsets"),
        _dev(group_padded_offsets, i32, "group_padded_offsets"),
        _dev(group_idx_for_bx, i32, "group_idx_for_bx"), _dev(workspace, f16, "workspace"),
        _dev(out, f16, "out"), _dev(sync, i32, "sync"), H, I, E, Tp,
        routed_expert_weights.numel(), M, int(max_wait_us), _HANDOVER[handover],
        _stream(x, stream))
    _check(st, "rmoe_forward_fused_f16")


def gate_up(stacked_expert_tokens, gate_w, up_w, group_sizes, group_padded_offsets,
            group_idx_for_bx, workspace, num_pairs, variant="auto", stream=None):
    """Stage 1 alone: workspace = fp16(silu(x Wg^T) * (x Wu^T)) on valid rows.
    ``num_pairs`` (routed rows, group_offsets[E]) feeds the family choice."""
    torch = _torch()
    x = stacked_expert_tokens
    E, I, H = gate_w.shape
    f16, i32 = torch.float16, torch.int32
    st = lib().rmoe_gate_up_f16(
        _dev(x, f16, "stacked_expert_tokens"), _dev(gate_w, f16, "gate_w"),
        _dev(up_w, f16, "up_w"), _dev(group_sizes, i32, "group_sizes"),
        _dev(group_padded_offsets, i32, "group_padded_offsets"),
        _dev(group_idx_for_bx, i32, "group_idx_for_bx"), _dev(workspace, f16, "workspace"),
        H, I, E, x.shape[0], int(num_pairs), group_idx_for_bx.numel(), _VARIANTS[variant],
        _stream(x, stream))
    _check(st, "rmoe_gate_up_f16")


def down(workspace, down_w, routed_expert_weights, group_sizes, group_offsets,
         group_padded_offsets, group_idx_for_bx, out, variant="auto", stream=None):
    """Stage 2 alone: out = fp16((hidden Wd^T) * w[compact row]) on valid rows."""
    torch = _torch()
    E, H, I = down_w.shape
    f16, i32 = torch.float16, torch.int32
    st = lib().rmoe_down_f16(
        _dev(workspace, f16, "workspace"), _dev(down_w, f16, "down_w"),
        _dev(routed_expert_weights, torch.float32, "routed_expert_weights"),
        _dev(group_sizes, i32, "group_sizes"), _dev(group_offsets, i32, "group_offsets"),
        _dev(group_padded_offsets, i32, "group_padded_offsets"),
        _dev(group_idx_for_bx, i32, "group_idx_for_bx"), _dev(out, f16, "out"), H, I, E,
        workspace.shape[0], routed_expert_weights.numel(), group_idx_for_bx.numel(),
        _VARIANTS[variant], _stream(workspace, stream))
    _check(st, "rmoe_down_f16")


def pack(x, topk_weights, padded_row_of_pair, compact_pos_of_pair, stacked, w_compact,
         stream=None):
    """Gather token rows into the padded expert-sorted layout and the routed
    weights into compact order (device tensors)."""
    torch = _torch()
    T, H = x.shape
    pairs = topk_weights.numel()
    k = pairs // T if T else 0
    st = lib().rmoe_pack_f16(
        _dev(x, torch.float16, "x"), _dev(topk_weights, torch.float32, "topk_weights"),
        _dev(padded_row_of_pair, torch.int32, "padded_row_of_pair"),
        _dev(compact_pos_of_pair, torch.int32, "compact_pos_of_pair"), T, k, H,
        _dev(stacked, torch.float16, "stacked"), _dev(w_compact, torch.float32, "w_compact"),
        stacked.shape[0], _stream(x, stream))
    _check(st, "rmoe_pack_f16")


def combine(out, padded_row_of_pair, top_k, y, stream=None):
    """y[t] = fp16(sum over the token's k slots of out[padded row])."""
    torch = _torch()
    T, H = y.shape
    st = lib().rmoe_combine_f16(
        _dev(out, torch.float16, "out"), _dev(padded_row_of_pair, torch.int32, "padded_row_of_pair"),
        T, int(top_k), H, _dev(y, torch.float16, "y"), out.shape[0], _stream(out, stream))
    _check(st, "rmoe_combine_f16")


def router(x, router_w, top_k: int, topk_ids=None, topk_weights=None, stream=None):
    """Top-k expert ids (int32) and softmax scores (fp32) of ``x @ router_w^T``
    for x [T, H] and router_w [E, H] fp16 device tensors; returns
    ``(topk_ids, topk_weights)``, both [T, top_k]."""
    torch = _torch()
    T, H = x.shape
    E = router_w.shape[0]
    if router_w.dim() != 2 or router_w.shape[1] != H:
        raise ValueError("router_w must be [E, H]")
    if topk_ids is None:
        topk_ids = torch.empty((T, top_k), dtype=torch.int32, device=x.device)
    if topk_weights is None:
        topk_weights = torch.empty((T, top_k), dtype=torch.float32, device=x.device)
    st = lib().rmoe_router_f16(_dev(x, torch.float16, "x"), _dev(router_w, torch.float16, "router_w"),
                               T, H, E, int(top_k), _dev(topk_ids, torch.int32, "topk_ids"),
                               _dev(topk_weights, torch.float32, "topk_weights"), _stream(x, stream))
    _check(st, "rmoe_router_f16")
    return topk_ids, topk_weights


def contract_workspace_bytes(num_pairs: int, num_experts: int) -> int:
    """Device scratch bytes ``build_contract_device`` needs."""
    return int(lib().rmoe_contract_workspace_bytes(num_pairs, num_experts))


def build_contract_device(topk_ids, num_experts: int, stream=None, out=None) -> dict:
    """The dispatch contract built on the GPU from device top-k ids
    ``[T, k]`` int32.  Returns device int32 tensors ``group_sizes``,
    ``group_offsets``, ``group_padded_offsets``, ``group_idx_for_bx``,
    ``order``, ``padded_row_of_pair``, ``compact_pos_of_pair``, ``bad_ids``
    (one entry: pairs with an expert id outside [0, E), which the tables
    leave out) and the host ints ``num_blocks_m``, ``total_padded_tokens``
    and ``pairs``.  Asynchronous on ``stream``; no host round trip.
    ``out``: a dict an earlier call returned for the same T, k and E; its
    tensors (scratch included) are filled again and returned, so the call
    allocates nothing.  The earlier tables are overwritten in stream order."""
    torch = _torch()
    if topk_ids.dim() != 2:
        raise ValueError("topk_ids must be [T, k]")
    T, k = topk_ids.shape
    pairs, E = T * k, int(num_experts)
    M, Tp = contract_sizes(pairs, E)
    dev = topk_ids.device
    nbytes = contract_workspace_bytes(pairs, E)
    if nbytes == 0:
        raise RmoeError(f"device contract: unsupported expert count {E}")
    if out is not None:
        if (out.get("pairs"), out.get("num_blocks_m"), out["group_sizes"].numel()) != (pairs, M, E) \
                or out["_workspace"].device != dev:
            raise ValueError("out was built for another shape or device")
        ws = out["_workspace"]
    else:
        i32 = lambda n: torch.empty(max(n, 1), dtype=torch.int32, device=dev)[:n]
        out = {"group_sizes": i32(E), "group_offsets": i32(E + 1), "group_padded_offsets": i32(E + 1),
               "group_idx_for_bx": i32(M), "order": i32(pairs), "padded_row_of_pair": i32(pairs),
               "compact_pos_of_pair": i32(pairs), "bad_ids": i32(1)}
        ws = torch.empty((nbytes + 3) // 4, dtype=torch.int32, device=dev)
    nb = ctypes.c_int32(0)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    st = lib().rmoe_build_contract_device(
        _dev(topk_ids.contiguous(), torch.int32, "topk_ids") if pairs else ctypes.c_void_p(0),
        T, k, E, ptr(out["group_sizes"]), ptr(out["group_offsets"]),
        ptr(out["group_padded_offsets"]), ptr(out["group_idx_for_bx"]), M, ctypes.byref(nb),
        ptr(out["order"]), ptr(out["padded_row_of_pair"]), ptr(out["compact_pos_of_pair"]),
        ptr(out["bad_ids"]), ptr(ws), nbytes, _stream(topk_ids, stream))
    _check(st, "rmoe_build_contract_device")
    out["_workspace"] = ws  # keeps the scratch alive until the stream has used it
    out.update(num_blocks_m=nb.value, total_padded_tokens=Tp, pairs=pairs)
    return out


def build_contract_device_noalloc(topk_ids, num_experts: int, out: dict, stream=None) -> dict:
    """rmoe_build_contract_device_noalloc: the same tables as
    ``build_contract_device``, written into the caller's ``out`` tensors
    (a dict as that function returns, for the same T, k and E), with the
    library's static scratch instead of a workspace: nothing is allocated.
    Calls that overlap in time on one GPU share that scratch and race."""
    torch = _torch()
    if topk_ids.dim() != 2:
        raise ValueError("topk_ids must be [T, k]")
    T, k = topk_ids.shape
    pairs, E = T * k, int(num_experts)
    if out.get("pairs") != pairs or out["group_sizes"].numel() != E:
        raise ValueError("out was built for another shape")
    nb = ctypes.c_int32(0)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    st = lib().rmoe_build_contract_device_noalloc(
        _dev(topk_ids, torch.int32, "topk_ids") if pairs else ctypes.c_void_p(0),
        T, k, E, ptr(out["group_sizes"]), ptr(out["group_offsets"]),
        ptr(out["group_padded_offsets"]), ptr(out["group_idx_for_bx"]),
        out["group_idx_for_bx"].numel(), ctypes.byref(nb), ptr(out["order"]),
        ptr(out["padded_row_of_pair"]), ptr(out["compact_pos_of_pair"]), ptr(out["bad_ids"]),
        _stream(topk_ids, stream))
    _check(st, "rmoe_build_contract_device_noalloc")
    out["num_blocks_m"] = nb.value
    return out


_WORKSPACE = {}


def _get_workspace(stacked_expert_tokens, intermediate):
    torch = _torch()
    x = stacked_expert_tokens
    key = (x.device.index or 0, int(x.shape[0]), int(intermediate), str(x.dtype))
    ws = _WORKSPACE.get(key)
    if ws is None:
        ws = torch.empty((int(x.shape[0]), int(intermediate)), device=x.device, dtype=x.dtype)
        _WORKSPACE[key] = ws
    return ws


def run_kernel(stacked_expert_tokens, gate_w, up_w, down_w, routed_expert_weights, group_sizes,
               group_offsets, group_padded_offsets, group_idx_for_bx, out):
    """Submission-style entry: derives the sizes from the tensors, uses a
    cached workspace, enqueues the forward; no sync, no return value."""
    ws = _get_workspace(stacked_expert_tokens, gate_w.shape[1])
    forward(stacked_expert_tokens, gate_w, up_w, down_w, routed_expert_weights, group_sizes,
            group_offsets, group_padded_offsets, group_idx_for_bx, ws, out)
