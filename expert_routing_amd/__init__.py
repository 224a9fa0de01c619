"""Python binding of libmoe.so, the MI355X MoE-layer forward pass.

Argument marshalling only: every function here takes torch tensors, passes their
device pointers and the current HIP stream to the C ABI of include/moe.h under the same
name, and raises MoeError on a non-zero status. All compute runs in the library's HIP
kernels; there is no fallback. Importing this package fails loudly when the library has
not been built (python expert_routing_amd/build.py).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# EXPERT_ROUTING_AMD_LIB may name another build of the same library (for example one built
# with different tile settings); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("EXPERT_ROUTING_AMD_LIB") or os.path.join(_HERE, "libmoe.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python expert_routing_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)

SCORE = {"softmax": 0, "sigmoid": 1}
DTYPE = {"f32": 0, "bf16": 1, "mxfp8": 2, "bf16_packed": 3}
# activations of each act_dtype (MX-FP8 and packed-weight problems keep bf16 activations)
_TORCH_DTYPE = {0: torch.float32, 1: torch.bfloat16, 2: torch.bfloat16, 3: torch.bfloat16}


class Problem(ctypes.Structure):
    """Mirror of `moe_problem`."""
    _fields_ = [
        ("T", ctypes.c_int64),
        ("h", ctypes.c_int32), ("E", ctypes.c_int32), ("K", ctypes.c_int32),
        ("score", ctypes.c_int32),
        ("renorm", ctypes.c_int32),
        ("n_groups", ctypes.c_int32), ("topk_groups", ctypes.c_int32),
        ("capacity_factor", ctypes.c_double),
        ("pad_to_capacity", ctypes.c_int32),
        ("n_ep", ctypes.c_int32), ("ep_rank", ctypes.c_int32),
        ("inter", ctypes.c_int32), ("n_shared", ctypes.c_int32), ("shared_inter", ctypes.c_int32),
        ("act_dtype", ctypes.c_int32),
    ]

    def __init__(self, T, h, E, K, score="softmax", renorm=True, n_groups=1, topk_groups=1,
                 capacity_factor=0.0, pad=False, n_ep=1, ep_rank=0, inter=0, n_shared=0,
                 shared_inter=0, dtype="bf16"):
        super().__init__(int(T), int(h), int(E), int(K), SCORE[score], int(bool(renorm)),
                         int(n_groups), int(topk_groups), float(capacity_factor), int(bool(pad)),
                         int(n_ep), int(ep_rank), int(inter), int(n_shared), int(shared_inter),
                         DTYPE[dtype])

    @property
    def torch_dtype(self):
        return _TORCH_DTYPE[self.act_dtype]

    @property
    def E_local(self):
        return self.E // self.n_ep


class Tensors(ctypes.Structure):
    """Mirror of `moe_tensors`."""
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "x", "w_router", "bias", "w13", "w2", "w13_sh", "w2_sh", "topk_ids", "topk_w",
        "counts", "offsets", "dest_row", "row_src", "send_bytes", "n_dropped", "xp", "yp",
        "y_sh", "y", "w13_scale", "w2_scale", "w13_sh_scale", "w2_sh_scale")]


class ReplicaMap(ctypes.Structure):
    """Mirror of `moe_replica_map` (device pointers)."""
    _fields_ = [("P", ctypes.c_int32), ("rep_start", ctypes.c_void_p),
                ("rep_list", ctypes.c_void_p), ("phys_expert", ctypes.c_void_p),
                ("phys_replica", ctypes.c_void_p)]


_P = ctypes.POINTER(Problem)
_V = ctypes.c_void_p
_SZ = ctypes.c_size_t


def _sig(name, args, res=ctypes.c_int):
    f = getattr(_lib, name)
    f.argtypes = args
    f.restype = res
    return f


_check_problem = _sig("moe_check_problem", [_P])
_capacity = _sig("moe_capacity", [_P, ctypes.POINTER(ctypes.c_int64)])
_max_rows = _sig("moe_max_rows", [_P, ctypes.POINTER(ctypes.c_int64)])
_workspace_bytes = _sig("moe_workspace_bytes", [_P, ctypes.POINTER(ctypes.c_size_t)])
_status_string = _sig("moe_status_string", [ctypes.c_int], ctypes.c_char_p)
_route = _sig("moe_route", [_P, _V, _V, _V, _V, _V, _V, _SZ, _V])
_select = _sig("moe_select", [_P, _V, _V, _V, _V, _V])
_dispatch = _sig("moe_dispatch", [_P, _V, _V, _V, _V, _V, _V, _V, _V, _V, _V, _SZ, _V])
_expert_ffn = _sig("moe_expert_ffn", [_P, _V, _V, _V, _V, _V, _V, _V, _V, _V, _V, _V, _SZ, _V])
_combine = _sig("moe_combine", [_P, _V, _V, _V, _V, _V, _V])
_layout_stats = _sig("moe_layout_stats", [_P, _V, _V, _V, _V, _V, _V, _SZ, _V])
_forward = _sig("moe_forward", [_P, ctypes.POINTER(Tensors), _V, _SZ, _V])
_forward_traced = _sig("moe_forward_traced",
                       [_P, ctypes.POINTER(Tensors), _V, _SZ, _V, ctypes.POINTER(_V)])
_forward_noalloc = _sig("moe_forward_noalloc", [_P, ctypes.POINTER(Tensors), _V])
_quantize_mx = _sig("moe_quantize_mx", [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _V, _V,
                                        _V, _V])
_pack_weights = _sig("moe_pack_weights", [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _V, _V,
                                          _V])
_RM = ctypes.POINTER(ReplicaMap)
_replica_plan = _sig("moe_replica_plan", [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                          _V, _V, _V, _V, _V, _V])
_replicated_sizes = _sig("moe_replicated_sizes", [_P, ctypes.c_int32,
                                                  ctypes.POINTER(ctypes.c_int64),
                                                  ctypes.POINTER(ctypes.c_size_t)])
_dispatch_replicated = _sig("moe_dispatch_replicated",
                            [_P, _RM, _V, _V, _V, _V, _V, _V, _V, _V, _V, _SZ, _V])
_forward_replicated = _sig("moe_forward_replicated", [_P, _RM, ctypes.POINTER(Tensors), _V, _SZ,
                                                      _V])
NOALLOC_SCRATCH_BYTES = 64 << 20   # MOE_NOALLOC_SCRATCH_BYTES
TRACE_POINTS = ["begin", "route", "dispatch", "ffn_prep", "ffn_gate_up", "ffn_down", "combine"]

EXPORTED = ["moe_check_problem", "moe_capacity", "moe_max_rows", "moe_workspace_bytes",
            "moe_status_string", "moe_route", "moe_select", "moe_dispatch", "moe_expert_ffn",
            "moe_combine", "moe_layout_stats", "moe_forward", "moe_forward_traced",
            "moe_forward_noalloc", "moe_replica_plan", "moe_replicated_sizes",
            "moe_dispatch_replicated", "moe_forward_replicated", "moe_quantize_mx",
            "moe_pack_weights"]


class MoeError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


def status_string(status: int) -> str:
    return _status_string(int(status)).decode()


def _ok(status, where):
    if status != 0:
        raise MoeError(status, where)


def _ptr(t):
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _ws(ws):
    return (None, 0) if ws is None else (ws.data_ptr(), ws.numel() * ws.element_size())


def check_problem(p: Problem) -> int:
    return _check_problem(ctypes.byref(p))


def capacity(p: Problem) -> int:
    v = ctypes.c_int64()
    _ok(_capacity(ctypes.byref(p), ctypes.byref(v)), "moe_capacity")
    return v.value


def max_rows(p: Problem) -> int:
    v = ctypes.c_int64()
    _ok(_max_rows(ctypes.byref(p), ctypes.byref(v)), "moe_max_rows")
    return v.value


def workspace_bytes(p: Problem) -> int:
    v = ctypes.c_size_t()
    _ok(_workspace_bytes(ctypes.byref(p), ctypes.byref(v)), "moe_workspace_bytes")
    return v.value


def moe_route(p, x, w_router, bias, topk_ids, topk_w, ws, stream=None):
    wp, wn = _ws(ws)
    _ok(_route(ctypes.byref(p), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(topk_ids),
               _ptr(topk_w), wp, wn, _stream(stream)), "moe_route")


def moe_select(p, logits, bias, topk_ids, topk_w, stream=None):
    _ok(_select(ctypes.byref(p), _ptr(logits), _ptr(bias), _ptr(topk_ids), _ptr(topk_w),
                _stream(stream)), "moe_select")


def moe_dispatch(p, x, topk_ids, counts, offsets, dest_row, row_src, send_bytes, n_dropped, xp,
                 ws, stream=None):
    wp, wn = _ws(ws)
    _ok(_dispatch(ctypes.byref(p), _ptr(x), _ptr(topk_ids), _ptr(counts), _ptr(offsets),
                  _ptr(dest_row), _ptr(row_src), _ptr(send_bytes), _ptr(n_dropped), _ptr(xp),
                  wp, wn, _stream(stream)), "moe_dispatch")


def moe_expert_ffn(p, xp, offsets, w13, w2, x, w13_sh, w2_sh, yp, y_sh, ws, stream=None,
                   row_src=None):
    """xp=None with row_src: the gate/up GEMM reads its rows from x through row_src."""
    wp, wn = _ws(ws)
    _ok(_expert_ffn(ctypes.byref(p), _ptr(xp), _ptr(row_src), _ptr(offsets), _ptr(w13),
                    _ptr(w2), _ptr(x), _ptr(w13_sh), _ptr(w2_sh), _ptr(yp), _ptr(y_sh), wp, wn,
                    _stream(stream)), "moe_expert_ffn")


def moe_combine(p, yp, dest_row, topk_w, y_sh, y, stream=None):
    _ok(_combine(ctypes.byref(p), _ptr(yp), _ptr(dest_row), _ptr(topk_w), _ptr(y_sh), _ptr(y),
                 _stream(stream)), "moe_combine")


def moe_layout_stats(p, topk_ids, tokens_to, recv_pairs, fanout_hist, busiest, ws,
                     stream=None):
    wp, wn = _ws(ws)
    _ok(_layout_stats(ctypes.byref(p), _ptr(topk_ids), _ptr(tokens_to), _ptr(recv_pairs),
                      _ptr(fanout_hist), _ptr(busiest), wp, wn, _stream(stream)),
        "moe_layout_stats")


def moe_quantize_mx(src, codes, scales, stream=None):
    """MX-FP8 codes [rows][cols] and scale bytes [rows][cols/32] (uint8 tensors) of a 2-D
    fp32 or bf16 tensor."""
    rows, cols = src.shape
    sd = {torch.float32: DTYPE["f32"], torch.bfloat16: DTYPE["bf16"]}.get(src.dtype)
    if sd is None or not src.is_contiguous():
        raise MoeError(-1, "moe_quantize_mx: src must be a contiguous fp32 or bf16 tensor")
    for t, shape in ((codes, (rows, cols)), (scales, (rows, cols // 32))):
        if t.dtype != torch.uint8 or tuple(t.shape) != shape or not t.is_contiguous():
            raise MoeError(-1, f"moe_quantize_mx: expected contiguous uint8 {shape}")
    _ok(_quantize_mx(rows, cols, sd, _ptr(src), _ptr(codes), _ptr(scales), _stream(stream)),
        "moe_quantize_mx")


def quantize_mx(src, stream=None):
    """(codes, scales) of src, allocated here."""
    rows, cols = src.shape
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=src.device)
    scales = torch.empty((rows, max(cols // 32, 0)), dtype=torch.uint8, device=src.device)
    moe_quantize_mx(src, codes, scales, stream)
    return codes, scales


def moe_pack_weights(src, dst, stream=None):
    """Packs bf16 matrices src [mats][rows][cols] (or one [rows][cols]) into dst (same shape
    and dtype) in the fragment order MOE_DTYPE_BF16_PACKED problems read."""
    if src.dtype != torch.bfloat16 or dst.dtype != torch.bfloat16 or src.shape != dst.shape:
        raise MoeError(-1, "moe_pack_weights: src and dst must be bf16 tensors of one shape")
    if not (src.is_contiguous() and dst.is_contiguous()) or src.dim() not in (2, 3):
        raise MoeError(-1, "moe_pack_weights: contiguous [mats][rows][cols] or [rows][cols]")
    mats, rows, cols = (1, *src.shape) if src.dim() == 2 else tuple(src.shape)
    _ok(_pack_weights(mats, rows, cols, _ptr(src), _ptr(dst), _stream(stream)),
        "moe_pack_weights")


def pack_weights(src, stream=None):
    """src packed into a tensor allocated here."""
    dst = torch.empty_like(src)
    moe_pack_weights(src, dst, stream)
    return dst


def moe_forward(p, t: dict, ws, stream=None):
    ts = Tensors(**{k: _ptr(t.get(k)) for k, _ in Tensors._fields_})
    wp, wn = _ws(ws)
    _ok(_forward(ctypes.byref(p), ctypes.byref(ts), wp, wn, _stream(stream)), "moe_forward")


def moe_forward_noalloc(p, t: dict, stream=None):
    """moe_forward with the library's own device scratch array as workspace (no ws)."""
    ts = Tensors(**{k: _ptr(t.get(k)) for k, _ in Tensors._fields_})
    _ok(_forward_noalloc(ctypes.byref(p), ctypes.byref(ts), _stream(stream)),
        "moe_forward_noalloc")


def moe_forward_traced(p, t: dict, ws, events, stream=None):
    """`events`: len(TRACE_POINTS) raw hipEvent_t handles (see HipEvents)."""
    ts = Tensors(**{k: _ptr(t.get(k)) for k, _ in Tensors._fields_})
    arr = (_V * len(TRACE_POINTS))(*events)
    wp, wn = _ws(ws)
    _ok(_forward_traced(ctypes.byref(p), ctypes.byref(ts), wp, wn, _stream(stream), arr),
        "moe_forward_traced")


def replica_plan(E, R, n_ep, load):
    """moe_replica_plan on host arrays: returns counts, rep_start, rep_list, phys_expert,
    phys_replica as int32 numpy arrays."""
    import numpy as np
    P = E + R
    ld = np.ascontiguousarray(np.asarray(load, dtype=np.int64))
    out = {"counts": np.zeros(E, np.int32), "rep_start": np.zeros(E + 1, np.int32),
           "rep_list": np.zeros(P, np.int32), "phys_expert": np.zeros(P, np.int32),
           "phys_replica": np.zeros(P, np.int32)}
    ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    _ok(_replica_plan(int(E), int(R), int(n_ep), ptr(ld), ptr(out["counts"]),
                      ptr(out["rep_start"]), ptr(out["rep_list"]), ptr(out["phys_expert"]),
                      ptr(out["phys_replica"])), "moe_replica_plan")
    return out


def replicated_sizes(p: Problem, P: int):
    rows, nb = ctypes.c_int64(), ctypes.c_size_t()
    _ok(_replicated_sizes(ctypes.byref(p), int(P), ctypes.byref(rows), ctypes.byref(nb)),
        "moe_replicated_sizes")
    return rows.value, nb.value


class DeviceReplicaMap:
    """A replica map copied to the device (keeps the tensors alive)."""

    def __init__(self, plan: dict, device="cuda"):
        self.t = {k: torch.as_tensor(plan[k]).to(device=device, dtype=torch.int32)
                  for k in ("rep_start", "rep_list", "phys_expert", "phys_replica")}
        self.P = int(len(plan["rep_list"]))
        self.c = ReplicaMap(self.P, *(self.t[k].data_ptr() for k in
                                      ("rep_start", "rep_list", "phys_expert", "phys_replica")))


def moe_dispatch_replicated(p, rmap: DeviceReplicaMap, topk_ids, counts, phys_counts, offsets,
                            dest_row, row_src, send_bytes, n_dropped, ws, stream=None):
    wp, wn = _ws(ws)
    _ok(_dispatch_replicated(ctypes.byref(p), ctypes.byref(rmap.c), _ptr(topk_ids), _ptr(counts),
                             _ptr(phys_counts), _ptr(offsets), _ptr(dest_row), _ptr(row_src),
                             _ptr(send_bytes), _ptr(n_dropped), wp, wn, _stream(stream)),
        "moe_dispatch_replicated")


def moe_forward_replicated(p, rmap: DeviceReplicaMap, t: dict, ws, stream=None):
    ts = Tensors(**{k: _ptr(t.get(k)) for k, _ in Tensors._fields_})
    wp, wn = _ws(ws)
    _ok(_forward_replicated(ctypes.byref(p), ctypes.byref(rmap.c), ctypes.byref(ts), wp, wn,
                            _stream(stream)), "moe_forward_replicated")


def alloc_buffers_replicated(p: Problem, P: int, device="cuda", send=True) -> dict:
    """alloc_buffers for a layer over P physical experts."""
    rows, nb = replicated_sizes(p, P)
    b = alloc_buffers(p, device, send)
    Pl = P // p.n_ep
    R = max(rows, 1)
    b["offsets"] = torch.empty((Pl + 1,), dtype=torch.int32, device=device)
    b["phys_counts"] = torch.empty((P,), dtype=torch.int32, device=device)
    b["row_src"] = torch.empty((R,), dtype=torch.int32, device=device)
    b["xp"] = torch.empty((R, p.h), dtype=p.torch_dtype, device=device)
    b["yp"] = torch.empty((R, p.h), dtype=p.torch_dtype, device=device)
    b["ws"] = torch.empty((max(nb, 256),), dtype=torch.uint8, device=device)
    return b


class HipEvents:
    """Raw hipEvent_t handles (timing enabled) from the HIP runtime, for the traced
    forward; elapsed(a, b) is hipEventElapsedTime in milliseconds."""

    def __init__(self, n):
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(_V)]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), _V, _V]
        self._hip.hipEventDestroy.argtypes = [_V]
        self.handles = []
        for _ in range(n):
            e = _V()
            if self._hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.handles.append(e.value)

    def record(self, i, stream=None):
        """hipEventRecord of handle i on `stream` (default: torch's current stream)."""
        self._hip.hipEventRecord.argtypes = [_V, _V]
        if self._hip.hipEventRecord(self.handles[i], _stream(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed(self, a, b):
        ms = ctypes.c_float()
        if self._hip.hipEventElapsedTime(ctypes.byref(ms), self.handles[a], self.handles[b]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self):
        for h in self.handles:
            self._hip.hipEventDestroy(h)
        self.handles = []


def alloc_buffers(p: Problem, device="cuda", send=True) -> dict:
    """Output and intermediate buffers of one layer call, plus its workspace."""
    T, K, E, El, h = p.T, p.K, p.E, p.E_local, p.h
    R = max_rows(p)
    dt = p.torch_dtype
    i32 = torch.int32
    b = {
        "topk_ids": torch.empty((T, K), dtype=i32, device=device),
        "topk_w": torch.empty((T, K), dtype=torch.float32, device=device),
        "counts": torch.empty((E,), dtype=i32, device=device),
        "offsets": torch.empty((El + 1,), dtype=i32, device=device),
        "dest_row": torch.empty((T, K), dtype=i32, device=device),
        "row_src": torch.empty((max(R, 1),), dtype=i32, device=device),
        "send_bytes": (torch.empty((p.n_ep, p.n_ep), dtype=torch.int64, device=device)
                       if send and T % p.n_ep == 0 else None),
        "n_dropped": torch.empty((1,), dtype=i32, device=device),
        "xp": torch.empty((max(R, 1), h), dtype=dt, device=device),
        "yp": torch.empty((max(R, 1), h), dtype=dt, device=device),
        "y_sh": (torch.empty((T // p.n_ep, h), dtype=dt, device=device) if p.n_shared else None),
        "y": torch.empty((T, h), dtype=dt, device=device),
    }
    nbytes = workspace_bytes(p)
    b["ws"] = torch.empty((max(nbytes, 256),), dtype=torch.uint8, device=device)
    return b


def problem_from_config(cfg, T=None, dtype=None) -> Problem:
    """Problem for a workload description with the fields of synth.MoEConfig (dtype, when
    given, overrides the workload's: "bf16_packed" for bf16 with packed expert weights)."""
    return Problem(T=cfg.T if T is None else T, h=cfg.h, E=cfg.E, K=cfg.K, score=cfg.score,
                   renorm=cfg.renorm, n_groups=cfg.n_groups, topk_groups=cfg.topk_groups,
                   capacity_factor=cfg.capacity_factor, pad=cfg.pad, n_ep=cfg.n_ep,
                   ep_rank=cfg.ep_rank, inter=cfg.inter, n_shared=cfg.n_shared,
                   shared_inter=cfg.shared_inter, dtype=dtype or cfg.dtype)
