"""int8 Hadamard-domain MoE gate_up on AMD Instinct MI355X (gfx950).

Thin Python binding over libi8h.so (C ABI declared in include/i8h.h). Every
function here only checks tensors, allocates outputs with torch and passes
device pointers plus torch's current HIP stream to the library; all of the
computation runs in the library's HIP kernels. There is no CPU fallback: if
the library is not built, or a tensor is not on the GPU, the call raises.

Functions (same names as the C entry points):
  moe_route_permute          top-k routing and the expert-sorted permutation
  moe_route_permute_noalloc  the same without a workspace (fixed device scratch)
  moe_route_permute_rotate   routing plus the rotation of the routed tokens' rows
  hadamard128_rotate         blockwise 128-wide Walsh-Hadamard rotation (bf16)
  moe_gateup_i8h_grouped     grouped int8 Hadamard-domain gate_up + GELU epilogue
  moe_gateup_i8h_grouped_fused  the same on unrotated activations (rotation fused)
  moe_route_gateup_i8h_decode   routing + rotation + gate_up in one launch (few tokens)
  fp8_quantize_activations   per-token, per-128 E4M3 activation quantizer
  moe_gateup_fp8blk_grouped  grouped FP8 E4M3 128x128-block gate_up + epilogue
  moe_down_bf16_combine      bf16 grouped down projection + weighted combine
                             (the step after the path)
  linear_i8f16               dense int8 linear with f16 group scales (the
                             drafter's linears)
  i8_quantize_activations    per-token, per-128 int8 activation quantizer (W8A8)
  moe_gateup_i8g_grouped     grouped W8A8 int8 g128 gate_up + epilogue
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libi8h.so")

I8H_OK, I8H_EINVAL, I8H_EUNSUPPORTED, I8H_EHIP = 0, -1, -2, -3
PATHS = {"auto": 0, "gemv": 1, "gemm": 2, "tall": 3, "skinny": 4}
DOWN_PATHS = {"auto": 0, "gemv": 1, "gemm": 2}

_lib = None


class I8HError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        msg = lib().i8h_status_string(status).decode()
        super().__init__(f"{fn} failed: {msg} ({status})")


def lib():
    """The loaded libi8h.so, with argument types set. Raises if not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                           "(python -m int8_hadamard_domain_amd.build_lib)")
    L = ctypes.CDLL(LIB_PATH)
    P, I, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "i8h_status_string": (ctypes.c_char_p, [I]),
        "moe_route_permute_workspace_size": (SZ, [I, I, I]),
        "moe_route_permute": (I, [P, I, I, I, P, P, P, P, P, P, SZ, P]),
        "moe_route_permute_noalloc": (I, [P, I, I, I, P, P, P, P, P, P]),
        "moe_route_permute_rotate": (I, [P, P, I, I, I, I, P, P, P, P, P, P, P, SZ, P]),
        "hadamard128_rotate": (I, [P, I64, P, I64, I, I, P]),
        "moe_gateup_i8h_grouped": (I, [P, I, I, P, P, I, I, I, P, P, P, P, P]),
        "moe_gateup_i8h_grouped_path": (I, [P, I, I, P, P, I, I, I, P, P, P, P, I, P]),
        "moe_gateup_i8h_grouped_act_bf16": (I, [P, I, I, P, P, I, I, I, P, P, P, P, I, P]),
        "moe_gateup_i8h_fused_workspace_size": (SZ, [I, I]),
        "moe_gateup_i8h_grouped_fused": (I, [P, I, I, P, P, I, I, I, P, P, P, P, P, SZ, P]),
        "moe_route_gateup_i8h_decode": (I, [P, P, I, I, P, P, I, I, I, P, P, P, P, P, P, P, P]),
        "fp8_quantize_activations": (I, [P, I, I, P, P, P]),
        "moe_gateup_fp8blk_workspace_size": (SZ, [I, I]),
        "moe_gateup_fp8blk_grouped": (I, [P, I, I, P, P, I, I, I, P, P, P, P, P, SZ, P]),
        "moe_gateup_fp8blk_grouped_path": (I, [P, I, I, P, P, I, I, I, P, P, P, P, P, SZ, I, P]),
        "moe_gateup_fp8blk_grouped_act_bf16": (I, [P, I, I, P, P, I, I, I, P, P, P, P, P, SZ, I, P]),
        "i8_quantize_activations": (I, [P, I, I, P, P, P]),
        "moe_gateup_i8g_workspace_size": (SZ, [I, I]),
        "moe_gateup_i8g_grouped": (I, [P, I, I, P, P, I, I, I, P, P, P, P, P, SZ, P]),
        "moe_gateup_i8g_grouped_act_bf16": (I, [P, I, I, P, P, I, I, I, P, P, P, P, P, SZ, P]),
        "moe_down_bf16_workspace_size": (SZ, [I, I, I, I]),
        "moe_down_bf16_combine": (I, [P, I, I, P, I, I, I, P, P, P, P, P, P, SZ, P]),
        "moe_down_bf16_combine_path": (I, [P, I, I, P, I, I, I, P, P, P, P, P, P, SZ, I, P]),
        "moe_down_bf16_act_bf16_workspace_size": (SZ, [I, I, I, I]),
        "moe_down_bf16_combine_act_bf16": (I, [P, I, I, P, I, I, I, P, P, P, P, P, P, SZ, I, P]),
        "linear_i8f16": (I, [P, I, I, P, P, I, P, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _check(fn, status):
    if status != I8H_OK:
        raise I8HError(fn, status)


def _dev(t, name, dtype, ndim=None, shape=None, device=None):
    """Check one tensor handed to the library: a torch.Tensor on the GPU (on
    `device` when given), of `dtype`, contiguous, with `ndim` dimensions or
    exactly `shape`. Raises TypeError / ValueError before anything is launched."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device} (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions (got {t.dim()})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _workspace(ws, name, need, device):
    """A caller's byte workspace (uint8, 1-D, at least `need` bytes, on
    `device`), or a new one when ws is None."""
    if ws is None:
        return torch.empty((max(need, 1),), dtype=torch.uint8, device=device)
    _dev(ws, name, torch.uint8, 1, device=device)
    if ws.numel() < need:
        raise ValueError(f"{name} must hold at least {need} bytes (got {ws.numel()})")
    return ws


def _routing_outputs(out, T, E, topk, device):
    """The five routing tensors (from `out` where given, checked, else new)."""
    o = dict(out or {})
    i32, f32 = torch.int32, torch.float32
    want = {"topk_ids": (i32, (T, topk)), "topk_w": (f32, (T, topk)), "expert_off": (i32, (E + 1,)),
            "sorted_pairs": (i32, (T * topk,)), "pair_pos": (i32, (T * topk,))}
    for key, (dt, shape) in want.items():
        if key in o:
            _dev(o[key], key, dt, shape=shape, device=device)
        else:
            o[key] = torch.empty(shape, dtype=dt, device=device)
    return o


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def moe_route_permute(logits, topk, out=None):
    """logits [T, E] float32 -> dict of topk_ids [T, k] int32, topk_w [T, k]
    float32, expert_off [E+1] int32, sorted_pairs [T*k] int32, pair_pos
    [T*k] int32 (and the workspace used). `out` may hold preallocated
    tensors under the same keys."""
    _dev(logits, "logits", torch.float32, 2)
    T, E = logits.shape
    dev = logits.device
    o = _routing_outputs(out, T, E, topk, dev)
    ws_bytes = lib().moe_route_permute_workspace_size(T, E, topk)
    o["workspace"] = _workspace(o.get("workspace"), "workspace", ws_bytes, dev)
    _check("moe_route_permute", lib().moe_route_permute(
        _ptr(logits), T, E, topk, _ptr(o["topk_ids"]), _ptr(o["topk_w"]), _ptr(o["expert_off"]),
        _ptr(o["sorted_pairs"]), _ptr(o["pair_pos"]), _ptr(o["workspace"]), o["workspace"].numel(),
        _stream(dev)))
    return o


def moe_route_permute_rotate(logits, x, topk, out=None, x_rot=None):
    """moe_route_permute on logits [T, E] float32, and the 128-wide Hadamard
    rotation of the activation rows x [T, K] bf16 in the same pass: returns
    the routing dict with "x_rot" [T, K] bf16 added (x_rot may be x itself)."""
    _dev(logits, "logits", torch.float32, 2)
    T, E = logits.shape
    dev = logits.device
    _dev(x, "x", torch.bfloat16, 2, device=dev)
    K = x.shape[1]
    _dev(x, "x", torch.bfloat16, shape=(T, K))
    o = _routing_outputs(out, T, E, topk, dev)
    xr = torch.empty_like(x) if x_rot is None else _dev(x_rot, "x_rot", torch.bfloat16, shape=(T, K), device=dev)
    ws_bytes = lib().moe_route_permute_workspace_size(T, E, topk)
    o["workspace"] = _workspace(o.get("workspace"), "workspace", ws_bytes, dev)
    _check("moe_route_permute_rotate", lib().moe_route_permute_rotate(
        _ptr(logits), _ptr(x), T, E, topk, K, _ptr(o["topk_ids"]), _ptr(o["topk_w"]), _ptr(o["expert_off"]),
        _ptr(o["sorted_pairs"]), _ptr(o["pair_pos"]), _ptr(xr), _ptr(o["workspace"]), o["workspace"].numel(),
        _stream(dev)))
    o["x_rot"] = xr
    return o


def moe_route_permute_noalloc(logits, topk, out=None):
    """moe_route_permute without a workspace: the library's own fixed device
    scratch holds the histograms (1 MiB per GPU; calls that overlap on one
    GPU race on it). Same results; `out` may hold the five output tensors."""
    _dev(logits, "logits", torch.float32, 2)
    T, E = logits.shape
    dev = logits.device
    o = _routing_outputs(out, T, E, topk, dev)
    _check("moe_route_permute_noalloc", lib().moe_route_permute_noalloc(
        _ptr(logits), T, E, topk, _ptr(o["topk_ids"]), _ptr(o["topk_w"]), _ptr(o["expert_off"]),
        _ptr(o["sorted_pairs"]), _ptr(o["pair_pos"]), _stream(dev)))
    return o


def hadamard128_rotate(x, out=None):
    """bf16 [T, K] (K % 128 == 0) -> bf16 [T, K], blockwise H x / sqrt(128).
    `out` may be x itself (in place)."""
    _dev(x, "x", torch.bfloat16, 2)
    T, K = x.shape
    y = torch.empty_like(x) if out is None else _dev(out, "out", torch.bfloat16, shape=(T, K), device=x.device)
    _check("hadamard128_rotate", lib().hadamard128_rotate(
        _ptr(x), K, _ptr(y), y.shape[1], T, K, _stream(x.device)))
    return y


def moe_gateup_i8h_grouped(x_rot, codes, scales, topk, expert_off, sorted_pairs,
                           gate_up=True, act=True, path="auto", act_dtype=torch.float32):
    """Grouped int8 Hadamard-domain gate_up.

    x_rot [T, K] bf16 (rotated), codes [E, N, K] int8, scales [E, N, K/128]
    bf16, expert_off [E+1] / sorted_pairs [T*topk] int32 from
    moe_route_permute. gate_up / act: True to allocate, a tensor to write
    into, or False/None to skip. act is float32, or bfloat16 (act_dtype, or
    the dtype of a given tensor: each value rounded to nearest even from the
    float32 one, the input moe_down_bf16_combine takes without rounding it
    again). Returns (gate_up, act) in expert-sorted row order (None for
    skipped outputs).
    """
    _dev(x_rot, "x_rot", torch.bfloat16, 2)
    T, K = x_rot.shape
    dev = x_rot.device
    _dev(codes, "codes", torch.int8, 3, device=dev)
    E, N, _ = codes.shape
    _dev(codes, "codes", torch.int8, shape=(E, N, K))
    _dev(scales, "scales", torch.bfloat16, shape=(E, N, K // 128), device=dev)
    _dev(expert_off, "expert_off", torch.int32, shape=(E + 1,), device=dev)
    _dev(sorted_pairs, "sorted_pairs", torch.int32, shape=(T * topk,), device=dev)
    gu = _out(gate_up, (T * topk, N), dev)
    adt = _act_dtype(act, act_dtype)
    ac = _out(act, (T * topk, N // 2), dev, adt)
    fn = "moe_gateup_i8h_grouped_act_bf16" if adt == torch.bfloat16 else "moe_gateup_i8h_grouped_path"
    _check(fn, getattr(lib(), fn)(
        _ptr(x_rot), T, K, _ptr(codes), _ptr(scales), E, N, topk, _ptr(expert_off), _ptr(sorted_pairs),
        _ptr(gu), _ptr(ac), PATHS[path], _stream(dev)))
    return gu, ac


def moe_gateup_i8h_grouped_fused(x, codes, scales, topk, expert_off, sorted_pairs,
                                 gate_up=True, act=True, workspace=None):
    """moe_gateup_i8h_grouped on UNROTATED bf16 activations x [T, K]: the
    128-wide Hadamard rotation is applied inside the call. Returns
    (gate_up, act)."""
    _dev(x, "x", torch.bfloat16, 2)
    T, K = x.shape
    dev = x.device
    _dev(codes, "codes", torch.int8, 3, device=dev)
    E, N, _ = codes.shape
    _dev(codes, "codes", torch.int8, shape=(E, N, K))
    _dev(scales, "scales", torch.bfloat16, shape=(E, N, K // 128), device=dev)
    _dev(expert_off, "expert_off", torch.int32, shape=(E + 1,), device=dev)
    _dev(sorted_pairs, "sorted_pairs", torch.int32, shape=(T * topk,), device=dev)
    need = lib().moe_gateup_i8h_fused_workspace_size(T, K)
    if need > 0 or workspace is not None:
        workspace = _workspace(workspace, "workspace", need, dev)
    gu = _out(gate_up, (T * topk, N), dev)
    ac = _out(act, (T * topk, N // 2), dev)
    _check("moe_gateup_i8h_grouped_fused", lib().moe_gateup_i8h_grouped_fused(
        _ptr(x), T, K, _ptr(codes), _ptr(scales), E, N, topk, _ptr(expert_off), _ptr(sorted_pairs),
        _ptr(gu), _ptr(ac), _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(dev)))
    return gu, ac


def moe_route_gateup_i8h_decode(logits, x, codes, scales, topk, gate_up=True, act=True, out=None):
    """Decode step in one launch: moe_route_permute on logits [T, E] float32,
    then the fused-rotation gate_up on UNROTATED x [T, K] bf16 (T*topk <= 64,
    E <= 256, K <= 4096). Returns (routing dict as moe_route_permute's,
    gate_up, act). `out` may hold preallocated routing tensors."""
    _dev(logits, "logits", torch.float32, 2)
    T, E = logits.shape
    dev = logits.device
    _dev(x, "x", torch.bfloat16, 2, device=dev)
    K = x.shape[1]
    _dev(x, "x", torch.bfloat16, shape=(T, K))
    _dev(codes, "codes", torch.int8, 3, device=dev)
    N = codes.shape[1]
    _dev(codes, "codes", torch.int8, shape=(E, N, K))
    _dev(scales, "scales", torch.bfloat16, shape=(E, N, K // 128), device=dev)
    o = _routing_outputs(out, T, E, topk, dev)
    gu = _out(gate_up, (T * topk, N), dev)
    ac = _out(act, (T * topk, N // 2), dev)
    _check("moe_route_gateup_i8h_decode", lib().moe_route_gateup_i8h_decode(
        _ptr(logits), _ptr(x), T, K, _ptr(codes), _ptr(scales), E, N, topk, _ptr(o["topk_ids"]),
        _ptr(o["topk_w"]), _ptr(o["expert_off"]), _ptr(o["sorted_pairs"]), _ptr(o["pair_pos"]),
        _ptr(gu), _ptr(ac), _stream(dev)))
    return o, gu, ac


def _out(spec, shape, dev, dtype=torch.float32):
    if spec is None or spec is False:
        return None
    if spec is True:
        return torch.empty(shape, dtype=dtype, device=dev)
    return _dev(spec, "output", dtype, shape=shape, device=dev)


def _act_dtype(act, act_dtype):
    """The act output's dtype: a given tensor's own, else act_dtype (float32 or bfloat16)."""
    dt = act.dtype if isinstance(act, torch.Tensor) else act_dtype
    if dt not in (torch.float32, torch.bfloat16):
        raise TypeError(f"act must be float32 or bfloat16 (got {dt})")
    return dt


def fp8_quantize_activations(x, qx=None, sx=None):
    """bf16 [T, K] -> (E4M3 codes uint8 [T, K], float32 scales [T, K/128])."""
    _dev(x, "x", torch.bfloat16, 2)
    T, K = x.shape
    dev = x.device
    qx = (torch.empty((T, K), dtype=torch.uint8, device=dev) if qx is None
          else _dev(qx, "qx", torch.uint8, shape=(T, K), device=dev))
    sx = (torch.empty((T, K // 128), dtype=torch.float32, device=dev) if sx is None
          else _dev(sx, "sx", torch.float32, shape=(T, K // 128), device=dev))
    _check("fp8_quantize_activations", lib().fp8_quantize_activations(
        _ptr(x), T, K, _ptr(qx), _ptr(sx), _stream(x.device)))
    return qx, sx


def moe_gateup_fp8blk_grouped(x, codes, scales, topk, expert_off, sorted_pairs,
                              gate_up=True, act=True, workspace=None, path="auto", act_dtype=torch.float32):
    """Grouped FP8 E4M3 128x128-block gate_up.

    x [T, K] bf16 (not rotated), codes [E, N, K] uint8 (E4M3 bytes), scales
    [E, N/128, K/128] bf16. path: "auto", "gemm" or "skinny". act float32 or
    bfloat16 as for moe_gateup_i8h_grouped. Returns (gate_up, act,
    workspace); the workspace holds the quantized activations (see
    fp8_workspace_views).
    """
    _dev(x, "x", torch.bfloat16, 2)
    T, K = x.shape
    dev = x.device
    _dev(codes, "codes", torch.uint8, 3, device=dev)
    E, N, _ = codes.shape
    _dev(codes, "codes", torch.uint8, shape=(E, N, K))
    _dev(scales, "scales", torch.bfloat16, shape=(E, N // 128, K // 128), device=dev)
    _dev(expert_off, "expert_off", torch.int32, shape=(E + 1,), device=dev)
    _dev(sorted_pairs, "sorted_pairs", torch.int32, shape=(T * topk,), device=dev)
    need = lib().moe_gateup_fp8blk_workspace_size(T, K)
    workspace = _workspace(workspace, "workspace", need, dev)
    gu = _out(gate_up, (T * topk, N), dev)
    adt = _act_dtype(act, act_dtype)
    ac = _out(act, (T * topk, N // 2), dev, adt)
    fn = "moe_gateup_fp8blk_grouped_act_bf16" if adt == torch.bfloat16 else "moe_gateup_fp8blk_grouped_path"
    _check(fn, getattr(lib(), fn)(
        _ptr(x), T, K, _ptr(codes), _ptr(scales), E, N, topk, _ptr(expert_off), _ptr(sorted_pairs),
        _ptr(gu), _ptr(ac), _ptr(workspace), workspace.numel(), PATHS[path], _stream(dev)))
    return gu, ac, workspace


def fp8_workspace_views(workspace, T, K):
    """(qx [T, K] uint8, sx [T, K/128] float32, xq [T, K] bf16) views of a
    moe_gateup_fp8blk_grouped workspace: codes, scales and the codes' exact
    bf16 values."""
    up = lambda v: (v + 255) // 256 * 256
    a = up(T * K)
    b = a + up(T * (K // 128) * 4)
    qx = workspace[:T * K].view(T, K)
    sx = workspace[a:a + T * (K // 128) * 4].view(torch.float32).view(T, K // 128)
    xq = workspace[b:b + T * K * 2].view(torch.bfloat16).view(T, K)
    return qx, sx, xq


def moe_down_bf16_combine(act, w_down, routing, out=None, workspace=None, path="auto"):
    """bf16 grouped down projection of the expert-sorted act rows [P, I]
    float32 (rounded to bf16 for the product), or bfloat16 (taken as they
    are: the gate_up calls' bf16 act), against w_down [E, H, I] bf16, merged
    per token with the router weights: returns out [T, H] float32.
    `routing` is moe_route_permute's dict (topk_ids, topk_w, expert_off,
    pair_pos); `path` is "auto", "gemv" (one launch) or "gemm" (GEMM +
    combine)."""
    if not isinstance(act, torch.Tensor) or act.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("act must be a float32 or bfloat16 tensor")
    bf = act.dtype == torch.bfloat16
    _dev(act, "act", act.dtype, 2)
    P, I = act.shape
    dev = act.device
    _dev(w_down, "w_down", torch.bfloat16, 3, device=dev)
    E, H, _ = w_down.shape
    _dev(w_down, "w_down", torch.bfloat16, shape=(E, H, I))
    ids = _dev(routing["topk_ids"], "topk_ids", torch.int32, 2, device=dev)
    T, topk = ids.shape
    if P != T * topk:
        raise ValueError(f"act must have T * topk = {T * topk} rows (got {P})")
    tw = _dev(routing["topk_w"], "topk_w", torch.float32, shape=(T, topk), device=dev)
    off = _dev(routing["expert_off"], "expert_off", torch.int32, shape=(E + 1,), device=dev)
    pos = _dev(routing["pair_pos"], "pair_pos", torch.int32, shape=(P,), device=dev)
    need = (lib().moe_down_bf16_act_bf16_workspace_size if bf else lib().moe_down_bf16_workspace_size)(T, I, H, topk)
    if path != "gemv" or workspace is not None:
        workspace = _workspace(workspace, "workspace", need, dev)
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=dev)
    else:
        _dev(out, "out", torch.float32, shape=(T, H), device=dev)
    fn = "moe_down_bf16_combine_act_bf16" if bf else "moe_down_bf16_combine_path"
    _check(fn, getattr(lib(), fn)(
        _ptr(act), T, I, _ptr(w_down), E, H, topk, _ptr(ids), _ptr(tw), _ptr(off), _ptr(pos), _ptr(out),
        _ptr(workspace), 0 if workspace is None else workspace.numel(), DOWN_PATHS[path], _stream(dev)))
    return out


def linear_i8f16(x, codes, scales, out=None):
    """Dense int8 linear: x [T, K] bf16 (unrotated), codes [N, K] int8,
    scales [N, K/128] float16 -> y [T, N] float32."""
    _dev(x, "x", torch.bfloat16, 2)
    T, K = x.shape
    dev = x.device
    _dev(codes, "codes", torch.int8, 2, device=dev)
    N = codes.shape[0]
    _dev(codes, "codes", torch.int8, shape=(N, K))
    _dev(scales, "scales", torch.float16, shape=(N, K // 128), device=dev)
    if out is None:
        out = torch.empty((T, N), dtype=torch.float32, device=dev)
    else:
        _dev(out, "out", torch.float32, shape=(T, N), device=dev)
    _check("linear_i8f16", lib().linear_i8f16(_ptr(x), T, K, _ptr(codes), _ptr(scales), N, _ptr(out), _stream(dev)))
    return out


def i8_quantize_activations(x):
    """x [T, K] bf16 -> (qx int8 [T, K], sx float32 [T, K/128])."""
    _dev(x, "x", torch.bfloat16, 2)
    T, K = x.shape
    qx = torch.empty((T, K), dtype=torch.int8, device=x.device)
    sx = torch.empty((T, K // 128), dtype=torch.float32, device=x.device)
    _check("i8_quantize_activations", lib().i8_quantize_activations(
        _ptr(x), T, K, _ptr(qx), _ptr(sx), _stream(x.device)))
    return qx, sx


def moe_gateup_i8g_grouped(x, codes, scales, topk, expert_off, sorted_pairs,
                           gate_up=True, act=True, workspace=None, act_dtype=torch.float32):
    """Grouped W8A8 int8 g128 gate_up.

    x [T, K] bf16 (not rotated), codes [E, N, K] int8, scales [E, N, K/128]
    bf16. act float32 or bfloat16 as for moe_gateup_i8h_grouped. Returns
    (gate_up, act, workspace); the workspace holds the int8 activations and
    their scales (see i8g_workspace_views).
    """
    _dev(x, "x", torch.bfloat16, 2)
    T, K = x.shape
    dev = x.device
    _dev(codes, "codes", torch.int8, 3, device=dev)
    E, N, _ = codes.shape
    _dev(codes, "codes", torch.int8, shape=(E, N, K))
    _dev(scales, "scales", torch.bfloat16, shape=(E, N, K // 128), device=dev)
    _dev(expert_off, "expert_off", torch.int32, shape=(E + 1,), device=dev)
    _dev(sorted_pairs, "sorted_pairs", torch.int32, shape=(T * topk,), device=dev)
    need = lib().moe_gateup_i8g_workspace_size(T, K)
    workspace = _workspace(workspace, "workspace", need, dev)
    gu = _out(gate_up, (T * topk, N), dev)
    adt = _act_dtype(act, act_dtype)
    ac = _out(act, (T * topk, N // 2), dev, adt)
    fn = "moe_gateup_i8g_grouped_act_bf16" if adt == torch.bfloat16 else "moe_gateup_i8g_grouped"
    _check(fn, getattr(lib(), fn)(
        _ptr(x), T, K, _ptr(codes), _ptr(scales), E, N, topk, _ptr(expert_off), _ptr(sorted_pairs),
        _ptr(gu), _ptr(ac), _ptr(workspace), workspace.numel(), _stream(dev)))
    return gu, ac, workspace


def i8g_workspace_views(workspace, T, K):
    """(qx [T, K] int8, sx [T, K/128] float32) views of a moe_gateup_i8g_grouped workspace."""
    a = (T * K + 255) // 256 * 256
    qx = workspace[:T * K].view(torch.int8).view(T, K)
    sx = workspace[a:a + T * (K // 128) * 4].view(torch.float32).view(T, K // 128)
    return qx, sx
