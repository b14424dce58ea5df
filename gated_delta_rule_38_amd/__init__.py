"""MI355X (gfx950) Kimi Delta Attention chunked prefill.

A thin ctypes binding over ``libkda.so`` (C ABI in ``include/kda.h``): it only
turns torch tensors into descriptors, allocates outputs/workspace with torch
and passes the current HIP stream.  Every step of the computation runs in the
library's HIP kernels; there is no fallback.  Importing works without a GPU
(so the ABI can be inspected on a CPU host), but every compute entry point
raises if the library or a GPU is missing.

Names follow the C ABI: ``prefill`` (kda_prefill / kda_prefill_ws),
``prefill_noalloc`` (kda_prefill_noalloc), ``workspace_size``, ``prep``
(kda_prep), ``decode`` (kda_decode),
``profile_enable``/``profile_read``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkda.so")

KDA_BF16, KDA_F32, KDA_I32 = 0, 1, 2
STATUS = {0: "KDA_OK", 1: "KDA_ERR_NULL", 2: "KDA_ERR_SHAPE", 3: "KDA_ERR_DTYPE", 4: "KDA_ERR_LAYOUT",
          5: "KDA_ERR_ALIAS", 6: "KDA_ERR_UNSUPPORTED", 7: "KDA_ERR_WORKSPACE", 8: "KDA_ERR_HIP",
          9: "KDA_ERR_RANGE"}
EXPORTS = ("kda_prefill", "kda_prefill_workspace_size", "kda_prefill_ws", "kda_prefill_noalloc", "kda_prep", "kda_decode",
           "kda_release_cached_workspace", "kda_profile_enable", "kda_profile_read", "kda_profile_read_kernels",
           "kda_status_string", "kda_last_error", "kda_abi_version",
           # measurement probes (include/kda_peak.h)
           "kda_peak_stream", "kda_peak_mfma")


class KdaTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


class KdaOptions(ctypes.Structure):
    _fields_ = [("nseg", ctypes.c_int32), ("prep", ctypes.c_int32),
                ("stall_wave", ctypes.c_int32), ("stall_cycles", ctypes.c_int32), ("variant", ctypes.c_int32),
                ("gate_act", ctypes.c_int32), ("gate_lower_bound", ctypes.c_float), ("beta_act", ctypes.c_int32),
                ("out_gate", ctypes.POINTER(KdaTensor)), ("norm_weight", ctypes.POINTER(KdaTensor)),
                ("norm_eps", ctypes.c_float), ("split_chains", ctypes.c_int32)]


class KdaProfileEntry(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double)]


class KdaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH):
    """Loads libkda.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m gated_delta_rule_38_amd.build`")
    lib = ctypes.CDLL(path)
    T = ctypes.POINTER(KdaTensor)
    O = ctypes.POINTER(KdaOptions)
    V = ctypes.c_void_p
    lib.kda_prefill.argtypes = [T, T, T, T, T, T, T, T, T, V]
    lib.kda_prefill.restype = ctypes.c_int
    lib.kda_prefill_ws.argtypes = [T, T, T, T, T, T, T, T, T, O, V, ctypes.c_size_t, V]
    lib.kda_prefill_ws.restype = ctypes.c_int
    lib.kda_prefill_noalloc.argtypes = [T, T, T, T, T, T, T, T, T, O, V]
    lib.kda_prefill_noalloc.restype = ctypes.c_int
    lib.kda_prefill_workspace_size.argtypes = [T, T, T, T, T, T, T, T, T, O, ctypes.POINTER(ctypes.c_size_t)]
    lib.kda_prefill_workspace_size.restype = ctypes.c_int
    lib.kda_decode.argtypes = [T, T, T, T, T, T, T, T, T, ctypes.c_int32, O, V]
    lib.kda_decode.restype = ctypes.c_int
    lib.kda_prep.argtypes = [T, T, ctypes.c_int32, T, V]
    lib.kda_prep.restype = ctypes.c_int
    lib.kda_release_cached_workspace.argtypes = []
    lib.kda_release_cached_workspace.restype = None
    lib.kda_profile_enable.argtypes = [ctypes.c_int]
    lib.kda_profile_enable.restype = None
    lib.kda_profile_read.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    lib.kda_profile_read.restype = ctypes.c_int
    lib.kda_profile_read_kernels.argtypes = [ctypes.POINTER(KdaProfileEntry), ctypes.c_int32,
                                             ctypes.POINTER(ctypes.c_int32)]
    lib.kda_profile_read_kernels.restype = ctypes.c_int
    lib.kda_peak_stream.argtypes = [ctypes.POINTER(ctypes.c_void_p), V, ctypes.c_int64, V]
    lib.kda_peak_stream.restype = ctypes.c_int
    lib.kda_peak_mfma.argtypes = [V, ctypes.c_int32, ctypes.c_int32, V]
    lib.kda_peak_mfma.restype = ctypes.c_int
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_last_error.argtypes = []
    lib.kda_last_error.restype = ctypes.c_char_p
    lib.kda_abi_version.argtypes = []
    lib.kda_abi_version.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        raise KdaError(status, load_library().kda_last_error().decode())


_DTYPE_CODES = None
_I64x4 = ctypes.c_int64 * 4


def describe(t, dtype_code: Optional[int] = None) -> KdaTensor:
    """A torch tensor as a kda_tensor_t (strides in elements)."""
    global _DTYPE_CODES
    if _DTYPE_CODES is None:
        import torch
        _DTYPE_CODES = {torch.bfloat16: KDA_BF16, torch.float32: KDA_F32, torch.int32: KDA_I32}
    n = t.dim()
    if n > 4:
        raise ValueError("at most 4 dimensions")
    code = _DTYPE_CODES.get(t.dtype, -1) if dtype_code is None else dtype_code
    pad = (0,) * (4 - n)
    return KdaTensor(t.data_ptr() if t.numel() > 0 else None, code, n,
                     _I64x4(*t.shape, *pad), _I64x4(*t.stride(), *pad))


def _ptr(d: Optional[KdaTensor]):
    return ctypes.byref(d) if d is not None else None


def _descs(q, k, v, g, beta, initial_state, cu_seqlens, out, final_state):
    return [describe(q), describe(k), describe(v), describe(g), describe(beta),
            describe(initial_state) if initial_state is not None else None,
            describe(cu_seqlens) if cu_seqlens is not None else None,
            describe(out), describe(final_state) if final_state is not None else None]


def _require_gpu(*tensors):
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("gated_delta_rule_38_amd needs a ROCm GPU (gfx950); none is visible")
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")


def _stream(device, stream):
    """(torch stream, raw hipStream_t) for a call: the current stream when None, else a
    torch.cuda.Stream or a raw handle (wrapped as an external stream)."""
    import torch
    if stream is None:
        s = torch.cuda.current_stream(device)
    elif isinstance(stream, torch.cuda.Stream):
        s = stream
    else:
        s = torch.cuda.ExternalStream(int(stream), device=device)
    return s, s.cuda_stream


def options(nseg: int = 0, prep: int = 0, stall_wave: int = -1, stall_cycles: int = 0, variant: int = 0,
            gate_logits: bool = False, gate_lower_bound: float = -5.0, beta_logits: bool = False,
            out_gate=None, norm_weight=None, norm_eps: float = 1e-6, split_chains: int = 0) -> KdaOptions:
    o = KdaOptions()
    o.nseg, o.prep, o.variant, o.split_chains = nseg, prep, variant, split_chains
    o.gate_act, o.gate_lower_bound, o.beta_act = int(bool(gate_logits)), gate_lower_bound, int(bool(beta_logits))
    o.norm_eps = norm_eps
    if out_gate is not None or norm_weight is not None:
        # the descriptors live as long as the options object
        o._norm = (describe(out_gate) if out_gate is not None else None,
                   describe(norm_weight) if norm_weight is not None else None)
        if o._norm[0] is not None:
            o.out_gate = ctypes.pointer(o._norm[0])
        if o._norm[1] is not None:
            o.norm_weight = ctypes.pointer(o._norm[1])
    o.stall_wave = stall_wave + 1 if stall_wave >= 0 else 0
    o.stall_cycles = stall_cycles
    return o


def _alloc_outputs(q, v, cu_seqlens, initial_state, out, final_state, want_final):
    import torch
    if out is None:
        out = torch.empty(v.shape, dtype=v.dtype, device=v.device)
    if final_state is None and want_final:
        N = (cu_seqlens.numel() - 1) if cu_seqlens is not None else q.shape[0]
        H, D = q.shape[-2], q.shape[-1]
        final_state = torch.empty((N, H, D, v.shape[-1]), dtype=torch.float32, device=q.device)
    return out, final_state


def workspace_size(q, k, v, g, beta, initial_state=None, cu_seqlens=None, out=None, final_state=None,
                   nseg: int = 0, prep: int = 0, variant: int = 0, gate_logits: bool = False,
                   gate_lower_bound: float = -5.0, beta_logits: bool = False, split_chains: int = 0) -> int:
    lib = load_library()
    out, final_state = _alloc_outputs(q, v, cu_seqlens, initial_state, out, final_state, False)
    ds = _descs(q, k, v, g, beta, initial_state, cu_seqlens, out, final_state)
    n = ctypes.c_size_t(0)
    opts = options(nseg, prep, variant=variant, gate_logits=gate_logits, gate_lower_bound=gate_lower_bound,
                   beta_logits=beta_logits, split_chains=split_chains)
    _check(lib.kda_prefill_workspace_size(*[_ptr(d) for d in ds], ctypes.byref(opts), ctypes.byref(n)))
    return n.value


def prefill(q, k, v, g, beta, initial_state=None, cu_seqlens=None, out=None, final_state=None,
            output_final_state: bool = True, nseg: int = 0, prep: int = 0, stall_wave: int = -1,
            stall_cycles: int = 0, variant: int = 0, gate_logits: bool = False, gate_lower_bound: float = -5.0,
            beta_logits: bool = False, out_gate=None, norm_weight=None, norm_eps: float = 1e-6,
            split_chains: int = 0, workspace=None, stream=None) -> Tuple:
    """KDA chunked prefill.  Returns (out, final_state).

    Dense layout: q, k, g [B, T, H, K], v [B, T, H, V], beta [B, T, H].
    Packed layout: q, k, g [T, H, K], v [T, H, V], beta [T, H] and int32
    ``cu_seqlens`` [N + 1] on the GPU.  States are fp32 [N, H, K, V].
    ``gate_logits``: g holds logits x, the log decay is gate_lower_bound * sigmoid(x);
    ``beta_logits``: beta holds logits, beta = sigmoid(beta) (both fused into the gate scan).
    ``out_gate``, ``norm_weight``, ``norm_eps``: the gated RMS norm output epilogue,
    out = o * rsqrt(mean(o^2) + eps) * norm_weight * sigmoid(out_gate) per (token, head).
    With the default knobs this calls ``kda_prefill`` (library-cached
    workspace); any knob or a ``workspace`` tensor routes through
    ``kda_prefill_ws`` with a torch-allocated workspace.
    ``stream``: None (torch's current stream), a torch.cuda.Stream or a raw
    hipStream_t handle; outputs and workspace this call allocates are allocated
    on that stream.
    """
    import torch
    lib = load_library()
    _require_gpu(q, k, v, g, beta, initial_state, cu_seqlens, out, final_state)
    sobj, st = _stream(q.device, stream)
    # Everything allocated here is allocated on the stream the kernels run on, so torch's
    # caching allocator never hands a block to another stream while they may still use it.
    with torch.cuda.stream(sobj):
        out, final_state = _alloc_outputs(q, v, cu_seqlens, initial_state, out, final_state, output_final_state)
    ds = _descs(q, k, v, g, beta, initial_state, cu_seqlens, out, final_state)
    plain = (nseg == 0 and prep == 0 and stall_wave < 0 and variant == 0 and workspace is None
             and not gate_logits and not beta_logits and out_gate is None and norm_weight is None
             and split_chains == 0)
    if plain:
        _check(lib.kda_prefill(*[_ptr(d) for d in ds], ctypes.c_void_p(st)))
        return out, final_state
    opts = options(nseg, prep, stall_wave, stall_cycles, variant, gate_logits, gate_lower_bound, beta_logits,
                   out_gate, norm_weight, norm_eps, split_chains)
    need = ctypes.c_size_t(0)
    _check(lib.kda_prefill_workspace_size(*[_ptr(d) for d in ds], ctypes.byref(opts), ctypes.byref(need)))
    if workspace is None and need.value:
        with torch.cuda.stream(sobj):
            workspace = torch.empty(need.value + 256, dtype=torch.uint8, device=q.device)
    wptr, wbytes = None, 0
    if workspace is not None:
        base = workspace.data_ptr()
        aligned = (base + 255) // 256 * 256
        wptr, wbytes = aligned, workspace.numel() - (aligned - base)
    _check(lib.kda_prefill_ws(*[_ptr(d) for d in ds], ctypes.byref(opts), ctypes.c_void_p(wptr),
                              ctypes.c_size_t(wbytes), ctypes.c_void_p(st)))
    return out, final_state


NOALLOC_SCRATCH_BYTES = 64 << 20


def prefill_noalloc(q, k, v, g, beta, initial_state=None, cu_seqlens=None, out=None, final_state=None,
                    nseg: int = 0, prep: int = 0, variant: int = 0, gate_logits: bool = False,
                    gate_lower_bound: float = -5.0, beta_logits: bool = False, out_gate=None, norm_weight=None,
                    norm_eps: float = 1e-6, stream=None) -> Tuple:
    """kda_prefill_noalloc: the prefill with its scratch in the library's fixed device array
    (no allocation in the library).  ``out`` and ``final_state`` must be given: the call
    allocates nothing, here either.  Returns (out, final_state)."""
    lib = load_library()
    _require_gpu(q, k, v, g, beta, initial_state, cu_seqlens, out, final_state)
    if out is None:
        raise ValueError("prefill_noalloc allocates nothing: pass out (and final_state, or None to skip it)")
    _, st = _stream(q.device, stream)
    ds = _descs(q, k, v, g, beta, initial_state, cu_seqlens, out, final_state)
    opts = options(nseg, prep, variant=variant, gate_logits=gate_logits, gate_lower_bound=gate_lower_bound,
                   beta_logits=beta_logits, out_gate=out_gate, norm_weight=norm_weight, norm_eps=norm_eps)
    _check(lib.kda_prefill_noalloc(*[_ptr(d) for d in ds], ctypes.byref(opts), ctypes.c_void_p(st)))
    return out, final_state


def decode(q, k, v, g, beta, state_pool, state_indices, num_tokens=None, out=None, update_state: bool = True,
           write_out: bool = True, gate_logits: bool = False, gate_lower_bound: float = -5.0,
           beta_logits: bool = False, stall_wave: int = -1, stall_cycles: int = 0, out_gate=None,
           norm_weight=None, norm_eps: float = 1e-6, stream=None):
    """Recurrent decode / draft verify against a state pool (kda_decode).

    q, k, g [R, T, H, K]; v [R, T, H, V]; beta [R, T, H]; 1 <= T <= 8.
    state_pool [P, H, K, V] fp32 or bf16; state_indices int32 [R] (negative:
    skip the request); num_tokens int32 [R] or None (all T tokens).
    update_state=False is the verify pass (the pool is only read);
    write_out=False with update_state=True is the replay-only commit.
    Returns out (allocated when not given and write_out), or None.
    """
    import torch
    lib = load_library()
    _require_gpu(q, k, v, g, beta, state_pool, state_indices, num_tokens, out)
    sobj, st = _stream(q.device, stream)
    if out is None and write_out:
        with torch.cuda.stream(sobj):
            out = torch.empty(v.shape, dtype=v.dtype, device=v.device)
    opts = options(stall_wave=stall_wave, stall_cycles=stall_cycles, gate_logits=gate_logits,
                   gate_lower_bound=gate_lower_bound, beta_logits=beta_logits, out_gate=out_gate,
                   norm_weight=norm_weight, norm_eps=norm_eps)
    do = describe(out) if out is not None else None
    dn = describe(num_tokens) if num_tokens is not None else None
    _check(lib.kda_decode(ctypes.byref(describe(q)), ctypes.byref(describe(k)), ctypes.byref(describe(v)),
                          ctypes.byref(describe(g)), ctypes.byref(describe(beta)), ctypes.byref(describe(state_pool)),
                          ctypes.byref(describe(state_indices)), _ptr(dn), _ptr(do), ctypes.c_int32(int(update_state)),
                          ctypes.byref(opts), ctypes.c_void_p(st)))
    return out


def prep(g, cu_seqlens=None, gamma=None, chunk: int = 64, stream=None):
    """Standalone PREP kernel: in-chunk (``chunk`` = 32 or 64 tokens) inclusive cumsum of g."""
    import torch
    lib = load_library()
    _require_gpu(g, cu_seqlens, gamma)
    sobj, st = _stream(g.device, stream)
    if gamma is None:
        with torch.cuda.stream(sobj):
            gamma = torch.empty_like(g)
    dc = describe(cu_seqlens) if cu_seqlens is not None else None
    _check(lib.kda_prep(ctypes.byref(describe(g)), _ptr(dc), ctypes.c_int32(chunk), ctypes.byref(describe(gamma)),
                        ctypes.c_void_p(st)))
    return gamma


def profile_enable(on: bool = True) -> None:
    load_library().kda_profile_enable(1 if on else 0)


def profile_read(kernel: Optional[str] = None) -> Tuple[float, int]:
    """(summed milliseconds, launches) of the library's kernels whose name
    contains ``kernel`` (None: all) since the last read; synchronises their
    events.  Every read clears all recorded launches, counted or not."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    _check(load_library().kda_profile_read(kernel.encode() if kernel else None, ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def profile_read_kernels() -> dict:
    """{kernel name: (launches, summed milliseconds)} of every launch recorded since the last
    read, grouped by kernel; synchronises their events and clears them all."""
    entries = (KdaProfileEntry * 16)()
    n = ctypes.c_int32(0)
    _check(load_library().kda_profile_read_kernels(entries, 16, ctypes.byref(n)))
    return {entries[i].name.decode(): (entries[i].launches, entries[i].total_ms) for i in range(n.value)}


def peak_stream(inputs, out, stream=None) -> None:
    """Measurement probe: out = xor of the five inputs (16-byte elements, equal sizes)."""
    import torch
    if len(inputs) != 5 or any(t.numel() * t.element_size() != out.numel() * out.element_size() for t in inputs):
        raise ValueError("five inputs of out's size")
    _require_gpu(*inputs, out)
    arr = (ctypes.c_void_p * 5)(*[t.data_ptr() for t in inputs])
    _, st = _stream(out.device, stream)
    n16 = out.numel() * out.element_size() // 16
    _check(load_library().kda_peak_stream(arr, ctypes.c_void_p(out.data_ptr()), n16, ctypes.c_void_p(st)))


def peak_mfma(out, workgroups: int, iters: int, stream=None) -> None:
    """Measurement probe: a loop of independent bf16 MFMAs (out: fp32, workgroups * 4 floats)."""
    _require_gpu(out)
    if out.numel() < workgroups * 4:
        raise ValueError("out holds one float per wave")
    _, st = _stream(out.device, stream)
    _check(load_library().kda_peak_mfma(ctypes.c_void_p(out.data_ptr()), workgroups, iters, ctypes.c_void_p(st)))


def release_cached_workspace() -> None:
    load_library().kda_release_cached_workspace()
