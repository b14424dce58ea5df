"""C-ABI checks that need no GPU: the library loads, exports every function
include/kda.h declares, and the host-side validator returns the documented
status codes (nothing is launched on an error, so these run on any host).
"""
import ctypes
import os
import re

import pytest

import gated_delta_rule_38_amd as kda
from gated_delta_rule_38_amd import KdaTensor, KDA_BF16, KDA_F32, KDA_I32

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.LIB_PATH):
        from gated_delta_rule_38_amd import build
        build.build(verbose=False)
    return kda.load_library()


def header_functions():
    text = "\n".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    """Every function declared in include/*.h (kda.h and the measurement probes of
    kda_peak.h) is exported by libkda.so and bound by the Python package."""
    assert len(HEADERS) >= 2
    names = header_functions()
    assert set(names) == set(kda.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), f"libkda.so does not export {n}"


def test_abi_version_and_status_strings(lib):
    assert lib.kda_abi_version() == 4
    assert lib.kda_status_string(0) == b"KDA_OK"
    assert lib.kda_status_string(5) == b"KDA_ERR_ALIAS"
    assert lib.kda_status_string(8) == b"KDA_ERR_HIP"
    assert lib.kda_status_string(9) == b"KDA_ERR_RANGE"


FAKE = 1 << 40   # a non-NULL, 256-aligned address; never dereferenced on the error paths


def desc(shape, dtype=KDA_BF16, base=FAKE, strides=None):
    d = KdaTensor()
    d.data = base
    d.dtype = dtype
    d.ndim = len(shape)
    if strides is None:
        strides, acc = [], 1
        for s in reversed(shape):
            strides.insert(0, acc)
            acc *= s
    for i, (s, st) in enumerate(zip(shape, strides)):
        d.shape[i] = s
        d.stride[i] = st
    return d


def packed_set(T=100, H=2, D=128, N=3, dt=KDA_BF16):
    gap = 1 << 32
    return dict(q=desc([T, H, D], dt, FAKE), k=desc([T, H, D], dt, FAKE + gap),
                v=desc([T, H, D], dt, FAKE + 2 * gap), g=desc([T, H, D], KDA_F32, FAKE + 3 * gap),
                beta=desc([T, H], KDA_F32, FAKE + 4 * gap), s0=desc([N, H, D, D], KDA_F32, FAKE + 5 * gap),
                cu=desc([N + 1], KDA_I32, FAKE + 6 * gap), out=desc([T, H, D], dt, FAKE + 7 * gap),
                sT=desc([N, H, D, D], KDA_F32, FAKE + 8 * gap))


def call_prefill(lib, s):
    r = lambda d: ctypes.byref(d) if d is not None else None
    return lib.kda_prefill(r(s["q"]), r(s["k"]), r(s["v"]), r(s["g"]), r(s["beta"]), r(s["s0"]),
                           r(s["cu"]), r(s["out"]), r(s["sT"]), None)


def test_null_descriptor(lib):
    s = packed_set()
    s["q"] = None
    assert call_prefill(lib, s) == 1
    assert b"q" in lib.kda_last_error()


def test_dtype_mismatch(lib):
    s = packed_set()
    s["k"] = desc([100, 2, 128], KDA_F32, s["k"].data)
    assert call_prefill(lib, s) == 3
    s = packed_set()
    s["g"] = desc([100, 2, 128], KDA_BF16, s["g"].data)
    assert call_prefill(lib, s) == 3
    s = packed_set()
    s["cu"] = desc([4], KDA_F32, s["cu"].data)
    assert call_prefill(lib, s) == 3


def test_shape_errors(lib):
    s = packed_set()
    s["v"] = desc([100, 2, 64], KDA_BF16, s["v"].data)
    assert call_prefill(lib, s) == 2
    s = packed_set()
    s["beta"] = desc([99, 2], KDA_F32, s["beta"].data)
    assert call_prefill(lib, s) == 2
    s = packed_set()
    s["s0"] = desc([2, 2, 128, 128], KDA_F32, s["s0"].data)   # N mismatch
    assert call_prefill(lib, s) == 2


def test_unsupported_head_size_and_fp32_d128(lib):
    s = packed_set(D=96)
    assert call_prefill(lib, s) == 6
    s = packed_set(D=128, dt=KDA_F32)
    assert call_prefill(lib, s) == 6


def test_layout_errors(lib):
    s = packed_set()
    s["q"] = desc([100, 2, 128], KDA_BF16, s["q"].data, strides=[256, 128, 2])
    assert call_prefill(lib, s) == 4
    s = packed_set()
    s["q"] = desc([100, 2, 128], KDA_BF16, s["q"].data, strides=[256, 129, 1])   # misaligned rows
    assert call_prefill(lib, s) == 4


def test_alias_errors(lib):
    s = packed_set()
    s["out"] = desc([100, 2, 128], KDA_BF16, s["v"].data + 64)   # overlaps v
    assert call_prefill(lib, s) == 5
    s = packed_set()
    s["sT"] = desc([3, 2, 128, 128], KDA_F32, s["s0"].data + 1024)   # partial overlap
    assert call_prefill(lib, s) == 5


def test_row_padded_views_validate(lib):
    """Row-padded strides (the cudnn-frontend review's [33, 2, 256][..., :128]
    probe) are legal; the workspace query walks the whole validator + planner."""
    s = packed_set(T=33, H=2, D=128, N=3)
    s["q"] = desc([33, 2, 128], KDA_BF16, s["q"].data, strides=[512, 256, 1])
    s["s0"] = desc([3, 2, 128, 128], KDA_F32, s["s0"].data, strides=[2 * 128 * 256, 128 * 256, 256, 1])
    r = lambda d: ctypes.byref(d)
    n = ctypes.c_size_t(7)
    opts = kda.options(nseg=1)
    st = lib.kda_prefill_workspace_size(r(s["q"]), r(s["k"]), r(s["v"]), r(s["g"]), r(s["beta"]), r(s["s0"]),
                                        r(s["cu"]), r(s["out"]), r(s["sT"]), ctypes.byref(opts), ctypes.byref(n))
    assert st == 0, lib.kda_last_error()
    assert n.value == 0


def test_in_place_state_allowed(lib):
    s = packed_set()
    s["sT"] = desc([3, 2, 128, 128], KDA_F32, s["s0"].data)
    r = lambda d: ctypes.byref(d)
    n = ctypes.c_size_t(0)
    opts = kda.options(nseg=1)
    st = lib.kda_prefill_workspace_size(*(r(s[x]) for x in ("q", "k", "v", "g", "beta", "s0", "cu", "out", "sT")),
                                        ctypes.byref(opts), ctypes.byref(n))
    assert st == 0, lib.kda_last_error()


def test_workspace_size_of_segmented_plan(lib):
    """Forced nseg = 8 on B=2, H=16, T=4096, d=128: (M, C) for segments 0 .. nseg - 2 (COMBINE
    never reads the last segment's maps) + a start state per segment, plus Gamma (fp32, one per
    token-head-channel) when the standalone PREP kernel is asked for."""
    B, T, H, D = 2, 4096, 16, 128
    gap = 1 << 34
    s = dict(q=desc([B, T, H, D]), k=desc([B, T, H, D], base=FAKE + gap), v=desc([B, T, H, D], base=FAKE + 2 * gap),
             g=desc([B, T, H, D], KDA_F32, FAKE + 3 * gap), beta=desc([B, T, H], KDA_F32, FAKE + 4 * gap),
             s0=None, cu=None, out=desc([B, T, H, D], base=FAKE + 5 * gap), sT=None)
    r = lambda d: ctypes.byref(d) if d is not None else None
    n = ctypes.c_size_t(0)
    opts = kda.options(nseg=8)
    st = lib.kda_prefill_workspace_size(*(r(s[x]) for x in ("q", "k", "v", "g", "beta", "s0", "cu", "out", "sT")),
                                        ctypes.byref(opts), ctypes.byref(n))
    assert st == 0, lib.kda_last_error()
    chains, dd = B * H, D * D * 4
    want = chains * 7 * 2 * dd + chains * 8 * dd
    assert n.value == want
    opts = kda.options(nseg=8, prep=1)
    st = lib.kda_prefill_workspace_size(*(r(s[x]) for x in ("q", "k", "v", "g", "beta", "s0", "cu", "out", "sT")),
                                        ctypes.byref(opts), ctypes.byref(n))
    assert st == 0 and n.value == B * T * H * D * 4 + want
    opts = kda.options(nseg=1, prep=2)
    st = lib.kda_prefill_workspace_size(*(r(s[x]) for x in ("q", "k", "v", "g", "beta", "s0", "cu", "out", "sT")),
                                        ctypes.byref(opts), ctypes.byref(n))
    assert st == 0 and n.value == 0     # single segment with the in-chunk scan: no workspace


def test_pipelined_kernel_needs_32bit_chunk_offsets(lib):
    """The pipelined kernel addresses each 32-token chunk with 32-bit byte offsets: a token
    stride of 2^25 bf16 elements (32 rows = 2 GiB) is refused when that kernel is forced,
    and planned onto the 64-token kernel otherwise."""
    big = 1 << 25
    gap = 1 << 38
    s = dict(q=desc([100, 2, 128], KDA_BF16, FAKE, strides=[big, 128, 1]),
             k=desc([100, 2, 128], base=FAKE + gap), v=desc([100, 2, 128], base=FAKE + 2 * gap),
             g=desc([100, 2, 128], KDA_F32, FAKE + 3 * gap), beta=desc([100, 2], KDA_F32, FAKE + 4 * gap),
             s0=None, cu=desc([4], KDA_I32, FAKE + 6 * gap), out=desc([100, 2, 128], base=FAKE + 7 * gap), sT=None)
    r = lambda d: ctypes.byref(d) if d is not None else None
    n = ctypes.c_size_t(0)
    args = [r(s[x]) for x in ("q", "k", "v", "g", "beta", "s0", "cu", "out", "sT")]
    opts = kda.options(nseg=1, variant=2)
    assert lib.kda_prefill_workspace_size(*args, ctypes.byref(opts), ctypes.byref(n)) == 6
    assert b"token strides" in lib.kda_last_error()
    opts = kda.options(nseg=1, variant=0)
    assert lib.kda_prefill_workspace_size(*args, ctypes.byref(opts), ctypes.byref(n)) == 0, lib.kda_last_error()
    s["q"] = desc([100, 2, 128], KDA_BF16, FAKE, strides=[big // 2, 128, 1])      # 1 GiB per 32 rows: fits
    args = [r(s[x]) for x in ("q", "k", "v", "g", "beta", "s0", "cu", "out", "sT")]
    opts = kda.options(nseg=1, variant=2)
    assert lib.kda_prefill_workspace_size(*args, ctypes.byref(opts), ctypes.byref(n)) == 0, lib.kda_last_error()


def test_python_binding_refuses_without_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("GPU present")
    x = torch.zeros(4, 1, 64)
    with pytest.raises(RuntimeError):
        kda.prefill(x, x, x, x, torch.zeros(4, 1), cu_seqlens=torch.tensor([0, 4], dtype=torch.int32))


def test_activation_options_validated(lib):
    """gate_act / beta_act must be 0 or 1 and the gate lower bound must lie in
    [-5, 0] (the range the kernels' gate factorisation is guaranteed on); the
    check runs on the host before anything is enqueued."""
    s = packed_set()
    r = lambda d: ctypes.byref(d) if d is not None else None
    n = ctypes.c_size_t(0)

    def size(**kw):
        opts = kda.options(**kw)
        return lib.kda_prefill_workspace_size(*(r(s[x]) for x in ("q", "k", "v", "g", "beta", "s0", "cu", "out", "sT")),
                                              ctypes.byref(opts), ctypes.byref(n))
    assert size(gate_logits=True, gate_lower_bound=-5.0, beta_logits=True) == 0
    assert size(gate_logits=True, gate_lower_bound=0.0) == 0
    for bad in (-5.5, 0.25, float("nan"), float("-inf")):
        assert size(gate_logits=True, gate_lower_bound=bad) == 6, bad
        assert b"gate_lower_bound" in lib.kda_last_error()
    assert size(gate_logits=False, gate_lower_bound=-9.0) == 0     # the bound is unused without logits
    opts = kda.options()
    opts.gate_act = 2
    assert lib.kda_prefill_workspace_size(*(r(s[x]) for x in ("q", "k", "v", "g", "beta", "s0", "cu", "out", "sT")),
                                          ctypes.byref(opts), ctypes.byref(n)) == 6


def decode_set(R=4, T=3, H=2, D=128, P=6, dt=KDA_BF16, pool_dt=KDA_F32):
    gap = 1 << 32
    return dict(q=desc([R, T, H, D], dt, FAKE), k=desc([R, T, H, D], dt, FAKE + gap),
                v=desc([R, T, H, D], dt, FAKE + 2 * gap), g=desc([R, T, H, D], KDA_F32, FAKE + 3 * gap),
                beta=desc([R, T, H], KDA_F32, FAKE + 4 * gap), pool=desc([P, H, D, D], pool_dt, FAKE + 5 * gap),
                idx=desc([R], KDA_I32, FAKE + 6 * gap), ntok=desc([R], KDA_I32, FAKE + 7 * gap),
                out=desc([R, T, H, D], dt, FAKE + 8 * gap))


def call_decode(lib, s, update=1):
    r = lambda d: ctypes.byref(d) if d is not None else None
    return lib.kda_decode(r(s["q"]), r(s["k"]), r(s["v"]), r(s["g"]), r(s["beta"]), r(s["pool"]), r(s["idx"]),
                          r(s["ntok"]), r(s["out"]), update, None, None)


def test_decode_validation(lib):
    """kda_decode's host checks; none of these calls reaches a launch."""
    s = decode_set(T=9)
    for x in ("q", "k", "v", "g", "out"):
        s[x] = desc([4, 9, 2, 128], s[x].dtype, s[x].data)
    s["beta"] = desc([4, 9, 2], KDA_F32, s["beta"].data)
    assert call_decode(lib, s) == 6 and b"1..8" in lib.kda_last_error()
    s = decode_set(pool_dt=KDA_I32)
    assert call_decode(lib, s) == 3
    s = decode_set()
    s["idx"] = desc([4], KDA_F32, s["idx"].data)
    assert call_decode(lib, s) == 3
    s = decode_set()
    s["pool"] = desc([6, 2, 128, 64], KDA_F32, s["pool"].data)
    assert call_decode(lib, s) == 2
    s = decode_set()
    s["ntok"] = desc([3], KDA_I32, s["ntok"].data)
    assert call_decode(lib, s) == 2
    s = decode_set()
    s["out"] = desc([4, 3, 2, 128], KDA_BF16, s["pool"].data)
    assert call_decode(lib, s) == 5
    s = decode_set()
    s["pool"] = desc([6, 2, 128, 128], KDA_F32, s["q"].data)
    assert call_decode(lib, s) == 5
    s = decode_set(D=96)
    assert call_decode(lib, s) == 6
    s = decode_set()
    s["state_dummy"] = None
    s["idx"] = None
    assert call_decode(lib, s) == 1


def test_decode_vector_alignment(lib):
    """state_pool and out rows move as 4-element vectors: a row stride or base that
    is not a multiple of 4 elements is refused before any launch."""
    s = decode_set()
    s["pool"] = desc([6, 2, 128, 128], KDA_F32, s["pool"].data, strides=[2 * 128 * 130, 128 * 130, 130, 1])
    assert call_decode(lib, s) == 4
    s = decode_set()
    s["out"] = desc([4, 3, 2, 128], KDA_BF16, s["out"].data + 2)
    assert call_decode(lib, s) == 4


def test_state_dtypes(lib):
    """Initial and final states may each be fp32 or bf16; other dtypes are refused.
    (Workspace sizing runs the full validation and launches nothing.)"""
    r = lambda d: ctypes.byref(d) if d is not None else None
    n = ctypes.c_size_t(0)
    for s0_dt, sT_dt, want in [(KDA_BF16, KDA_BF16, 0), (KDA_BF16, KDA_F32, 0), (KDA_F32, KDA_BF16, 0),
                               (KDA_I32, KDA_F32, 3), (KDA_F32, KDA_I32, 3)]:
        s = packed_set()
        s["s0"] = desc([3, 2, 128, 128], s0_dt, s["s0"].data)
        s["sT"] = desc([3, 2, 128, 128], sT_dt, s["sT"].data)
        st = lib.kda_prefill_workspace_size(*(r(s[x]) for x in ("q", "k", "v", "g", "beta", "s0", "cu", "out", "sT")),
                                            None, ctypes.byref(n))
        assert st == want, (s0_dt, sT_dt, st, lib.kda_last_error())


def test_output_norm_options_validated(lib):
    """The gated RMS norm epilogue's descriptors: out_gate like out, fp32 [V] weight,
    positive eps, no overlap with out, and only on the pipelined kernel; checked on
    the host (workspace sizing launches nothing)."""
    r = lambda d: ctypes.byref(d) if d is not None else None
    n = ctypes.c_size_t(0)
    gap = 1 << 32

    def size(z, w, eps=1e-6, variant=0, dt=KDA_BF16, D=128):
        s = packed_set(D=D, dt=dt)
        opts = kda.options(variant=variant)
        opts.norm_eps = eps
        keep = (z, w)
        if z is not None:
            opts.out_gate = ctypes.pointer(z)
        if w is not None:
            opts.norm_weight = ctypes.pointer(w)
        st = lib.kda_prefill_workspace_size(*(r(s[x]) for x in ("q", "k", "v", "g", "beta", "s0", "cu", "out", "sT")),
                                            ctypes.byref(opts), ctypes.byref(n))
        del keep
        return st
    z = lambda shape=(100, 2, 128), dt=KDA_BF16, base=FAKE + 10 * gap: desc(list(shape), dt, base)
    w = lambda D=128, dt=KDA_F32, base=FAKE + 11 * gap: desc([D], dt, base)
    assert size(z(), w()) == 0
    assert size(z(), None) == 1
    assert size(z(dt=KDA_F32), w()) == 3
    assert size(z(shape=(100, 2, 64)), w()) == 2
    assert size(z(), w(D=64)) == 2
    assert size(z(), w(dt=KDA_BF16)) == 2
    assert size(z(), w(), eps=0.0) == 6
    assert size(z(base=FAKE + 7 * gap), w()) == 5          # out_gate is out
    assert size(z(base=FAKE + 8 * gap), w()) == 5          # out_gate inside final_state
    assert size(z(), w(base=FAKE + 8 * gap + 4096)) == 5   # norm_weight inside final_state
    assert size(z(base=FAKE + 10 * gap + 2), w()) == 4     # misaligned rows
    assert size(z(), w(), variant=1) == 6                   # single-role kernel: unsupported


def test_plan_log(tmp_path):
    """KDA_LOG=1 prints each plan to stderr (the planner runs on the host: a
    workspace-size query shows it without a GPU)."""
    import subprocess, sys, textwrap
    code = textwrap.dedent(f"""
        import ctypes, sys
        sys.path.insert(0, {ROOT!r}); sys.path.insert(0, {os.path.join(ROOT, 'tests')!r})
        import test_abi as t
        import gated_delta_rule_38_amd as kda
        lib = kda.load_library()
        s = t.packed_set(T=4096, H=2, N=2)
        r = lambda d: ctypes.byref(d) if d is not None else None
        n = ctypes.c_size_t(0)
        st = lib.kda_prefill_workspace_size(*(r(s[x]) for x in ("q", "k", "v", "g", "beta", "s0", "cu", "out", "sT")),
                                            None, ctypes.byref(n))
        print("status", st, n.value)
    """)
    env = dict(os.environ, KDA_LOG="1")
    p = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert p.returncode == 0, p.stderr[-2000:]
    assert "status 0" in p.stdout
    assert "kda: plan N=2 H=2 D=128 packed chains=4 nseg=" in p.stderr and "kernel=pipelined" in p.stderr


def test_segment_grid_beyond_one_launch_is_refused(lib):
    """2^25 chains (B = 2^20 dense sequences of one token, H = 32) with 64 forced segments
    would need 2^32 segment-build workgroups: refused before any launch."""
    B, T, H, D = 1 << 20, 1, 32, 128
    gap = 1 << 36
    s = [desc([B, T, H, D]), desc([B, T, H, D], base=FAKE + gap), desc([B, T, H, D], base=FAKE + 2 * gap),
         desc([B, T, H, D], KDA_F32, FAKE + 3 * gap), desc([B, T, H], KDA_F32, FAKE + 4 * gap), None, None,
         desc([B, T, H, D], base=FAKE + 5 * gap), None]
    n = ctypes.c_size_t(0)
    r = lambda d: ctypes.byref(d) if d is not None else None
    st = lib.kda_prefill_workspace_size(*(r(d) for d in s), ctypes.byref(kda.options(nseg=64)), ctypes.byref(n))
    assert st == 6 and "segments" in lib.kda_last_error().decode()
    st = lib.kda_prefill_workspace_size(*(r(d) for d in s), ctypes.byref(kda.options(nseg=0)), ctypes.byref(n))
    assert st == 0 and n.value == 0       # the planner's choice: one segment, no workspace


def test_plan_chain_order(tmp_path):
    """The planner starts the longest sequences first exactly when a packed single-segment
    launch has more chains than CUs (256 without a GPU) and at most 512 sequences;
    KDA_ORDER overrides it."""
    import subprocess, sys, textwrap
    code = textwrap.dedent(f"""
        import ctypes, os, sys
        sys.path.insert(0, {ROOT!r}); sys.path.insert(0, {os.path.join(ROOT, 'tests')!r})
        import test_abi as t
        import gated_delta_rule_38_amd as kda
        lib = kda.load_library()
        r = lambda d: ctypes.byref(d) if d is not None else None
        def plan(T, H, N, env=None, nseg=0):
            os.environ.pop("KDA_ORDER", None)
            if env: os.environ["KDA_ORDER"] = env
            s = t.packed_set(T=T, H=H, N=N)
            n = ctypes.c_size_t(0)
            st = lib.kda_prefill_workspace_size(*(r(s[x]) for x in ("q", "k", "v", "g", "beta", "s0", "cu", "out", "sT")),
                                                ctypes.byref(kda.options(nseg=nseg)), ctypes.byref(n))
            sys.stderr.flush()
            print("case", T, H, N, env, nseg, "status", st, flush=True)
        plan(4096, 128, 3)               # 384 chains > 256 CUs: longest first
        plan(4096, 32, 8)                # 256 chains: every chain resident, natural
        plan(4096, 1, 600)               # 600 sequences > 512: natural
        plan(4096, 128, 3, "natural")
        plan(4096, 2, 2, "longest", 1)   # forced on a small single-segment plan
        plan(4096, 2, 2, "longest")      # the planner segments it: order not applicable
    """)
    env = dict(os.environ, KDA_LOG="1")
    p = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert p.returncode == 0 and p.stdout.count("status 0") == 6, p.stdout + p.stderr[-2000:]
    orders = [l.split("order=")[1].split()[0] for l in p.stderr.splitlines() if l.startswith("kda: plan")]
    assert orders == ["longest-first", "natural", "natural", "natural", "longest-first", "natural"], orders


@pytest.mark.parametrize("B,H,T,nseg", [(2, 16, 4096, 8), (1, 8, 65536, 32), (3, 32, 4096, 1), (4, 32, 4096, 1),
                                        (8, 32, 8192, 1), (1, 2, 256, 1), (1, 8, 16384, 32), (2, 16, 1024, 4),
                                        (1, 16, 8192, 16), (4, 16, 8192, 4), (1, 8, 4096, 16)])
def test_planner_segment_counts(lib, B, H, T, nseg):
    """The planner's segment count (read off the workspace size, chains x (3 nseg - 2) states)
    on 256 CUs: the fastest forced count measured on MI355X for each shape (equal-length 8, long
    32; 32 chains of 1,024 tokens 4, where one segment pays its pass's fixed cost too; 16 chains
    of 8,192 tokens 16; 64 chains of 8,192 tokens 4; 8 chains of 4,096 tokens 16), one segment
    where the segment passes would need more rounds than they save (96 and 128 chains)."""
    D = 128
    gap = 1 << 36
    s = [desc([B, T, H, D]), desc([B, T, H, D], base=FAKE + gap), desc([B, T, H, D], base=FAKE + 2 * gap),
         desc([B, T, H, D], KDA_F32, FAKE + 3 * gap), desc([B, T, H], KDA_F32, FAKE + 4 * gap), None, None,
         desc([B, T, H, D], base=FAKE + 5 * gap), None]
    n = ctypes.c_size_t(0)
    r = lambda d: ctypes.byref(d) if d is not None else None
    st = lib.kda_prefill_workspace_size(*(r(d) for d in s), None, ctypes.byref(n))
    assert st == 0, lib.kda_last_error()
    got = (n.value // (B * H * D * D * 4) + 2) // 3 if n.value else 1     # chains (3 nseg - 2) states
    assert got == nseg


def test_decode_pool_may_not_overlap_norm_operands(lib):
    """The pool is written while other workgroups read the output gate and the norm
    weight: an overlap with either is refused on the host."""
    gap = 1 << 32
    for which in ("out_gate", "norm_weight"):
        s = decode_set()
        z = desc([4, 3, 2, 128], KDA_BF16, FAKE + 10 * gap)
        w = desc([128], KDA_F32, FAKE + 11 * gap)
        if which == "out_gate":
            z = desc([4, 3, 2, 128], KDA_BF16, s["pool"].data + 4096)
        else:
            w = desc([128], KDA_F32, s["pool"].data + 4096)
        opts = kda.options()
        opts.out_gate, opts.norm_weight, opts.norm_eps = ctypes.pointer(z), ctypes.pointer(w), 1e-6
        r = lambda d: ctypes.byref(d) if d is not None else None
        st = lib.kda_decode(r(s["q"]), r(s["k"]), r(s["v"]), r(s["g"]), r(s["beta"]), r(s["pool"]), r(s["idx"]),
                            r(s["ntok"]), r(s["out"]), 1, ctypes.byref(opts), None)
        assert st == 5 and b"state_pool" in lib.kda_last_error(), (which, st, lib.kda_last_error())


def test_peak_probes_validate(lib):
    """The probes refuse NULL pointers and empty sizes before any launch."""
    arr = (ctypes.c_void_p * 5)(*([FAKE] * 5))
    assert lib.kda_peak_stream(arr, None, 16, None) == 1
    assert lib.kda_peak_stream(arr, ctypes.c_void_p(FAKE), 0, None) == 2
    assert lib.kda_peak_mfma(None, 4, 4, None) == 1
    assert lib.kda_peak_mfma(ctypes.c_void_p(FAKE), 0, 4, None) == 2


def test_profile_read_kernels_without_records(lib):
    entries = (kda.KdaProfileEntry * 4)()
    n = ctypes.c_int32(-1)
    assert lib.kda_profile_read_kernels(entries, 4, ctypes.byref(n)) == 0 and n.value == 0
    assert lib.kda_profile_read_kernels(None, 4, ctypes.byref(n)) == 1


def test_planner_splits_chains_just_above_the_cu_count(tmp_path):
    """288 equal chains (B=9, H=32, T=4096) on 256 CUs: instead of a second round of 32 chains on
    32 CUs, only the last 32 chains are cut into segments (8) and the other 256 run whole; the
    workspace holds the 32 chains' maps and start states.  256 chains (one full round) and the
    packed layout (lengths unknown on the host) are not split; a forced split is refused without a
    forced segment count or on the single-role kernel."""
    import subprocess, sys, textwrap
    code = textwrap.dedent(f"""
        import ctypes, sys
        sys.path.insert(0, {ROOT!r}); sys.path.insert(0, {os.path.join(ROOT, 'tests')!r})
        import test_abi as t
        import gated_delta_rule_38_amd as kda
        lib = kda.load_library()
        r = lambda d: ctypes.byref(d) if d is not None else None
        D = 128
        def dense(B, H, T):
            gap = 1 << 36
            return [t.desc([B, T, H, D]), t.desc([B, T, H, D], base=t.FAKE + gap), t.desc([B, T, H, D], base=t.FAKE + 2 * gap),
                    t.desc([B, T, H, D], t.KDA_F32, t.FAKE + 3 * gap), t.desc([B, T, H], t.KDA_F32, t.FAKE + 4 * gap), None, None,
                    t.desc([B, T, H, D], base=t.FAKE + 5 * gap), None]
        for B, H, T, kw in ((9, 32, 4096, {{}}), (8, 32, 4096, {{}}), (2, 3, 300, dict(nseg=3, split_chains=2)),
                            (2, 3, 300, dict(split_chains=2)), (2, 3, 300, dict(nseg=3, split_chains=2, variant=1))):
            n = ctypes.c_size_t(0)
            st = lib.kda_prefill_workspace_size(*(r(d) for d in dense(B, H, T)), ctypes.byref(kda.options(**kw)), ctypes.byref(n))
            sys.stderr.flush()
            print("case", B, H, T, sorted(kw.items()), "status", st, "bytes", n.value, flush=True)
    """)
    env = dict(os.environ, KDA_LOG="1")
    p = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert p.returncode == 0, p.stderr[-2000:]
    cases = [l for l in p.stdout.splitlines() if l.startswith("case")]
    plans = [l for l in p.stderr.splitlines() if l.startswith("kda: plan")]
    dd = 128 * 128 * 4
    assert "status 0" in cases[0] and f"bytes {32 * (3 * 8 - 2) * dd}" in cases[0], cases[0]
    assert "nseg=8 segmented=32" in plans[0], plans[0]
    assert "status 0 bytes 0" in cases[1] and "nseg=1 segmented=0" in plans[1]
    assert "status 0" in cases[2] and f"bytes {2 * (3 * 3 - 2) * dd}" in cases[2] and "nseg=3 segmented=2" in plans[2]
    assert "status 6" in cases[3] and "status 6" in cases[4]


def test_plan_capped_concurrency(tmp_path):
    """A packed single-segment launch with every chain resident (<= 256 without a GPU) and
    more chains than the cap (160) plans the capped schedule: groups of H workgroups, a
    8-byte flag per chain last in the workspace.  Not with at most 160 chains, more chains
    than CUs (longest first instead), the dense layout, more than 16 groups, or KDA_CAP=0."""
    import subprocess, sys, textwrap
    code = textwrap.dedent(f"""
        import ctypes, os, sys
        sys.path.insert(0, {ROOT!r}); sys.path.insert(0, {os.path.join(ROOT, 'tests')!r})
        import test_abi as t
        import gated_delta_rule_38_amd as kda
        lib = kda.load_library()
        r = lambda d: ctypes.byref(d) if d is not None else None
        def plan(T, H, N, cap=None):
            os.environ.pop("KDA_CAP", None)
            if cap is not None: os.environ["KDA_CAP"] = str(cap)
            s = t.packed_set(T=T, H=H, N=N)
            n = ctypes.c_size_t(0)
            st = lib.kda_prefill_workspace_size(*(r(s[x]) for x in ("q", "k", "v", "g", "beta", "s0", "cu", "out", "sT")),
                                                ctypes.byref(kda.options(nseg=1)), ctypes.byref(n))
            sys.stderr.flush()
            print("case", T, H, N, cap, "status", st, "bytes", n.value, flush=True)
        plan(32768, 32, 8)               # 256 chains: 5 groups of 32
        plan(32768, 32, 8, 0)            # turned off
        plan(32768, 32, 4)               # 128 chains: under the cap
        plan(32768, 64, 5)               # 320 chains > 256 CUs: longest first
        plan(32768, 2, 100)              # 200 chains in 80 groups of 2: more than 16 groups
        plan(32768, 16, 12, 96)          # a cap of 96 chains: 6 groups of 16
    """)
    env = dict(os.environ, KDA_LOG="1")
    p = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert p.returncode == 0 and p.stdout.count("status 0") == 6, p.stdout + p.stderr[-2000:]
    caps = [int(l.split("cap=")[1].split()[0]) for l in p.stderr.splitlines() if l.startswith("kda: plan")]
    assert caps == [160, 0, 0, 0, 0, 96], caps
    sizes = [int(l.split("bytes ")[1]) for l in p.stdout.splitlines() if l.startswith("case")]
    assert sizes == [2048, 0, 0, 0, 0, 1536], sizes
