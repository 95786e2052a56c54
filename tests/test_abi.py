"""The C-ABI library loads and exports every symbol include/gdn.h declares, and its
host-side checks reject bad arguments before any launch (no GPU needed: none of
these calls reaches the HIP runtime)."""
import ctypes
import os
import re
import subprocess

import pytest

import gated_deltanet_prefill_gdn_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted(gdn.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = gdn.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", gdn.LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    exported = set(re.findall(r" T (\w+)$", nm, flags=re.M))
    for name in declared_functions():
        assert name in exported, name


def test_library_carries_gfx950_code():
    blob = open(gdn.LIB_PATH, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in blob


def test_status_strings_and_version():
    for code in range(6):
        assert gdn.status_str(code)
    assert gdn.gdn_version() >= 100


def prob(**kw):
    base = dict(N=16384, B=4, H=16, HV=16, dk=128, dv=128, pool=4, dtype=gdn.GDN_DTYPE_BF16,
                flags=0)
    base.update(kw)
    return gdn.make_problem(base["N"], base["B"], base["H"], base["HV"], base["dk"], base["dv"],
                            base["pool"], base["dtype"], base["flags"])


def test_workspace_size():
    ws = gdn.gdn_prefill_workspace_size(prob())
    assert ws > 0 and ws % 256 == 0
    # the chunk-everything flag needs no other workspace (the bound covers every request)
    assert gdn.gdn_prefill_workspace_size(prob(flags=gdn.GDN_FLAG_CHUNK_ALL)) == ws
    assert gdn.gdn_prefill_workspace_size(prob(flags=2)) == 0
    # grows with the chunk upper bound N / C + B
    assert gdn.gdn_prefill_workspace_size(prob(B=40)) > ws
    assert gdn.gdn_prefill_workspace_size(prob(), 32) == 0          # C = 64 or 128 only
    assert gdn.gdn_prefill_workspace_size(prob(HV=24)) == 0         # HV % H != 0
    assert gdn.gdn_prefill_workspace_size(prob(dk=96)) == 0         # unsupported head dim
    assert gdn.gdn_prefill_workspace_size(prob(dtype=7)) == 0


def call(p, chunk=64, ws_bytes=1 << 30, nonnull=True, ws_ptr=1 << 20):
    lib = gdn.load_library()
    P = ctypes.c_void_p
    x = P(4096) if nonnull else P(0)
    return lib.gdn_prefill_fwd(x, x, x, x, x, x, x, x, x, x, chunk, x, ctypes.byref(p),
                               P(ws_ptr), ws_bytes, P(0))


def test_error_paths_return_before_launch():
    # every one of these is rejected by host checks before any HIP call
    assert call(prob(HV=24)) == gdn.GDN_ERR_INVALID_ARG
    assert call(prob(H=0)) == gdn.GDN_ERR_INVALID_ARG
    assert call(prob(N=-1)) == gdn.GDN_ERR_INVALID_ARG
    assert call(prob(dtype=3)) == gdn.GDN_ERR_INVALID_ARG
    assert call(prob(), chunk=0) == gdn.GDN_ERR_INVALID_ARG
    assert call(prob(), chunk=96) == gdn.GDN_ERR_UNSUPPORTED
    assert call(prob(dk=96)) == gdn.GDN_ERR_UNSUPPORTED
    assert call(prob(dv=512)) == gdn.GDN_ERR_UNSUPPORTED
    assert call(prob(pool=0)) == gdn.GDN_ERR_INVALID_ARG
    assert call(prob(flags=2)) == gdn.GDN_ERR_INVALID_ARG     # an undefined flag bit
    assert call(prob(flags=1 | 4)) == gdn.GDN_ERR_INVALID_ARG
    assert call(prob(), nonnull=False) == gdn.GDN_ERR_INVALID_ARG
    assert call(prob(), ws_bytes=1024) == gdn.GDN_ERR_WORKSPACE
    assert call(prob(), ws_ptr=(1 << 20) + 64) == gdn.GDN_ERR_WORKSPACE   # not 256-aligned
    lib = gdn.load_library()
    assert lib.gdn_prefill_fwd(None, None, None, None, None, None, None, None, None, None, 64,
                               None, None, None, 0, None) == gdn.GDN_ERR_INVALID_ARG


def test_state_schedule():
    """The state-pass schedule is a function of the descriptor: column slices where those
    fill the device (the dense batch), segments for few long requests (the long-decay
    request), column slices at dk = 256 and above 64 requests, the fp32 kernels for fp32."""
    S = gdn.gdn_prefill_state_schedule
    assert S(prob()) == gdn.GDN_SCHEDULE_COLUMN_SLICES
    assert S(prob(N=131072, B=1, HV=32, pool=1)) == gdn.GDN_SCHEDULE_SEGMENTS
    assert S(prob(N=16384, B=1, H=8, HV=8, dk=256, dv=256, pool=1)) == \
        gdn.GDN_SCHEDULE_COLUMN_SLICES
    assert S(prob(N=8192, B=65, H=1, HV=1, pool=65)) == gdn.GDN_SCHEDULE_COLUMN_SLICES
    assert S(prob(N=8192, B=63, H=1, HV=1, pool=63)) == gdn.GDN_SCHEDULE_SEGMENTS
    assert S(prob(dtype=gdn.GDN_DTYPE_F32)) == gdn.GDN_SCHEDULE_FP32
    assert S(prob(HV=24)) == -1
    assert S(prob(), 96) == -1
    # C = 128: column slices, never segments
    assert S(prob(N=131072, B=1, HV=32, pool=1), 128) == gdn.GDN_SCHEDULE_COLUMN_SLICES


def test_chunk_size_128():
    """C = 128 serves bf16 inputs with dk of 128 or 256; fp32 inputs, dk = 64 and the
    backward take C = 64 only. Its workspace holds half as many chunks, each with twice the
    rows of A_qk."""
    ws64 = gdn.gdn_prefill_workspace_size(prob())
    ws128 = gdn.gdn_prefill_workspace_size(prob(), 128)
    assert ws128 > 0 and ws128 % 256 == 0 and ws128 != ws64
    assert gdn.gdn_prefill_workspace_size(prob(dk=256, dv=64), 128) > 0
    assert gdn.gdn_prefill_workspace_size(prob(dtype=gdn.GDN_DTYPE_F32), 128) == 0
    assert gdn.gdn_prefill_workspace_size(prob(dk=64), 128) == 0
    assert gdn.gdn_prefill_bwd_workspace_size(prob(), 128) == 0
    assert call(prob(dtype=gdn.GDN_DTYPE_F32), chunk=128) == gdn.GDN_ERR_UNSUPPORTED
    assert call(prob(dk=64), chunk=128) == gdn.GDN_ERR_UNSUPPORTED
    assert call(prob(), chunk=128, ws_bytes=1024) == gdn.GDN_ERR_WORKSPACE


def test_grids_beyond_launch_limits_are_refused():
    """Shapes whose kernel grids would exceed 2^32 work-items are refused on the host,
    before the workspace is even looked at."""
    huge = prob(N=1 << 30, B=1 << 24, H=1, HV=1024, dk=128, dv=256, pool=1 << 24)
    assert call(huge, ws_bytes=0, ws_ptr=0) == gdn.GDN_ERR_UNSUPPORTED
    huge32 = prob(N=(1 << 31) - (1 << 26), B=1, H=1, HV=65535, pool=1,
                  dtype=gdn.GDN_DTYPE_F32)
    assert call(huge32, ws_bytes=0, ws_ptr=0) == gdn.GDN_ERR_UNSUPPORTED


def test_validate_inputs_refuses_what_it_cannot_copy():
    """gdn_validate_inputs copies the arrays to the host: a descriptor with more requests
    than it copies is refused with a status (no exception through the C ABI, no HIP call);
    the pool size plays no part in its memory."""
    lib = gdn.load_library()
    P = ctypes.c_void_p
    for B in (1 << 40, (1 << 26) + 1):
        p = prob(N=0, B=B, pool=B)
        assert lib.gdn_validate_inputs(P(4096), P(4096), ctypes.byref(p), P(0)) == \
            gdn.GDN_ERR_UNSUPPORTED


def test_nonfinite_flag_argument_checks():
    lib = gdn.load_library()
    P = ctypes.c_void_p
    flag = ctypes.c_int32(7)
    assert lib.gdn_prefill_nonfinite(P(0), 1024, ctypes.byref(flag), P(0)) == \
        gdn.GDN_ERR_INVALID_ARG
    assert lib.gdn_prefill_nonfinite(P(4096), 1024, None, P(0)) == gdn.GDN_ERR_INVALID_ARG
    assert lib.gdn_prefill_nonfinite(P(4096), 2, ctypes.byref(flag), P(0)) == \
        gdn.GDN_ERR_WORKSPACE
    assert flag.value == 7


def test_empty_problem_is_a_no_op():
    # N == 0 or B == 0: nothing to read or write, so null pointers are fine
    assert call(prob(N=0, B=3), nonnull=False, ws_bytes=0, ws_ptr=0) == gdn.GDN_OK
    assert call(prob(N=0, B=0, pool=0), nonnull=False, ws_bytes=0, ws_ptr=0) == gdn.GDN_OK


def call_decode(p, nonnull=True, misalign=0):
    lib = gdn.load_library()
    P = ctypes.c_void_p
    x = P(4096) if nonnull else P(0)
    return lib.gdn_decode_fwd(P(4096 + misalign), x, x, x, x, x, x, x, x, x, ctypes.byref(p),
                              P(0))


def test_decode_error_paths_return_before_launch():
    dec = dict(N=512, B=512, H=16, HV=32, pool=512)
    assert call_decode(prob(**{**dec, "N": 511})) == gdn.GDN_ERR_INVALID_ARG  # one token each
    assert call_decode(prob(**{**dec, "HV": 24})) == gdn.GDN_ERR_INVALID_ARG
    assert call_decode(prob(**{**dec, "dtype": 2})) == gdn.GDN_ERR_INVALID_ARG
    assert call_decode(prob(**{**dec, "pool": 0})) == gdn.GDN_ERR_INVALID_ARG
    assert call_decode(prob(**{**dec, "dk": 32})) == gdn.GDN_ERR_UNSUPPORTED
    assert call_decode(prob(**dec), nonnull=False) == gdn.GDN_ERR_INVALID_ARG
    assert call_decode(prob(**dec), misalign=8) == gdn.GDN_ERR_INVALID_ARG   # q not 16-aligned
    lib = gdn.load_library()
    assert lib.gdn_decode_fwd(None, None, None, None, None, None, None, None, None, None, None,
                              None) == gdn.GDN_ERR_INVALID_ARG


def test_decode_empty_batch_is_a_no_op():
    assert call_decode(prob(N=0, B=0, pool=0), nonnull=False) == gdn.GDN_OK


def call_promote(scans=4, F=8, n=64, dk=128, dv=128, dtype=gdn.GDN_DTYPE_BF16, reserved=0,
                 nonnull=True, misalign=0):
    lib = gdn.load_library()
    P = ctypes.c_void_p
    x = P(4096) if nonnull else P(0)
    p = gdn.GdnPromoteProblem(scans, F, n, dk, dv, dtype, reserved)
    return lib.gdn_promote_scan(P(4096 + misalign), x, x, x, x, x, x, ctypes.byref(p), P(0))


def test_promote_error_paths_return_before_launch():
    assert call_promote(dtype=5) == gdn.GDN_ERR_INVALID_ARG
    assert call_promote(reserved=1) == gdn.GDN_ERR_INVALID_ARG
    assert call_promote(scans=-1) == gdn.GDN_ERR_INVALID_ARG
    assert call_promote(n=0) == gdn.GDN_ERR_INVALID_ARG
    assert call_promote(dtype=gdn.GDN_DTYPE_F32) == gdn.GDN_ERR_UNSUPPORTED
    assert call_promote(dk=256) == gdn.GDN_ERR_UNSUPPORTED
    assert call_promote(dv=96) == gdn.GDN_ERR_UNSUPPORTED
    assert call_promote(n=24) == gdn.GDN_ERR_UNSUPPORTED          # not a multiple of 16
    assert call_promote(dk=64, n=80) == gdn.GDN_ERR_UNSUPPORTED   # more pairs than key rows
    assert call_promote(nonnull=False) == gdn.GDN_ERR_INVALID_ARG
    assert call_promote(misalign=8) == gdn.GDN_ERR_INVALID_ARG    # K not 16-byte aligned
    lib = gdn.load_library()
    assert lib.gdn_promote_scan(None, None, None, None, None, None, None, None,
                                None) == gdn.GDN_ERR_INVALID_ARG


def test_promote_empty_is_a_no_op():
    assert call_promote(scans=0, nonnull=False) == gdn.GDN_OK


def test_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    z = torch.zeros(4, 1, 64)
    with pytest.raises(ValueError):
        gdn.gdn_prefill_fwd(z, z, z, torch.zeros(4, 1), torch.zeros(4, 1), torch.zeros(1),
                            torch.zeros(1), torch.zeros(1, 1, 64, 64),
                            torch.zeros(1, dtype=torch.int64), torch.tensor([0, 4]))


def test_package_has_no_oracle_dependency():
    """The product path never imports the oracle or any CPU fallback."""
    pkg_dir = os.path.join(ROOT, "gated_deltanet_prefill_gdn_amd")
    for dirpath, _, files in os.walk(pkg_dir):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "gdn_oracle" not in text, f


def call_recurrent(p, nonnull=True, misalign=0):
    lib = gdn.load_library()
    P = ctypes.c_void_p
    x = P(4096) if nonnull else P(0)
    return lib.gdn_recurrent_fwd(P(4096 + misalign), x, x, x, x, x, x, x, x, x, x,
                                 ctypes.byref(p), P(0))


def test_recurrent_error_paths_return_before_launch():
    assert call_recurrent(prob(HV=24)) == gdn.GDN_ERR_INVALID_ARG
    assert call_recurrent(prob(N=-1)) == gdn.GDN_ERR_INVALID_ARG
    assert call_recurrent(prob(dtype=3)) == gdn.GDN_ERR_INVALID_ARG
    assert call_recurrent(prob(pool=0)) == gdn.GDN_ERR_INVALID_ARG
    assert call_recurrent(prob(dk=96)) == gdn.GDN_ERR_UNSUPPORTED
    assert call_recurrent(prob(dv=32)) == gdn.GDN_ERR_UNSUPPORTED
    assert call_recurrent(prob(), nonnull=False) == gdn.GDN_ERR_INVALID_ARG
    assert call_recurrent(prob(), misalign=8) == gdn.GDN_ERR_INVALID_ARG   # q not 16-aligned
    assert call_recurrent(prob(N=0, B=3), nonnull=False) == gdn.GDN_OK
    assert call_recurrent(prob(N=5, B=0, pool=0), nonnull=False) == gdn.GDN_OK
    lib = gdn.load_library()
    assert lib.gdn_recurrent_fwd(None, None, None, None, None, None, None, None, None, None, None,
                                 None, None) == gdn.GDN_ERR_INVALID_ARG


def test_header_constants_match_the_binding():
    text = open(HEADER).read()
    for name in ("GDN_FLAG_CHUNK_ALL", "GDN_SHORT_REQUEST", "GDN_SPLIT_MEAN_LENGTH"):
        m = re.search(rf"#define {name} (\d+)", text)
        assert m and int(m.group(1)) == getattr(gdn, name), name
