"""CPU tests of the C-ABI boundary: the library loads, exports every declared entry point, and
validates arguments on the host (returning a status before touching the GPU)."""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ffpa.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:ffpa_status_t|size_t|int|const char\*)\s+(ffpa_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    from head_dim_attention_amd import _binding
    path = _binding.library_path()
    if not os.path.exists(path):
        pytest.fail(f"libffpa.so is not built at {path}: run python -m head_dim_attention_amd.build")
    return _binding.load_library()


def test_header_declares_expected_entry_points():
    names = _declared()
    for n in ("ffpa_fwd", "ffpa_bwd", "ffpa_bwd_stage", "ffpa_varlen_fwd", "ffpa_varlen_bwd", "ffpa_status_string",
              "ffpa_bwd_workspace_bytes", "ffpa_varlen_bwd_workspace_bytes", "ffpa_decode_fwd",
              "ffpa_decode_workspace_bytes", "ffpa_decode_fwd_strided", "ffpa_fwd_strided", "ffpa_fwd_masked",
              "ffpa_bwd_masked", "ffpa_fwd_fp8", "ffpa_fwd_fp8_workspace_bytes", "ffpa_fwd_split",
              "ffpa_fwd_split_workspace_bytes", "ffpa_varlen_bwd_workspace_bytes_exact", "ffpa_bwd_fused_products"):
        assert n in names


def test_header_is_valid_c_and_cxx():
    """include/ffpa.h compiles as C11 and as C++17 (declarations only, no library needed)."""
    import shutil
    import subprocess
    import tempfile
    for cc, std, ext in (("gcc", "-std=c11", "c"), ("g++", "-std=c++17", "cpp")):
        if shutil.which(cc) is None:
            pytest.skip(f"{cc} not available")
        with tempfile.TemporaryDirectory() as td:
            src = os.path.join(td, f"t.{ext}")
            with open(src, "w") as f:
                f.write('#include "ffpa.h"\nint main(void) { ffpa_status_t s = FFPA_OK; ffpa_dtype_t t = '
                        'FFPA_DTYPE_BF16; hipStream_t st = 0; (void)st; return (int)s + (int)t; }\n')
            r = subprocess.run([cc, std, "-fsyntax-only", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                                "-I", "/opt/rocm/include", src], capture_output=True, text=True)
            assert r.returncode == 0, r.stderr


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), f"{name} declared in include/ffpa.h but not exported"


def test_status_strings(lib):
    from head_dim_attention_amd import _binding as B
    for code in (0, 1, 2, 3, 99):
        s = B.ffpa_status_string(code)
        assert isinstance(s, str) and s
    assert "INVALID" in B.ffpa_status_string(1)
    assert "NOT_SUPPORTED" in B.ffpa_status_string(2)


# A fake non-null device pointer: validation returns before anything dereferences it.
P = ctypes.c_void_p(0x1000)
N = ctypes.c_void_p(0)
S = ctypes.c_void_p(0)


def _fwd(lib, b=1, hq=2, hkv=2, nq=64, nkv=64, d=512, dtype=0, scale=0.04, causal=0, ptrs=None):
    ptrs = ptrs or [P] * 5
    return lib.ffpa_fwd(*ptrs, b, hq, hkv, nq, nkv, d, dtype, scale, causal, S)


@pytest.mark.parametrize("kw,expect", [
    (dict(b=0), 1), (dict(nq=0), 1), (dict(nkv=0), 1), (dict(hq=3, hkv=2), 1), (dict(hkv=0), 1),
    (dict(dtype=2), 1), (dict(dtype=-1), 1), (dict(causal=2), 1), (dict(scale=0.0), 1), (dict(scale=-1.0), 1),
    (dict(scale=float("nan")), 1), (dict(scale=float("inf")), 1),
    (dict(d=288), 2), (dict(d=1056), 2), (dict(d=336), 2), (dict(d=64), 2),
])
def test_fwd_validation(lib, kw, expect):
    assert _fwd(lib, **kw) == expect


def test_fwd_null_pointers(lib):
    for i in range(5):
        ptrs = [P] * 5
        ptrs[i] = N
        assert _fwd(lib, ptrs=ptrs) == 1


# q, k, v, o, dout, lse, dlse, delta, dq, dk, dv; dlse (index 6) may be NULL.
BWD_PTRS = 11
DLSE = 6


def _bwd(lib, stage=None, b=1, hq=2, hkv=1, nq=64, nkv=64, d=640, dtype=1, scale=0.04, causal=1, ptrs=None,
         ws=N, ws_bytes=0):
    ptrs = ptrs or [P] * BWD_PTRS
    args = (*ptrs, b, hq, hkv, nq, nkv, d, dtype, scale, causal, ws, ws_bytes, S)
    return lib.ffpa_bwd(*args) if stage is None else lib.ffpa_bwd_stage(stage, *args)


@pytest.mark.parametrize("kw,expect", [
    (dict(b=0), 1), (dict(hq=3, hkv=2), 1), (dict(d=300), 2), (dict(dtype=5), 1), (dict(scale=0.0), 1),
    (dict(stage=5), 1), (dict(stage=-1), 1), (dict(stage=2, d=2048), 2),
    # a workspace smaller than ffpa_bwd_workspace_bytes() is rejected before any launch
    (dict(ws=P, ws_bytes=2 * 2 * 64 * 64 * 2 - 1), 1), (dict(stage=3, ws=P, ws_bytes=16), 1),
])
def test_bwd_validation(lib, kw, expect):
    assert _bwd(lib, **kw) == expect


def test_workspace_sizes(lib):
    from head_dim_attention_amd import _binding as B
    # two blocks (dS, P), stored transposed: B * Hq * Nkv * round_up(Nq, 8) dtype-sized elements
    assert B.ffpa_bwd_workspace_bytes(1, 32, 8192, 8192) == 2 * 32 * 8192 * 8192 * 2
    assert B.ffpa_bwd_workspace_bytes(2, 3, 13, 5) == 2 * 2 * 3 * 5 * 16 * 2
    assert B.ffpa_bwd_workspace_bytes(1, 1, 8, 7) == 2 * 7 * 8 * 2
    assert B.ffpa_bwd_workspace_bytes(0, 1, 7, 8) == 0
    # a head's block above 2^31 bytes: not available (the library then recomputes)
    assert B.ffpa_bwd_workspace_bytes(1, 1, 40000, 40000) == 0
    # varlen: bounded by total_k * round_up(max_seqlen_q, 8) per head and block
    assert B.ffpa_varlen_bwd_workspace_bytes(4, 100, 90, 41, 60) == 2 * 4 * 90 * 48 * 2
    assert B.ffpa_varlen_bwd_workspace_bytes(4, 0, 0, 0, 41) == 0
    # exact: sum over sequences of Lk * round_up(Lq, 8) per head and block
    cq, ck = [0, 41, 41, 100], [0, 30, 60, 90]
    assert B.ffpa_varlen_bwd_workspace_bytes_exact(4, cq, ck, 100, 90, 59, 30) == \
        2 * 4 * (30 * 48 + 30 * 0 + 30 * 64) * 2
    assert B.ffpa_varlen_bwd_workspace_bytes_exact(4, cq, None, 100, 100, 59, 59) == \
        2 * 4 * (41 * 48 + 0 + 59 * 64) * 2
    assert B.ffpa_varlen_bwd_workspace_bytes_exact(4, cq, ck, 100, 90, 40, 30) == 0   # max_seqlen_q too small
    assert B.ffpa_varlen_bwd_workspace_bytes_exact(4, cq, ck, 101, 90, 59, 30) == 0   # wrong total


def test_store_ds_policy():
    """The backward stores P and dS only when the workspace exists and fits with headroom."""
    from head_dim_attention_amd import _binding as B
    gib = 1 << 30
    assert B.choose_store_ds(8 * gib, 200 * gib)
    assert not B.choose_store_ds(8 * gib, 8 * gib)                  # no headroom left
    assert B.choose_store_ds(8 * gib, 9 * gib)
    assert not B.choose_store_ds(0, 200 * gib)                      # not available for these sizes
    assert not B.choose_store_ds(275 * gib, 280 * gib, headroom=8 * gib)
    assert B.choose_store_ds(100, 200, headroom=0)


def test_masked_backward_workspace_check():
    """The masked backward needs the P/dS workspace: a clear error when it cannot fit."""
    from head_dim_attention_amd import _binding as B
    dev = torch.device("cpu")
    need = B.ffpa_bwd_workspace_bytes(8, 32, 16384, 16384)
    assert B.masked_bwd_workspace_check(8, 32, 16384, 16384, dev, available=need) == need
    with pytest.raises(MemoryError):
        B.masked_bwd_workspace_check(8, 32, 16384, 16384, dev, available=need - 1)
    with pytest.raises(NotImplementedError):
        B.masked_bwd_workspace_check(1, 1, 40000, 40000, dev, available=1 << 40)


def test_bwd_null_pointers(lib):
    for i in range(BWD_PTRS):
        if i == DLSE:
            continue
        ptrs = [P] * BWD_PTRS
        ptrs[i] = N
        assert _bwd(lib, ptrs=ptrs) == 1


def _vfwd(lib, batch=2, mq=64, mk=64, tq=128, tk=128, hq=4, hkv=2, d=512, dtype=0, scale=0.04, causal=1,
          ptrs=None):
    ptrs = ptrs or [P] * 7
    return lib.ffpa_varlen_fwd(*ptrs, batch, mq, mk, tq, tk, hq, hkv, d, dtype, scale, causal, S)


@pytest.mark.parametrize("kw,expect", [
    (dict(batch=0), 1), (dict(mq=-1), 1), (dict(tq=-1), 1), (dict(mq=200), 1), (dict(mk=300), 1),
    (dict(hq=5), 1), (dict(d=100), 2), (dict(causal=-1), 1),
])
def test_varlen_fwd_validation(lib, kw, expect):
    assert _vfwd(lib, **kw) == expect


def test_varlen_null_pointers(lib):
    for i in range(6):  # q, k, v, o, lse, cu_seqlens_q are required; cu_seqlens_k may be NULL
        ptrs = [P] * 7
        ptrs[i] = N
        assert _vfwd(lib, ptrs=ptrs) == 1
    # q, k, v, o, dout, lse, dlse, delta, dq, dk, dv, cu_q, cu_k, then the two host copies (NULL)
    args = [P] * 13 + [N, N]
    args[3] = N
    assert lib.ffpa_varlen_bwd(*args, 2, 64, 64, 128, 128, 4, 2, 512, 0, 0.04, 1, N, 0, S) == 1
    # too small a dS workspace
    assert lib.ffpa_varlen_bwd(*([P] * 13), N, N, 2, 64, 64, 128, 128, 4, 2, 512, 0, 0.04, 1, P, 1024, S) == 1


def test_varlen_null_cu_seqlens_k_needs_equal_totals(lib):
    """cu_seqlens_k = NULL reuses the query offsets for the keys: total_k != total_q would index K
    and V out of range, so it is an invalid argument (forward and backward)."""
    ptrs = [P] * 7
    ptrs[6] = N
    assert _vfwd(lib, ptrs=ptrs, tq=128, tk=96, mk=64) == 1
    bargs = [P] * 12 + [N, N, N]
    assert lib.ffpa_varlen_bwd(*bargs, 2, 64, 64, 128, 96, 4, 2, 512, 0, 0.04, 1, N, 0, S) == 1
    # host copy of k without one of q is rejected
    cu = (ctypes.c_int32 * 3)(0, 64, 128)
    hargs = [P] * 13 + [N, ctypes.cast(cu, ctypes.c_void_p)]
    assert lib.ffpa_varlen_bwd(*hargs, 2, 64, 64, 128, 128, 4, 2, 512, 0, 0.04, 1, N, 0, S) == 1


def test_varlen_host_cu_seqlens_checked(lib):
    """Host copies of cu_seqlens are validated before anything is launched."""
    def call(cq, ck, tq=128, tk=128, mq=64, mk=64, ws=N, nws=0):
        aq = (ctypes.c_int32 * len(cq))(*cq)
        ak = (ctypes.c_int32 * len(ck))(*ck)
        args = [P] * 13 + [ctypes.cast(aq, ctypes.c_void_p), ctypes.cast(ak, ctypes.c_void_p)]
        return lib.ffpa_varlen_bwd(*args, len(cq) - 1, mq, mk, tq, tk, 4, 2, 512, 0, 0.04, 1, ws, nws, S)
    assert call([1, 64, 128], [0, 64, 128]) == 1        # does not start at 0
    assert call([0, 70, 128], [0, 64, 128]) == 1        # a length above max_seqlen_q
    assert call([0, 64, 120], [0, 64, 128]) == 1        # does not end at total_q
    assert call([0, 64, 128], [0, 80, 60]) == 1         # decreasing
    # a workspace of the exact size passes validation only when it is large enough
    from head_dim_attention_amd import _binding as B
    need = B.ffpa_varlen_bwd_workspace_bytes_exact(4, [0, 64, 128], [0, 64, 128], 128, 128, 64, 64)
    assert need == 2 * 4 * (64 * 64 + 64 * 64) * 2
    assert call([0, 64, 128], [0, 64, 128], ws=P, nws=need - 1) == 1


def test_varlen_empty_batch_is_a_noop(lib):
    # total_q == 0: nothing to compute, no launch, OK (no GPU needed).
    assert _vfwd(lib, tq=0, mq=0) == 0


def test_binding_rejects_cpu_tensors():
    import head_dim_attention_amd as F
    q = torch.zeros(1, 2, 8, 512, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        F.ffpa_fwd(q, q, q)


def test_binding_rejects_bad_dtype_before_launch():
    from head_dim_attention_amd import _binding as B
    with pytest.raises(NotImplementedError):
        B._dtype_code(torch.zeros(1, dtype=torch.float32))


def test_binding_checks_cu_seqlens_on_host():
    from head_dim_attention_amd import _binding as B
    ok = torch.tensor([0, 3, 3, 8], dtype=torch.int32)
    assert B._check_cu(ok, 8, "cu") == [0, 3, 3, 8]
    for bad, total in ((torch.tensor([1, 3, 8], dtype=torch.int32), 8),
                       (torch.tensor([0, 5, 3, 8], dtype=torch.int32), 8),
                       (torch.tensor([0, 3, 7], dtype=torch.int32), 8),
                       (torch.tensor([0, 3, 8], dtype=torch.int64), 8)):
        with pytest.raises(ValueError):
            B._check_cu(bad, total, "cu")


def test_bench_refuses_multi_gpu():
    import bench
    assert bench.main(["--gpus", "2"]) == 2


def test_bench_refuses_workloads_it_cannot_step():
    """A step is forward + backward on a dense batch: forward-only and varlen workloads are refused
    before any device work."""
    import bench
    assert bench.main(["--workload", "fwd_d320_n512"]) == 2
    assert bench.main(["--workload", "varlen_causal_d512"]) == 2


def test_bench_legal_pair_count():
    import bench
    assert bench.legal_pairs(4, 4, False) == 16
    assert bench.legal_pairs(4, 4, True) == 10
    assert bench.legal_pairs(5, 3, True) == 0 + 0 + 1 + 2 + 3
    assert bench.legal_pairs(3, 5, True) == 3 + 4 + 5
    n = 8192
    assert bench.legal_pairs(n, n, True) == n * (n + 1) // 2


def test_decode_workspace_sizes(lib):
    from head_dim_attention_amd import _binding as B
    # batch * hq * nq * nsplit * (d + 1) * 4 bytes: one fp32 O row and one LSE per key range
    n = B.ffpa_decode_workspace_bytes(1, 32, 8, 1, 65536, 512)
    assert n > 0 and n % (32 * 513 * 4) == 0
    nsplit = n // (32 * 513 * 4)
    assert 1 <= nsplit <= 256 and 2048 // nsplit >= 4  # at least four 32-key tiles per range
    assert B.ffpa_decode_workspace_bytes(1, 2, 2, 1, 40, 512) == 2 * 1 * 513 * 4  # two tiles: one range
    assert B.ffpa_decode_workspace_bytes(0, 2, 2, 1, 40, 512) == 0
    assert B.ffpa_decode_workspace_bytes(1, 3, 2, 1, 40, 512) == 0  # hq % hkv != 0


def test_decode_validation(lib):
    args = [P] * 5 + [1, 2, 2, 1, 64, 512, 0, 0.04, 0]
    assert lib.ffpa_decode_fwd(*args, N, 1 << 20, S) == 1            # NULL workspace
    assert lib.ffpa_decode_fwd(*args, P, 16, S) == 1                 # too small
    bad_d = [P] * 5 + [1, 2, 2, 1, 64, 300, 0, 0.04, 0]
    assert lib.ffpa_decode_fwd(*bad_d, P, 1 << 20, S) == 2          # unsupported head dim


def _strided_args(strides, ptrs=None):
    ptrs = ptrs or [P] * 5
    return (*ptrs, 1, 2, 2, 64, 64, 512, strides, 0, 0.04, 0, S)


def test_strided_validation(lib):
    ok = [64 * 2 * 512, 512, 2 * 512] * 4          # [B, N, H, D] viewed as [B, H, N, D]
    arr = lambda xs: (ctypes.c_int64 * 12)(*xs)
    assert lib.ffpa_fwd_strided(*_strided_args(None)) == 1                     # NULL strides
    for i in range(12):
        bad = list(ok)
        bad[i] = 4                                                              # not a multiple of 8
        assert lib.ffpa_fwd_strided(*_strided_args(arr(bad))) == 1
        bad[i] = -8                                                             # negative
        assert lib.ffpa_fwd_strided(*_strided_args(arr(bad))) == 1
    huge = list(ok)
    huge[5] = 1 << 26                                                           # K rows beyond 2^31 bytes
    assert lib.ffpa_fwd_strided(*_strided_args(arr(huge))) == 1
    mis = [P, ctypes.c_void_p(0x1008), P, P, P]                                 # k not 16-byte aligned
    assert lib.ffpa_fwd_strided(*_strided_args(arr(ok), mis)) == 1
    args = (P, P, P, P, P, 1, 2, 2, 1, 64, 512, arr(ok), 0, 0.04, 0)
    assert lib.ffpa_decode_fwd_strided(*args, N, 1 << 20, S) == 1             # NULL workspace
    assert lib.ffpa_decode_fwd_strided(P, P, P, P, P, 1, 2, 2, 1, 64, 512, None, 0, 0.04, 0, P, 1 << 20, S) == 1


def test_mask_validation(lib):
    arr = lambda *xs: (ctypes.c_int64 * 4)(*xs)
    base = (P, P, P, P, P, 1, 2, 2, 64, 64, 512)
    tail = (0, 0.04, 0, S)
    good = arr(0, 64 * 64, 64, 1)
    assert lib.ffpa_fwd_masked(*base, N, 1, good, *tail) == 1                 # NULL mask
    assert lib.ffpa_fwd_masked(*base, P, 3, good, *tail) == 1                 # unknown kind
    assert lib.ffpa_fwd_masked(*base, P, 1, None, *tail) == 1                 # NULL strides
    assert lib.ffpa_fwd_masked(*base, P, 1, arr(0, 64 * 64, 64, 2), *tail) == 1   # key stride 2
    assert lib.ffpa_fwd_masked(*base, P, 1, arr(0, 64 * 64, 60, 1), *tail) == 1  # row stride % 8
    assert lib.ffpa_fwd_masked(*base, P, 1, arr(-8, 0, 64, 1), *tail) == 1       # negative
    assert lib.ffpa_fwd_masked(*base, ctypes.c_void_p(0x1008), 1, good, *tail) == 1  # 8-byte aligned bias
    bw = (P,) * 11 + (1, 2, 2, 64, 64, 512)
    assert lib.ffpa_bwd_masked(*bw, P, 1, good, N, 0, 0.04, 0, N, 0, S) == 1       # no workspace
    assert lib.ffpa_bwd_masked(*bw, P, 2, good, P, 0, 0.04, 0, P, 1 << 30, S) == 1  # gradient of a bool mask


def test_fp8_workspace_sizes(lib):
    """ffpa_fwd_fp8_workspace_bytes: amax of Q, K, V (fp32), K8 (one byte per element) and V8^T with
    the key count padded to 64, each part 256-byte aligned; 0 outside the supported sizes."""
    lib.ffpa_fwd_fp8_workspace_bytes.restype = ctypes.c_size_t
    al = lambda x: (x + 255) // 256 * 256
    for b, hq, hkv, nkv, d in ((1, 32, 32, 8192, 512), (2, 4, 2, 150, 320), (1, 4, 1, 333, 448), (3, 6, 3, 1, 384),
                               (1, 32, 8, 8192, 1024), (2, 4, 2, 150, 544)):
        want = al(4 * (b * hq + 2 * b * hkv)) + al(b * hkv * nkv * d) + al(b * hkv * d * ((nkv + 63) // 64 * 64))
        assert lib.ffpa_fwd_fp8_workspace_bytes(b, hq, hkv, 7, nkv, d) == want
    for bad in ((1, 2, 2, 8, 8, 1056), (1, 2, 2, 8, 8, 300), (1, 3, 2, 8, 8, 512), (0, 2, 2, 8, 8, 512),
                (1, 2, 2, 0, 8, 512), (1, 2, 2, 8, 0, 512)):
        assert lib.ffpa_fwd_fp8_workspace_bytes(*bad) == 0


def test_fp8_validation(lib):
    """Host checks of ffpa_fwd_fp8 (no launch happens for any of these)."""
    def call(b=1, hq=2, hkv=2, nq=64, nkv=64, d=512, dtype=0, scale=0.04, causal=0, ptrs=None, ws=P, nws=1 << 30):
        ptrs = ptrs or [P] * 5
        return lib.ffpa_fwd_fp8(*ptrs, b, hq, hkv, nq, nkv, d, dtype, ctypes.c_float(scale), causal, ws, nws, S)
    assert call(ws=N) == 1                                   # no workspace
    assert call(nws=1024) == 1                               # workspace too small
    assert call(d=1056) == 2 and call(d=300) == 2            # head dims the FP8 path does not cover
    assert call(d=1024, nkv=8192, nws=1 << 20) == 1          # workspace too small at D = 1024
    assert call(b=2048, hq=64, hkv=64, nq=1, nkv=1) == 2     # batch x heads beyond one grid dimension
    assert call(hq=3, hkv=2) == 1 and call(dtype=7) == 1 and call(scale=-1.0) == 1 and call(causal=2) == 1
    assert call(nq=0) == 1 and call(nkv=0) == 1
    for i in range(5):
        ptrs = [P] * 5
        ptrs[i] = N
        assert call(ptrs=ptrs) == 1


def test_fwd_split_workspace_and_validation(lib):
    """ffpa_fwd_split_workspace_bytes: B Hq Nq nsplit (D + 1) fp32 values when the grid has fewer
    than two workgroups per compute unit (128 queries per workgroup for D <= 512, 64 above), else 0;
    ffpa_fwd_split then needs a workspace of that size, and is ffpa_fwd when it is 0."""
    lib.ffpa_fwd_split_workspace_bytes.restype = ctypes.c_size_t
    f = lib.ffpa_fwd_split_workspace_bytes
    assert f(1, 32, 32, 8192, 8192, 512) == 0                      # 2048 workgroups: no split
    assert f(1, 2, 2, 128, 128, 512) == 0                          # 4 key tiles: too short to split
    # 8 heads x 32 tiles = 256 workgroups -> 2 ranges
    assert f(1, 8, 8, 4096, 4096, 512) == 1 * 8 * 4096 * 2 * 513 * 4
    assert f(1, 2, 2, 300, 4096, 768) == 2 * 300 * 8 * 769 * 4    # 10 workgroups -> 8 ranges
    assert f(1, 2, 2, 300, 4096, 300) == 0 and f(1, 3, 2, 300, 4096, 512) == 0
    def call(b=1, hq=8, hkv=8, nq=4096, nkv=4096, d=512, ws=P, nws=1 << 30):
        return lib.ffpa_fwd_split(P, P, P, P, P, b, hq, hkv, nq, nkv, d, 0, ctypes.c_float(0.04), 1, ws, nws, S)
    assert call(ws=N) == 1 and call(nws=1024) == 1
    assert call(hq=3, hkv=2, ws=N) == 1       # no split for invalid sizes: ffpa_fwd's checks apply


def test_decode_noalloc_validation(lib):
    """ffpa_decode_fwd_noalloc checks every argument, then its sizes against the fixed scratch,
    before it touches the device (fake pointers: nothing is dereferenced)."""
    from head_dim_attention_amd import _binding as B
    args = lambda b, hq, hkv, nq, nkv, d, dt=0, scale=0.04, causal=1: (P, P, P, P, P, b, hq, hkv, nq, nkv, d, dt,
                                                                         scale, causal, S)
    assert lib.ffpa_decode_fwd_noalloc(*args(0, 32, 8, 1, 4096, 512)) == 1
    assert lib.ffpa_decode_fwd_noalloc(*args(1, 32, 8, 1, 4096, 300)) == 2
    assert lib.ffpa_decode_fwd_noalloc(*args(1, 32, 8, 1, 4096, 512, dt=3)) == 1
    assert lib.ffpa_decode_fwd_noalloc(N, P, P, P, P, 1, 32, 8, 1, 4096, 512, 0, 0.04, 1, S) == 1
    assert B.ffpa_decode_workspace_bytes(64, 32, 8, 7, 4096, 1024) > B.NOALLOC_SCRATCH_BYTES
    assert lib.ffpa_decode_fwd_noalloc(*args(64, 32, 8, 7, 4096, 1024)) == B.FFPA_ERR_TOO_LARGE
    assert "TOO_LARGE" in B.ffpa_status_string(B.FFPA_ERR_TOO_LARGE)


def test_fused_products_decision(lib):
    """One-launch dK/dV/dQ for dense grids below two workgroups per CU per pass, with a workspace."""
    from head_dim_attention_amd import _binding as B
    assert B.ffpa_bwd_fused_products(1, 8, 8, 4096, 4096, 512)          # 256 items per pass
    assert not B.ffpa_bwd_fused_products(1, 32, 32, 8192, 8192, 512)    # 2048 items per pass
    assert not B.ffpa_bwd_fused_products(1, 32, 8, 8192, 8192, 1024)
    assert not B.ffpa_bwd_fused_products(1, 1, 1, 40000, 40000, 512)    # no workspace for these sizes
    assert not B.ffpa_bwd_fused_products(1, 8, 8, 4096, 4096, 300)      # unsupported head dim
    # stage 5 without a workspace is an invalid argument (nothing launched)
    args = [P] * 11 + [1, 2, 2, 64, 64, 512, 0, 0.04, 1, N, 0, S]
    assert lib.ffpa_bwd_stage(5, *args) == 1
