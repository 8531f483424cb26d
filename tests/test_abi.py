"""The C ABI on the CPU: the library loads, exports what include/fa.h
declares, and rejects bad arguments synchronously, before any HIP call (so no
GPU is needed).  No compute call is made here."""
import ctypes
import math
import os
import re

import pytest

from exact_io_aware_33_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

INVALID, UNSUPPORTED = _lib.FA_ERR_INVALID, _lib.FA_ERR_UNSUPPORTED
A = 0x10000          # fake, 16-byte aligned "device" address (never dereferenced)


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(fa_[a-z_]+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def prob(**kw):
    p = dict(batch=2, heads=3, seqlen=256, head_dim=64, stride_b=3 * 256 * 64, stride_h=256 * 64,
             stride_n=64, scale=0.125, causal=0, dtype=_lib.FA_DTYPE_BF16, key_lens=None)
    p.update(kw)
    return _lib.FaProblem(**p)


def fwd(lib, p, q=A, k=A, v=A, o=A, lse=A):
    return lib.fa_fwd(ctypes.byref(p), q, k, v, o, lse, None)


def bwd(lib, p, ws_bytes=None, **ptrs):
    a = dict(q=A, k=A, v=A, o=A, lse=A, do=A, dq=A, dk=A, dv=A, ws=A)
    a.update(ptrs)
    if ws_bytes is None:
        ws_bytes = lib.fa_bwd_workspace_bytes(ctypes.byref(p))
    return lib.fa_bwd(ctypes.byref(p), a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"],
                      a["dk"], a["dv"], a["ws"], ws_bytes, None)


def test_exports_match_header(lib):
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n
    assert lib.fa_abi_version() == _lib.ABI_VERSION == 4


def test_status_strings(lib):
    for s in range(4):
        assert lib.fa_status_string(s)
    assert lib.fa_status_string(99)


@pytest.mark.parametrize("field,value,status", [
    ("batch", 0, INVALID), ("heads", -1, INVALID), ("seqlen", 0, INVALID),
    ("head_dim", 0, INVALID), ("head_dim", 96, UNSUPPORTED), ("head_dim", 256, UNSUPPORTED),
    ("dtype", 7, INVALID), ("scale", float("nan"), INVALID), ("scale", float("inf"), INVALID),
    ("scale", -0.5, INVALID), ("stride_n", 60, INVALID), ("stride_n", 36, INVALID),
    ("stride_h", -64, INVALID), ("key_lens", 0x10004, UNSUPPORTED),
    ("stride_b", 4, UNSUPPORTED), ("stride_h", 3 * 256 * 64 + 4, UNSUPPORTED),
    ("stride_n", 68, UNSUPPORTED),
    ("seqlen", 1 << 30, UNSUPPORTED),
    ("dropout_p", -0.1, INVALID), ("dropout_p", 1.0, INVALID), ("dropout_p", 1.5, INVALID),
    ("dropout_p", float("nan"), INVALID), ("dropout_p", float("inf"), INVALID),
    ("seqlen_k", -1, INVALID), ("seqlen_k", 1 << 30, UNSUPPORTED), ("fwd_query_tile", 1, INVALID),
    ("fwd_query_tile", 96, INVALID), ("fwd_query_tile", -64, INVALID),
    ("k_stride_n", 60, INVALID), ("k_stride_h", -64, INVALID), ("k_stride_b", 4, INVALID),
])
def test_problem_rejected_before_any_hip_call(lib, field, value, status):
    p = prob(**{field: value})
    assert fwd(lib, p) == status
    assert lib.fa_last_error()
    assert bwd(lib, p, ws_bytes=1 << 40) == status
    assert lib.fa_bwd_workspace_bytes(ctypes.byref(p)) == 0


def test_null_problem(lib):
    assert lib.fa_fwd(None, A, A, A, A, A, None) == INVALID


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "lse"])
@pytest.mark.parametrize("bad,status", [(0, INVALID), (A + 8, UNSUPPORTED)])
def test_forward_pointers(lib, which, bad, status):
    """NULL is an invalid argument; a pointer off the 16-byte grid is a
    layout the vector path is not built for."""
    kw = {which: bad}
    assert fwd(lib, prob(), **kw) == status
    assert which in lib.fa_last_error().decode()


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "lse", "do", "dq", "dk", "dv", "ws"])
def test_backward_pointers(lib, which):
    assert bwd(lib, prob(), **{which: 0}) == INVALID
    assert bwd(lib, prob(), **{which: A + 4}) == UNSUPPORTED


def test_workspace_size_and_too_small(lib):
    p = prob()
    need = lib.fa_bwd_workspace_bytes(ctypes.byref(p))
    rows = 2 * 3 * 256
    assert rows * 8 <= need <= rows * 8 + 512         # two floats per row: O(N)
    assert bwd(lib, p, ws_bytes=need - 1) == INVALID


def test_fp32_strides_need_16_bytes(lib):
    p = prob(dtype=_lib.FA_DTYPE_F32, stride_n=66, stride_h=256 * 66, stride_b=3 * 256 * 66)
    assert fwd(lib, p) == UNSUPPORTED


def _bnhd(N, H, d, **kw):
    """[B=1, N, H, d] storage seen as [B, H, N, d]: stride_n = H d."""
    return prob(batch=1, heads=H, seqlen=N, head_dim=d, stride_b=N * H * d, stride_h=d,
                stride_n=H * d, **kw)


@pytest.mark.parametrize("case", ["packed_qkv_bf16", "bnhd_fp32", "bnhd_keys_fp32"])
def test_row_byte_offsets_over_31_bits_rejected(lib, case):
    """The kernels address one (batch, head) slice's rows with 32-bit byte
    offsets (buffer record count, tile offsets), tiles overrunning the end by
    up to 256 rows: (N + 256) * stride_n * element size must stay below 2^31.
    Layouts whose elements fit the 2^31 index bound can still break that."""
    if case == "packed_qkv_bf16":
        # [B, N, 3, H, d] bf16 packed QKV, H = 32, N = 512K: B*H*N*d = 2^30,
        # but a slice spans (N - 1) * 6144 * 2 bytes ~ 6.4e9
        N, H, d = 1 << 19, 32, 64
        p = prob(batch=1, heads=H, seqlen=N, head_dim=d, stride_b=N * 3 * H * d, stride_h=d,
                 stride_n=3 * H * d)
    elif case == "bnhd_fp32":
        p = _bnhd(1 << 20, 16, 64, dtype=_lib.FA_DTYPE_F32)        # 4 GiB slice span
    else:
        # queries small, keys in a [B, N_k, H, d] fp32 layout over 4 GiB
        Nk, H, d = 131072, 127, 128
        p = prob(batch=1, heads=H, seqlen=64, head_dim=d, stride_b=H * 64 * d, stride_h=64 * d,
                 stride_n=d, dtype=_lib.FA_DTYPE_F32, seqlen_k=Nk, k_stride_b=Nk * H * d,
                 k_stride_h=d, k_stride_n=H * d)
    assert fwd(lib, p) == UNSUPPORTED
    assert "2^31" in lib.fa_last_error().decode()
    assert bwd(lib, p, ws_bytes=1 << 40) == UNSUPPORTED
    assert lib.fa_bwd_workspace_bytes(ctypes.byref(p)) == 0


def test_row_byte_offsets_at_the_bound(lib):
    """(N + 256) * stride_n * e just below 2^31 passes, at 2^31 fails."""
    H, d = 16, 64                      # bf16 [1, N, 16, 64]: 2048 bytes per row
    N_ok = (1 << 31) // 2048 - 256 - 1
    # the argument checks alone (a passing fwd call would launch on these fake
    # addresses): the workspace-size query runs exactly those checks
    assert lib.fa_bwd_workspace_bytes(ctypes.byref(_bnhd(N_ok, H, d))) > 0
    assert lib.fa_bwd_workspace_bytes(ctypes.byref(_bnhd(N_ok + 1, H, d))) == 0


@pytest.mark.parametrize("mb,hstride,status", [
    (100, 0, INVALID),        # does not divide N = 256
    (64, 0, UNSUPPORTED),     # divides N but is not a multiple of 128
    (0, 0, INVALID),
    (128, -1, INVALID),
])
def test_block_mask_arguments(lib, mb, hstride, status):
    p = prob()
    assert lib.fa_fwd_blocksparse(ctypes.byref(p), A, mb, hstride, A, A, A, A, A, None) == status
    ws = lib.fa_bwd_workspace_bytes(ctypes.byref(p))
    assert lib.fa_bwd_blocksparse(ctypes.byref(p), A, mb, hstride, A, A, A, A, A, A, A, A, A, A, ws,
                                  None) == status


def test_null_block_mask(lib):
    p = prob()
    assert lib.fa_fwd_blocksparse(ctypes.byref(p), None, 128, 0, A, A, A, A, A, None) == INVALID


def test_too_many_mask_blocks(lib):
    p = prob(batch=1, heads=1, seqlen=128 * 1025, stride_h=128 * 1025 * 64, stride_b=128 * 1025 * 64)
    assert lib.fa_fwd_blocksparse(ctypes.byref(p), A, 128, 0, A, A, A, A, A, None) == UNSUPPORTED


def test_error_message_cleared_by_next_call(lib):
    assert fwd(lib, prob(batch=0)) == INVALID
    assert lib.fa_last_error()
    lib.fa_bwd_workspace_bytes(ctypes.byref(prob()))
    assert lib.fa_last_error() == b""


def test_python_binding_refuses_missing_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libfa.so"))
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load()


def test_problem_struct_layout_matches_header(tmp_path):
    """The ctypes mirror of fa_problem_t has the C compiler's field offsets."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    fields = [f[0] for f in _lib.FaProblem._fields_]
    src = tmp_path / "layout.c"
    src.write_text("#include <stdio.h>\n#include <stddef.h>\n#include \"fa.h\"\nint main(void) {\n"
                   + "".join(f'  printf("%zu\\n", offsetof(fa_problem_t, {f}));\n' for f in fields)
                   + '  printf("%zu\\n", sizeof(fa_problem_t));\n  return 0;\n}\n')
    exe = tmp_path / "layout"
    subprocess.run([cc, "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]
    want = [getattr(_lib.FaProblem, f).offset for f in fields] + [ctypes.sizeof(_lib.FaProblem)]
    assert got == want


@pytest.mark.parametrize("nq,nk,mb", [
    (256, 320, 128),  # does not divide N_k
    (384, 256, 256),  # does not divide N_q
])
def test_block_mask_must_divide_both_lengths(lib, nq, nk, mb):
    p = prob(seqlen=nq, seqlen_k=nk, stride_b=3 * nq * 64, stride_h=nq * 64,
             k_stride_b=3 * nk * 64, k_stride_h=nk * 64, k_stride_n=64)
    assert lib.fa_fwd_blocksparse(ctypes.byref(p), A, mb, 0, A, A, A, A, A, None) == INVALID
    assert "divide" in lib.fa_last_error().decode()


def test_workspace_counts_query_rows_only(lib):
    p = prob(seqlen=100, seqlen_k=5000, stride_b=3 * 100 * 64, stride_h=100 * 64,
             k_stride_b=3 * 5000 * 64, k_stride_h=5000 * 64, k_stride_n=64)
    need = lib.fa_bwd_workspace_bytes(ctypes.byref(p))
    assert 2 * 3 * 100 * 8 <= need <= 2 * 3 * 100 * 8 + 512


def _splitkv(lib, p, splits=0, ws=A, ws_bytes=None, mask=None, mb=128):
    if ws_bytes is None:
        ws_bytes = lib.fa_fwd_splitkv_workspace_bytes(ctypes.byref(p), splits)
    return lib.fa_fwd_splitkv(ctypes.byref(p), mask, mb, 0, splits, A, A, A, A, A, ws, ws_bytes, None)


def test_splitkv_choice_and_workspace(lib):
    p = prob(seqlen=1, seqlen_k=32768, stride_b=3 * 64, stride_h=64,
             k_stride_b=3 * 32768 * 64, k_stride_h=32768 * 64, k_stride_n=64)
    n = lib.fa_fwd_splitkv_num_splits(ctypes.byref(p))
    assert 1 <= n <= 128
    rows = 2 * 3 * 1
    assert lib.fa_fwd_splitkv_workspace_bytes(ctypes.byref(p), 0) == \
        lib.fa_fwd_splitkv_workspace_bytes(ctypes.byref(p), n)
    need7 = lib.fa_fwd_splitkv_workspace_bytes(ctypes.byref(p), 7)
    assert 7 * rows * (64 + 1) * 4 <= need7 <= 7 * rows * (64 + 1) * 4 + 512
    assert lib.fa_fwd_splitkv_workspace_bytes(ctypes.byref(p), 1025) == 0
    # a large problem gets a single split (the query tiles already fill the GPU)
    big = prob(seqlen=16384, batch=4, heads=16, stride_b=16 * 16384 * 64, stride_h=16384 * 64)
    assert lib.fa_fwd_splitkv_num_splits(ctypes.byref(big)) == 1


@pytest.mark.parametrize("case,status", [
    ("too_many_splits", INVALID), ("workspace_small", INVALID), ("workspace_null", INVALID),
    ("dropout", UNSUPPORTED), ("mask_block", INVALID), ("bad_problem", INVALID),
])
def test_splitkv_rejected_before_any_hip_call(lib, case, status):
    p = prob()
    if case == "too_many_splits":
        assert _splitkv(lib, p, splits=1025, ws_bytes=1 << 40) == status
    elif case == "workspace_small":
        need = lib.fa_fwd_splitkv_workspace_bytes(ctypes.byref(p), 4)
        assert _splitkv(lib, p, splits=4, ws_bytes=need - 1) == status
    elif case == "workspace_null":
        assert _splitkv(lib, p, ws=0) == status
    elif case == "dropout":
        assert _splitkv(lib, prob(dropout_p=0.1), ws_bytes=1 << 40) == status
    elif case == "mask_block":
        assert _splitkv(lib, p, mask=A, mb=100, ws_bytes=1 << 40) == status
    else:
        assert _splitkv(lib, prob(seqlen=0), ws_bytes=1 << 40) == status
    assert lib.fa_last_error()


@pytest.mark.parametrize("args,status", [
    (dict(dtype=7), INVALID), (dict(rows=0), INVALID), (dict(cols=0), INVALID),
    (dict(ld_x=7, cols=8), INVALID), (dict(ld_y=12), INVALID), (dict(x=0), INVALID),
    (dict(y=A + 1), INVALID), (dict(rows=1 << 31), UNSUPPORTED),
])
def test_softmax_rows_rejected(lib, args, status):
    a = dict(dtype=_lib.FA_DTYPE_BF16, rows=4, cols=64, x=A, ld_x=64, y=A, ld_y=64, lse=A)
    a.update(args)
    assert lib.fa_softmax_rows(a["dtype"], a["rows"], a["cols"], a["x"], a["ld_x"], a["y"], a["ld_y"],
                               a["lse"], None) == status
    assert lib.fa_last_error()


@pytest.mark.parametrize("args,status", [
    (dict(eps=-1.0), INVALID), (dict(eps=float("nan")), INVALID), (dict(groups=0), INVALID),
    (dict(inner=0), INVALID), (dict(inner=5), INVALID), (dict(gamma=A + 1), INVALID),
    (dict(mean=A + 2), INVALID), (dict(cols=0), INVALID),
])
def test_layernorm_rows_rejected(lib, args, status):
    a = dict(dtype=_lib.FA_DTYPE_F16, rows=4, cols=64, x=A, ld_x=64, gamma=None, beta=None, eps=1e-5,
             groups=1, inner=1, y=A, ld_y=64, mean=None, rstd=None)
    a.update(args)
    assert lib.fa_layernorm_rows(a["dtype"], a["rows"], a["cols"], a["x"], a["ld_x"], a["gamma"],
                                 a["beta"], a["eps"], a["groups"], a["inner"], a["y"], a["ld_y"],
                                 a["mean"], a["rstd"], None) == status
    assert lib.fa_last_error()


def _noalloc(lib, p, mask=None, mb=128, **ptrs):
    a = dict(q=A, k=A, v=A, o=A, lse=A, do=A, dq=A, dk=A, dv=A)
    a.update(ptrs)
    return lib.fa_bwd_noalloc(ctypes.byref(p), mask, mb, 0, a["q"], a["k"], a["v"], a["o"], a["lse"],
                              a["do"], a["dq"], a["dk"], a["dv"], None)


@pytest.mark.parametrize("case,status", [
    ("bad_problem", INVALID), ("null_q", INVALID), ("misaligned_dk", UNSUPPORTED),
    ("mask_block", INVALID), ("too_many_rows", UNSUPPORTED),
])
def test_noalloc_rejected_before_any_hip_call(lib, case, status):
    """The allocation-free backward runs every check of fa_bwd, then refuses
    a workspace beyond its static array -- all before any HIP call.  (A call
    that passes the checks would launch, so none is made here.)"""
    if case == "bad_problem":
        assert _noalloc(lib, prob(head_dim=96)) == UNSUPPORTED
        assert _noalloc(lib, prob(seqlen=0)) == status
    elif case == "null_q":
        assert _noalloc(lib, prob(), q=0) == status
    elif case == "misaligned_dk":
        assert _noalloc(lib, prob(), dk=A + 4) == status
    elif case == "mask_block":
        assert _noalloc(lib, prob(), mask=A, mb=100) == status
    else:
        # 32 heads x 65600 queries = 2,099,200 rows: 2 floats each exceed 16 MiB
        N, H = 65600, 32
        p = prob(batch=1, heads=H, seqlen=N, stride_b=H * N * 64, stride_h=N * 64, stride_n=64)
        need = lib.fa_bwd_workspace_bytes(ctypes.byref(p))
        assert need > _lib.FA_BWD_NOALLOC_MAX_WORKSPACE_BYTES
        assert _noalloc(lib, p) == status
        assert "static" in lib.fa_last_error().decode()
    assert lib.fa_last_error()


def test_noalloc_limit_matches_header():
    src = open(HEADER).read()
    m = re.search(r"#define FA_BWD_NOALLOC_MAX_WORKSPACE_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.FA_BWD_NOALLOC_MAX_WORKSPACE_BYTES


def _merge(lib, p, parts, lse_parts, o=A, lse=A, n=None):
    S = len(parts) if n is None else n
    op = None if parts is None else (ctypes.c_void_p * max(1, len(parts)))(*parts)
    lp = None if lse_parts is None else (ctypes.c_void_p * max(1, len(lse_parts)))(*lse_parts)
    return lib.fa_merge_partials(ctypes.byref(p), S, op, lp, o, lse, None)


@pytest.mark.parametrize("case,status", [
    ("zero_parts", INVALID), ("too_many", INVALID), ("null_arrays", INVALID),
    ("null_part", INVALID), ("misaligned_part", UNSUPPORTED), ("misaligned_lse_part", UNSUPPORTED),
    ("null_out", INVALID), ("bad_problem", UNSUPPORTED),
])
def test_merge_rejected_before_any_hip_call(lib, case, status):
    p = prob()
    two = [A, A + 1024]
    if case == "zero_parts":
        st = _merge(lib, p, two, two, n=0)
    elif case == "too_many":
        st = _merge(lib, p, [A] * 65, [A] * 65)
    elif case == "null_arrays":
        st = _merge(lib, p, None, None, n=2)
    elif case == "null_part":
        st = _merge(lib, p, [A, 0], two)
    elif case == "misaligned_part":
        st = _merge(lib, p, [A, A + 8], two)
    elif case == "misaligned_lse_part":
        st = _merge(lib, p, two, [A, A + 4])
    elif case == "null_out":
        st = _merge(lib, p, two, two, o=0)
    else:
        st = _merge(lib, prob(head_dim=80), two, two)
    assert st == status
    assert lib.fa_last_error()


@pytest.mark.parametrize("kw,sparse", [
    (dict(fwd_query_tile=64, dtype=_lib.FA_DTYPE_F32), False),
    (dict(fwd_query_tile=256, dtype=_lib.FA_DTYPE_F32), False),
    (dict(fwd_query_tile=64, dropout_p=0.1), False),
    (dict(fwd_query_tile=256), True),
])
def test_query_tile_not_built_is_refused(lib, kw, sparse):
    """Query tiles other than 128 exist for fp16 / bf16 without dropout; 256
    not with a block mask (a workgroup must lie within one mask block row)."""
    p = prob(**kw)
    if sparse:
        st = lib.fa_fwd_blocksparse(ctypes.byref(p), A, 128, 0, A, A, A, A, A, None)
    else:
        st = fwd(lib, p)
    assert st == UNSUPPORTED
    assert "fwd_query_tile" in lib.fa_last_error().decode()
