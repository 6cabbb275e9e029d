"""The C-ABI library loads, exports every declared entry point, and rejects bad
arguments before touching the GPU (CPU only: no compute calls are made)."""
import ctypes
import os
import re

import pytest

from tiled_exact_attention_bf16_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa_gfx950.h")

pytestmark = pytest.mark.skipif(not os.path.exists(L.LIB_PATH), reason="library not built")

P = 0x100000  # aligned stand-in device addresses; never dereferenced on these paths


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = L.lib()
    names = declared_functions()
    assert {"fa_fwd", "fa_bwd", "fa_fwd_workspace_size", "fa_bwd_workspace_size", "fa_status_str"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(L.SIGNATURES) == set(names)


def test_check_build_exports_the_same_symbols():
    serial = L.load(L.SERIAL_LIB_PATH)  # the serial-loads check build
    for n in declared_functions():
        assert hasattr(serial, n), n


def test_status_strings():
    for code, name in [(0, "FA_OK"), (1, "FA_ERR_INVALID_ARGUMENT"), (2, "FA_ERR_UNSUPPORTED"),
                       (3, "FA_ERR_WORKSPACE_TOO_SMALL"), (4, "FA_ERR_HIP")]:
        assert L.status_str(code) == name
    assert L.lib().fa_version().startswith(b"fa_gfx950")


def fwd_args(b=2, s=256, h=4, d=128, causal=0, scale=0.088):
    a = L.FwdArgs()
    a.q, a.k, a.v, a.o, a.lse = P, P + 0x1000000, P + 0x2000000, P + 0x3000000, P + 0x4000000
    st = L.Strides(s * h * d, h * d, d)
    a.q_stride = a.k_stride = a.v_stride = a.o_stride = st
    a.batch, a.seqlen_q, a.seqlen_k, a.num_heads, a.head_dim = b, s, s, h, d
    a.softmax_scale, a.causal = scale, causal
    return a


def ws_size(a, tuning=None):
    n = ctypes.c_size_t(123)
    t = tuning if tuning is not None else L.FwdTuning(-1, -1, -1, -1)
    st = L.lib().fa_fwd_workspace_size(ctypes.byref(a), ctypes.byref(t), ctypes.byref(n))
    return st, n.value


def fwd_status(a, tuning=None, ws=None, ws_bytes=0):
    t = tuning if tuning is not None else L.FwdTuning(-1, -1, -1)
    return L.lib().fa_fwd(ctypes.byref(a), ctypes.byref(t), ws, ws_bytes, None)


def v16_bytes(h, total_k, d):
    """Workspace of the fp16 copy of V and its per-tile exponents (256-byte aligned parts)."""
    r = lambda x: (x + 255) // 256 * 256
    return r(h * total_k * d * 2) + r(h * total_k * 4)


def test_fixed_length_forward_workspace_is_the_fp16_v_copy():
    # the PV product runs in fp16: the workspace holds V converted to fp16 (2 bytes per
    # element) and one int32 exponent slot per key row and head
    assert ws_size(fwd_args()) == (L.FA_OK, v16_bytes(4, 2 * 256, 128))
    assert ws_size(fwd_args(d=64)) == (L.FA_OK, v16_bytes(4, 2 * 256, 64))
    assert fwd_status(fwd_args(), ws=None, ws_bytes=0) == L.FA_ERR_WORKSPACE_TOO_SMALL
    assert fwd_status(fwd_args(), ws=P, ws_bytes=v16_bytes(4, 512, 128) - 1) == L.FA_ERR_WORKSPACE_TOO_SMALL
    empty = fwd_args(b=0)
    assert ws_size(empty) == (L.FA_OK, 0)


@pytest.mark.parametrize("mutate,expect", [
    (lambda a: setattr(a, "q", None), L.FA_ERR_INVALID_ARGUMENT),
    (lambda a: setattr(a, "lse", None), L.FA_ERR_INVALID_ARGUMENT),
    (lambda a: setattr(a, "k", P + 8), L.FA_ERR_INVALID_ARGUMENT),          # misaligned
    (lambda a: setattr(a, "head_dim", 96), L.FA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "head_dim", 0), L.FA_ERR_INVALID_ARGUMENT),
    (lambda a: setattr(a, "num_heads", 0), L.FA_ERR_INVALID_ARGUMENT),
    (lambda a: setattr(a, "batch", -1), L.FA_ERR_INVALID_ARGUMENT),
    (lambda a: setattr(a, "seqlen_q", -5), L.FA_ERR_INVALID_ARGUMENT),
    (lambda a: setattr(a, "softmax_scale", float("nan")), L.FA_ERR_INVALID_ARGUMENT),
    (lambda a: setattr(a, "softmax_scale", float("inf")), L.FA_ERR_INVALID_ARGUMENT),
    (lambda a: setattr(a, "softmax_scale", -1.0), L.FA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "softmax_scale", 0.0), L.FA_ERR_UNSUPPORTED),    # scale must be > 0
    (lambda a: setattr(a, "softmax_scale", -0.0), L.FA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "causal", 2), L.FA_ERR_INVALID_ARGUMENT),
    (lambda a: setattr(a, "q_stride", L.Strides(256 * 512, 500, 128)), L.FA_ERR_INVALID_ARGUMENT),  # stride % 8
    (lambda a: setattr(a, "o_stride", L.Strides(256 * 512, 64, 128)), L.FA_ERR_INVALID_ARGUMENT),   # rows overlap D
    (lambda a: setattr(a, "cu_seqlens_k", P), L.FA_ERR_INVALID_ARGUMENT),   # k offsets without q offsets
    (lambda a: setattr(a, "v_stride", L.Strides(0, 1 << 24, 128)), L.FA_ERR_UNSUPPORTED),  # 32-bit offsets
])
def test_forward_validation(mutate, expect):
    a = fwd_args()
    mutate(a)
    assert fwd_status(a) == expect
    assert ws_size(a)[0] == expect


def test_fp32_output_option():
    # o_dtype selects bf16 (default) or fp32 O; anything else is rejected before any
    # device work, and fp32 strides count fp32 elements (multiples of 4 for 16 bytes)
    a = fwd_args()
    a.o_dtype = 2
    assert fwd_status(a) == L.FA_ERR_INVALID_ARGUMENT
    assert ws_size(a)[0] == L.FA_ERR_INVALID_ARGUMENT
    a = fwd_args()
    a.o_dtype = L.FA_DTYPE_F32
    a.o_stride = L.Strides(256 * 4 * 132, 4 * 132, 132)
    assert ws_size(a) == (L.FA_OK, v16_bytes(4, 2 * 256, 128))
    a.o_stride = L.Strides(256 * 4 * 130, 4 * 130, 130)   # 520 bytes: not a 16-byte multiple
    assert ws_size(a)[0] == L.FA_ERR_INVALID_ARGUMENT
    b = fwd_args()                                         # the same strides in bf16 elements
    b.o_stride = L.Strides(256 * 4 * 132, 4 * 132, 132)   # 264 bytes: not a 16-byte multiple
    assert ws_size(b)[0] == L.FA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("tuning,expect", [
    ((3, -1, -1), L.FA_ERR_UNSUPPORTED),
    ((2, 0, -1), L.FA_ERR_UNSUPPORTED),
    ((-1, 5, -1), L.FA_ERR_UNSUPPORTED),
    ((-1, -1, 3), L.FA_ERR_UNSUPPORTED),
    ((-1, -1, -1, 65), L.FA_ERR_UNSUPPORTED),
])
def test_forward_tuning_validation(tuning, expect):
    assert fwd_status(fwd_args(), L.FwdTuning(*tuning)) == expect


@pytest.mark.parametrize("tuning", [(2, 8, -1), (4, -1, 1), (0, 0, 2)])
def test_measurement_variants_need_d128_fixed_length(tuning):
    # the exp2-share and eager-threshold instances exist for head_dim 128, fixed length
    t = L.FwdTuning(*tuning)
    assert ws_size(fwd_args(d=128), t)[0] == L.FA_OK
    assert ws_size(fwd_args(d=64), t)[0] == L.FA_ERR_UNSUPPORTED
    assert fwd_status(fwd_args(d=64), t) == L.FA_ERR_UNSUPPORTED
    assert ws_size(varlen_args(), t)[0] == L.FA_ERR_UNSUPPORTED
    assert ws_size(varlen_args(), L.FwdTuning(0, 8, -1))[0] == L.FA_OK


def test_tile_rows():
    lib = L.lib()
    assert lib.fa_fwd_tile_rows(ctypes.byref(L.FwdTuning(-1, -1, 1))) == 128
    assert lib.fa_fwd_tile_rows(ctypes.byref(L.FwdTuning(-1, -1, 2))) == 256
    assert lib.fa_fwd_tile_rows(ctypes.byref(L.FwdTuning(-1, -1, 7))) == 0
    assert lib.fa_fwd_tile_rows(ctypes.byref(L.FwdTuning(-1, -1, -1, 4))) == 128   # key split: 128-row tiles


def varlen_args(n_seq=32, total=131072, max_len=16384, causal=1, h=16, d=128):
    a = fwd_args(b=n_seq, h=h, d=d, causal=causal)
    a.cu_seqlens_q = P + 0x5000000
    a.total_q = a.total_k = total
    a.max_seqlen_q = a.max_seqlen_k = max_len
    st = L.Strides(0, h * d, d)
    a.q_stride = a.k_stride = a.v_stride = a.o_stride = st
    return a


def test_varlen_workspace_and_checks():
    a = varlen_args()
    st, n = ws_size(a)                                  # default: 256-row work items
    assert st == L.FA_OK
    assert n >= 4 * (1 + 2 * ((131072 + 255) // 256 + 32)) and n % 256 == 0
    t1 = L.FwdTuning(-1, -1, 1)
    st, n1 = ws_size(a, t1)                             # 128-row work items: a longer list
    assert st == L.FA_OK and n1 >= 4 * (1 + 2 * ((131072 + 127) // 128 + 32)) and n1 % 256 == 0
    assert fwd_status(a, ws=None, ws_bytes=0) == L.FA_ERR_WORKSPACE_TOO_SMALL
    assert fwd_status(a, t1, ws=P, ws_bytes=n1 - 256) == L.FA_ERR_WORKSPACE_TOO_SMALL
    assert fwd_status(a, ws=P + 16, ws_bytes=n) == L.FA_ERR_INVALID_ARGUMENT  # workspace alignment
    a.cu_seqlens_k = P + 0x6000000        # separate key offsets under the causal mask (bottom-right)
    assert ws_size(a)[0] == L.FA_OK
    b = varlen_args()
    b.cu_seqlens_q = P + 2                                                   # int32 alignment
    assert ws_size(b)[0] == L.FA_ERR_INVALID_ARGUMENT
    c = varlen_args(max_len=1 << 20)                                         # longest-first histogram range
    assert ws_size(c)[0] == L.FA_ERR_UNSUPPORTED
    d = varlen_args()
    d.max_seqlen_q = -1
    assert ws_size(d)[0] == L.FA_ERR_INVALID_ARGUMENT


def test_build_schedule_rejects_fixed_length_and_small_workspace():
    lib = L.lib()
    t = L.FwdTuning(-1, -1, -1)
    assert lib.fa_fwd_build_schedule(ctypes.byref(fwd_args()), ctypes.byref(t), P, 1 << 20, None) == \
        L.FA_ERR_INVALID_ARGUMENT
    assert lib.fa_fwd_build_schedule(ctypes.byref(varlen_args()), ctypes.byref(t), P, 64, None) == \
        L.FA_ERR_WORKSPACE_TOO_SMALL


def bwd_args(b=2, s=256, h=4, d=128, causal=1, det=0, gd=L.FA_DTYPE_F32):
    a = L.BwdArgs()
    for i, f in enumerate(["q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv"]):
        setattr(a, f, P + i * 0x1000000)
    st = L.Strides(s * h * d, h * d, d)
    for f in ["q", "k", "v", "o", "do", "dq", "dk", "dv"]:
        setattr(a, f + "_stride", st)
    a.batch, a.seqlen_q, a.seqlen_k, a.num_heads, a.head_dim = b, s, s, h, d
    a.softmax_scale, a.causal, a.deterministic, a.grad_dtype = 0.088, causal, det, gd
    return a


def bwd_ws(a):
    n = ctypes.c_size_t(0)
    return L.lib().fa_bwd_workspace_size(ctypes.byref(a), ctypes.byref(n)), n.value


def test_backward_workspace_sizes():
    st, n_atomic = bwd_ws(bwd_args(det=0))
    assert st == L.FA_OK
    rows = 2 * 256 * 4
    copies = 2 * rows * 128 * 2                           # fp16 copies of Q and K
    assert n_atomic >= rows * 128 * 4 + rows * 4 + copies  # fp32 dQ accumulator + row terms + copies
    st, n_det = bwd_ws(bwd_args(det=1))
    assert st == L.FA_OK and rows * 4 + copies <= n_det < n_atomic  # no accumulator in deterministic mode


def test_key_split_workspace_and_validation():
    a = fwd_args(b=2, s=256, h=4, d=128)
    a.seqlen_q, a.seqlen_k = 8, 16384
    base = v16_bytes(4, 2 * 16384, 128)
    assert ws_size(a, L.FwdTuning(-1, -1, -1, 1)) == (L.FA_OK, base)           # split off: the V copy only
    st, n = ws_size(a, L.FwdTuning(-1, -1, -1, 4))
    rows = 4 * 4 * 2 * 8                                                   # splits * heads * total_q
    # the key-split path reads V itself: partial O and LSE only, no V copy
    assert st == L.FA_OK and n >= rows * 4 + rows * 128 * 4 and n < base and n % 256 == 0
    st, n_auto = ws_size(a)                                                # 8 work items: split chosen
    assert st == L.FA_OK and 0 < n_auto < base
    assert ws_size(a, L.FwdTuning(-1, -1, -1, 65))[0] == L.FA_ERR_UNSUPPORTED
    assert fwd_status(a, L.FwdTuning(-1, -1, -1, 4), ws=None, ws_bytes=0) == L.FA_ERR_WORKSPACE_TOO_SMALL
    big = fwd_args()                                                       # many work items: no split
    assert ws_size(big) == (L.FA_OK, v16_bytes(4, 512, 128))


@pytest.mark.parametrize("b,h,lq,lk,expect", [
    (4, 16, 1, 16384, 8),     # 64 items of 128 rows: ~512 workgroups, chunks of 32 tiles
    (1, 16, 1, 65536, 32),    # 16 items: 32 chunks of 32 tiles
    (16, 16, 1, 4096, 2),     # 256 items: two chunks
    (8, 8, 128, 8192, 4),     # capped at 32 key tiles per chunk
    (1, 8, 64, 4096, 4),      # 8 items: chunks of 16 tiles, as 32-tile chunks leave the GPU idle
    (4, 16, 1, 2048, 2),      # 32 key tiles: two 16-tile chunks
    (4, 16, 1, 1984, 1),      # fewer than 32 key tiles: no split
    (32, 16, 1, 16384, 1),    # 512 items: no split
])
def test_automatic_key_split_count(b, h, lq, lk, expect):
    # the automatic choice shows in the workspace size, which holds one partial O and
    # LSE per chunk: it equals the size for the expected explicit count
    a = fwd_args(b=b, s=256, h=h, d=128)
    a.seqlen_q, a.seqlen_k = lq, lk
    st, n_auto = ws_size(a)
    assert st == L.FA_OK
    assert ws_size(a, L.FwdTuning(-1, -1, -1, expect)) == (L.FA_OK, n_auto)
    for other in (expect - 1, expect + 1):
        if 1 <= other <= 64:
            assert ws_size(a, L.FwdTuning(-1, -1, -1, other))[1] != n_auto


def test_causal_with_unequal_lengths_is_accepted():
    # the causal mask aligns the diagonal to the bottom-right corner, so L_q != L_k is valid
    a = fwd_args()
    a.causal, a.seqlen_k = 1, 1000
    assert ws_size(a) == (L.FA_OK, v16_bytes(4, 2 * 1000, 128))
    b = bwd_args()
    b.seqlen_k = 100
    assert bwd_ws(b)[0] == L.FA_OK


@pytest.mark.parametrize("mutate,expect", [
    (lambda a: setattr(a, "dout", None), L.FA_ERR_INVALID_ARGUMENT),
    (lambda a: setattr(a, "dq", P + 4), L.FA_ERR_INVALID_ARGUMENT),
    (lambda a: setattr(a, "deterministic", 3), L.FA_ERR_INVALID_ARGUMENT),
    (lambda a: setattr(a, "grad_dtype", 7), L.FA_ERR_INVALID_ARGUMENT),
    (lambda a: setattr(a, "head_dim", 256), L.FA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "softmax_scale", 0.0), L.FA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "dk_stride", L.Strides(256 * 512, 130, 128)), L.FA_ERR_INVALID_ARGUMENT),
])
def test_backward_validation(mutate, expect):
    a = bwd_args()
    mutate(a)
    assert bwd_ws(a)[0] == expect
    assert L.lib().fa_bwd(ctypes.byref(a), P, 1 << 30, None) == expect


def test_backward_workspace_too_small():
    a = bwd_args()
    st, n = bwd_ws(a)
    assert L.lib().fa_bwd(ctypes.byref(a), P, n - 1, None) == L.FA_ERR_WORKSPACE_TOO_SMALL
    assert L.lib().fa_bwd(ctypes.byref(a), None, 0, None) == L.FA_ERR_WORKSPACE_TOO_SMALL


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(L.FaLibraryMissing):
        L.lib()


def test_exp2_probe_validation():
    lib = L.lib()
    assert lib.fa_exp2_probe(None, None, None, -1, None) == L.FA_ERR_INVALID_ARGUMENT
    assert lib.fa_exp2_probe(None, None, None, 5, None) == L.FA_ERR_INVALID_ARGUMENT
    assert lib.fa_exp2_probe(None, None, None, 0, None) == L.FA_OK  # nothing to do, no device call


def test_noalloc_backward_rejects_before_touching_the_gpu():
    lib = L.lib()
    assert lib.fa_bwd_noalloc_scratch_bytes() == 64 << 20
    assert lib.fa_bwd_noalloc(None, None) == L.FA_ERR_INVALID_ARGUMENT
    bad = bwd_args()
    bad.head_dim = 96
    assert lib.fa_bwd_noalloc(ctypes.byref(bad), None) == L.FA_ERR_UNSUPPORTED
    # deterministic mode: 4 + 2 * head_dim bytes per query row and head, 2 * head_dim per
    # key row and head (row terms and the fp16 copies of Q and K): B=1, S=4096, H=16
    # fits in 64 MiB, B=2, S=8192 does not
    fits = bwd_args(b=1, s=4096, h=16, det=1)
    assert bwd_ws(fits)[1] <= 64 << 20
    big = bwd_args(b=2, s=8192, h=16, det=1)
    st, need = bwd_ws(big)
    assert st == L.FA_OK and need > 64 << 20
    assert lib.fa_bwd_noalloc(ctypes.byref(big), None) == L.FA_ERR_WORKSPACE_TOO_SMALL
    atomic = bwd_args(b=1, s=8192, h=16, det=0)         # + 4 * head_dim per query row and head
    assert bwd_ws(atomic)[1] > 64 << 20
    assert lib.fa_bwd_noalloc(ctypes.byref(atomic), None) == L.FA_ERR_WORKSPACE_TOO_SMALL
