"""The C ABI on the host: exports, status strings, argument checks (no GPU needed).

Every check here is taken on the host before any HIP call, so a bad argument
returns an error code and enqueues nothing. Pointer values used below are
never dereferenced.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

aa = pytest.importorskip("aware_attention_amd")
from aware_attention_amd import _lib  # noqa: E402

INV, UNS, HIP = _lib.FA_ERR_INVALID_ARGUMENT, _lib.FA_ERR_UNSUPPORTED, _lib.FA_ERR_HIP
P = 0x10000          # a 16-byte aligned stand-in pointer; never dereferenced


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def _lib_or_skip():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libfa.so not built")
    return _lib.load()


def test_header_declares_the_abi():
    assert _declared_functions() == sorted(_lib.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = _lib_or_skip()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert lib.fa_abi_version() == 1


def test_status_strings():
    lib = _lib_or_skip()
    for s in range(4):
        assert lib.fa_status_string(s)
    assert lib.fa_status_string(99) == b"unknown status"
    assert lib.fa_last_error() is not None


def _fwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Nq=128, Nk=128, H=2, d=64, scale=0.125,
             causal=0, stream=None)
    a.update(kw)
    return _lib.raw_fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Nq"], a["Nk"],
                           a["H"], a["d"], a["scale"], a["causal"], a["stream"])


def _varlen(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, cu=P, num_seqs=2, max_seqlen=100, total=150, H=2, d=128,
             scale=0.1, causal=0, stream=None)
    a.update(kw)
    return _lib.raw_fa_fwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cu"], a["num_seqs"],
                                  a["max_seqlen"], a["total"], a["H"], a["d"], a["scale"],
                                  a["causal"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INV), (dict(k=None), INV), (dict(v=None), INV), (dict(o=None), INV),
    (dict(lse=None), INV),
    (dict(B=0), INV), (dict(Nq=0), INV), (dict(Nk=-1), INV), (dict(H=0), INV),
    (dict(causal=2), INV), (dict(causal=1, Nq=128, Nk=64), INV),
    (dict(scale=float("nan")), INV), (dict(scale=float("inf")), INV),
    (dict(q=P + 8), INV), (dict(o=P + 2), INV), (dict(lse=P + 4), INV),
    (dict(d=48), UNS), (dict(d=192), UNS), (dict(d=512), UNS),
])
def test_fa_fwd_rejects_bad_arguments(kw, code):
    _lib_or_skip()
    assert _fwd(**kw) == code
    assert _lib.load().fa_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(cu=None), INV), (dict(num_seqs=0), INV), (dict(total=-1), INV),
    (dict(max_seqlen=-1), INV), (dict(max_seqlen=200, total=150), INV),
    (dict(q=None), INV), (dict(v=P + 4), INV), (dict(cu=P + 2), INV),
    (dict(causal=3), INV), (dict(scale=float("nan")), INV), (dict(d=80), UNS),
])
def test_fa_fwd_varlen_rejects_bad_arguments(kw, code):
    _lib_or_skip()
    assert _varlen(**kw) == code


def test_varlen_empty_batch_enqueues_nothing():
    _lib_or_skip()
    assert _varlen(total=0, max_seqlen=0, q=None, k=None, v=None, o=None, lse=None) == _lib.FA_OK
    assert _varlen(max_seqlen=0) == _lib.FA_OK


def test_valid_call_without_a_device_is_a_hip_error():
    _lib_or_skip()
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; this case covers hosts without one")
    assert _fwd(scale=-0.5) == HIP      # any finite scale, negative included
    assert _fwd() == HIP
    assert b"hip" in _lib.load().fa_last_error().lower()


def test_binding_rejects_host_tensors_and_wrong_dtype():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 8, 1, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        aa.fa_fwd(x, x, x)
    with pytest.raises(TypeError):
        aa.fa_fwd(x.float(), x, x)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libfa.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(OSError, match="libfa.so"):
        _lib.load()


def test_product_path_never_touches_the_oracle():
    """The package and the oracle share no code and import nothing from each other."""
    pkg = os.path.join(ROOT, "aware_attention_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b", src, re.M), f
                assert "oracle/" not in src, f
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith(".py"):
            src = open(os.path.join(ROOT, "oracle", f), encoding="utf-8").read()
            assert "aware_attention_amd" not in src and "workloads" not in src, f


def _band(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Nq=128, Nk=96, H=2, d=64, scale=0.125,
             left=16, right=0, stream=None)
    a.update(kw)
    return _lib.raw_fa_fwd_band(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Nq"],
                                a["Nk"], a["H"], a["d"], a["scale"], a["left"], a["right"],
                                a["stream"])


def _varlen_band(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, cu=P, num_seqs=2, max_seqlen=100, total=150, H=2, d=32,
             scale=0.1, left=-1, right=7, stream=None)
    a.update(kw)
    return _lib.raw_fa_fwd_varlen_band(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cu"],
                                       a["num_seqs"], a["max_seqlen"], a["total"], a["H"], a["d"],
                                       a["scale"], a["left"], a["right"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(left=-2), INV), (dict(right=-5), INV), (dict(q=None), INV), (dict(Nk=0), INV),
    (dict(lse=P + 4), INV), (dict(scale=float("nan")), INV), (dict(d=96), UNS),
    (dict(Nq=(1 << 29) + 1), UNS), (dict(Nk=(1 << 29) + 1), UNS),
])
def test_fa_fwd_band_rejects_bad_arguments(kw, code):
    _lib_or_skip()
    assert _band(**kw) == code
    assert _lib.load().fa_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(left=-3), INV), (dict(cu=None), INV), (dict(max_seqlen=200, total=150), INV),
    (dict(d=16), UNS), (dict(max_seqlen=(1 << 29) + 1, total=1 << 30), UNS),
])
def test_fa_fwd_varlen_band_rejects_bad_arguments(kw, code):
    _lib_or_skip()
    assert _varlen_band(**kw) == code


def test_band_valid_call_without_a_device_is_a_hip_error():
    _lib_or_skip()
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; this case covers hosts without one")
    for left, right in [(-1, -1), (-1, 0), (0, 0), (2**31 - 1, 5)]:
        assert _band(left=left, right=right) == HIP
    assert _varlen_band() == HIP


def test_binding_window_arguments():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 8, 1, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        aa._window((None, 0), causal=True)
    with pytest.raises(ValueError):
        aa._window((-1, 0), causal=False)
    assert aa._window((None, None), causal=False) == (-1, -1)
    assert aa._window((3, 10**12), causal=False) == (3, 2**31 - 1)
    with pytest.raises(ValueError):
        aa.fa_fwd(x, x, x, window=(4, 4))   # host tensors are refused before any window use


def _strided(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=2, Nq=100, Nk=80, H=3, d=64,
             qs=(100 * 3 * 64, 3 * 64, 64), ks=(80 * 3 * 64, 3 * 64, 64),
             vs=(80 * 3 * 64, 3 * 64, 64), os=(100 * 3 * 64, 3 * 64, 64),
             dtype=_lib.FA_DTYPE_F16, scale=0.125, causal=0, left=-1, right=-1, stream=None)
    a.update(kw)
    return _lib.raw_fa_fwd_strided(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Nq"],
                                   a["Nk"], a["H"], a["d"], a["qs"], a["ks"], a["vs"], a["os"],
                                   a["dtype"], a["scale"], a["causal"], a["left"], a["right"],
                                   a["stream"])


def _varlen_strided(**kw):
    # packed (total, 3, H, d) QKV: token stride 3*H*d, head stride d
    t = 3 * 2 * 128
    a = dict(q=P, k=P + 256, v=P + 512, o=P, lse=P, cu=P, num_seqs=2, max_seqlen=100, total=150,
             H=2, d=128, qs=(t, 128), ks=(t, 128), vs=(t, 128), os=(2 * 128, 128),
             dtype=_lib.FA_DTYPE_BF16, scale=0.1, causal=1, left=-1, right=-1, stream=None)
    a.update(kw)
    return _lib.raw_fa_fwd_varlen_strided(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cu"],
                                          a["num_seqs"], a["max_seqlen"], a["total"], a["H"],
                                          a["d"], a["qs"], a["ks"], a["vs"], a["os"], a["dtype"],
                                          a["scale"], a["causal"], a["left"], a["right"],
                                          a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(qs=None), INV), (dict(os=None), INV),
    (dict(qs=(0, 3 * 64 + 4, 64)), INV), (dict(ks=(80 * 3 * 64, 3 * 64, 60)), INV),
    (dict(vs=(-8, 3 * 64, 64)), INV), (dict(os=(1, 3 * 64, 64)), INV),
    (dict(ks=(0, (1 << 24) + 8, 64)), UNS),
    (dict(dtype=2), INV), (dict(dtype=-1), INV),
    (dict(causal=1), INV),                             # causal needs Nq == Nk
    (dict(causal=1, Nq=80, left=5), INV),              # causal with a window
    (dict(causal=2), INV), (dict(left=-2), INV),
    (dict(d=16), UNS), (dict(q=P + 8), INV), (dict(B=0), INV),
    (dict(Nq=(1 << 29) + 1, left=3), UNS),
])
def test_fa_fwd_strided_rejects_bad_arguments(kw, code):
    _lib_or_skip()
    assert _strided(**kw) == code
    assert _lib.load().fa_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(qs=None), INV), (dict(ks=(3 * 2 * 128, 129)), INV), (dict(dtype=7), INV),
    (dict(causal=1, right=0), INV), (dict(cu=None), INV), (dict(d=96), UNS),
])
def test_fa_fwd_varlen_strided_rejects_bad_arguments(kw, code):
    _lib_or_skip()
    assert _varlen_strided(**kw) == code


def _packed_bwd_strides(B, S, H, d, varlen=False):
    """Strides of q, k, v (views of a packed (B, S, 3, H, d) tensor), o and dout
    (contiguous) and dq, dk, dv (views of a packed gradient), flattened."""
    t = 3 * H * d
    packed = (S * t, t, d)[1 if varlen else 0:]
    plain = (S * H * d, H * d, d)[1 if varlen else 0:]
    return [x for s_ in (packed, packed, packed, plain, plain, packed, packed, packed) for x in s_]


def _bwd_strided(**kw):
    a = dict(q=P, k=P + 256, v=P + 512, o=P, dout=P, lse=P, dq=P, dk=P, dv=P, delta=P, B=2, Nq=90,
             Nk=90, H=2, d=64, st=_packed_bwd_strides(2, 90, 2, 64), dtype=_lib.FA_DTYPE_BF16,
             scale=0.125, causal=1, left=-1, right=-1, stream=None)
    a.update(kw)
    return _lib.raw_fa_bwd_strided(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"],
                                   a["dk"], a["dv"], a["delta"], a["B"], a["Nq"], a["Nk"], a["H"],
                                   a["d"], a["st"], a["dtype"], a["scale"], a["causal"], a["left"],
                                   a["right"], a["stream"])


def _bwd_varlen_strided(**kw):
    a = dict(q=P, k=P + 256, v=P + 512, o=P, dout=P, lse=P, dq=P, dk=P, dv=P, delta=P, cu=P,
             num_seqs=2, max_seqlen=100, total=150, H=2, d=128,
             st=_packed_bwd_strides(1, 150, 2, 128, varlen=True), dtype=_lib.FA_DTYPE_F16,
             scale=0.1, causal=0, left=-1, right=-1, stream=None)
    a.update(kw)
    return _lib.raw_fa_bwd_varlen_strided(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"],
                                          a["dq"], a["dk"], a["dv"], a["delta"], a["cu"],
                                          a["num_seqs"], a["max_seqlen"], a["total"], a["H"],
                                          a["d"], a["st"], a["dtype"], a["scale"], a["causal"],
                                          a["left"], a["right"], a["stream"])


def _with(st, i, value):
    st = list(st)
    st[i] = value
    return st


_BWD_ST = _packed_bwd_strides(2, 90, 2, 64)


@pytest.mark.parametrize("kw,code", [
    (dict(st=None), INV),
    (dict(st=_with(_BWD_ST, 1, 3 * 2 * 64 + 4)), INV),        # q token stride not a multiple of 8
    (dict(st=_with(_BWD_ST, 14, -8)), INV),                  # dout head stride negative
    (dict(st=_with(_BWD_ST, 21, 1)), INV),                   # dv batch stride odd
    (dict(st=_with(_BWD_ST, 19, (1 << 24) + 8)), UNS),       # dk token stride above 2^24
    (dict(causal=1, left=4), INV),                           # causal with a window
    (dict(causal=0, left=-2), INV), (dict(causal=2), INV),
    (dict(causal=1, Nk=80), INV),                            # causal needs Nq == Nk
    (dict(dtype=3), INV), (dict(d=512), UNS), (dict(d=48), UNS), (dict(B=0), INV),
    (dict(dk=None), INV), (dict(v=P + 4), INV), (dict(scale=float("nan")), INV),
    (dict(causal=0, left=3, Nq=(1 << 29) + 1, Nk=5), UNS),
])
def test_fa_bwd_strided_rejects_bad_arguments(kw, code):
    _lib_or_skip()
    assert _bwd_strided(**kw) == code
    assert _lib.load().fa_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(st=None), INV), (dict(st=_with(_packed_bwd_strides(1, 150, 2, 128, True), 3, 130)), INV),
    (dict(causal=1, right=0), INV), (dict(cu=None), INV), (dict(d=96), UNS), (dict(dtype=9), INV),
    (dict(num_seqs=0), INV),
])
def test_fa_bwd_varlen_strided_rejects_bad_arguments(kw, code):
    _lib_or_skip()
    assert _bwd_varlen_strided(**kw) == code


def test_bwd_strided_valid_calls_without_a_device_are_hip_errors():
    _lib_or_skip()
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; this case covers hosts without one")
    assert _bwd_strided() == HIP                                  # causal
    assert _bwd_strided(causal=0, left=10, right=0) == HIP        # band
    assert _bwd_strided(causal=0, Nq=30, dtype=_lib.FA_DTYPE_F16) == HIP
    assert _bwd_strided(st=[0] * 24) == HIP                       # zero strides are allowed
    assert _bwd_varlen_strided() == HIP
    assert _bwd_varlen_strided(total=0, max_seqlen=0) == _lib.FA_OK


def test_strided_valid_calls_without_a_device_are_hip_errors():
    _lib_or_skip()
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; this case covers hosts without one")
    assert _strided() == HIP                                   # fp16, unmasked
    assert _strided(dtype=_lib.FA_DTYPE_BF16, causal=1, Nq=80) == HIP
    assert _strided(left=0, right=7) == HIP                     # band
    assert _strided(qs=(0, 0, 0)) == HIP                        # zero strides are allowed
    assert _varlen_strided() == HIP
    assert _varlen_strided(total=0, max_seqlen=0) == _lib.FA_OK


def test_binding_accepts_f16_and_views_but_not_bad_ones():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 8, 1, 32, dtype=torch.float16)
    with pytest.raises(ValueError):            # host tensors are refused
        aa.fa_fwd(x, x, x)
    with pytest.raises(TypeError):             # neither bf16 nor fp16 (checked first)
        aa.fa_fwd(x.float(), x.float(), x.float())
    qkv = torch.zeros(2, 5, 3, 4, 32)          # packed (B, S, 3, H, d)
    assert aa._strides(qkv[:, :, 1]) == [5 * 3 * 4 * 32, 3 * 4 * 32, 32]
    assert aa._strides(torch.zeros(1, 5, 1, 32)) == [0, 32, 0]
    assert aa._dtype_code(torch.float16) == _lib.FA_DTYPE_F16
    assert aa._dtype_code(torch.bfloat16) == _lib.FA_DTYPE_BF16


def _bwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, delta=P, B=1, Nq=128, Nk=128, H=2,
             d=64, dtype=_lib.FA_DTYPE_BF16, scale=0.125, causal=0, stream=None)
    a.update(kw)
    return _lib.raw_fa_bwd(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"],
                           a["dv"], a["delta"], a["B"], a["Nq"], a["Nk"], a["H"], a["d"],
                           a["dtype"], a["scale"], a["causal"], a["stream"])


def _bwd_varlen(**kw):
    a = dict(q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, delta=P, cu=P, num_seqs=2,
             max_seqlen=100, total=150, H=2, d=128, dtype=_lib.FA_DTYPE_F16, scale=0.1, causal=1,
             stream=None)
    a.update(kw)
    return _lib.raw_fa_bwd_varlen(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"],
                                  a["dk"], a["dv"], a["delta"], a["cu"], a["num_seqs"],
                                  a["max_seqlen"], a["total"], a["H"], a["d"], a["dtype"],
                                  a["scale"], a["causal"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INV), (dict(do=None), INV), (dict(lse=None), INV), (dict(delta=None), INV),
    (dict(dq=None), INV), (dict(dv=P + 8), INV), (dict(delta=P + 4), INV),
    (dict(B=0), INV), (dict(Nk=0), INV), (dict(H=0), INV), (dict(causal=2), INV),
    (dict(causal=1, Nk=64), INV), (dict(dtype=3), INV), (dict(scale=float("nan")), INV),
    (dict(d=48), UNS),
])
def test_fa_bwd_rejects_bad_arguments(kw, code):
    _lib_or_skip()
    assert _bwd(**kw) == code
    assert _lib.load().fa_last_error()


@pytest.mark.parametrize("kw,code", [
    (dict(cu=None), INV), (dict(num_seqs=0), INV), (dict(max_seqlen=200), INV),
    (dict(dk=None), INV), (dict(dtype=-1), INV), (dict(d=16), UNS),
])
def test_fa_bwd_varlen_rejects_bad_arguments(kw, code):
    _lib_or_skip()
    assert _bwd_varlen(**kw) == code


def test_bwd_valid_calls_without_a_device_are_hip_errors():
    _lib_or_skip()
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; this case covers hosts without one")
    assert _bwd() == HIP
    assert _bwd(causal=1, dtype=_lib.FA_DTYPE_F16) == HIP
    assert _bwd_varlen() == HIP
    assert _bwd_varlen(total=0, max_seqlen=0) == _lib.FA_OK


def _padded(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, mask=P, B=2, S=100, H=2, d=64, dtype=_lib.FA_DTYPE_BF16,
             scale=0.125, causal=0, stream=None)
    a.update(kw)
    return _lib.raw_fa_fwd_padded(a["q"], a["k"], a["v"], a["o"], a["lse"], a["mask"], a["B"],
                                  a["S"], a["H"], a["d"], a["dtype"], a["scale"], a["causal"],
                                  a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(mask=None), INV), (dict(q=None), INV), (dict(causal=2), INV), (dict(dtype=5), INV),
    (dict(S=0), INV), (dict(B=0), INV), (dict(o=P + 2), INV), (dict(d=80), UNS),
])
def test_fa_fwd_padded_rejects_bad_arguments(kw, code):
    _lib_or_skip()
    assert _padded(**kw) == code


def test_padded_valid_call_without_a_device_is_a_hip_error():
    _lib_or_skip()
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; this case covers hosts without one")
    assert _padded() == HIP
    assert _padded(causal=1, dtype=_lib.FA_DTYPE_F16, mask=P + 1) == HIP   # mask bytes unaligned


def test_head_dim_256_checks():
    """d = 256 runs every forward mask (unmasked, causal, varlen, bands,
    padding masks) and the backward's; other head dimensions are refused."""
    _lib_or_skip()
    for d in (16, 96, 192, 512):
        assert _bwd(d=d) == UNS
        assert _bwd_varlen(d=d) == UNS
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        return
    assert _bwd(d=256) == HIP and _bwd(d=256, causal=1, dtype=_lib.FA_DTYPE_F16) == HIP
    assert _bwd_varlen(d=256) == HIP
    assert _bwd_strided(d=256, st=_packed_bwd_strides(2, 90, 2, 256)) == HIP
    assert _fwd(d=256) == HIP and _fwd(d=256, causal=1) == HIP
    assert _varlen(d=256) == HIP
    assert _band(d=256) == HIP
    assert _padded(d=256) == HIP
    assert _varlen_band(d=256) == HIP
    assert _strided(d=256, left=0, right=3, qs=(100 * 3 * 256, 3 * 256, 256),
                    ks=(80 * 3 * 256, 3 * 256, 256), vs=(80 * 3 * 256, 3 * 256, 256),
                    os=(100 * 3 * 256, 3 * 256, 256)) == HIP
    assert _strided(d=256, qs=(100 * 3 * 256, 3 * 256, 256), ks=(80 * 3 * 256, 3 * 256, 256),
                    vs=(80 * 3 * 256, 3 * 256, 256), os=(100 * 3 * 256, 3 * 256, 256)) == HIP


def _decode(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, sl=None, B=2, Nk=1000, H=4, d=128,
             dtype=_lib.FA_DTYPE_BF16, scale=0.088, ws=P, wsb=1 << 30, stream=None)
    a.update(kw)
    return _lib.raw_fa_decode(a["q"], a["k"], a["v"], a["o"], a["lse"], a["sl"], a["B"], a["Nk"],
                              a["H"], a["d"], a["dtype"], a["scale"], a["ws"], a["wsb"],
                              a["stream"])


def test_decode_workspace_plan():
    _lib_or_skip()
    ws = _lib.decode_workspace_bytes
    assert ws(0, 10, 1, 64) == 0 and ws(1, 0, 1, 64) == 0
    assert ws(1, 100, 1, 64) == 1 * 1 * 1 * 65 * 4              # one chunk of 128 keys
    # 1 x 1 head, 8192 keys: chunks of >= 256 keys -> 32 splits
    assert ws(1, 8192, 1, 128) == 32 * 129 * 4
    # 16 x 32 heads = 512 units: 4 splits each reach 2048 workgroups
    assert ws(16, 8192, 32, 128) == 16 * 32 * 4 * 129 * 4
    # a long cache is cut into chunks of at most 4096 keys
    assert ws(64, 100000, 32, 128) == 64 * 32 * 25 * 129 * 4


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INV), (dict(ws=None), INV), (dict(wsb=100), INV), (dict(B=0), INV),
    (dict(Nk=0), INV), (dict(H=0), INV), (dict(dtype=9), INV), (dict(scale=float("inf")), INV),
    (dict(d=48), UNS), (dict(sl=P + 2), INV), (dict(ws=P + 8), INV),
])
def test_fa_decode_rejects_bad_arguments(kw, code):
    _lib_or_skip()
    assert _decode(**kw) == code


def test_decode_valid_call_without_a_device_is_a_hip_error():
    _lib_or_skip()
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; this case covers hosts without one")
    assert _decode() == HIP
    assert _decode(d=256, sl=P, dtype=_lib.FA_DTYPE_F16) == HIP


def test_bwd_band_and_padded_argument_checks():
    _lib_or_skip()
    lib = _lib
    args = [P] * 10
    # window side below -1, bad dtype, d unsupported, null mask, causal out of range
    assert lib.raw_fa_bwd_band(*args, 1, 128, 128, 2, 64, lib.FA_DTYPE_BF16, 0.1, -2, 0, None) == INV
    assert lib.raw_fa_bwd_band(*args, 1, 128, 128, 2, 48, lib.FA_DTYPE_BF16, 0.1, 4, 0, None) == UNS
    assert lib.raw_fa_bwd_band(*args, 1, (1 << 29) + 1, 128, 2, 64, lib.FA_DTYPE_BF16, 0.1, 4, 0,
                               None) == UNS
    assert lib.raw_fa_bwd_varlen_band(*args, None, 2, 100, 150, 2, 64, lib.FA_DTYPE_BF16, 0.1, 3,
                                      3, None) == INV
    assert lib.raw_fa_bwd_padded(*args, None, 2, 100, 2, 64, lib.FA_DTYPE_BF16, 0.1, 0, None) == INV
    assert lib.raw_fa_bwd_padded(*args, P, 2, 100, 2, 64, lib.FA_DTYPE_BF16, 0.1, 2, None) == INV
    assert lib.raw_fa_bwd_padded(*args, P, 2, 100, 2, 64, 7, 0.1, 0, None) == INV
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        assert lib.raw_fa_bwd_band(*args, 1, 128, 96, 2, 64, lib.FA_DTYPE_F16, 0.1, -1, 0, None) == HIP
        assert lib.raw_fa_bwd_varlen_band(*args, P, 2, 100, 150, 2, 32, lib.FA_DTYPE_BF16, 0.1, 8,
                                          8, None) == HIP
        assert lib.raw_fa_bwd_padded(*args, P, 2, 100, 2, 128, lib.FA_DTYPE_BF16, 0.1, 1,
                                     None) == HIP


def test_local_argument_checks():
    _lib_or_skip()
    lib = _lib
    args = [P] * 5
    bf = lib.FA_DTYPE_BF16
    # null pointer, N < 1, causal out of range, bad dtype, negative scale, negative or
    # zero pattern sizes, unsupported d, N above 2^28
    assert lib.raw_fa_fwd_local(None, P, P, P, P, 1, 100, 2, 64, bf, 0.1, 0, 4, 10, 2, 2,
                                None) == INV
    assert lib.raw_fa_fwd_local(*args, 1, 0, 2, 64, bf, 0.1, 0, 4, 10, 2, 2, None) == INV
    assert lib.raw_fa_fwd_local(*args, 1, 100, 2, 64, bf, 0.1, 2, 4, 10, 2, 2, None) == INV
    assert lib.raw_fa_fwd_local(*args, 1, 100, 2, 64, 9, 0.1, 0, 4, 10, 2, 2, None) == INV
    assert lib.raw_fa_fwd_local(*args, 1, 100, 2, 64, bf, 0.1, 0, -1, 10, 2, 2, None) == INV
    assert lib.raw_fa_fwd_local(*args, 1, 100, 2, 64, bf, 0.1, 0, 4, 0, 2, 2, None) == INV
    assert lib.raw_fa_fwd_local(*args, 1, 100, 2, 64, bf, 0.1, 0, 4, 10, -1, 2, None) == INV
    assert lib.raw_fa_fwd_local(*args, 1, 100, 2, 64, bf, 0.1, 0, 4, 10, 2, -3, None) == INV
    assert lib.raw_fa_fwd_local(*args, 1, 100, 2, 48, bf, 0.1, 0, 4, 10, 2, 2, None) == UNS
    assert lib.raw_fa_fwd_local(*args, 1, (1 << 28) + 1, 2, 64, bf, 0.1, 0, 4, 10, 2, 2,
                                None) == UNS
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():   # every check passed: the device lookup fails
        assert lib.raw_fa_fwd_local(*args, 2, 1608, 4, 32, bf, 0.1, 1, 8, 40, 2, 2, None) == HIP
        assert lib.raw_fa_fwd_local(*args, 1, 100, 2, 256, lib.FA_DTYPE_F16, 0.0, 0, 1000, 1, 0,
                                    0, None) == HIP


def test_bwd_local_argument_checks():
    _lib_or_skip()
    lib = _lib
    args = [P] * 10
    bf = lib.FA_DTYPE_BF16
    assert lib.raw_fa_bwd_local(*args, 1, 100, 2, 64, bf, 0.1, 0, -1, 10, 2, 2, None) == INV
    assert lib.raw_fa_bwd_local(*args, 1, 100, 2, 64, bf, 0.1, 0, 4, 0, 2, 2, None) == INV
    assert lib.raw_fa_bwd_local(*args, 1, 100, 2, 64, bf, 0.1, 0, 4, 10, -1, 2, None) == INV
    assert lib.raw_fa_bwd_local(*args, 1, 100, 2, 64, bf, 0.1, 2, 4, 10, 2, 2, None) == INV
    assert lib.raw_fa_bwd_local(*args, 1, 100, 2, 192, bf, 0.1, 0, 4, 10, 2, 2, None) == UNS
    assert lib.raw_fa_bwd_local(*args, 1, (1 << 28) + 1, 2, 64, bf, 0.1, 0, 4, 10, 2, 2,
                                None) == UNS
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        assert lib.raw_fa_bwd_local(*args, 2, 408, 2, 64, bf, 0.1, 1, 8, 20, 2, 2, None) == HIP


# ---------------------------------------------------------------------------
# Outputs and auxiliary tensors on another device than q are refused by the
# binding before any library call (a host pointer must never reach a kernel).
# The host stands in for "q's GPU" here: _on_gpu is patched to accept CPU
# tensors, and "meta" tensors play a tensor on another device.
# ---------------------------------------------------------------------------

@pytest.fixture
def host_as_gpu(monkeypatch):
    torch = pytest.importorskip("torch")
    monkeypatch.setattr(aa, "_on_gpu", lambda t: t.device.type == "cpu")

    def refuse(*a, **k):
        raise AssertionError("a library call was reached")
    for name in dir(aa):
        if name.startswith("raw_fa_"):
            monkeypatch.setattr(aa, name, refuse)
    return torch


def _meta(torch, shape, dtype):
    return torch.empty(shape, dtype=dtype, device="meta")


def test_forward_outputs_on_another_device_are_refused(host_as_gpu):
    torch = host_as_gpu
    bf, f32 = torch.bfloat16, torch.float32
    q = torch.zeros(1, 8, 2, 32, dtype=bf)
    with pytest.raises(ValueError, match="^out must be on"):
        aa.fa_fwd(q, q, q, out=_meta(torch, (1, 8, 2, 32), bf))
    with pytest.raises(ValueError, match="^lse must be on"):
        aa.fa_fwd(q, q, q, lse=_meta(torch, (1, 2, 8), f32))
    with pytest.raises(ValueError, match="^lse must be contiguous"):  # strided lse
        aa.fa_fwd(q, q, q, lse=torch.zeros(1, 8, 2, dtype=f32).transpose(1, 2))
    with pytest.raises(ValueError, match="^k must be on"):
        aa.fa_fwd(q, _meta(torch, (1, 8, 2, 32), bf), q)
    qv = torch.zeros(8, 2, 32, dtype=bf)
    cu = torch.tensor([0, 8], dtype=torch.int32)
    with pytest.raises(ValueError, match="^v must be on"):
        aa.fa_fwd_varlen(qv, qv, _meta(torch, (8, 2, 32), bf), cu, 8)
    with pytest.raises(ValueError, match="^lse must be on"):
        aa.fa_fwd_varlen(qv, qv, qv, cu, 8, lse=_meta(torch, (2, 8), f32))
    with pytest.raises(ValueError, match="^out must be on"):
        aa.fa_fwd_varlen(qv, qv, qv, cu, 8, out=_meta(torch, (8, 2, 32), bf))
    with pytest.raises(ValueError, match="^lse must be on"):
        aa.fa_fwd_local(q, q, q, 2, 3, (1, 1), lse=_meta(torch, (1, 2, 8), f32))
    with pytest.raises(ValueError, match="^out must be on"):
        aa.fa_fwd_local(q, q, q, 2, 3, (1, 1), out=_meta(torch, (1, 8, 2, 32), bf))


@pytest.mark.parametrize("name", ["lse", "delta", "dq", "dk", "dv", "o", "dout"])
def test_backward_tensors_on_another_device_are_refused(host_as_gpu, name):
    torch = host_as_gpu
    bf, f32 = torch.bfloat16, torch.float32
    x = torch.zeros(1, 8, 2, 32, dtype=bf)
    kw = dict(q=x, k=x, v=x, o=x, lse=torch.zeros(1, 2, 8, dtype=f32), dout=x)
    extra = {}
    meta = _meta(torch, (1, 2, 8), f32) if name in ("lse", "delta") else \
        _meta(torch, (1, 8, 2, 32), bf)
    if name in ("lse", "o", "dout"):
        kw[name] = meta
    else:
        extra[name] = meta
    with pytest.raises(ValueError, match=f"^{name} must be on"):
        aa.fa_bwd(kw["q"], kw["k"], kw["v"], kw["o"], kw["lse"], kw["dout"], **extra)
    # the same through the packed entry point
    xv = torch.zeros(8, 2, 32, dtype=bf)
    cu = torch.tensor([0, 8], dtype=torch.int32)
    kw = dict(q=xv, k=xv, v=xv, o=xv, lse=torch.zeros(2, 8, dtype=f32), dout=xv)
    extra = {}
    meta = _meta(torch, (2, 8), f32) if name in ("lse", "delta") else _meta(torch, (8, 2, 32), bf)
    if name in ("lse", "o", "dout"):
        kw[name] = meta
    else:
        extra[name] = meta
    with pytest.raises(ValueError, match=f"^{name} must be on"):
        aa.fa_bwd_varlen(kw["q"], kw["k"], kw["v"], kw["o"], kw["lse"], kw["dout"], cu, 8, **extra)


def test_decode_tensors_on_another_device_or_strided_are_refused(host_as_gpu):
    torch = host_as_gpu
    bf, f32 = torch.bfloat16, torch.float32
    q = torch.zeros(2, 1, 4, 64, dtype=bf)
    kv = torch.zeros(2, 100, 4, 64, dtype=bf)
    with pytest.raises(ValueError, match="^out must be on"):
        aa.fa_decode(q, kv, kv, out=_meta(torch, (2, 1, 4, 64), bf))
    with pytest.raises(ValueError, match="^lse must be on"):
        aa.fa_decode(q, kv, kv, lse=_meta(torch, (2, 4), f32))
    with pytest.raises(ValueError, match="^workspace must be on"):
        aa.fa_decode(q, kv, kv, workspace=_meta(torch, (1 << 20,), torch.uint8))
    with pytest.raises(ValueError, match="^seqlens_k must be on"):
        aa.fa_decode(q, kv, kv, seqlens_k=_meta(torch, (2,), torch.int32))
    with pytest.raises(ValueError, match="^seqlens_k must be contiguous"):  # a strided view
        aa.fa_decode(q, kv, kv, seqlens_k=torch.zeros(4, dtype=torch.int32)[::2])
    with pytest.raises(ValueError, match="^seqlens_k must be torch.int32"):  # wrong dtype
        aa.fa_decode(q, kv, kv, seqlens_k=torch.zeros(2, dtype=torch.int64))


# ---------------------------------------------------------------------------
# fa_decode_noalloc: the decode without a workspace argument (host checks)
# ---------------------------------------------------------------------------

def _decode_noalloc(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, sl=None, B=2, Nk=1000, H=4, d=128,
             dtype=_lib.FA_DTYPE_BF16, scale=0.088, stream=None)
    a.update(kw)
    return _lib.raw_fa_decode_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["sl"], a["B"],
                                      a["Nk"], a["H"], a["d"], a["dtype"], a["scale"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INV), (dict(lse=None), INV), (dict(B=0), INV), (dict(Nk=0), INV),
    (dict(dtype=5), INV), (dict(scale=float("inf")), INV), (dict(o=P + 8), INV),
    (dict(sl=P + 2), INV), (dict(d=48), UNS),
    # partial results above the 8 MiB array: 8192 (batch, head) pairs at d = 256,
    # and one pair over a cache split into 9766 chunks of 4096 keys
    (dict(B=64, H=128, Nk=100, d=256), UNS), (dict(B=1, H=1, Nk=40_000_000, d=256), UNS),
])
def test_fa_decode_noalloc_rejects_bad_arguments(kw, code):
    _lib_or_skip()
    assert _decode_noalloc(**kw) == code


def test_decode_noalloc_limit_matches_the_workspace_plan():
    _lib_or_skip()
    lim = _lib.FA_DECODE_NOALLOC_SCRATCH_BYTES
    assert "FA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)" in open(HEADER).read()
    assert _lib.decode_workspace_bytes(64, 100, 128, 256) > lim
    assert _lib.decode_workspace_bytes(16, 32768, 32, 256) <= lim   # the decode workloads fit


def test_decode_noalloc_valid_call_without_a_device_is_a_hip_error():
    _lib_or_skip()
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; this case covers hosts without one")
    assert _decode_noalloc() == HIP
    assert _decode_noalloc(d=32, sl=P, dtype=_lib.FA_DTYPE_F16) == HIP


def test_backward_gradient_views_on_another_device_are_refused(host_as_gpu):
    """Caller-supplied dq/dk/dv may be strided views, but still only on q's device."""
    torch = host_as_gpu
    B, N, H, d = 1, 16, 2, 64
    packed = torch.zeros(B, N, 3, H, d, dtype=torch.bfloat16)
    q, k, v = packed.unbind(2)
    o, do = torch.zeros(B, N, H, d, dtype=torch.bfloat16), torch.zeros(B, N, H, d, dtype=torch.bfloat16)
    lse = torch.zeros(B, H, N)
    meta = _meta(torch, (B, N, 3, H, d), torch.bfloat16)
    for i, name in enumerate(("dq", "dk", "dv")):
        kw = {name: meta.unbind(2)[i]}
        with pytest.raises(ValueError, match=f"^{name} must be on"):
            aa.fa_bwd(q, k, v, o, lse, do, **kw)
    with pytest.raises(TypeError, match="^dk must be"):
        aa.fa_bwd(q, k, v, o, lse, do, dk=torch.zeros(B, N, H, d, dtype=torch.float16))


def test_attention_qkvpacked_argument_checks():
    torch = pytest.importorskip("torch")
    x4 = torch.zeros(10, 3, 2, 64, dtype=torch.bfloat16)
    x5 = torch.zeros(1, 10, 3, 2, 64, dtype=torch.bfloat16)
    cu = torch.tensor([0, 10], dtype=torch.int32)
    with pytest.raises(ValueError, match="qkv must be a"):
        aa.attention_qkvpacked(x4)                                  # varlen layout without cu_seqlens
    with pytest.raises(ValueError, match="qkv must be a"):
        aa.attention_qkvpacked(x5, cu_seqlens=cu, max_seqlen=10)    # dense layout with cu_seqlens
    with pytest.raises(ValueError, match="qkv must be a"):
        aa.attention_qkvpacked(torch.zeros(1, 10, 4, 2, 64))        # not three tensors
    with pytest.raises(ValueError, match="max_seqlen"):
        aa.attention_qkvpacked(x4, cu_seqlens=cu)


def test_kernel_view_keeps_readable_views_and_copies_the_rest():
    """Views the strided entry points read in place are passed as they are; others are copied."""
    torch = pytest.importorskip("torch")
    packed = torch.zeros(2, 33, 3, 4, 64, dtype=torch.bfloat16)
    q = packed.unbind(2)[0]                                         # token stride 3*4*64, head stride 64
    assert aa._kernel_view(q).data_ptr() == q.data_ptr()
    assert aa._kernel_view(packed, token_dim=-4).data_ptr() == packed.data_ptr()
    bhsd = torch.zeros(2, 4, 33, 64, dtype=torch.bfloat16).permute(0, 2, 1, 3)
    assert aa._kernel_view(bhsd).data_ptr() == bhsd.data_ptr()      # head stride 33*64
    ones = torch.ones(64, dtype=torch.bfloat16).expand(2, 33, 4, 64)
    assert aa._kernel_view(ones).data_ptr() == ones.data_ptr()      # zero strides are readable
    col = torch.zeros(2, 33, 4, 64, dtype=torch.bfloat16).transpose(-1, -2).contiguous().transpose(-1, -2)
    out = aa._kernel_view(col)                                      # d not contiguous
    assert out.is_contiguous() and out.data_ptr() != col.data_ptr()
    odd = torch.zeros(2, 33, 4, 68, dtype=torch.bfloat16)[..., :64]  # token stride 272, head 68
    out = aa._kernel_view(odd)                                      # 68 is not a multiple of 8
    assert out.is_contiguous() and out.data_ptr() != odd.data_ptr()
