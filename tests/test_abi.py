"""The C ABI without a GPU: libfa.so loads, exports every function that
include/fa.h declares, and rejects bad arguments on the host (before any
HIP call) with the documented codes. No compute call is made here: every
call below is one the library must refuse."""
import ctypes
import os
import re

import pytest

import exact_attention_28_amd as fa
from exact_attention_28_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

# fake, aligned, never-dereferenced device addresses
P = 0x7F0000000000


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_\w+)\s*\(", src)))


def _codes():
    src = open(HEADER).read()
    return {m[0]: int(m[1]) for m in
            re.findall(r"#define\s+(FA_\w+)\s+\(?(-?\d+)\)?", src)}


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("libfa.so not built")
    return fa.load_library()


def test_exports_every_declared_function(lib):
    declared = _declared()
    assert declared == sorted(L.EXPORTS)
    so = ctypes.CDLL(L.LIB_PATH)
    for name in declared:
        assert hasattr(so, name), name


def test_python_constants_match_header():
    codes = _codes()
    for name, val in codes.items():
        assert getattr(L, name) == val, name


def test_strerror(lib):
    for name, val in _codes().items():
        if name.startswith("FA_E") or name == "FA_OK":
            msg = fa.fa_strerror(val)
            assert msg and msg != "unknown error code", name
    assert "HIP" in fa.fa_strerror(1)
    assert fa.fa_strerror(-999) == "unknown error code"


def fwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=4, Hkv=2, Nq=8, Nk=8, d=128,
             scale=0.1, causal=0, dtype=L.FA_DTYPE_BF16, qkv_descale=None,
             stream=None)
    a.update(kw)
    return fa.fa_fwd(**a, check=False)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), L.FA_EINVAL_NULL),
    (dict(k=None), L.FA_EINVAL_NULL),
    (dict(v=None), L.FA_EINVAL_NULL),
    (dict(o=None), L.FA_EINVAL_NULL),
    (dict(B=0), L.FA_EINVAL_DIM),
    (dict(Hq=-1), L.FA_EINVAL_DIM),
    (dict(Nq=0), L.FA_EINVAL_DIM),
    (dict(Nk=0), L.FA_EINVAL_DIM),
    (dict(d=96), L.FA_EUNSUPPORTED_D),
    (dict(d=256), L.FA_EUNSUPPORTED_D),
    (dict(Hq=6, Hkv=4), L.FA_EGQA),
    (dict(dtype=3), L.FA_EDTYPE),
    (dict(dtype=L.FA_DTYPE_FP8_E4M3), L.FA_EDESCALE),
    (dict(dtype=L.FA_DTYPE_FP8_E4M3, qkv_descale=(1.0, 0.0, 1.0)), L.FA_EDESCALE),
    (dict(dtype=L.FA_DTYPE_FP8_E4M3, qkv_descale=(1.0, float("nan"), 1.0)), L.FA_EDESCALE),
    (dict(qkv_descale=(1.0, 1.0, 1.0)), L.FA_EDESCALE),
    (dict(scale=0.0), L.FA_ESCALE),
    (dict(scale=-1.0), L.FA_ESCALE),
    (dict(scale=float("inf")), L.FA_ESCALE),
    (dict(scale=float("nan")), L.FA_ESCALE),
    (dict(q=P + 8), L.FA_EALIGN),
    (dict(o=P + 2), L.FA_EALIGN),
    (dict(lse=P + 2), L.FA_EALIGN),
    (dict(Nq=1 << 25), L.FA_EINVAL_DIM),          # Nq*d beyond 32-bit offsets
    (dict(B=1 << 20, Hq=1 << 10, Hkv=1 << 10, Nq=1 << 14), L.FA_EINVAL_DIM),
])
def test_fwd_rejects(lib, kw, code):
    assert fwd(**kw) == code


def test_fwd_raises_with_message(lib):
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd(P, P, P, P, P, 1, 1, 1, 1, 1, 100, 0.1, 0, 1)
    assert e.value.code == L.FA_EUNSUPPORTED_D
    assert "64 or 128" in str(e.value)


def bwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, dout=P, lse=P, dq=P, dk=P, dv=P, B=1, Hq=4,
             Hkv=2, Nq=8, Nk=8, d=128, scale=0.1, causal=0,
             dtype=L.FA_DTYPE_BF16, workspace=P, workspace_bytes=1 << 30,
             stream=None)
    a.update(kw)
    return fa.fa_bwd(**a, check=False)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), L.FA_EINVAL_NULL),
    (dict(dout=None), L.FA_EINVAL_NULL),
    (dict(lse=None), L.FA_EINVAL_NULL),
    (dict(dq=None), L.FA_EINVAL_NULL),
    (dict(dv=None), L.FA_EINVAL_NULL),
    (dict(B=0), L.FA_EINVAL_DIM),
    (dict(Nk=0), L.FA_EINVAL_DIM),
    (dict(d=32), L.FA_EUNSUPPORTED_D),
    (dict(Hq=6, Hkv=4), L.FA_EGQA),
    (dict(dtype=L.FA_DTYPE_F32), L.FA_EDTYPE),
    (dict(dtype=L.FA_DTYPE_FP8_E4M3), L.FA_EDTYPE),
    (dict(scale=float("nan")), L.FA_ESCALE),
    (dict(dk=P + 8), L.FA_EALIGN),
    (dict(lse=P + 1), L.FA_EALIGN),
    (dict(workspace=None), L.FA_EWORKSPACE),
    (dict(workspace_bytes=64), L.FA_EWORKSPACE),
    (dict(workspace=P + 64), L.FA_EWORKSPACE),
    (dict(Nq=1 << 25), L.FA_EINVAL_DIM),
])
def test_bwd_rejects(lib, kw, code):
    assert bwd(**kw) == code


def test_bwd_workspace_size(lib):
    # two fp32 arrays of B*Hq*Nq rows, each with at least 32 rows of padding,
    # rounded up to 64 rows (the documented layout)
    up = lambda x: -(-(x + 32) // 64) * 64
    assert fa.fa_bwd_workspace_size(1, 1, 1) == 8 * up(1)
    assert fa.fa_bwd_workspace_size(2, 16, 2048) == 8 * up(2 * 16 * 2048)
    assert fa.fa_bwd_workspace_size(1, 32, 16384) == 8 * up(32 * 16384)
    assert fa.fa_bwd_workspace_size(0, 1, 1) == 0
    assert fa.fa_bwd_workspace_size(1, 1, -5) == 0


def dec(**kw):
    a = dict(q=P, k_pool=P, v_pool=P, block_table=P, seq_lens=P, page_size=16,
             num_pages=100, B=4, Hq=32, Hkv=8, d=128, max_pages_per_seq=512,
             scale=0.1, o=P, lse=P, workspace=P, workspace_bytes=1 << 40,
             num_splits=0, stream=None)
    a.update(kw)
    return fa.fa_paged_decode(**a, check=False)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), L.FA_EINVAL_NULL),
    (dict(block_table=None), L.FA_EINVAL_NULL),
    (dict(seq_lens=None), L.FA_EINVAL_NULL),
    (dict(o=None), L.FA_EINVAL_NULL),
    (dict(B=0), L.FA_EINVAL_DIM),
    (dict(max_pages_per_seq=0), L.FA_EINVAL_DIM),
    (dict(d=80), L.FA_EUNSUPPORTED_D),
    (dict(Hq=12, Hkv=8), L.FA_EGQA),
    (dict(Hq=64, Hkv=2), L.FA_EGQA),                 # group of 32 > 16
    (dict(page_size=32), L.FA_EPAGE),
    (dict(num_pages=0), L.FA_EPAGE),
    (dict(num_splits=-1), L.FA_ESPLITS),
    (dict(num_splits=65537), L.FA_ESPLITS),          # above the range cap
    (dict(B=1 << 22, Hq=8, Hkv=8), L.FA_EINVAL_DIM),  # B * max_pages > 2^31 - 1
    (dict(scale=0.0), L.FA_ESCALE),
    (dict(workspace=None), L.FA_EWORKSPACE),
    (dict(workspace_bytes=16), L.FA_EWORKSPACE),
    (dict(workspace=P + 16), L.FA_EWORKSPACE),       # not 256-byte aligned
    (dict(k_pool=P + 4), L.FA_EALIGN),
    (dict(seq_lens=P + 2), L.FA_EALIGN),
])
def test_decode_rejects(lib, kw, code):
    assert dec(**kw) == code


def _ws_bytes(B, Hq, Hkv, d, R):
    """Workspace of the decode plan, from its documented layout: 64 header
    words and two per-request ints, rounded up to 64 words; then the partial
    outputs (B + R) * Hq * d fp32 and their (B + R) * Hq log-sum-exps. R is
    rounded up to a multiple of the waves per KV head."""
    G = Hq // Hkv
    nw = 8 if (Hkv % 8 == 0 and G <= 8) else 4
    hh = max((c for c in range(1, nw + 1) if Hkv % c == 0),
             key=lambda c: (c * (nw // c), c))
    wph = nw // hh
    R = -(-R // wph) * wph
    off_o = -(-(64 + 2 * B) // 64) * 64
    return 4 * (off_o + (B + R) * Hq * d + (B + R) * Hq)


def test_workspace_size(lib):
    ws = fa.fa_paged_decode_workspace_size
    # explicit range counts (one KV head: four ranges per workgroup)
    assert ws(2, 4, 1, 64, 10, 16, 1) == _ws_bytes(2, 4, 1, 64, 1)
    assert ws(2, 4, 1, 64, 10, 16, 3) == _ws_bytes(2, 4, 1, 64, 4)
    assert ws(2, 4, 1, 64, 10, 16, 8) == _ws_bytes(2, 4, 1, 64, 8)
    assert ws(64, 32, 8, 128, 512, 16, 512) == _ws_bytes(64, 32, 8, 128, 512)
    assert ws(3, 6, 2, 128, 7, 16, 5) == _ws_bytes(3, 6, 2, 128, 6)
    # auto: some positive size, at least that of one range
    assert ws(64, 32, 8, 128, 512, 16, 0) >= _ws_bytes(64, 32, 8, 128, 1)
    # rejected arguments report 0
    assert ws(0, 4, 1, 64, 10, 16, 0) == 0
    assert ws(1, 4, 1, 64, 10, 8, 0) == 0
    assert ws(1, 4, 1, 64, 10, 16, 70000) == 0        # above the range cap


def dec8(**kw):
    a = dict(q=P, k_pool=P, v_pool=P, block_table=P, seq_lens=P, page_size=16,
             num_pages=100, B=4, Hq=32, Hkv=8, d=128, max_pages_per_seq=512,
             scale=0.1, kv_descale=(0.01, 0.02), o=P, lse=P, workspace=P,
             workspace_bytes=1 << 40, num_splits=0, stream=None)
    a.update(kw)
    return fa.fa_paged_decode_fp8kv(**a, check=False)


@pytest.mark.parametrize("kw,code", [
    (dict(kv_descale=None), L.FA_EDESCALE),
    (dict(kv_descale=(0.0, 1.0)), L.FA_EDESCALE),
    (dict(kv_descale=(1.0, -2.0)), L.FA_EDESCALE),
    (dict(kv_descale=(float("inf"), 1.0)), L.FA_EDESCALE),
    (dict(q=None), L.FA_EINVAL_NULL),
    (dict(d=96), L.FA_EUNSUPPORTED_D),
    (dict(page_size=8), L.FA_EPAGE),
    (dict(workspace_bytes=8), L.FA_EWORKSPACE),
    (dict(v_pool=P + 8), L.FA_EALIGN),
])
def test_decode_fp8kv_rejects(lib, kw, code):
    assert dec8(**kw) == code


def naive(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, Hq=4, Hkv=2, Nq=8, Nk=64, d=128,
             scale=0.1, causal=0, workspace=P, workspace_bytes=1 << 30,
             stream=None)
    a.update(kw)
    return fa.fa_naive_attention(**a, check=False)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), L.FA_EINVAL_NULL),
    (dict(Nq=0), L.FA_EINVAL_DIM),
    (dict(Nk=60), L.FA_EINVAL_DIM),          # not a multiple of 8
    (dict(Nk=16392), L.FA_EINVAL_DIM),       # above 16384
    (dict(d=80), L.FA_EUNSUPPORTED_D),
    (dict(Hq=3, Hkv=2), L.FA_EGQA),
    (dict(scale=-1.0), L.FA_ESCALE),
    (dict(o=P + 4), L.FA_EALIGN),
    (dict(workspace=None), L.FA_EWORKSPACE),
    (dict(workspace_bytes=100), L.FA_EWORKSPACE),
])
def test_naive_rejects(lib, kw, code):
    assert naive(**kw) == code


def test_naive_workspace_size(lib):
    assert fa.fa_naive_workspace_size(2, 3, 5, 64) == 2 * 3 * 5 * 64 * 2
    assert fa.fa_naive_workspace_size(1, 1, 0, 8) == 0


def ppf(**kw):
    a = dict(q=P, k_pool=P, v_pool=P, block_table=P, seq_lens=P, page_size=16,
             num_pages=100, B=2, Hq=8, Hkv=2, Nq=64, d=128,
             max_pages_per_seq=64, scale=0.1, causal=1, o=P, lse=P,
             stream=None)
    a.update(kw)
    return fa.fa_paged_prefill(**a, check=False)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), L.FA_EINVAL_NULL),
    (dict(seq_lens=None), L.FA_EINVAL_NULL),
    (dict(Nq=0), L.FA_EINVAL_DIM),
    (dict(max_pages_per_seq=8193), L.FA_EINVAL_DIM),   # page table cap
    (dict(d=32), L.FA_EUNSUPPORTED_D),
    (dict(Hq=6, Hkv=4), L.FA_EGQA),
    (dict(page_size=32), L.FA_EPAGE),
    (dict(num_pages=0), L.FA_EPAGE),
    (dict(scale=0.0), L.FA_ESCALE),
    (dict(o=P + 2), L.FA_EALIGN),
    (dict(block_table=P + 1), L.FA_EALIGN),
])
def test_paged_prefill_rejects(lib, kw, code):
    assert ppf(**kw) == code


def dec_na(**kw):
    a = dict(q=P, k_pool=P, v_pool=P, block_table=P, seq_lens=P, page_size=16,
             num_pages=100, B=4, Hq=32, Hkv=8, d=128, max_pages_per_seq=512,
             scale=0.1, o=P, lse=P, num_splits=0, stream=None)
    a.update(kw)
    return fa.fa_paged_decode_noalloc(**a, check=False)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), L.FA_EINVAL_NULL),
    (dict(o=None), L.FA_EINVAL_NULL),
    (dict(B=0), L.FA_EINVAL_DIM),
    (dict(d=96), L.FA_EUNSUPPORTED_D),
    (dict(Hq=12, Hkv=8), L.FA_EGQA),
    (dict(page_size=8), L.FA_EPAGE),
    (dict(num_splits=-1), L.FA_ESPLITS),
    (dict(scale=float("nan")), L.FA_ESCALE),
    (dict(k_pool=P + 4), L.FA_EALIGN),
    # an explicit range count whose partials exceed the 16 MiB built-in
    # workspace: (4 + 4096) * 32 * 129 * 4 bytes
    (dict(num_splits=4096), L.FA_ESCRATCH),
    # so many requests that even one range per KV head does not fit
    (dict(B=2000, max_pages_per_seq=64), L.FA_ESCRATCH),
])
def test_decode_noalloc_rejects(lib, kw, code):
    assert dec_na(**kw) == code


# The prototypes of include/fa.h, parameter by parameter. The first
# parameters of fa_fwd and fa_paged_decode are the boundary's fixed prefixes
# fa_fwd(q,k,v,o,lse,B,Hq,Hkv,Nq,Nk,d,scale,causal) and
# fa_paged_decode(q,k_pool,v_pool,block_table,seq_lens,page_size,...);
# what follows them (and the decode workspace query's Hkv) are the
# library's own choices.
PROTOTYPES = {
    "fa_fwd": ("int", [
        "const void* q", "const void* k", "const void* v", "void* o",
        "float* lse", "int B", "int Hq", "int Hkv", "int Nq", "int Nk",
        "int d", "float scale", "int causal", "int dtype",
        "const float* qkv_descale", "void* stream"]),
    "fa_bwd_workspace_size": ("size_t", ["int B", "int Hq", "int Nq"]),
    "fa_bwd": ("int", [
        "const void* q", "const void* k", "const void* v", "const void* o",
        "const void* dout", "const float* lse", "void* dq", "void* dk",
        "void* dv", "int B", "int Hq", "int Hkv", "int Nq", "int Nk", "int d",
        "float scale", "int causal", "int dtype", "void* workspace",
        "size_t workspace_bytes", "void* stream"]),
    "fa_paged_decode_workspace_size": ("size_t", [
        "int B", "int Hq", "int Hkv", "int d", "int max_pages_per_seq",
        "int page_size", "int num_splits"]),
    "fa_paged_decode": ("int", [
        "const void* q", "const void* k_pool", "const void* v_pool",
        "const int32_t* block_table", "const int32_t* seq_lens",
        "int page_size", "int num_pages", "int B", "int Hq", "int Hkv",
        "int d", "int max_pages_per_seq", "float scale", "void* o",
        "float* lse", "void* workspace", "size_t workspace_bytes",
        "int num_splits", "void* stream"]),
    "fa_paged_decode_noalloc": ("int", [
        "const void* q", "const void* k_pool", "const void* v_pool",
        "const int32_t* block_table", "const int32_t* seq_lens",
        "int page_size", "int num_pages", "int B", "int Hq", "int Hkv",
        "int d", "int max_pages_per_seq", "float scale", "void* o",
        "float* lse", "int num_splits", "void* stream"]),
    "fa_paged_decode_fp8kv": ("int", [
        "const void* q", "const void* k_pool", "const void* v_pool",
        "const int32_t* block_table", "const int32_t* seq_lens",
        "int page_size", "int num_pages", "int B", "int Hq", "int Hkv",
        "int d", "int max_pages_per_seq", "float scale",
        "const float* kv_descale", "void* o", "float* lse", "void* workspace",
        "size_t workspace_bytes", "int num_splits", "void* stream"]),
    "fa_paged_prefill": ("int", [
        "const void* q", "const void* k_pool", "const void* v_pool",
        "const int32_t* block_table", "const int32_t* seq_lens",
        "int page_size", "int num_pages", "int B", "int Hq", "int Hkv",
        "int Nq", "int d", "int max_pages_per_seq", "float scale",
        "int causal", "void* o", "float* lse", "void* stream"]),
    "fa_naive_workspace_size": ("size_t", [
        "int B", "int Hq", "int Nq", "int Nk"]),
    "fa_naive_attention": ("int", [
        "const void* q", "const void* k", "const void* v", "void* o",
        "float* lse", "int B", "int Hq", "int Hkv", "int Nq", "int Nk",
        "int d", "float scale", "int causal", "void* workspace",
        "size_t workspace_bytes", "void* stream"]),
    "fa_strerror": ("const char*", ["int code"]),
}


def _header_prototypes():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    out = {}
    for ret, name, params in re.findall(
            r"(const char\s*\*|size_t|int)\s+(fa_\w+)\s*\(([^;]*?)\)\s*;",
            src, flags=re.S):
        plist = [re.sub(r"\s+", " ", p.strip()).replace(" *", "*")
                 for p in params.split(",")]
        out[name] = (re.sub(r"\s+", "", ret).replace("char*", "char*")
                     .replace("constchar*", "const char*"), plist)
    return out


def test_header_prototypes():
    got = _header_prototypes()
    assert sorted(got) == sorted(PROTOTYPES)
    for name, (ret, params) in PROTOTYPES.items():
        assert got[name] == (ret, params), name
    # the fixed prefixes of the boundary
    assert [p.split()[-1] for p in got["fa_fwd"][1][:13]] == [
        "q", "k", "v", "o", "lse", "B", "Hq", "Hkv", "Nq", "Nk", "d", "scale",
        "causal"]
    assert [p.split()[-1] for p in got["fa_paged_decode"][1][:6]] == [
        "q", "k_pool", "v_pool", "block_table", "seq_lens", "page_size"]


def test_binding_argument_counts(lib):
    for name, (_, params) in PROTOTYPES.items():
        assert len(getattr(lib, name).argtypes) == len(params), name
