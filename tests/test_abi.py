"""The C ABI of libfa2.so on the CPU: it loads, exports every declared entry
point, and rejects bad arguments with the documented status codes before any
HIP call (so no GPU is needed).  Nothing here launches a kernel."""
import os
import re

import pytest

import tiled_attention_fwd_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa2.h")

A = 0x10000  # a fake, 16-byte aligned, never dereferenced address
MIS = 0x10008  # a fake misaligned address


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa2_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fa.LIB_PATH):
        from tiled_attention_fwd_amd import build
        build.build()
    return fa.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert names == ["fa2_backward", "fa2_backward_ex", "fa2_backward_noalloc", "fa2_backward_stage",
                     "fa2_backward_stage_ex",
                     "fa2_backward_stage_varlen", "fa2_backward_varlen", "fa2_backward_workspace_size",
                     "fa2_backward_workspace_size_ex", "fa2_backward_workspace_size_varlen", "fa2_decode",
                     "fa2_decode_workspace_size", "fa2_forward", "fa2_forward_ex", "fa2_forward_varlen",
                     "fa2_status_string"]
    for n in names:
        assert hasattr(L, n), n


def fwd(L, q=A, k=A, v=A, o=A, lse=A, B=1, H=2, N=64, d=64, scale=0.125, causal=1, dtype=1):
    return L.fa2_forward(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, None)


def bwd(L, ptr=A, B=1, H=2, N=64, d=64, scale=0.125, causal=1, dtype=1, ws=A, wsb=None, **over):
    p = dict(q=ptr, k=ptr, v=ptr, o=ptr, dO=ptr, lse=ptr, dq=ptr, dk=ptr, dv=ptr)
    p.update(over)
    if wsb is None:
        wsb = L.fa2_backward_workspace_size(B, H, N, d, dtype)
    return L.fa2_backward(p["q"], p["k"], p["v"], p["o"], p["dO"], p["lse"], p["dq"], p["dk"], p["dv"],
                          B, H, N, d, scale, causal, dtype, ws, wsb, None)


@pytest.mark.parametrize("arg", ["q", "k", "v", "o", "lse"])
def test_forward_null_pointer(L, arg):
    assert fwd(L, **{arg: None}) == fa.FA2_ERR_INVALID_ARG


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), fa.FA2_ERR_INVALID_ARG), (dict(H=-2), fa.FA2_ERR_INVALID_ARG),
    (dict(N=-3), fa.FA2_ERR_INVALID_ARG), (dict(d=0), fa.FA2_ERR_INVALID_ARG),
    (dict(d=48), fa.FA2_ERR_UNSUPPORTED), (dict(d=256), fa.FA2_ERR_UNSUPPORTED),
    (dict(dtype=3), fa.FA2_ERR_INVALID_ARG), (dict(dtype=-1), fa.FA2_ERR_INVALID_ARG),
    (dict(scale=0.0), fa.FA2_ERR_INVALID_ARG), (dict(scale=-0.0), fa.FA2_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA2_ERR_INVALID_ARG), (dict(scale=float("inf")), fa.FA2_ERR_INVALID_ARG),
    (dict(q=MIS), fa.FA2_ERR_UNSUPPORTED), (dict(lse=MIS), fa.FA2_ERR_UNSUPPORTED),
    (dict(N=1 << 24, d=128), fa.FA2_ERR_INVALID_ARG),
])
def test_forward_rejects(L, kw, status):
    assert fwd(L, **kw) == status


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(N=0)])
def test_empty_problem_is_noop(L, kw):
    # null data pointers are fine for an empty problem: nothing is launched
    assert fwd(L, q=None, k=None, v=None, o=None, lse=None, **kw) == fa.FA2_OK
    assert bwd(L, ptr=None, ws=None, wsb=0, **kw) == fa.FA2_OK


@pytest.mark.parametrize("arg", ["q", "k", "v", "o", "dO", "lse", "dq", "dk", "dv"])
def test_backward_null_and_misaligned(L, arg):
    assert bwd(L, **{arg: None}) == fa.FA2_ERR_INVALID_ARG
    assert bwd(L, **{arg: MIS}) == fa.FA2_ERR_UNSUPPORTED


@pytest.mark.parametrize("dtype", [0, 1])
def test_backward_workspace_checks(L, dtype):
    need = L.fa2_backward_workspace_size(1, 2, 64, 64, dtype)
    assert need > 0
    assert bwd(L, dtype=dtype, ws=None, wsb=need) == fa.FA2_ERR_WORKSPACE
    assert bwd(L, dtype=dtype, wsb=need - 1) == fa.FA2_ERR_WORKSPACE
    assert bwd(L, dtype=dtype, ws=MIS, wsb=need) == fa.FA2_ERR_UNSUPPORTED


def test_workspace_size_formula(L):
    def al(x):
        return (x + 255) // 256 * 256
    B, H, N, d = 4, 16, 4096, 128
    rows = B * H * N
    assert L.fa2_backward_workspace_size(B, H, N, d, 1) == 2 * al(rows * 4)
    assert L.fa2_backward_workspace_size(B, H, N, d, 0) == 2 * al(rows * 4)
    assert L.fa2_backward_workspace_size(B, H, N, d, 2) == 2 * al(rows * 4)
    assert L.fa2_backward_workspace_size(0, H, N, d, 1) == 0
    assert L.fa2_backward_workspace_size(B, H, N, 40, 1) == 0
    assert L.fa2_backward_workspace_size(-1, H, N, d, 1) == 0


def test_workspace_size_ex_formula(L):
    """Grouped-query sizes: the plain size, plus fp32 partial dK and dV when a
    bf16 d=128 group is split over S workgroups (S the smallest divisor of G
    giving 1024 key-tile workgroups, else G), or an fp32 key tile's walk over
    the query tiles is cut into S pieces."""
    def al(x):
        return (x + 255) // 256 * 256
    B, H, N, d = 4, 16, 4096, 128
    plain = 2 * al(B * H * N * 4)
    assert L.fa2_backward_workspace_size_ex(B, H, H, N, d, 1) == L.fa2_backward_workspace_size(B, H, N, d, 1)
    # 32 key tiles x 4 x 2 = 256 workgroups -> S = 4 of G = 8
    assert L.fa2_backward_workspace_size_ex(B, H, 2, N, d, 1) == plain + 2 * al(4 * B * 2 * N * d * 4)
    # 32 x 4 x 1 = 128 -> S = 8 of G = 16
    assert L.fa2_backward_workspace_size_ex(B, H, 1, N, d, 1) == plain + 2 * al(8 * B * 1 * N * d * 4)
    # tiny problem: S = G
    assert L.fa2_backward_workspace_size_ex(1, 8, 1, 64, 128, 1) == 2 * al(8 * 64 * 4) + 2 * al(8 * 64 * 128 * 4)
    # G = 6 with 1 key tile: S runs 2, 3, 6
    assert L.fa2_backward_workspace_size_ex(1, 6, 1, 64, 128, 1) == 2 * al(6 * 64 * 4) + 2 * al(6 * 64 * 128 * 4)
    # enough workgroups already (16 x 8 x 8 = 1024) or another head size: no partials
    assert L.fa2_backward_workspace_size_ex(8, 16, 8, 2048, d, 1) == 2 * al(8 * 16 * 2048 * 4)
    # fp32 splits query tiles instead, to 512 workgroups while the longest walk
    # keeps 4 query tiles (32 rows at d >= 64, 64 below) per piece:
    # 32 key tiles x 4 x 2 = 256 -> S = 2
    assert L.fa2_backward_workspace_size_ex(B, H, 2, N, d, 0) == plain + 2 * al(2 * B * 2 * N * d * 4)
    # fp32 at d <= 64 with fewer than 512 unsplit workgroups and N >= 256
    # first pairs the walks inside each workgroup (64 keys or 64 query rows
    # per workgroup, no partial sums), then splits what is left while every
    # wave keeps 4 query steps (dK/dV) or 8 key tiles (dQ) per piece.
    # The 8x8x512x64 shape: 8 key tiles x 64 = 512 paired workgroups, no split
    assert L.fa2_backward_workspace_size(8, 8, 512, 64, 0) == 2 * al(64 * 512 * 4)
    # 4x4x256x32: paired, walks of 4 query steps / 8 key tiles: no split
    assert L.fa2_backward_workspace_size(4, 4, 256, 32, 0) == 2 * al(16 * 256 * 4)
    # 2048 workgroups already: no split
    assert L.fa2_backward_workspace_size_ex(8, 16, 16, 2048, d, 0) == 2 * al(8 * 16 * 2048 * 4)
    # 1x2x2048x64, paired: 32 x 2 = 64 workgroups each side; dK/dV walks of
    # 64 query steps -> S = 8 (512 workgroups, 64 / 8 >= 8), dQ walks of 64
    # key tiles -> S = 4 (64 / 4 >= 16); the larger of the two partial sets
    # sizes the area
    assert L.fa2_backward_workspace_size(1, 2, 2048, 64, 0) == \
        2 * al(2 * 2048 * 4) + max(2 * al(8 * 2 * 2048 * 64 * 4), al(4 * 2 * 2048 * 64 * 4))
    # the unpaired rule still holds at d = 128 and below N = 256: 1x2x2048x128
    # dK/dV 16 query tiles x 2 = 32 -> S = 16, dQ S = 7
    assert L.fa2_backward_workspace_size(1, 2, 2048, 128, 0) == \
        2 * al(2 * 2048 * 4) + max(2 * al(16 * 2 * 2048 * 128 * 4), al(7 * 2 * 2048 * 128 * 4))
    assert L.fa2_backward_workspace_size_ex(B, H, 2, N, d, 2) == plain + 2 * al(4 * B * 2 * N * d * 4)
    assert L.fa2_backward_workspace_size_ex(B, H, 2, N, 64, 1) == plain
    assert L.fa2_backward_workspace_size_ex(B, H, 3, N, d, 1) == 0
    assert L.fa2_backward_workspace_size_ex(0, H, 2, N, d, 1) == 0


def test_backward_ex_wants_the_ex_workspace(L):
    need = L.fa2_backward_workspace_size_ex(1, 8, 1, 64, 128, 1)
    short = L.fa2_backward_workspace_size(1, 8, 64, 128, 1)
    assert need > short
    args = (A,) * 9 + (1, 8, 1, 64, 128, 0.125, 1, 1, A)
    assert L.fa2_backward_ex(*args, short, None) == fa.FA2_ERR_WORKSPACE
    assert L.fa2_backward_stage_ex(2, *args, need - 1, None) == fa.FA2_ERR_WORKSPACE


def test_status_strings(L):
    for s in range(5):
        txt = L.fa2_status_string(s).decode()
        assert txt.startswith("FA2_")
    assert b"unknown" in L.fa2_status_string(99)


def test_python_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 8, 16)
    with pytest.raises(ValueError):
        fa.forward(q, q, q)


@pytest.mark.parametrize("stage", [0, 3, 4, -1])
def test_backward_stage_rejects_bad_stage(L, stage):
    n = L.fa2_backward_workspace_size(1, 2, 64, 64, 1)
    assert L.fa2_backward_stage(stage, A, A, A, A, A, A, A, A, A, 1, 2, 64, 64, 0.125, 1, 1, A, n, None) \
        == fa.FA2_ERR_INVALID_ARG


def test_backward_stage_validates_like_backward(L):
    n = L.fa2_backward_workspace_size(1, 2, 64, 64, 1)
    assert L.fa2_backward_stage(2, A, A, A, A, A, A, A, A, A, 1, 2, 64, 48, 0.125, 1, 1, A, n, None) \
        == fa.FA2_ERR_UNSUPPORTED
    assert L.fa2_backward_stage(1, A, A, A, A, A, A, A, A, A, 1, 2, 64, 64, 0.125, 1, 1, A, n - 1, None) \
        == fa.FA2_ERR_WORKSPACE


# Grouped-query entry points: H_kv must divide H (validated before any HIP
# call, so these run without a GPU).
def fwd_ex(L, H=4, H_kv=2, ptr=A, **over):
    p = dict(B=1, N=64, d=64, scale=0.125, causal=1, dtype=1)
    p.update(over)
    return L.fa2_forward_ex(ptr, ptr, ptr, ptr, ptr, p["B"], H, H_kv, p["N"], p["d"], p["scale"], p["causal"],
                            p["dtype"], None)


def bwd_ex(L, H=4, H_kv=2, ptr=A, stage=None):
    wsb = L.fa2_backward_workspace_size_ex(1, H, max(H_kv, 1), 64, 64, 1)
    args = (ptr,) * 9 + (1, H, H_kv, 64, 64, 0.125, 1, 1, A, wsb, None)
    if stage is None:
        return L.fa2_backward_ex(*args)
    return L.fa2_backward_stage_ex(stage, *args)


@pytest.mark.parametrize("H,H_kv", [(4, 3), (4, 0), (4, -1), (4, 8), (6, 4)])
def test_ex_rejects_bad_kv_heads(L, H, H_kv):
    assert fwd_ex(L, H, H_kv) == fa.FA2_ERR_INVALID_ARG
    assert bwd_ex(L, H, H_kv) == fa.FA2_ERR_INVALID_ARG
    assert bwd_ex(L, H, H_kv, stage=2) == fa.FA2_ERR_INVALID_ARG


def test_ex_checks_like_the_plain_calls(L):
    assert fwd_ex(L, 4, 2, ptr=None) == fa.FA2_ERR_INVALID_ARG
    assert fwd_ex(L, 4, 2, ptr=MIS) == fa.FA2_ERR_UNSUPPORTED
    assert fwd_ex(L, 4, 2, d=48) == fa.FA2_ERR_UNSUPPORTED
    assert fwd_ex(L, 0, 0, B=1) == fa.FA2_OK  # empty: a no-op
    assert bwd_ex(L, 4, 1, stage=4) == fa.FA2_ERR_INVALID_ARG


# Decoding: validation happens before any HIP call.
def dec(L, B=1, H=4, H_kv=2, Nq=1, Nk=100, d=128, scale=0.125, causal=0, dtype=1, ptr=A, ws=A, wsb=1 << 30):
    return L.fa2_decode(ptr, ptr, ptr, ptr, ptr, B, H, H_kv, Nq, Nk, d, scale, causal, dtype, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), fa.FA2_ERR_INVALID_ARG), (dict(Nq=-1), fa.FA2_ERR_INVALID_ARG),
    (dict(Nk=-1), fa.FA2_ERR_INVALID_ARG), (dict(H_kv=3), fa.FA2_ERR_INVALID_ARG),
    (dict(H_kv=0), fa.FA2_ERR_INVALID_ARG), (dict(scale=0.0), fa.FA2_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA2_ERR_INVALID_ARG), (dict(dtype=5), fa.FA2_ERR_INVALID_ARG),
    (dict(Nk=0), fa.FA2_ERR_INVALID_ARG), (dict(Nq=5, Nk=4, causal=1), fa.FA2_ERR_INVALID_ARG),
    (dict(dtype=3), fa.FA2_ERR_INVALID_ARG), (dict(d=48, dtype=0), fa.FA2_ERR_UNSUPPORTED),
    (dict(d=48), fa.FA2_ERR_UNSUPPORTED), (dict(d=256, dtype=2), fa.FA2_ERR_UNSUPPORTED),
    (dict(ptr=None), fa.FA2_ERR_INVALID_ARG), (dict(ptr=None, dtype=0, d=64), fa.FA2_ERR_INVALID_ARG),
    (dict(ptr=MIS), fa.FA2_ERR_UNSUPPORTED), (dict(Nk=1 << 24), fa.FA2_ERR_INVALID_ARG),
])
def test_decode_rejects(L, kw, status):
    assert dec(L, **kw) == status


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0, H_kv=0), dict(Nq=0)])
def test_decode_empty_is_noop(L, kw):
    assert dec(L, ptr=None, ws=None, wsb=0, **kw) == fa.FA2_OK


def test_decode_workspace(L):
    """Partial results of the split cache: S chunks x (O rows in fp32 and
    their LSE), S from the sizes; none when the cache is one chunk."""
    def al(x):
        return (x + 255) // 256 * 256
    # 16 x 8 key/value heads, one row block each: 512 / 128 = 4 chunks of 128 blocks
    rows = 16 * 64 * 1
    assert L.fa2_decode_workspace_size(16, 64, 8, 1, 16384, 128, 1) == al(4 * rows * 128 * 4) + al(4 * rows * 4)
    # 4 blocks of keys: a single chunk, no workspace
    assert L.fa2_decode_workspace_size(1, 8, 1, 4, 100, 128, 1) == 0
    # 33 blocks, at most 8 chunks of >= 4 blocks: chunks of 5 blocks, 7 of them
    assert L.fa2_decode_workspace_size(1, 1, 1, 100, 1040, 128, 1) == al(7 * 100 * 128 * 4) + al(7 * 100 * 4)
    assert L.fa2_decode_workspace_size(1, 4, 2, 1, 100, 64, 1) == 0
    assert L.fa2_decode_workspace_size(16, 64, 8, 1, 16384, 128, 2) == al(4 * rows * 128 * 4) + al(4 * rows * 4)
    assert L.fa2_decode_workspace_size(16, 64, 8, 1, 16384, 128, 0) == 0
    assert L.fa2_decode_workspace_size(1, 4, 3, 1, 100, 128, 1) == 0
    need = L.fa2_decode_workspace_size(16, 64, 8, 1, 16384, 128, 1)
    assert dec(L, B=16, H=64, H_kv=8, Nk=16384, wsb=need - 1) == fa.FA2_ERR_WORKSPACE
    assert dec(L, B=16, H=64, H_kv=8, Nk=16384, ws=None, wsb=need) == fa.FA2_ERR_WORKSPACE
    assert dec(L, B=16, H=64, H_kv=8, Nk=16384, ws=MIS, wsb=need) == fa.FA2_ERR_UNSUPPORTED


# Packed ragged batches: host-side validation (the offsets themselves live on
# the device and are never read here).
def fwd_vl(L, cu=A, B=2, H=4, H_kv=2, T=100, mx=60, d=64, dtype=1, ptr=A):
    return L.fa2_forward_varlen(ptr, ptr, ptr, ptr, ptr, cu, B, H, H_kv, T, mx, d, 0.125, 1, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(cu=None), fa.FA2_ERR_INVALID_ARG), (dict(T=-1), fa.FA2_ERR_INVALID_ARG),
    (dict(mx=-1), fa.FA2_ERR_INVALID_ARG), (dict(mx=101), fa.FA2_ERR_INVALID_ARG),
    (dict(H_kv=3), fa.FA2_ERR_INVALID_ARG), (dict(d=48), fa.FA2_ERR_UNSUPPORTED),
    (dict(dtype=3), fa.FA2_ERR_INVALID_ARG), (dict(ptr=None), fa.FA2_ERR_INVALID_ARG),
    (dict(ptr=MIS), fa.FA2_ERR_UNSUPPORTED), (dict(cu=A + 2), fa.FA2_ERR_UNSUPPORTED),
    (dict(T=1 << 24, mx=10, d=128), fa.FA2_ERR_INVALID_ARG),
])
def test_varlen_rejects(L, kw, status):
    assert fwd_vl(L, **kw) == status


def test_varlen_empty_is_noop(L):
    assert fwd_vl(L, ptr=None, cu=None, B=0) == fa.FA2_OK
    assert fwd_vl(L, ptr=None, mx=0) == fa.FA2_OK
    assert fwd_vl(L, ptr=None, H=0, H_kv=0) == fa.FA2_OK


def test_varlen_workspace(L):
    def al(x):
        return (x + 255) // 256 * 256
    # rows = H * T for D and LSE * log2(e)
    assert L.fa2_backward_workspace_size_varlen(3, 4, 4, 1000, 600, 64, 1) == 2 * al(4 * 1000 * 4)
    # grouped bf16 d=128: 5 key tiles x 3 x 2 = 30 workgroups -> split S = G = 2, partials [2][H_kv * T, d]
    assert L.fa2_backward_workspace_size_varlen(3, 4, 2, 1000, 600, 128, 1) == \
        2 * al(4 * 1000 * 4) + 2 * al(2 * 2 * 1000 * 128 * 4)
    assert L.fa2_backward_workspace_size_varlen(3, 4, 2, 1000, 1001, 128, 1) == 0
    need = L.fa2_backward_workspace_size_varlen(3, 4, 2, 1000, 600, 128, 1)
    args = (A,) * 10 + (3, 4, 2, 1000, 600, 128, 0.125, 1, 1, A)
    assert L.fa2_backward_varlen(*args, need - 1, None) == fa.FA2_ERR_WORKSPACE
    assert L.fa2_backward_stage_varlen(4, *args, need, None) == fa.FA2_ERR_INVALID_ARG


# fa2_backward_noalloc validates before any HIP call: bad arguments and
# problems that need more than its static workspace are rejected on a host
# without a GPU.
def bwd_noalloc(L, B=1, H=2, H_kv=2, N=64, d=64, scale=0.125, dtype=1, ptr=A):
    return L.fa2_backward_noalloc(ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, B, H, H_kv, N, d, scale, 1, dtype,
                                  None)


def test_noalloc_rejects_problems_beyond_its_buffer(L):
    # 64 x 64 x 4096 query rows: D and LSE*log2(e) alone take 128 MiB
    assert fa.NOALLOC_SCRATCH_BYTES == 64 << 20
    assert L.fa2_backward_workspace_size_ex(64, 64, 64, 4096, 128, 1) > fa.NOALLOC_SCRATCH_BYTES
    assert bwd_noalloc(L, B=64, H=64, H_kv=64, N=4096, d=128) == fa.FA2_ERR_SCRATCH
    assert "static buffer" in fa.fa2_status_string(fa.FA2_ERR_SCRATCH)


def test_noalloc_validates_like_backward(L):
    assert bwd_noalloc(L, d=48) == fa.FA2_ERR_UNSUPPORTED
    assert bwd_noalloc(L, H=4, H_kv=3) == fa.FA2_ERR_INVALID_ARG
    assert bwd_noalloc(L, scale=float("nan")) == fa.FA2_ERR_INVALID_ARG
    assert bwd_noalloc(L, dtype=7) == fa.FA2_ERR_INVALID_ARG
    assert bwd_noalloc(L, ptr=None) == fa.FA2_ERR_INVALID_ARG
    assert bwd_noalloc(L, ptr=A + 8) == fa.FA2_ERR_UNSUPPORTED
    assert bwd_noalloc(L, B=0, ptr=None) == fa.FA2_OK
