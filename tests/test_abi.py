"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/dsa.h declares, sizes workspaces, and rejects bad
arguments before launching anything."""
import ctypes
import os
import re

import pytest

import long_context_02_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")


def _declared():
    text = open(HEADER).read()
    return re.findall(r"DSA_API\s+[\w\s\*]+?\b(dsa_\w+)\s*\(", text)


def test_header_declares_the_boundary():
    names = set(_declared())
    assert {"dsa_indexer_scores", "dsa_topk_select", "dsa_sparse_mla_attn", "dsa_forward",
            "dsa_workspace_size", "dsa_status_string", "dsa_version"} <= names


def test_library_exports_every_declared_symbol():
    L = dsa.lib()
    for name in _declared():
        assert hasattr(L, name), name


def test_status_strings_and_version():
    L = dsa.lib()
    for code, name in dsa._STATUS.items():
        assert L.dsa_status_string(code).decode().startswith(name)
    assert L.dsa_status_string(99).decode().startswith("unknown")
    assert L.dsa_version() >> 16 == 1


def test_workspace_sizes():
    # top-k needs none for long batches; batches of at most 255 rows hold
    # a per-row histogram, counters and candidate lists
    assert dsa.workspace_size(dsa.OP_TOPK, 1, 8192, 8192, 8, 128, 512, 2048) == 0
    seg = dsa.workspace_size(dsa.OP_TOPK, 64, 1, 131072, 8, 128, 512, 2048)
    assert seg >= 64 * (4096 + 2048 + 2 * 12288) * 4
    # forward holds the fp32 score matrix and the indices
    fwd = dsa.workspace_size(dsa.OP_FORWARD, 1, 4096, 131072, 8, 128, 512, 2048)
    assert fwd >= 4096 * 131072 * 4 + 4096 * 2048 * 4
    # decode splits the 2048 slots of its 64 rows over 4 workgroups each:
    # bf16 O rows plus fp32 (max, sum) per split and head
    att = dsa.workspace_size(dsa.OP_ATTN, 64, 1, 131072, 8, 128, 512, 2048)
    assert att >= 64 * 4 * 128 * (512 * 2 + 2 * 4)
    # prefill-sized batches need no split workspace; f32 shapes never do
    assert dsa.workspace_size(dsa.OP_ATTN, 1, 8192, 8192, 8, 128, 512, 2048) == 0
    assert dsa.workspace_size(dsa.OP_ATTN, 1, 4, 256, 8, 16, 64, 64) == 0
    # the fused selection holds the scores and, for few rows, the row lists
    sel = dsa.workspace_size(dsa.OP_SELECT, 64, 1, 131072, 8, 1, 1, 2048)
    assert sel >= 64 * 131072 * 4 + seg
    assert dsa.workspace_size(dsa.OP_SELECT, 1, 4096, 131072, 8, 1, 1, 2048) >= 4096 * 131072 * 4
    with pytest.raises(ValueError):
        dsa.workspace_size(dsa.OP_FORWARD, 1, 1, 1, 8, 128, 512, 4096)
    with pytest.raises(ValueError):
        dsa.workspace_size(7, 1, 1, 1, 8, 1, 1, 1)
    with pytest.raises(ValueError):  # indexer heads must be >= 1
        dsa.workspace_size(dsa.OP_SELECT, 64, 1, 131072, 0, 128, 512, 2048)


def test_workspace_size_takes_eight_sizes():
    # the C signature is (op, B, T, N, H_I, H, d_v, k): called directly
    # through ctypes with explicit argument types
    L = ctypes.CDLL(dsa.lib_path())
    f = L.dsa_workspace_size
    f.argtypes = [ctypes.c_int] * 8
    f.restype = ctypes.c_size_t
    fwd = f(dsa.OP_FORWARD, 64, 1, 131072, 8, 128, 512, 2048)
    assert fwd == dsa.workspace_size(dsa.OP_FORWARD, 64, 1, 131072, 8, 128, 512, 2048)
    assert fwd >= 64 * 131072 * 4 + 64 * 2048 * 4 + 64 * 4 * 128 * 512 * 2
    assert f(dsa.OP_SELECT, 64, 1, 131072, 0, 128, 512, 2048) == ctypes.c_size_t(-1).value
    assert f(dsa.OP_ATTN, 64, 1, 131072, 8, 0, 512, 2048) == ctypes.c_size_t(-1).value


# Fake 16-byte-aligned device addresses: these calls must fail validation on
# the host, so nothing is ever dereferenced or launched.
P = ctypes.c_void_p(0x10000)


def test_indexer_rejects_bad_arguments():
    L = dsa.lib()
    f = L.dsa_indexer_scores
    ok = dict(B=1, T=4, N=8, H_I=8, d_I=128, q_offset=4, dt=dsa.FP8_E4M3FN)

    def call(**kw):
        a = {**ok, **kw}
        ptrs = kw.get("ptrs", [P, P, P, P, P, P])
        return f(*ptrs, a["B"], a["T"], a["N"], a["H_I"], a["d_I"], a["q_offset"], a["dt"], None)

    assert call(ptrs=[None, P, P, P, P, P]) == 1
    assert call(ptrs=[P, None, P, P, P, P]) == 1          # FP8 needs scales
    assert call(ptrs=[P, P, P, P, P, ctypes.c_void_p(0x10004)]) == 1  # misaligned
    assert call(q_offset=5) == 1                          # q_offset + T > N
    assert call(T=0) == 1
    assert call(q_offset=-1) == 1
    assert call(H_I=4) == 2 and call(d_I=64) == 2         # FP8 supports (8, 128)
    assert call(N=1 << 24, q_offset=(1 << 24) - 4) == 2   # FP8 keys: 32-bit byte offsets
    assert call(dt=dsa.BF16) == 2
    assert call(dt=9) == 1
    assert call(dt=dsa.F32) == 1                          # f32 takes no scales
    assert call(dt=dsa.F32, ptrs=[P, None, P, None, P, P], H_I=17) == 2


def test_topk_rejects_bad_arguments():
    f = dsa.lib().dsa_topk_select
    assert f(None, P, 1, 1, 8, 4, 0, None, 0, None) == 1
    assert f(P, P, 1, 1, 8, 0, 0, None, 0, None) == 1
    assert f(P, P, 1, 1, 8, 4096, 0, None, 0, None) == 2
    assert f(P, P, 1, 2, 8, 4, 7, None, 0, None) == 1
    # batches of at most 255 rows need a 16-byte-aligned workspace
    need = dsa.workspace_size(dsa.OP_TOPK, 4, 1, 8, 8, 1, 1, 4)
    assert need > 0
    assert f(P, P, 4, 1, 8, 4, 7, None, need, None) == 3
    assert f(P, P, 4, 1, 8, 4, 7, P, need - 1, None) == 3
    assert f(P, P, 4, 1, 8, 4, 7, ctypes.c_void_p(0x10008), need, None) == 3


def test_attention_rejects_bad_arguments():
    f = dsa.lib().dsa_sparse_mla_attn

    def call(H=128, dqk=576, dv=512, k=2048, scale=0.04, dt=dsa.BF16, ptrs=None, N=10):
        ptrs = ptrs or [P, P, P, P, None]
        return f(*ptrs, 1, 1, N, H, dqk, dv, k, scale, dt, None, 0, None)

    assert call(ptrs=[P, None, P, P, None]) == 1
    assert call(H=64) == 2 and call(dqk=512) == 2 and call(dv=256) == 2
    assert call(k=0) == 1 and call(k=2049) == 2
    assert call(scale=float("nan")) == 1
    assert call(dt=dsa.FP8_E4M3FN) == 2
    assert call(H=16, dqk=80, dv=96, dt=dsa.F32) == 2     # d_v > d_qk
    assert call(N=(1 << 31) // 1152 + 1) == 2             # bf16 rows beyond 32-bit offsets


def test_attention_bwd_rejects_bad_arguments():
    f = dsa.lib().dsa_sparse_mla_attn_bwd
    need = dsa.workspace_size(dsa.OP_ATTN_BWD, 1, 4, 10, 8, 128, 512, 64)
    # P and dS tiles ([128 heads][32 slots] bf16 each) of every row
    assert need >= 2 * 4 * 2 * 128 * 32 * 2
    big = dsa.workspace_size(dsa.OP_ATTN_BWD, 1, 4096, 131072, 8, 128, 512, 2048)
    assert big >= 2 * 2048 * 64 * 128 * 32 * 2  # rows are processed 2048 at a time

    def call(H=128, dqk=576, dv=512, k=64, scale=0.04, dt=dsa.BF16, lse=P, dout=P, dq=P, dkv=P,
             ws=P, ws_bytes=None, N=10, T=4):
        wb = need if ws_bytes is None else ws_bytes
        return f(P, P, P, P, lse, dout, dq, dkv, 1, T, N, H, dqk, dv, k, scale, dt, ws, wb, None)

    assert call(lse=None) == 1 and call(dout=None) == 1 and call(dq=None) == 1 and call(dkv=None) == 1
    assert call(dq=ctypes.c_void_p(0x10004)) == 1          # misaligned
    assert call(H=64) == 2 and call(dqk=512) == 2 and call(dv=256) == 2
    assert call(k=0) == 1 and call(k=2049) == 2
    assert call(scale=float("inf")) == 1
    assert call(H=16, dqk=64, dv=64, dt=dsa.F32) == 2     # bf16 only
    assert call(ws=None) == 3 and call(ws_bytes=need - 1) == 3
    assert call(N=(1 << 31) // 1152 + 1) == 2


def test_indexer_select_rejects_bad_arguments():
    f = dsa.lib().dsa_indexer_select

    def call(ptrs=None, k=4, ws=P, wsb=1 << 20, q_offset=4, dt=dsa.FP8_E4M3FN):
        ptrs = ptrs or [P, P, P, P, P, P]
        return f(*ptrs, 1, 4, 8, 8, 128, k, q_offset, dt, ws, wsb, None)

    assert call(ptrs=[P, P, P, P, P, None]) == 1          # no idx
    assert call(ptrs=[None, P, P, P, P, P]) == 1
    assert call(k=0) == 1 and call(k=4096) == 2
    assert call(q_offset=5) == 1
    assert call(ws=None) == 3 and call(wsb=16) == 3
    assert call(dt=dsa.BF16) == 2


def test_forward_rejects_small_workspace():
    f = dsa.lib().dsa_forward
    st = f(P, P, P, P, P, P, P, P, None, None, 1, 4, 8, 8, 128, 128, 576, 512, 4, 4, 0.04,
           dsa.FP8_E4M3FN, dsa.BF16, P, 16, None)
    assert st == 3


def test_cache_append_rejects_bad_arguments():
    f = dsa.lib().dsa_cache_append

    def call(ptrs=None, d_I=128, d_qk=576, idt=dsa.FP8_E4M3FN, adt=dsa.BF16, B=2, T=1, N=8):
        ptrs = ptrs or [P, P, P, P, P, P]
        return f(*ptrs, B, T, N, d_I, d_qk, idt, adt, None)

    assert call(ptrs=[None, P, P, P, P, P]) == 1
    assert call(ptrs=[P, P, P, P, P, None]) == 1          # no positions
    assert call(ptrs=[P, P, P, None, P, P]) == 1          # FP8 needs the scales
    assert call(idt=dsa.F32, d_I=32) == 1                 # f32 keys take no scales
    assert call(d_I=64) == 2 and call(d_qk=512) == 2
    assert call(adt=dsa.F32, d_qk=300) == 2
    assert call(idt=dsa.BF16) == 2 and call(adt=dsa.FP8_E4M3FN) == 2
    assert call(B=0) == 1 and call(T=0) == 1


def test_indexer_kl_rejects_bad_arguments():
    f = dsa.lib().dsa_indexer_kl

    def call(ptrs=None, B=1, T=4, N=8, k=0, q_offset=4):
        ptrs = ptrs or [P, P, None, P, P]
        return f(*ptrs, B, T, N, k, q_offset, None)

    assert call(ptrs=[None, P, None, P, P]) == 1
    assert call(ptrs=[P, P, None, None, P]) == 1          # loss is required
    assert call(q_offset=5) == 1                          # dense: q_offset + T > N
    assert call(ptrs=[P, P, P, P, None], k=0) == 1        # selected slots need k >= 1
    assert call(ptrs=[P, P, P, P, None], k=4096) == 2
    assert call(B=0) == 1


def test_forward_noalloc_rejects_before_launching():
    f = dsa.lib().dsa_forward_noalloc
    f.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int] * 10 + [ctypes.c_float, ctypes.c_int,
                                                                 ctypes.c_int, ctypes.c_void_p]
    f.restype = ctypes.c_int

    def call(B=1, T=4, N=8, k=4, q_offset=4, ptrs=None):
        ptrs = ptrs or [P, P, P, P, P, P, P, P, None, None]
        return f(*ptrs, B, T, N, 8, 128, 128, 576, 512, k, q_offset, 0.04, dsa.FP8_E4M3FN, dsa.BF16,
                 None)

    assert call(ptrs=[None, P, P, P, P, P, P, P, None, None]) == 1
    assert call(q_offset=5) == 1
    assert call(k=4096) == 2
    # a [B,T,N] score matrix beyond the fixed 128 MiB array (prefill 8K)
    assert dsa.workspace_size(dsa.OP_FORWARD, 1, 8192, 8192, 8, 128, 512, 2048) > (128 << 20)
    assert call(T=8192, N=8192, k=2048, q_offset=0) == 2
    # decode of 64 sequences at 131072 tokens fits
    assert dsa.workspace_size(dsa.OP_FORWARD, 64, 1, 131072, 8, 128, 512, 2048) <= (128 << 20)


def test_attention_mha_rejects_bad_arguments():
    f = dsa.lib().dsa_sparse_mla_attn_mha
    need = dsa.workspace_size(dsa.OP_ATTN_MHA, 1, 4, 10, 8, 128, 128, 64)
    assert need >= 10 * 128 * (128 + 128) * 2
    with pytest.raises(ValueError):
        dsa.workspace_size(dsa.OP_ATTN_MHA, 1, 4, 10, 8, 64, 128, 64)

    def call(H=128, dc=512, dr=64, dn=128, dvh=128, k=64, scale=0.07, dt=dsa.BF16, ws=P, wsb=None,
             ptrs=None):
        ptrs = ptrs or [P, P, P, P, P, P, None]
        return f(*ptrs, 1, 4, 10, H, dc, dr, dn, dvh, k, scale, dt, ws, need if wsb is None else wsb,
                 None)

    assert call(ptrs=[P, P, None, P, P, P, None]) == 1      # no W_UK
    assert call(ptrs=[P, P, P, P, P, ctypes.c_void_p(0x10002), None]) == 1  # misaligned out
    assert call(H=64) == 2 and call(dc=256) == 2 and call(dr=32) == 2
    assert call(dn=64) == 2 and call(dvh=64) == 2
    assert call(k=0) == 1 and call(k=2049) == 2
    assert call(scale=float("nan")) == 1
    assert call(dt=dsa.F32) == 2 and call(dt=7) == 1
    assert call(ws=None) == 3 and call(wsb=need - 1) == 3
