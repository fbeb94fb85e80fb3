"""C-ABI checks that need no GPU: the library loads, exports every entry point declared in
include/sala.h, and rejects bad arguments before anything is enqueued (these paths make no
HIP call, so they run on a CPU-only host)."""

import ctypes
import os
import re

import pytest

from conftest import ROOT

LIB = os.environ.get("SALA_LIBRARY") or os.path.join(ROOT, "hybrid_sparse_linear_causal_amd", "libsala.so")
pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libsala.so not built")


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "sala.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sala_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    names = declared_symbols()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_status_strings():
    from hybrid_sparse_linear_causal_amd import sala as S

    L = S.lib()
    assert L.sala_abi_version() == 6
    for code in range(6):
        assert L.sala_status_str(code)
    assert L.sala_last_hip_error() == 0


def _lin(**kw):
    from hybrid_sparse_linear_causal_amd import sala as S

    base = dict(batch=1, seq_len=128, n_heads=2, n_kv_heads=2, head_dim=128, dtype=S.SALA_BF16,
                pos0=0, rope_base=10000.0, norm_eps=1e-6)
    base.update(kw)
    return S.LinearDesc(**base)


def _sp(**kw):
    from hybrid_sparse_linear_causal_amd import sala as S

    base = dict(batch=1, n_q=128, n_heads=4, n_kv_heads=2, head_dim=128, dtype=S.SALA_BF16, block=64,
                topk=8, n_local=2, norm_eps=1e-6, scale=0.0, reserved_=0, kv_len=128, kv_capacity=128)
    base.update(kw)
    return S.SparseDesc(**base)


FAKE = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: every call below fails validation


@pytest.mark.parametrize("kw,expect", [
    (dict(batch=0), 2), (dict(seq_len=-1), 2), (dict(head_dim=96), 3), (dict(dtype=7), 2),
    (dict(n_kv_heads=3), 2), (dict(n_heads=130, n_kv_heads=2), 3), (dict(rope_base=0.0), 2),
    (dict(norm_eps=-1.0), 2), (dict(pos0=-5), 2), (dict(head_dim=64), 3),
    # chunk sizes: 64 (or 0) built; 128 and 256 valid but not built; anything else invalid
    (dict(chunk=128), 3), (dict(chunk=256), 3), (dict(chunk=100), 2), (dict(chunk=-64), 2), (dict(reserved_=1), 2),
])
def test_linear_prefill_rejects(kw, expect):
    from hybrid_sparse_linear_causal_amd import sala as S

    d = _lin(**kw)
    st = S.lib().sala_linear_prefill(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, None, None, None,
                                     FAKE, FAKE, 1 << 30, None)
    assert st == expect


def test_linear_prefill_null_and_alignment_and_workspace():
    from hybrid_sparse_linear_causal_amd import sala as S

    L = S.lib()
    d = _lin(seq_len=1 << 16, n_heads=32, n_kv_heads=32)
    assert L.sala_linear_prefill(None, FAKE, FAKE, FAKE, FAKE, None, None, None, None, FAKE, FAKE, 0, None) == 1
    assert L.sala_linear_prefill(ctypes.byref(d), None, FAKE, FAKE, FAKE, None, None, None, None, FAKE,
                                 FAKE, 1 << 40, None) == 1
    odd = ctypes.c_void_p((1 << 20) + 2)
    assert L.sala_linear_prefill(ctypes.byref(d), odd, FAKE, FAKE, FAKE, None, None, None, None, FAKE,
                                 FAKE, 1 << 40, None) == 2
    need = S.workspace_bytes(S.OP_LINEAR_PREFILL, d)
    assert need > 0
    assert L.sala_linear_prefill(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, None, None, None, FAKE,
                                 FAKE, need - 1, None) == 4
    assert L.sala_linear_prefill(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, None, None, None, FAKE,
                                 None, need, None) == 4


def test_linear_grouped_heads_sizes():
    """Grouped (GQA) linear heads: the segment-state workspace is per KV head; the backward
    supports plain multi-head layers only."""
    from hybrid_sparse_linear_causal_amd import sala as S

    L = S.lib()
    mha = _lin(seq_len=1 << 16, n_heads=32, n_kv_heads=32)
    gqa = _lin(seq_len=1 << 16, n_heads=32, n_kv_heads=2)
    assert S.workspace_bytes(S.OP_LINEAR_PREFILL, gqa) * 16 == S.workspace_bytes(S.OP_LINEAR_PREFILL, mha)
    assert L.sala_workspace_bytes(S.OP_LINEAR_BACKWARD, ctypes.byref(gqa)) == ctypes.c_size_t(-1).value
    args = [FAKE] * 4 + [None, None, None, FAKE, None] + [FAKE] * 4 + [None, None, None]
    assert L.sala_linear_backward(ctypes.byref(gqa), *args, FAKE, 1 << 40, None) == 3
    assert L.sala_linear_prefill(ctypes.byref(_lin(chunk=256)), FAKE, FAKE, FAKE, FAKE, None, None, None, None,
                                 FAKE, FAKE, 1 << 30, None) == 3


def test_linear_decode_rejects():
    from hybrid_sparse_linear_causal_amd import sala as S

    L = S.lib()
    d = _lin(seq_len=2)
    assert L.sala_linear_decode_step(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, None) == 2
    d = _lin(seq_len=1)
    assert L.sala_linear_decode_step(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE, None) == 1


@pytest.mark.parametrize("kw,expect", [
    (dict(block=32), 3), (dict(n_local=3), 3), (dict(topk=2), 2), (dict(topk=257), 2),
    (dict(n_heads=3), 2), (dict(kv_len=100, n_q=128), 2), (dict(kv_capacity=100, kv_len=100, n_q=100), 2),
    (dict(kv_capacity=192, kv_len=160, n_q=128), 2), (dict(head_dim=80), 3), (dict(scale=-1.0), 2),
    (dict(n_heads=128, n_kv_heads=2), 3), (dict(n_q=0), 2),
])
def test_sparse_rejects(kw, expect):
    from hybrid_sparse_linear_causal_amd import sala as S

    L = S.lib()
    d = _sp(**kw)
    assert L.sala_kv_append(ctypes.byref(d), FAKE, FAKE, None, FAKE, FAKE, FAKE, None) == expect
    assert L.sala_block_select(ctypes.byref(d), FAKE, None, FAKE, FAKE, None, FAKE, 1 << 40, None) == expect
    assert L.sala_sparse_attn(ctypes.byref(d), FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40,
                              None) == expect
    assert L.sala_workspace_bytes(S.OP_BLOCK_SELECT, ctypes.byref(d)) == ctypes.c_size_t(-1).value


def test_sparse_null_workspace_and_pool_range():
    from hybrid_sparse_linear_causal_amd import sala as S

    L = S.lib()
    d = _sp()
    assert L.sala_block_select(ctypes.byref(d), None, None, FAKE, FAKE, None, FAKE, 1 << 30, None) == 1
    need = S.workspace_bytes(S.OP_BLOCK_SELECT, d)
    assert need > 0
    assert L.sala_block_select(ctypes.byref(d), FAKE, None, FAKE, FAKE, None, FAKE, need - 1, None) == 4
    assert L.sala_kv_pool(ctypes.byref(d), FAKE, FAKE, 0, 3, None) == 2  # 3*64 > kv_len
    assert L.sala_kv_pool(ctypes.byref(d), FAKE, FAKE, 2, 1, None) == 2
    assert L.sala_kv_pool(ctypes.byref(d), None, FAKE, 0, 1, None) == 1
    dd = _sp(n_q=1, kv_len=1000, kv_capacity=1024, n_heads=64, n_kv_heads=2)  # bf16 decode, group 32
    assert L.sala_sparse_attn(ctypes.byref(dd), FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30,
                              None) == 3
    assert S.workspace_bytes(S.OP_SPARSE_ATTN, _sp(n_q=1, kv_len=1000, kv_capacity=1024)) > 0


def test_dense_attn_arguments_and_mode_switch():
    """Argument errors of sala_dense_attn (no device work), and the dense/sparse switch rule
    (host-side): dense exactly while kv_len <= topk * 64."""
    import torch

    from hybrid_sparse_linear_causal_amd import sala as S

    L = S.lib()
    d = S.sparse_desc(batch=1, n_q=64, n_heads=8, n_kv_heads=2, head_dim=128, dtype=torch.bfloat16,
                      kv_len=640, kv_capacity=640, topk=10, n_local=2)
    assert L.sala_dense_attn(None, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    assert L.sala_dense_attn(ctypes.byref(d), None, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    bad = S.sparse_desc(batch=1, n_q=64, n_heads=8, n_kv_heads=3, head_dim=128, dtype=torch.bfloat16,
                        kv_len=640, kv_capacity=640, topk=10, n_local=2)
    assert L.sala_dense_attn(ctypes.byref(bad), FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == 2
    assert L.sala_sparse_layer_uses_dense(ctypes.byref(d)) == 1          # 640 <= 10 * 64
    d.kv_len = d.kv_capacity = 641 + 63  # 704 > 640
    d.n_q = 704 - 640
    assert L.sala_sparse_layer_uses_dense(ctypes.byref(d)) == 0
    assert L.sala_sparse_layer_uses_dense(ctypes.byref(bad)) == -1
    assert L.sala_workspace_bytes(S.OP_DENSE_ATTN, ctypes.byref(d)) == 0  # prefill: none


def test_linear_backward_arguments():
    """Argument errors of sala_linear_backward (no device work): bf16 and d = 128 only, the four
    input-gradient buffers are required, the workspace must be large enough."""
    from hybrid_sparse_linear_causal_amd import sala as S

    L = S.lib()
    d = _lin(seq_len=256)
    need = S.workspace_bytes(S.OP_LINEAR_BACKWARD, d)
    assert need > 0
    # q k v gate | q_norm_w k_norm_w state_in | dout dstate_out | dq dk dv dg | dqw dkw dstate_in
    args = [FAKE] * 4 + [None, None, None] + [FAKE, None] + [FAKE] * 4 + [None, None, None]
    assert L.sala_linear_backward(ctypes.byref(d), *args, FAKE, need - 1, None) == 4
    assert L.sala_linear_backward(ctypes.byref(d), *args, None, need, None) == 4
    bad = list(args)
    bad[9] = None  # dq
    assert L.sala_linear_backward(ctypes.byref(d), *bad, FAKE, need, None) == 1
    f32 = _lin(seq_len=256, dtype=S.SALA_F32)
    assert L.sala_linear_backward(ctypes.byref(f32), *args, FAKE, need, None) == 3
    assert L.sala_workspace_bytes(S.OP_LINEAR_BACKWARD, ctypes.byref(f32)) == ctypes.c_size_t(-1).value
    d64 = _lin(seq_len=256, head_dim=64, n_heads=2, n_kv_heads=2)
    assert L.sala_linear_backward(ctypes.byref(d64), *args, FAKE, need, None) == 3


def test_sparse_backward_arguments():
    """Argument errors of sala_sparse_attn_backward and sala_kv_norm_backward (no device work)."""
    import torch

    from hybrid_sparse_linear_causal_amd import sala as S

    L = S.lib()
    d = S.sparse_desc(batch=1, n_q=128, n_heads=4, n_kv_heads=2, head_dim=128, dtype=torch.bfloat16,
                      kv_len=128, kv_capacity=128, topk=3, n_local=2)
    need = S.workspace_bytes(S.OP_SPARSE_ATTN_BACKWARD, d)
    assert need > 0
    # q qw k v gate sel dout | out lse | dq dk dv dg dqw
    args = [FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, FAKE, None]
    assert L.sala_sparse_attn_backward(ctypes.byref(d), *args, FAKE, need - 1, None) == 4
    assert L.sala_sparse_attn_backward(ctypes.byref(d), *args, None, need, None) == 4
    bad = list(args)
    bad[5] = None  # sel
    assert L.sala_sparse_attn_backward(ctypes.byref(d), *bad, FAKE, need, None) == 1
    half = list(args)
    half[7] = FAKE  # the forward's out without its lse
    assert L.sala_sparse_attn_backward(ctypes.byref(d), *half, FAKE, need, None) == 1
    dec = S.sparse_desc(batch=1, n_q=1, n_heads=4, n_kv_heads=2, head_dim=128, dtype=torch.bfloat16,
                        kv_len=128, kv_capacity=128, topk=3, n_local=2)
    assert L.sala_sparse_attn_backward(ctypes.byref(dec), *args, FAKE, need, None) == 3  # decode: not built
    # the forward's lse output: bf16 prefill only
    assert L.sala_sparse_attn(ctypes.byref(dec), FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                              None) == 3
    f32 = S.sparse_desc(batch=1, n_q=128, n_heads=4, n_kv_heads=2, head_dim=128, dtype=torch.float32,
                        kv_len=128, kv_capacity=128, topk=3, n_local=2)
    assert L.sala_sparse_attn_backward(ctypes.byref(f32), *args, FAKE, need, None) == 3
    assert L.sala_workspace_bytes(S.OP_SPARSE_ATTN_BACKWARD, ctypes.byref(f32)) == ctypes.c_size_t(-1).value
    kneed = S.workspace_bytes(S.OP_KV_NORM_BACKWARD, d)
    assert kneed > 0
    assert L.sala_kv_norm_backward(ctypes.byref(d), FAKE, None, FAKE, None, None, FAKE, kneed, None) == 1
    assert L.sala_kv_norm_backward(ctypes.byref(d), FAKE, None, FAKE, FAKE, None, FAKE, kneed - 1, None) == 4


def test_varlen_arguments():
    """Argument errors of the packed variable-length entry points (no device work): the host
    arrays must describe the packed tokens, sparse positions must start a block and fit the
    cache, bf16 / d = 128 only, at most SALA_VARLEN_MAX_SEQS sequences."""
    import torch

    from hybrid_sparse_linear_causal_amd import sala as S

    L = S.lib()
    vl = S.Varlen([100, 0, 300], [0, 5, 64])
    d = S.LinearDesc(3, 400, 4, 4, 128, S.SALA_BF16, 0, 10000.0, 1e-6)
    need = S.varlen_workspace_bytes(S.OP_LINEAR_PREFILL, d, vl)
    assert need > 0
    # q k v gate | qw kw state_in state_out | out
    args = [FAKE] * 4 + [None, None, None, None] + [FAKE]
    assert L.sala_linear_prefill_varlen(ctypes.byref(d), *vl.args(), *args, FAKE, need - 1, None) == 4
    assert L.sala_linear_prefill_varlen(ctypes.byref(d), None, vl.args()[1], *args, FAKE, need, None) == 1
    bad = S.LinearDesc(3, 399, 4, 4, 128, S.SALA_BF16, 0, 10000.0, 1e-6)  # packed count != cu_seqlens[3]
    assert L.sala_linear_prefill_varlen(ctypes.byref(bad), *vl.args(), *args, FAKE, need, None) == 2
    f32 = S.LinearDesc(3, 400, 4, 4, 128, S.SALA_F32, 0, 10000.0, 1e-6)
    assert L.sala_linear_prefill_varlen(ctypes.byref(f32), *vl.args(), *args, FAKE, need, None) == 3
    down = S.Varlen([100, 300, 0], [0, 0, 0])
    down._cu[2], down._cu[3] = 50, 400  # cu_seqlens not nondecreasing
    assert L.sala_linear_prefill_varlen(ctypes.byref(d), *down.args(), *args, FAKE, need, None) == 2
    many = S.Varlen([1] * 65)
    dm = S.LinearDesc(65, 65, 4, 4, 128, S.SALA_BF16, 0, 10000.0, 1e-6)
    assert L.sala_linear_prefill_varlen(ctypes.byref(dm), *many.args(), *args, FAKE, 1 << 30, None) == 3

    svl = S.Varlen([100, 0, 300], [64, 0, 128])
    sd = S.sparse_desc(batch=3, n_q=400, n_heads=4, n_kv_heads=2, head_dim=128, dtype=torch.bfloat16, kv_len=0,
                       kv_capacity=512, topk=3, n_local=2)
    assert S.Varlen([100, 0, 300]).query_blocks() == 2 + 0 + 5
    sneed = S.varlen_workspace_bytes(S.OP_BLOCK_SELECT, sd, svl)
    assert sneed > 0 and S.varlen_workspace_bytes(S.OP_SPARSE_ATTN, sd, svl) == 0
    assert L.sala_block_select_varlen(ctypes.byref(sd), *svl.args(), FAKE, None, FAKE, FAKE, FAKE, sneed - 1,
                                      None) == 4
    assert L.sala_block_select_varlen(ctypes.byref(sd), *svl.args(), FAKE, None, FAKE, None, FAKE, sneed,
                                      None) == 1
    unaligned = S.Varlen([100, 0, 300], [64, 0, 100])  # a query start inside a block
    assert L.sala_sparse_attn_varlen(ctypes.byref(sd), *unaligned.args(), FAKE, None, FAKE, FAKE, FAKE, FAKE,
                                     FAKE, None) == 2
    over = S.Varlen([100, 0, 300], [64, 0, 256])  # 256 + 300 > capacity 512
    assert L.sala_kv_append_varlen(ctypes.byref(sd), *over.args(), FAKE, FAKE, None, FAKE, FAKE, FAKE, None) == 2
    assert L.sala_sparse_attn_varlen(ctypes.byref(sd), *svl.args(), FAKE, None, FAKE, FAKE, FAKE, None, FAKE,
                                     None) == 1
    sf = S.sparse_desc(batch=3, n_q=400, n_heads=4, n_kv_heads=2, head_dim=128, dtype=torch.float32, kv_len=0,
                       kv_capacity=512, topk=3, n_local=2)
    assert L.sala_kv_append_varlen(ctypes.byref(sf), *svl.args(), FAKE, FAKE, None, FAKE, FAKE, FAKE, None) == 3


def test_decode_at_arguments():
    """Argument errors of the decode calls with per-sequence positions (no device work)."""
    import torch

    from hybrid_sparse_linear_causal_amd import sala as S

    L = S.lib()
    d = S.LinearDesc(4, 1, 2, 2, 128, S.SALA_BF16, 0, 10000.0, 1e-6)
    args = [FAKE] * 4 + [None, None] + [FAKE, FAKE]  # q k v gate | qw kw | state out
    assert L.sala_linear_decode_step_at(ctypes.byref(d), None, *args, None) == 1
    two = S.LinearDesc(4, 2, 2, 2, 128, S.SALA_BF16, 0, 10000.0, 1e-6)
    assert L.sala_linear_decode_step_at(ctypes.byref(two), FAKE, *args, None) == 2  # one token per sequence
    sd = S.sparse_desc(batch=3, n_q=1, n_heads=8, n_kv_heads=2, head_dim=128, dtype=torch.bfloat16, kv_len=3000,
                       kv_capacity=3072, topk=16, n_local=2)
    need = S.workspace_bytes(S.OP_SPARSE_DECODE_STEP, sd)
    assert need > 0
    # q qw k_new v_new kw gate | k_cache v_cache k_pool sel out
    sargs = [FAKE, None, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE]
    assert L.sala_sparse_decode_step(ctypes.byref(sd), FAKE, *sargs, FAKE, need - 1, None) == 4
    assert L.sala_sparse_decode_step(ctypes.byref(sd), None, *sargs, FAKE, need, None) == 1
    pre = S.sparse_desc(batch=3, n_q=64, n_heads=8, n_kv_heads=2, head_dim=128, dtype=torch.bfloat16, kv_len=3000,
                        kv_capacity=3072, topk=16, n_local=2)
    assert L.sala_sparse_decode_step(ctypes.byref(pre), FAKE, *sargs, FAKE, need, None) == 2
    wide = S.sparse_desc(batch=3, n_q=1, n_heads=64, n_kv_heads=2, head_dim=128, dtype=torch.bfloat16, kv_len=3000,
                         kv_capacity=3072, topk=16, n_local=2)  # 32 query heads per KV head
    assert L.sala_sparse_decode_step(ctypes.byref(wide), FAKE, *sargs, FAKE, need, None) == 3
    # the variant without workspace: the same argument errors, and calls needing more scratch than
    # its static array (8 MiB) are refused before any device call
    assert L.sala_sparse_decode_step_noalloc(ctypes.byref(sd), None, *sargs, None) == 1
    assert L.sala_sparse_decode_step_noalloc(ctypes.byref(pre), FAKE, *sargs, None) == 2
    assert L.sala_sparse_decode_step_noalloc(ctypes.byref(wide), FAKE, *sargs, None) == 3
    big = S.sparse_desc(batch=64, n_q=1, n_heads=32, n_kv_heads=2, head_dim=128, dtype=torch.bfloat16,
                        kv_len=1 << 20, kv_capacity=1 << 20, topk=64, n_local=2)
    assert S.workspace_bytes(S.OP_SPARSE_DECODE_STEP, big) > (8 << 20)
    assert L.sala_sparse_decode_step_noalloc(ctypes.byref(big), FAKE, *sargs, None) == 4
    huge = S.sparse_desc(batch=1, n_q=1, n_heads=8, n_kv_heads=2, head_dim=128, dtype=torch.bfloat16,
                         kv_len=64 * 20000, kv_capacity=64 * 20000, topk=16, n_local=2)  # beyond 16,384 blocks
    assert S.lib().sala_workspace_bytes(S.OP_SPARSE_DECODE_STEP, ctypes.byref(huge)) == ctypes.c_size_t(-1).value
