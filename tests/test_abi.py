"""C-ABI checks that need no GPU: exports, host-only queries, table export, argument validation.

No call here reaches a kernel launch: every call either is host-only or fails
validation first (fake pointers are only ever passed to calls that are
rejected for another argument), or is a documented no-op (N == 0, B*H == 0).
"""

import ctypes
import math
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
import recurrent_state_amd as rs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "taylor_attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(rs.LIB_PATH), reason="library not built")


def _header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?(taylor_[a-z_0-9]+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported():
    declared = _header_functions()
    assert len(declared) == 18
    assert sorted(rs.EXPORTS) == declared
    out = subprocess.run(["nm", "-D", "--defined-only", rs.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(taylor_[a-z_0-9]+)$", out, re.M))
    assert set(declared) <= exported
    L = rs.lib()
    for name in declared:
        assert getattr(L, name) is not None


def test_status_strings():
    for st in (0, -1, -2, -3):
        assert rs.taylor_status_string(st).startswith("TAYLOR_")
    assert "unknown" in rs.taylor_status_string(7)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("d", [1, 2, 4, 16])
def test_feature_width(n, d):
    assert rs.taylor_feature_width(n, d) == sum(math.comb(d + m - 1, m) for m in range(n))


def test_feature_width_rejects():
    L = rs.lib()
    assert L.taylor_feature_width(0, 16) == rs.TAYLOR_ERR_INVALID_ARG
    assert L.taylor_feature_width(3, 0) == rs.TAYLOR_ERR_INVALID_ARG
    assert L.taylor_feature_width(40, 4096) == rs.TAYLOR_ERR_INVALID_ARG  # overflows int


def test_state_size_and_stride():
    cfg = rs.config(3, 16, 64)
    assert rs.taylor_state_elems(cfg) == 9945  # the Abstract's elements per head
    assert rs.taylor_state_stride(cfg) == 9948
    assert rs.taylor_state_stride(rs.config(3, 4, 4)) == 76
    for n in range(1, 6):
        c = rs.config(n, 16, 64)
        assert rs.taylor_state_stride(c) % 4 == 0 and rs.taylor_state_stride(c) >= rs.taylor_state_elems(c)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("d", [1, 2, 3, 4, 8, 16])
def test_monomial_table_bit_exact_against_oracle(n, d):
    idx, coef = rs.taylor_monomial_table(n, d)
    assert np.array_equal(idx, oracle.index_table(n, d))
    ref = oracle.coef_table(n, d)
    assert coef.dtype == np.float64
    assert np.array_equal(coef.view(np.uint64), ref.view(np.uint64))


def test_monomial_table_capacity_checked():
    L = rs.lib()
    idx = np.full((200, 2), 7, dtype=np.int32)
    assert L.taylor_monomial_table(3, 16, idx.ctypes.data, None, 152) == rs.TAYLOR_ERR_INVALID_ARG
    assert np.all(idx == 7)  # nothing written
    assert L.taylor_monomial_table(3, 16, idx.ctypes.data, None, 153) == 153
    assert L.taylor_monomial_table(6, 16, idx.ctypes.data, None, 200) == rs.TAYLOR_ERR_INVALID_ARG


def test_supported_configs():
    for n in range(1, 6):
        for dt in (rs.TAYLOR_F32, rs.TAYLOR_BF16):
            for C in (0, 64, 128):
                assert rs.taylor_supported(rs.config(n, 16, 64, C, 1.0, dt)) == rs.TAYLOR_OK
                assert rs.taylor_supported(rs.config(n, 4, 4, C, 1.0, dt)) == rs.TAYLOR_OK
    assert rs.taylor_supported(rs.config(3, 16, 64, 96)) == rs.TAYLOR_ERR_UNSUPPORTED
    assert rs.taylor_supported(rs.config(3, 16, 6)) == rs.TAYLOR_ERR_UNSUPPORTED
    assert rs.taylor_supported(rs.config(6, 16, 64)) == rs.TAYLOR_ERR_UNSUPPORTED
    assert rs.taylor_supported(rs.config(3, 5, 64)) == rs.TAYLOR_ERR_UNSUPPORTED
    assert rs.taylor_supported(rs.config(0, 16, 64)) == rs.TAYLOR_ERR_INVALID_ARG
    assert rs.taylor_supported(rs.config(3, 16, 64, -1)) == rs.TAYLOR_ERR_INVALID_ARG
    assert rs.taylor_supported(rs.config(3, 16, 64, 0, float("nan"))) == rs.TAYLOR_ERR_INVALID_ARG
    assert rs.taylor_supported(rs.config(3, 16, 64, 0, 1.0, 5)) == rs.TAYLOR_ERR_INVALID_ARG
    assert rs.lib().taylor_supported(None) == rs.TAYLOR_ERR_INVALID_ARG


def test_workspace_bytes():
    cfg = rs.config(3, 16, 64, 64)
    assert rs.taylor_prefill_workspace_bytes(cfg, 1, 8, 0) == 0
    assert rs.taylor_prefill_workspace_bytes(cfg, 0, 8, 4096) == 0
    assert rs.taylor_prefill_workspace_bytes(cfg, 1, 8, 4096) > 0
    L = rs.lib()
    assert L.taylor_prefill_workspace_bytes(ctypes.byref(cfg), -1, 8, 64) == rs.TAYLOR_ERR_INVALID_ARG
    assert L.taylor_prefill_workspace_bytes(ctypes.byref(cfg), 1, 8, -5) == rs.TAYLOR_ERR_INVALID_ARG
    assert L.taylor_prefill_workspace_bytes(ctypes.byref(cfg), 300, 300, 64) == rs.TAYLOR_ERR_UNSUPPORTED


FAKE = 1 << 20  # an aligned address; only ever passed to calls rejected for another reason
MIS = FAKE + 4  # misaligned


def _prefill(q, k, v, o, st, ws, B, H, N, cfg):
    return rs.lib().taylor_attn_prefill(q, k, v, o, st, ws, B, H, N, ctypes.byref(cfg) if cfg else None, None)


def test_prefill_validation():
    cfg = rs.config(3, 16, 64, 64)
    E = rs.TAYLOR_ERR_INVALID_ARG
    assert _prefill(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, None) == E
    assert _prefill(FAKE, FAKE, FAKE, None, None, FAKE, 1, 1, 64, cfg) == E  # nothing to produce
    assert _prefill(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, -1, 1, 64, cfg) == E
    assert _prefill(FAKE, None, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, cfg) == E
    assert _prefill(FAKE, FAKE, None, FAKE, FAKE, FAKE, 1, 1, 64, cfg) == E
    assert _prefill(None, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, cfg) == E  # q needed for outputs
    assert _prefill(MIS, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, cfg) == E
    assert _prefill(FAKE, MIS, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, cfg) == E
    assert _prefill(FAKE, FAKE, FAKE, MIS, FAKE, FAKE, 1, 1, 64, cfg) == E
    assert _prefill(FAKE, FAKE, FAKE, FAKE, MIS, FAKE, 1, 1, 64, cfg) == E
    assert _prefill(FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 1, 64, cfg) == E  # workspace required
    assert _prefill(FAKE, FAKE, FAKE, FAKE, FAKE, MIS, 1, 1, 64, cfg) == E
    assert _prefill(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, rs.config(3, 16, 64, 96)) == rs.TAYLOR_ERR_UNSUPPORTED
    assert _prefill(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, rs.config(7, 16, 64)) == rs.TAYLOR_ERR_UNSUPPORTED
    # documented no-ops (no launch): N == 0, B*H == 0
    assert _prefill(FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 1, 0, cfg) == rs.TAYLOR_OK
    assert _prefill(FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 4, 64, cfg) == rs.TAYLOR_OK


def _into(q, k, v, o, sin, sout, ws, B, H, N, cfg):
    return rs.lib().taylor_attn_prefill_into(q, k, v, o, sin, sout, ws, B, H, N, ctypes.byref(cfg) if cfg else None,
                                             None)


def test_prefill_into_validation():
    cfg = rs.config(3, 16, 64, 64)
    E = rs.TAYLOR_ERR_INVALID_ARG
    stride_bytes = 4 * rs.taylor_state_stride(cfg)
    assert _into(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, None) == E
    assert _into(FAKE, FAKE, FAKE, None, FAKE, None, FAKE, 1, 1, 64, cfg) == E  # nothing to produce
    assert _into(FAKE, FAKE, FAKE, FAKE, MIS, FAKE, FAKE, 1, 1, 64, cfg) == E
    assert _into(FAKE, FAKE, FAKE, FAKE, FAKE, MIS, FAKE, 1, 1, 64, cfg) == E
    # the two state arrays must be the same array or disjoint (2 x 2 heads here)
    assert _into(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 16, FAKE, 2, 2, 64, cfg) == E
    assert _into(FAKE, FAKE, FAKE, FAKE, FAKE + 4 * stride_bytes - 16, FAKE, FAKE, 2, 2, 64, cfg) == E
    assert _into(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, -1, 1, 64, cfg) == E
    assert _into(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 1, 64, cfg) == E  # workspace required
    assert _into(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, rs.config(7, 16, 64)) == rs.TAYLOR_ERR_UNSUPPORTED
    # no launch: B*H == 0; N == 0 in place or with the final state discarded
    assert _into(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 4, 64, cfg) == rs.TAYLOR_OK
    assert _into(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 4, 0, cfg) == rs.TAYLOR_OK
    assert _into(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 1, 4, 0, cfg) == rs.TAYLOR_OK


def test_readout_field():
    # TAYLOR_READOUT_CENTERED: orders 1, 2 (n_terms 2, 3) at d_k = 16, d_v = 64, either input type
    C = rs.TAYLOR_READOUT_CENTERED
    for n in (2, 3):
        for dt in (rs.TAYLOR_F32, rs.TAYLOR_BF16):
            cfg = rs.config(n, 16, 64, 0, 1.0, dt, C)
            assert rs.taylor_supported(cfg) == rs.TAYLOR_OK
            assert rs.taylor_prefill_workspace_bytes(cfg, 4, 16, 8192) > 0
            assert rs.taylor_prefill_varlen_workspace_bytes(cfg, 8, 16, 4096, 10000) > 0
    for n in (1, 4, 5):
        assert rs.taylor_supported(rs.config(n, 16, 64, 0, 1.0, 0, C)) == rs.TAYLOR_ERR_UNSUPPORTED
    assert rs.taylor_supported(rs.config(3, 8, 32, 0, 1.0, 0, C)) == rs.TAYLOR_ERR_UNSUPPORTED
    assert rs.taylor_supported(rs.config(3, 16, 64, 0, 1.0, 0, 2)) == rs.TAYLOR_ERR_INVALID_ARG
    assert rs.taylor_supported(rs.config(3, 16, 64, 0, 1.0, 0, -1)) == rs.TAYLOR_ERR_INVALID_ARG
    # the state layout does not depend on the readout
    assert rs.taylor_state_stride(rs.config(3, 16, 64, 0, 1.0, 0, C)) == rs.taylor_state_stride(rs.config(3, 16, 64))
    L = rs.lib()
    bad = rs.config(3, 8, 32, 0, 1.0, 0, C)
    assert L.taylor_attn_decode_step(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, ctypes.byref(bad), None) == \
        rs.TAYLOR_ERR_UNSUPPORTED
    assert _prefill(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, bad) == rs.TAYLOR_ERR_UNSUPPORTED


def test_varlen_workspace_bytes():
    cfg = rs.config(3, 16, 64, 64, 1.0, rs.TAYLOR_BF16)
    assert rs.taylor_prefill_varlen_workspace_bytes(cfg, 8, 16, 4096, 0) == 0
    assert rs.taylor_prefill_varlen_workspace_bytes(cfg, 0, 16, 4096, 0) == 0
    assert rs.taylor_prefill_varlen_workspace_bytes(cfg, 8, 16, 4096, 10000) > 0
    for n, dt in ((1, rs.TAYLOR_F32), (3, rs.TAYLOR_F32), (4, rs.TAYLOR_BF16), (5, rs.TAYLOR_F32)):
        assert rs.taylor_prefill_varlen_workspace_bytes(rs.config(n, 16, 64, 0, 1.0, dt), 8, 16, 4096, 10000) > 0
    L = rs.lib()

    def q(c, *a):
        return L.taylor_prefill_varlen_workspace_bytes(ctypes.byref(c) if c else None, *a)

    E = rs.TAYLOR_ERR_INVALID_ARG
    assert q(None, 8, 16, 4096, 100) == E
    assert q(cfg, -1, 16, 4096, 100) == E
    assert q(cfg, 8, -1, 4096, 100) == E
    assert q(cfg, 8, 16, -1, 100) == E
    assert q(cfg, 8, 16, 4096, -1) == E
    assert q(cfg, 8, 16, 100, 801) == E  # more tokens than n_seqs * max_seqlen
    assert q(cfg, 300, 300, 64, 100) == rs.TAYLOR_ERR_UNSUPPORTED  # too many (sequence, head) pairs
    # ragged batches run on the d_k = 16, d_v = 64 kernels only
    assert q(rs.config(3, 8, 32, 64), 8, 16, 4096, 100) == rs.TAYLOR_ERR_UNSUPPORTED
    assert q(rs.config(3, 4, 4, 64), 8, 16, 4096, 100) == rs.TAYLOR_ERR_UNSUPPORTED


def _varlen(q, k, v, o, st, ws, cu, n_seqs, H, N, T, cfg):
    return rs.lib().taylor_attn_prefill_varlen(q, k, v, o, st, ws, cu, n_seqs, H, N, T,
                                               ctypes.byref(cfg) if cfg else None, None)


def test_varlen_into_validation():
    cfg = rs.config(3, 16, 64, 64, 1.0, rs.TAYLOR_BF16)
    E = rs.TAYLOR_ERR_INVALID_ARG
    L = rs.lib()

    def call(o, sin, sout, ws, cu, n_seqs, H, N, T):
        return L.taylor_attn_prefill_varlen_into(FAKE, FAKE, FAKE, o, sin, sout, ws, cu, n_seqs, H, N, T,
                                                 ctypes.byref(cfg), None)

    assert call(None, FAKE, None, FAKE, FAKE, 4, 2, 100, 300) == E  # nothing to produce
    assert call(FAKE, MIS, FAKE, FAKE, FAKE, 4, 2, 100, 300) == E
    assert call(FAKE, FAKE, FAKE + 16, FAKE, FAKE, 4, 2, 100, 300) == E  # overlapping state arrays
    assert call(FAKE, FAKE, FAKE, FAKE, None, 4, 2, 100, 300) == E  # offsets required
    assert call(FAKE, FAKE, FAKE, FAKE, FAKE + 2, 4, 2, 100, 300) == E
    assert call(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 2, 100, 401) == E  # more tokens than n_seqs * max_seqlen
    assert call(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 2, 100, 0) == rs.TAYLOR_OK  # no rows
    assert call(FAKE, FAKE, FAKE, None, None, 4, 2, 100, 0) == rs.TAYLOR_OK  # in place, no tokens


def test_varlen_validation():
    cfg = rs.config(3, 16, 64, 64, 1.0, rs.TAYLOR_BF16)
    E = rs.TAYLOR_ERR_INVALID_ARG
    ok = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 2, 100, 300)
    assert _varlen(*ok, None) == E
    assert _varlen(FAKE, FAKE, FAKE, None, None, FAKE, FAKE, 4, 2, 100, 300, cfg) == E  # nothing to produce
    for i in range(7):
        args = list(ok)
        args[i] = MIS if i < 6 else FAKE + 2  # cu_seqlens needs 4-byte alignment only
        if i == 4 or i == 3:
            continue  # misaligned o / state checked below with the other argument present
        assert _varlen(*args, cfg) == E, i
    for i in (0, 1, 2, 6):  # q (outputs wanted), k, v, cu_seqlens
        args = list(ok)
        args[i] = None
        assert _varlen(*args, cfg) == E, i
    assert _varlen(FAKE, FAKE, FAKE, MIS, FAKE, FAKE, FAKE, 4, 2, 100, 300, cfg) == E
    assert _varlen(FAKE, FAKE, FAKE, FAKE, MIS, FAKE, FAKE, 4, 2, 100, 300, cfg) == E
    assert _varlen(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 4, 2, 100, 300, cfg) == E  # workspace required
    assert _varlen(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 2, 100, 401, cfg) == E  # T > n_seqs * max
    assert _varlen(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, -4, 2, 100, 300, cfg) == E
    assert _varlen(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 2, 100, -3, cfg) == E
    assert _varlen(*ok, rs.config(3, 8, 32, 64)) == rs.TAYLOR_ERR_UNSUPPORTED
    assert _varlen(*ok, rs.config(7, 16, 64)) == rs.TAYLOR_ERR_UNSUPPORTED
    # documented no-ops (no launch): no tokens, no pairs
    assert _varlen(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 4, 2, 100, 0, cfg) == rs.TAYLOR_OK
    assert _varlen(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, 2, 100, 0, cfg) == rs.TAYLOR_OK
    assert _varlen(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 4, 0, 100, 300, cfg) == rs.TAYLOR_OK


def test_backward_queries_and_validation():
    L = rs.lib()
    for n in (1, 2, 3, 4, 5):
        for dt in (rs.TAYLOR_F32, rs.TAYLOR_BF16):
            assert rs.taylor_prefill_backward_workspace_bytes(rs.config(n, 16, 64, 0, 1.0, dt), 4, 16, 8192) > 0
    # n = 4, 5: gh and delta (68 floats) plus per feature block a den, 16 dq / dk and 64 dv floats per token
    for n, blocks in ((4, 16), (5, 38)):
        assert rs.taylor_prefill_backward_workspace_bytes(rs.config(n, 16, 64), 2, 3, 100) == 600 * 4 * (68 + 81 * blocks)
    cfg = rs.config(3, 16, 64)
    assert rs.taylor_prefill_backward_workspace_bytes(cfg, 0, 16, 8192) == 0
    assert rs.taylor_prefill_backward_workspace_bytes(cfg, 4, 16, 0) == 0
    U = rs.TAYLOR_ERR_UNSUPPORTED
    E = rs.TAYLOR_ERR_INVALID_ARG

    def wsb(c, B=1, H=1, N=64):
        return L.taylor_prefill_backward_workspace_bytes(ctypes.byref(c) if c else None, B, H, N)

    assert wsb(rs.config(6, 16, 64)) == U
    assert wsb(rs.config(3, 8, 32)) == U
    assert wsb(rs.config(3, 16, 64, 0, 1.0, 0, rs.TAYLOR_READOUT_CENTERED)) == U
    assert wsb(None) == E
    assert wsb(cfg, -1) == E

    def bwd(args, B=1, H=1, N=64, c=cfg):
        return L.taylor_attn_prefill_backward(*args, B, H, N, ctypes.byref(c) if c else None, None)

    ok = [FAKE] * 11  # q k v o g state dstate dq dk dv ws
    for i in (0, 1, 2, 3, 4, 7, 8, 9):  # required pointers
        a = list(ok)
        a[i] = None
        assert bwd(a) == E, i
        a[i] = MIS
        assert bwd(a) == E, i
    for i in (5, 6, 10):  # optional, but aligned when given
        a = list(ok)
        a[i] = MIS
        assert bwd(a) == E, i
    a = list(ok)
    a[10] = None
    assert bwd(a) == E  # workspace required
    assert bwd(ok, c=None) == E
    assert bwd(ok, c=rs.config(6, 16, 64)) == U
    assert bwd(ok, c=rs.config(3, 16, 64, 0, 1.0, 0, rs.TAYLOR_READOUT_CENTERED)) == U
    assert bwd(ok, c=rs.config(4, 8, 32)) == U
    # documented no-ops: no pairs, no tokens
    assert bwd([None] * 11, B=0) == rs.TAYLOR_OK
    assert bwd([None] * 11, N=0) == rs.TAYLOR_OK


def test_decode_validation():
    cfg = rs.config(3, 16, 64)
    L = rs.lib()
    E = rs.TAYLOR_ERR_INVALID_ARG

    def dec(q, k, v, o, st, B, H, c=cfg):
        return L.taylor_attn_decode_step(q, k, v, o, st, B, H, ctypes.byref(c) if c else None, None)

    assert dec(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, None) == E
    for i in range(5):
        args = [FAKE] * 5
        args[i] = None
        assert dec(*args, 1, 1) == E
        args[i] = MIS
        assert dec(*args, 1, 1) == E
    assert dec(FAKE, FAKE, FAKE, FAKE, FAKE, -1, 1) == E
    assert dec(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, rs.config(3, 16, 60)) == rs.TAYLOR_ERR_UNSUPPORTED
    assert dec(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 16) == rs.TAYLOR_OK


def test_state_init_validation():
    L = rs.lib()
    cfg = rs.config(3, 16, 64)
    assert L.taylor_state_init(None, 1, 1, ctypes.byref(cfg), None) == rs.TAYLOR_ERR_INVALID_ARG
    assert L.taylor_state_init(MIS, 1, 1, ctypes.byref(cfg), None) == rs.TAYLOR_ERR_INVALID_ARG
    assert L.taylor_state_init(FAKE, 1, 1, None, None) == rs.TAYLOR_ERR_INVALID_ARG
    assert L.taylor_state_init(FAKE, -2, 1, ctypes.byref(cfg), None) == rs.TAYLOR_ERR_INVALID_ARG
    assert L.taylor_state_init(None, 0, 3, ctypes.byref(cfg), None) == rs.TAYLOR_OK


def test_prefill_chunk_is_what_the_kernels_walk():
    # the matrix-core kernels walk a fixed chunk whatever cfg.chunk asks; the portable ones honour it
    for chunk in (0, 64, 128):
        for n in (1, 2, 3):
            assert rs.taylor_prefill_chunk(rs.config(n, 16, 64, chunk, 1.0, rs.TAYLOR_BF16)) == 64
        for n in (1, 2, 3, 4, 5):
            assert rs.taylor_prefill_chunk(rs.config(n, 16, 64, chunk, 1.0, rs.TAYLOR_F32)) == 32
        for n in (4, 5):
            assert rs.taylor_prefill_chunk(rs.config(n, 16, 64, chunk, 1.0, rs.TAYLOR_BF16)) == 32
        assert rs.taylor_prefill_chunk(rs.config(3, 4, 4, chunk)) == (chunk or 64)
    L = rs.lib()
    assert L.taylor_prefill_chunk(ctypes.byref(rs.config(3, 16, 64, 96))) == rs.TAYLOR_ERR_UNSUPPORTED
    assert L.taylor_prefill_chunk(ctypes.byref(rs.config(0, 16, 64))) == rs.TAYLOR_ERR_INVALID_ARG


def test_static_workspace_variant_rejects_sizes_beyond_its_array():
    # the allocation-free prefill checks the workspace its sizes need against the static array before
    # any HIP call: float32 n = 5 over 16 heads of 16,384 tokens needs gigabytes
    L = rs.lib()
    cfg = rs.config(5, 16, 64, 0, 1.0, rs.TAYLOR_F32)
    assert rs.taylor_prefill_workspace_bytes(cfg, 1, 16, 16384) > (32 << 20)
    rc = L.taylor_attn_prefill_into_static(FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 16, 16384, ctypes.byref(cfg), None)
    assert rc == rs.TAYLOR_ERR_INVALID_ARG
    # the bf16 n = 3 benchmark shape fits, and so do 843 (sequence, head) pairs
    b3 = rs.config(3, 16, 64, 0, 1.0, rs.TAYLOR_BF16)
    assert rs.taylor_prefill_workspace_bytes(b3, 4, 16, 8192) <= (32 << 20)
    assert rs.taylor_prefill_workspace_bytes(b3, 1, 843, 8192) <= (32 << 20)
    # invalid configurations and sizes fail as in taylor_attn_prefill_into
    assert L.taylor_attn_prefill_into_static(FAKE, FAKE, FAKE, FAKE, None, FAKE, -1, 16, 64, ctypes.byref(b3),
                                             None) == rs.TAYLOR_ERR_INVALID_ARG
    assert L.taylor_attn_prefill_into_static(FAKE, FAKE, FAKE, FAKE, None, FAKE, 1, 1, 64, None,
                                             None) == rs.TAYLOR_ERR_INVALID_ARG
