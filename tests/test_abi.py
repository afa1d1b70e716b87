"""CPU-side tests of the C ABI: the library loads, exports every symbol the
header declares, rejects invalid arguments before touching the GPU, and its
integer plan matches the oracle's bit for bit. No compute call runs here."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from depth_wise_attention_rms_amd import binding as b
from depth_wise_attention_rms_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attnres.h")

FAKE = ctypes.c_void_p(0x10000)     # aligned, never dereferenced: validation fails first
MISALIGNED = ctypes.c_void_p(0x10008)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"\b(attnres_[a-z0-9_]+)\s*\(", text))
    names.discard("attnres_sublayer_fn")
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("attnres_aggregate", "attnres_phase1_batched", "attnres_phase2_merge",
                     "attnres_block_stack_forward"):
        assert required in names


def test_library_exports_every_declared_symbol():
    L = b.lib()
    for name in declared_functions():
        assert hasattr(L, name), f"libattnres.so does not export {name}"
    assert set(declared_functions()) == set(b.EXPORTS)


def test_inputs_library_loads():
    L = inputs.lib()
    for name in ("attnres_inputs_fill_normal", "attnres_inputs_gather_rows",
                 "attnres_inputs_ring_sublayer", "attnres_inputs_record_sublayer"):
        assert hasattr(L, name)


def _last():
    return b.lib().attnres_last_error().decode()


def _agg(n=2, R=4, D=16, dt=1, w=FAKE, out=FAKE, eps=1e-8, srcs=None, m=None, lse=None):
    arr = (ctypes.c_void_p * max(n, 1))(*([0x20000 + 0x1000 * i for i in range(max(n, 1))] if srcs is None else srcs))
    return b.lib().attnres_aggregate(arr, n, R, D, dt, w, None, eps, out, m, lse, None)


@pytest.mark.parametrize("kwargs,code,msg", [
    (dict(n=0), -1, "n = 0"),
    (dict(n=65), -1, "n = 65"),
    (dict(R=-1), -1, "R = -1"),
    (dict(D=12), -1, "D = 12"),
    (dict(D=4, dt=1), -1, "D = 4"),
    (dict(dt=7), -1, "dtype"),
    (dict(w=None), -1, "w is NULL"),
    (dict(out=None), -1, "out is NULL"),
    (dict(out=MISALIGNED), -1, "not 16-byte aligned"),
    (dict(eps=-1.0), -1, "eps"),
    (dict(eps=float("nan")), -1, "eps"),
    (dict(D=16384 + 8), -2, "exceeds"),
    (dict(srcs=[0x20000, 0x20008]), -1, "not 16-byte aligned"),
    (dict(srcs=[0x20000, 0x10000]), -1, "aliases"),
    (dict(m=MISALIGNED), -1, "m_out"),
])
def test_aggregate_rejects_invalid_arguments(kwargs, code, msg):
    assert _agg(**kwargs) == code
    assert msg in _last()


def test_zero_rows_is_a_successful_noop():
    assert _agg(R=0) == 0
    assert b.lib().attnres_phase2_merge(FAKE, FAKE, FAKE, None, 1e-8, None, ctypes.c_void_p(0x50000),
                                        None, ctypes.c_void_p(0x60000), 0, 16, 1, None) == 0


def test_phase1_rejects_invalid_arguments():
    L = b.lib()
    arr = (ctypes.c_void_p * 2)(0x20000, 0x30000)
    assert L.attnres_phase1_batched(arr, 2, 4, 16, 1, FAKE, None, 0, 1e-8, FAKE, None, FAKE, None) == -1
    assert "S = 0" in _last()
    assert L.attnres_phase1_batched(arr, 2, 4, 16, 1, FAKE, None, 3, 1e-8, FAKE, None, None, None) == -1
    assert "lse_out is NULL" in _last()


def test_phase2_rejects_invalid_arguments():
    L = b.lib()
    f = L.attnres_phase2_merge
    # p_out required when p_prev is given
    assert f(FAKE, FAKE, FAKE, None, 1e-8, ctypes.c_void_p(0x50000), FAKE, None,
             ctypes.c_void_p(0x60000), 4, 16, 1, None) == -1
    assert "p_out is NULL" in _last()
    # p_out must be NULL on the first merge
    assert f(FAKE, FAKE, FAKE, None, 1e-8, None, ctypes.c_void_p(0x50000), ctypes.c_void_p(0x70000),
             ctypes.c_void_p(0x60000), 4, 16, 1, None) == -1
    # h_out may not alias an input
    assert f(FAKE, FAKE, FAKE, None, 1e-8, None, ctypes.c_void_p(0x50000), None, FAKE, 4, 16, 1, None) == -1
    assert "aliases" in _last()


def test_stack_rejects_invalid_arguments():
    L = b.lib()
    fn = ctypes.cast(L.attnres_table_sublayer, ctypes.c_void_p)
    ws_need = L.attnres_stack_workspace_bytes(8, 4, 4, 16, 1)
    bs = (ctypes.c_void_p * 2)(0x80000, 0x90000)
    ws = ctypes.c_void_p(0x100000)

    def call(Lr=8, S=4, block_sums=bs, ws_bytes=ws_need, workspace=ws, f=fn):
        return L.attnres_block_stack_forward(FAKE, Lr, S, 4, 16, 1, FAKE, None, 1e-8, f, None,
                                             block_sums, ctypes.c_void_p(0xA0000), workspace,
                                             ws_bytes, None)
    assert call(S=0) == -1
    assert call(Lr=0) == -1
    assert call(block_sums=None) == -1 and "block_sums" in _last()
    assert call(ws_bytes=ws_need - 1) == -3
    assert call(workspace=ctypes.c_void_p(0x100010)) == -1 and "256-byte" in _last()
    assert call(f=None) == -1
    assert call(Lr=64, S=1, block_sums=None) == -1 and "exceed" in _last()


def test_status_strings():
    L = b.lib()
    for code in (0, -1, -2, -3, -4, -5):
        assert L.attnres_status_string(code).decode() != "unknown status"


def test_plan_matches_oracle_bit_exactly():
    for L in range(1, 40):
        for S in range(1, L + 3):
            nb, starts, ns = b.attnres_block_layout(L, S)
            onb, ostarts, ons = oracle.block_plan(L, S)
            assert nb == onb and starts == list(ostarts) and ns == list(ons), (L, S)
    for Ldec in range(1, 200):
        for per in (None, 1, 2, 3, 12):
            assert b.attnres_atomic_block_size(Ldec, per) == oracle.atomic_block_size(Ldec, per)


def test_workspace_bytes_cover_the_regions():
    L = b.lib()
    R, D = 16384, 4096
    ws = L.attnres_stack_workspace_bytes(48, 8, R, D, 1)
    row = R * D * 2
    assert ws >= 8 * row + row + row + 49 * D * 4 + 2 * 8 * R * 4
    assert L.attnres_stack_workspace_bytes(0, 8, R, D, 1) == 0
    assert L.attnres_stack_workspace_bytes(16, 1, 2048, 1024, 1) >= 2048 * 1024 * 2


def _a256(x):
    return (x + 255) // 256 * 256


@pytest.mark.parametrize("L_,S,R,D,dt,ast", [
    (186, 24, 131072, 7168, 1, 8),       # long context: the matrix-core scores pass, 8 blocks
    (96, 12, 128, 7168, 1, 0),           # decode: too few rows, streamed Phase 1
    (48, 8, 16384, 4096, 1, 0),          # register-tile Phase 1
    (72, 8, 8192, 4096, 1, 16),          # 9 blocks: the last Phase 1 has 9 sources
    (40, 4, 4096, 1024, 1, 16),          # 10 blocks
    (40, 3, 4096, 1024, 1, 0),           # 14 blocks of 3 queries: register tile up to 8 sources, streamed beyond
    (20, 9, 4096, 4096, 1, 8),           # 9 queries at D = 4096
    (20, 9, 4096, 4096, 0, 0),           # fp32 never takes it
    (20, 9, 4096, 4000, 1, 0),           # D not a multiple of 256
    (40, 33, 8192, 1024, 1, 0),          # more than 32 queries
])
def test_workspace_bytes_layout(L_, S, R, D, dt, ast):
    """The stack workspace is the 256-byte-aligned regions the header lists:
    folded queries, one block's Phase-1 outputs and statistics, the partial,
    h, and -- where some block takes the matrix-core scores pass -- the query
    parts [32 ceil(S/8), D] bf16 and the weights [S, R, ast] fp32 (ast = 16
    when a Phase 1 has more than 8 sources)."""
    es = 2 if dt == 1 else 4
    Sk = min(S, L_)
    row = R * D * es
    want = _a256((L_ + 1) * D * 4) + _a256(Sk * row if Sk > 1 else 0) + 2 * _a256(Sk * R * 4)
    want += _a256(row if Sk > 2 else 0) + _a256(row)
    if ast:
        want += _a256(_a256(32 * ((Sk + 7) // 8) * D * 2) + Sk * R * ast * 4)
    assert b.lib().attnres_stack_workspace_bytes(L_, S, R, D, dt) == want


@pytest.mark.parametrize("L_,C,R,D,dt,ast", [
    (16, 4, 16384, 4096, 1, 16),   # chunks over 1, 5, 9 and 13 sources: the last two take the scores pass
    (16, 4, 2048, 1024, 1, 0),     # too few rows
    (8, 4, 16384, 4096, 1, 0),     # chunks over 1 and 5 sources: the register-tile Phase 1
    (12, 3, 8192, 7168, 1, 8),     # D = 7168: chunks of up to 8 sources; 10 with 3 queries stay streamed
    (17, 4, 4096, 1024, 1, 16),    # the last chunk has one sublayer: no Phase 1 over 17 sources
    (16, 1, 16384, 4096, 1, 0),    # the naive schedule
])
def test_full_workspace_bytes_layout(L_, C, R, D, dt, ast):
    """The Full workspace: folded queries, one chunk's Phase-1 outputs and
    statistics, h and -- where some chunk takes the scores pass -- its query
    parts and weights [C, R, ast] fp32."""
    es = 2 if dt == 1 else 4
    Ck = min(C, L_)
    row = R * D * es
    want = _a256((L_ + 1) * D * 4) + _a256(Ck * row if Ck > 1 else 0) + 2 * _a256(Ck * R * 4) + _a256(row)
    if ast:
        want += _a256(_a256(32 * ((Ck + 7) // 8) * D * 2) + Ck * R * ast * 4)
    assert b.lib().attnres_full_workspace_bytes(L_, C, R, D, dt) == want


def test_generator_twin_rounding_and_distribution():
    # bf16 rounding of the twin equals torch's nearest-even fp32 -> bf16 for fp32 values
    import torch
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(20000) * 7).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(inputs.bf16_bits(x.astype(np.float64)), ref)
    z = inputs.normal(0, inputs.ROLE_V, 3, np.arange(400000))
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01
    u = inputs.uniform(0, inputs.ROLE_SCALE, 0, np.arange(100000))
    assert u.min() >= 0 and u.max() < 1 and abs(u.mean() - 0.5) < 0.01
    # distinct streams differ, the same stream repeats
    assert not np.array_equal(inputs.normal(0, 2, 1, np.arange(10)), inputs.normal(0, 2, 2, np.arange(10)))
    assert np.array_equal(inputs.normal(5, 2, 1, np.arange(10)), inputs.normal(5, 2, 1, np.arange(10)))


def test_noalloc_backward_validates_on_the_host():
    """The no-allocation backward checks its arguments and its scratch limit
    before it looks up any device."""
    L = b.lib()
    assert L.attnres_noalloc_scratch_bytes() == 33 << 20
    src = (ctypes.c_void_p * 1)(0x20000)
    dv = (ctypes.c_void_p * 1)(0x40000)
    # a bf16 row of 8200 elements needs more scratch than the fixed array holds
    rc = L.attnres_aggregate_backward_noalloc(src, 1, 4096, 8200, 1, FAKE, None, 1e-8, ctypes.c_void_p(0x30000),
                                              dv, 0, ctypes.c_void_p(0x50000), None, None)
    assert rc == -2 and "scratch" in _last()
    assert b.lib().attnres_aggregate_backward_workspace_bytes(4096, 8200, 1) > (33 << 20)
    assert b.lib().attnres_aggregate_backward_workspace_bytes(1 << 27, 8192, 1) <= (33 << 20)
    assert b.lib().attnres_aggregate_backward_workspace_bytes(1 << 27, 8192, 0) <= (33 << 20)
    rc = L.attnres_aggregate_backward_noalloc(src, 0, 64, 1024, 1, FAKE, None, 1e-8, ctypes.c_void_p(0x30000),
                                              dv, 0, ctypes.c_void_p(0x50000), None, None)
    assert rc == -1 and "n = 0" in _last()
    rc = L.attnres_aggregate_backward_noalloc(src, 1, 64, 1024, 1, FAKE, None, 1e-8, ctypes.c_void_p(0x30000),
                                              dv, 0, None, None, None)
    assert rc == -1 and "dw is NULL" in _last()


@pytest.mark.parametrize("L_,S,R,D,dt", [(48, 8, 16384, 4096, 1), (20, 6, 600, 2048, 1), (13, 5, 65, 1024, 0),
                                         (30, 7, 90, 1000, 1), (64, 8, 50, 1000, 1), (9, 4, 2100, 2048, 1)])
def test_stack_backward_workspace_holds_a_slot_per_merge(L_, S, R, D, dt):
    """The stack backward reduces a block's merge-backward query gradients
    together, each merge's dq~ partial rows in a slot the size of one
    aggregate backward's workspace: beyond the recomputed Phase-1 outputs
    (min(S, L) rows of [R, D]) the workspace holds min(S, L) - 1 such slots."""
    lib = b.lib()
    slot = lib.attnres_aggregate_backward_workspace_bytes(R, D, dt)
    total = lib.attnres_stack_backward_workspace_bytes(L_, S, R, D, dt)
    sk = min(S, L_)
    assert slot > 0 and total % 256 == 0
    assert total >= (sk - 1) * slot + sk * R * D * (2 if dt == 1 else 4)
