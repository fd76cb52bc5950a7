"""CPU tests of the C-ABI library: it loads, exports every entry point the
header declares, and rejects bad arguments on the host before any launch
(no GPU needed: every case here fails validation, so nothing is enqueued)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ba.h")

lib_mod = pytest.importorskip("cached_split_attention_amd._lib")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(lib_mod.LIB_PATH):
        pytest.skip("libba.so not built")
    return lib_mod.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ba_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ("ba_prefix_attn", "ba_block_attn", "ba_lse_merge", "ba_reuse_gate", "ba_varlen_pack"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in ba.h but not exported"
        assert name in lib_mod.EXPORTS, f"{name} has no binding prototype"


def test_version(lib):
    assert lib.ba_version() >> 16 == 1


FAKE = 0x10000  # a non-NULL pointer value that is never dereferenced here


def good_desc():
    d = lib_mod.AttnDesc()
    d.dtype, d.n_seq, d.hq, d.hkv, d.d, d.max_q, d.max_k = 0, 1, 4, 2, 128, 32, 8192
    d.q = d.k = d.v = FAKE
    for i, s in enumerate((32 * 4 * 128, 4 * 128, 128)):
        d.q_stride[i] = s
    for i, s in enumerate((2 * 8192 * 128, 128, 8192 * 128)):
        d.k_stride[i] = s
        d.v_stride[i] = s
    return d


def status_of(lib, fn, *args):
    st = fn(*args)
    return st, lib.ba_last_error().decode()


@pytest.mark.parametrize("mutate,code,text", [
    (lambda d: setattr(d, "hkv", 3), 2, "multiple"),
    (lambda d: setattr(d, "d", 96), 4, "head dim"),
    (lambda d: setattr(d, "dtype", 7), 3, "dtype"),
    (lambda d: setattr(d, "max_q", -1), 2, "negative"),
    (lambda d: setattr(d, "q", None), 1, "q is NULL"),
    (lambda d: setattr(d, "cu_q", FAKE), 2, "cu_q and cu_k"),
    (lambda d: d.k_stride.__setitem__(1, 100), 4, "16 bytes"),
    (lambda d: setattr(d, "q", FAKE + 2), 4, "aligned"),
])
def test_prefix_validation(lib, mutate, code, text):
    d = good_desc()
    mutate(d)
    st, msg = status_of(lib, lib.ba_prefix_attn, ctypes.byref(d), FAKE, FAKE, None, 0, None)
    assert st == code and text in msg, (st, msg)


def test_prefix_null_desc_and_outputs(lib):
    st, msg = status_of(lib, lib.ba_prefix_attn, None, FAKE, FAKE, None, 0, None)
    assert st == 1
    d = good_desc()
    st, msg = status_of(lib, lib.ba_prefix_attn, ctypes.byref(d), None, FAKE, None, 0, None)
    assert st == 1 and "a_out" in msg


def test_prefix_workspace_required(lib):
    d = good_desc()
    need = lib.ba_prefix_attn_workspace(ctypes.byref(d))
    assert need > 0  # an 8192-key prefix for 2 KV heads is split across workgroups
    st, msg = status_of(lib, lib.ba_prefix_attn, ctypes.byref(d), FAKE, FAKE, FAKE, need - 1, None)
    assert st == 5 and "workspace" in msg


def test_prefix_workspace_covers_gated_split(lib):
    # Eight sequences of 16 rows (8 heads) over 4096 prefix keys: the split
    # pass plans 8 key splits, a gated fused step with a valid cache 16 (it
    # plans for a step that recomputes part of the sequences or heads).  The
    # workspace query covers the finer split: 16 x rows x heads x (d + 1)
    # float32 partials.
    d = lib_mod.AttnDesc()
    d.dtype, d.n_seq, d.hq, d.hkv, d.d, d.max_q, d.max_k = 0, 8, 8, 8, 128, 16, 4096
    d.q = d.k = d.v = FAKE
    for i, s in enumerate((16 * 8 * 128, 8 * 128, 128)):
        d.q_stride[i] = s
    for i, s in enumerate((8 * 4096 * 128, 128, 4096 * 128)):
        d.k_stride[i] = s
        d.v_stride[i] = s
    need = lib.ba_prefix_attn_workspace(ctypes.byref(d))
    assert need >= 16 * (8 * 16 * 8) * 129 * 4


def test_prefix_workspace_covers_gated_single_split(lib):
    # A 64-key prefix needs one key split, so an ungated pass needs no
    # workspace; a gated fused step still writes its prefix part as split
    # partials (a prefix workgroup that gave up waiting for the gate must
    # not overwrite a reused head's cache), and the query covers that.
    d = good_desc()
    d.max_k = 64
    for i, s in enumerate((2 * 64 * 128, 128, 64 * 128)):
        d.k_stride[i] = s
        d.v_stride[i] = s
    need = lib.ba_prefix_attn_workspace(ctypes.byref(d))
    assert need >= (32 * 4) * 129 * 4


def f32_pair():
    """A float32 prefix / block descriptor pair for one fused step (4 heads,
    32 block rows) and its matching count gate."""
    p = good_desc()
    p.dtype = 1
    for i, s in enumerate((32 * 4 * 128, 4 * 128, 128)):
        p.q_stride[i] = s
    b = good_desc()
    b.dtype, b.max_k = 1, 32
    for i, s in enumerate((32 * 2 * 128, 2 * 128, 128)):
        b.k_stride[i] = s
        b.v_stride[i] = s
    g = good_gate()
    g.dtype, g.n_seq, g.hq = 1, 1, 4
    return p, b, g


def test_fused_f32_validates_before_the_gate(lib):
    # The float32 fused step runs the gate and then the split pass as two
    # launches; a bad prefix descriptor must be rejected before the gate is
    # enqueued (with no GPU here, an enqueued gate would report a HIP error
    # instead of the validation failure).
    p, b, g = f32_pair()
    p.d = 96
    gws = lib.ba_gated_split_attn_gate_workspace(ctypes.byref(g))
    st, msg = status_of(lib, lib.ba_gated_split_attn, ctypes.byref(g), FAKE, None, FAKE, FAKE, gws,
                        ctypes.byref(p), ctypes.byref(b), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == 4 and "head dim" in msg, (st, msg)
    p, b, g = f32_pair()
    st, msg = status_of(lib, lib.ba_gated_split_attn, ctypes.byref(g), FAKE, None, FAKE, FAKE, gws,
                        ctypes.byref(p), ctypes.byref(b), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == 1 and "a_in" in msg, (st, msg)


def test_noalloc_rejects_scratch_beyond_its_limit(lib):
    # 16 query heads of 3000 block rows on one KV head over a 30000-key
    # prefix: 48000 rows per KV head in few workgroups, so the split plan's
    # partials exceed the static scratch and the no-allocation call refuses
    # it on the host (nothing is enqueued); the workspace call would take it.
    d = lib_mod.AttnDesc()
    d.dtype, d.n_seq, d.hq, d.hkv, d.d, d.max_q, d.max_k = 0, 1, 16, 1, 128, 3000, 30000
    d.q = d.k = d.v = FAKE
    for i, s in enumerate((3000 * 16 * 128, 16 * 128, 128)):
        d.q_stride[i] = s
    for i, s in enumerate((30000 * 128, 128, 30000 * 128)):
        d.k_stride[i] = s
        d.v_stride[i] = s
    assert lib.ba_prefix_attn_workspace(ctypes.byref(d)) > lib_mod.BA_NOALLOC_SCRATCH_BYTES
    st, msg = status_of(lib, lib.ba_prefix_attn_noalloc, ctypes.byref(d), FAKE, FAKE, None)
    assert st == 5 and "static scratch" in msg, (st, msg)
    d.d = 96
    st, msg = status_of(lib, lib.ba_prefix_attn_noalloc, ctypes.byref(d), FAKE, FAKE, None)
    assert st == 4 and "head dim" in msg, (st, msg)


def test_prefix_empty_is_ok_without_launch(lib):
    d = good_desc()
    d.n_seq = 0
    assert lib.ba_prefix_attn(ctypes.byref(d), FAKE, FAKE, None, 0, None) == 0


def test_block_validation(lib):
    d = good_desc()
    st, msg = status_of(lib, lib.ba_block_attn, ctypes.byref(d), None, None, None, None, None, None, None)
    assert st == 1 and "no output" in msg
    st, msg = status_of(lib, lib.ba_block_attn, ctypes.byref(d), FAKE, None, None, None, FAKE, None, None)
    assert st == 1 and "a_cache" in msg
    st, msg = status_of(lib, lib.ba_block_attn, ctypes.byref(d), None, None, None, None, FAKE, None, None)
    assert st == 1 and "cache" in msg


def test_merge_validation(lib):
    assert lib.ba_lse_merge(-1, 128, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == 2
    assert lib.ba_lse_merge(4, 6, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == 4
    assert lib.ba_lse_merge(4, 128, None, FAKE, FAKE, FAKE, FAKE, None, None) == 1
    assert lib.ba_lse_merge(0, 128, None, None, None, None, None, None, None) == 0


def good_gate():
    g = lib_mod.GateDesc()
    g.mode, g.dtype, g.n_seq, g.n_blk, g.hq, g.hkv, g.d = 0, 0, 2, 32, 4, 2, 128
    g.q_cur = g.q_prev = g.k_cur = g.k_prev = g.v_cur = g.v_prev = FAKE
    for i, s in enumerate((32 * 4 * 128, 4 * 128, 128)):
        g.q_stride[i] = s
    for i, s in enumerate((32 * 2 * 128, 2 * 128, 128)):
        g.kv_stride[i] = s
    g.tau = 4
    return g


def test_gate_validation(lib):
    g = good_gate()
    need = lib.ba_reuse_gate_workspace(ctypes.byref(g))
    assert need == 2 * 4
    st, msg = status_of(lib, lib.ba_reuse_gate, ctypes.byref(g), FAKE, None, None, FAKE, need, None)
    assert st == 1 and "decision" in msg
    st, msg = status_of(lib, lib.ba_reuse_gate, ctypes.byref(g), FAKE, None, FAKE, FAKE, need - 1, None)
    assert st == 5
    g.k_prev = None
    st, msg = status_of(lib, lib.ba_reuse_gate, ctypes.byref(g), FAKE, None, FAKE, FAKE, need, None)
    assert st == 1 and "pairs" in msg
    g = good_gate()
    g.n_blk = 0
    assert lib.ba_reuse_gate(ctypes.byref(g), FAKE, None, FAKE, FAKE, 64, None) == 2
    g = good_gate()
    g.mode = 5
    assert lib.ba_reuse_gate(ctypes.byref(g), FAKE, None, FAKE, FAKE, 64, None) == 2
    g = good_gate()
    g.mode = 1
    assert lib.ba_reuse_gate_workspace(ctypes.byref(g)) > 2 * 4 * 4


def test_pack_validation(lib):
    sizes = (ctypes.c_int32 * 3)(4, -1, 2)
    st, msg = status_of(lib, lib.ba_varlen_pack, 3, sizes, FAKE, FAKE, FAKE, FAKE, 0, 0, 0, None, None, None, None)
    assert st == 2 and "negative" in msg
    sizes = (ctypes.c_int32 * 1)(4)
    assert lib.ba_varlen_pack(600, sizes, FAKE, FAKE, FAKE, FAKE, 0, 0, 0, None, None, None, None) == 2
    assert lib.ba_varlen_pack(1, sizes, None, FAKE, FAKE, FAKE, 0, 0, 0, None, None, None, None) == 1
    assert lib.ba_varlen_pack(1, sizes, FAKE, FAKE, FAKE, FAKE, 0, 0, 0, FAKE, None, None, None) == 1


def test_rows_validation(lib):
    # partial refresh: dense descriptors only, no decision, both lists given
    d = good_desc()
    st, msg = status_of(lib, lib.ba_prefix_attn_rows, ctypes.byref(d), None, FAKE, FAKE, FAKE, None, 0, None)
    assert st == 1 and "cu_rows" in msg
    d.decision = FAKE
    st, msg = status_of(lib, lib.ba_prefix_attn_rows, ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, 0, None)
    assert st == 2 and "decision" in msg
    d = good_desc()
    d.cu_q = d.cu_k = FAKE
    st, msg = status_of(lib, lib.ba_prefix_attn_rows, ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, 0, None)
    assert st == 4 and "dense" in msg
    d = good_desc()
    need = lib.ba_prefix_attn_workspace(ctypes.byref(d))
    st, msg = status_of(lib, lib.ba_prefix_attn_rows, ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None)
    assert st == 5 and "workspace" in msg
    d.n_seq = 0
    assert lib.ba_prefix_attn_rows(ctypes.byref(d), None, None, FAKE, FAKE, None, 0, None) == 0


def test_gate_variant_validation(lib):
    g = good_gate()
    g.mode = 2   # count since the last refresh: needs its marks
    need = lib.ba_reuse_gate_workspace(ctypes.byref(g))
    assert need == 2 * 4
    st, msg = status_of(lib, lib.ba_reuse_gate, ctypes.byref(g), FAKE, None, FAKE, FAKE, need, None)
    assert st == 1 and "since_refresh" in msg
    g = good_gate()
    g.mode = 3   # rows: Q only
    st, msg = status_of(lib, lib.ba_reuse_gate, ctypes.byref(g), FAKE, None, FAKE, FAKE, need, None)
    assert st == 2 and "Q only" in msg
    g.k_cur = g.k_prev = g.v_cur = g.v_prev = None
    st, msg = status_of(lib, lib.ba_reuse_gate, ctypes.byref(g), None, None, FAKE, FAKE, need, None)
    assert st == 1 and "m_count" in msg
    # the rows gate feeds the partial refresh, not the fused step
    d = good_desc()
    gws = lib.ba_gated_split_attn_gate_workspace(ctypes.byref(g))
    g.n_seq, g.hq, g.n_blk = d.n_seq, d.hq, d.max_q
    st, msg = status_of(lib, lib.ba_gated_split_attn, ctypes.byref(g), FAKE, None, FAKE, FAKE, gws,
                        ctypes.byref(d), ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None)
    assert st == 4 and "rows gate" in msg


def test_kl_validation(lib):
    kl = lib.ba_kl_lock
    assert kl(-1, 100, 0, FAKE, FAKE, 100, None, 1e-3, FAKE, None, None) == 2
    assert kl(4, 0, 0, FAKE, FAKE, 100, None, 1e-3, FAKE, None, None) == 2
    assert kl(4, 100, 9, FAKE, FAKE, 100, None, 1e-3, FAKE, None, None) == 3
    st, msg = status_of(lib, kl, 4, 100, 0, FAKE, FAKE, 99, None, 1e-3, FAKE, None, None)
    assert st == 2 and "row_stride" in msg
    st, msg = status_of(lib, kl, 4, 100, 0, FAKE, FAKE, 100, None, 1e-3, None, None, None)
    assert st == 1 and "no output" in msg
    st, msg = status_of(lib, kl, 4, 100, 0, None, FAKE, 100, None, 1e-3, FAKE, None, None)
    assert st == 1 and "logits" in msg
    st, msg = status_of(lib, kl, 4, 100, 0, FAKE, FAKE, 100, None, -1.0, FAKE, None, None)
    assert st == 2 and "eps" in msg
    assert kl(0, 100, 0, None, None, 100, None, 1e-3, FAKE, None, None) == 0


def test_sparse_validation(lib):
    d = good_desc()
    n_max = (d.max_k + 63) // 64
    fn = lib.ba_sparse_prefix_attn
    st, msg = status_of(lib, fn, ctypes.byref(d), FAKE, n_max + 1, FAKE, FAKE, None, 0, None)
    assert st == 2 and "n_blocks" in msg
    st, msg = status_of(lib, fn, ctypes.byref(d), None, 3, FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == 1 and "blocks" in msg
    d.dtype = 1
    st, msg = status_of(lib, fn, ctypes.byref(d), FAKE, 3, FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == 4 and "bf16" in msg
    d = good_desc()
    d.cu_q = d.cu_k = FAKE
    st, msg = status_of(lib, fn, ctypes.byref(d), FAKE, 3, FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == 4 and "dense" in msg


def test_prefix_rejects_entries_beyond_32_bit_indexing(lib):
    # The kernels number rows per KV head and, in the 256-row kernel's
    # epilogue, (split, row, head) entries with 32-bit integers; shapes beyond
    # either are refused on the host (nothing is enqueued).
    def desc(n_seq, hq, hkv, max_q):
        d = lib_mod.AttnDesc()
        d.dtype, d.n_seq, d.hq, d.hkv, d.d, d.max_q, d.max_k = 0, n_seq, hq, hkv, 128, max_q, 64
        d.q = d.k = d.v = FAKE
        for i, s in enumerate((max_q * hq * 128, hq * 128, 128)):
            d.q_stride[i] = s
        for i, s in enumerate((hkv * 64 * 128, 128, 64 * 128)):
            d.k_stride[i] = s
            d.v_stride[i] = s
        return d
    # 1024 query heads on one KV head over 3,000,000 rows: 3.07e9 rows per KV head
    d = desc(1, 1024, 1, 3_000_000)
    st, msg = status_of(lib, lib.ba_prefix_attn, ctypes.byref(d), FAKE, FAKE, FAKE, 1 << 62, None)
    assert st == 4 and "rows per KV head" in msg, (st, msg)
    # 4 sequences x 600,000 rows x 1024 heads = 2.46e9 entries (38.4e6 rows per KV head)
    d = desc(4, 1024, 16, 600_000)
    st, msg = status_of(lib, lib.ba_prefix_attn, ctypes.byref(d), FAKE, FAKE, FAKE, 1 << 62, None)
    assert st == 4 and "entries" in msg, (st, msg)
