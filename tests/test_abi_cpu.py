"""Host-side checks of the C ABI (no kernel launches): the library loads, exports
every function include/kvq.h declares, sizes buffers as the layout says and
rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

from oracle import kivi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _cfg(B, **kw):
    base = dict(batch=8, num_q_heads=32, num_kv_heads=32, head_dim=128, k_bits=2, v_bits=2, k_group=32,
                v_group=32, residual=128, res_capacity=160, max_blocks=128, num_pages=0, dtype=0)
    base.update(kw)
    return B.kvq_config(**base)


def test_library_exports_every_declared_function(kvq_lib):
    header = open(os.path.join(ROOT, "include", "kvq.h")).read()
    declared = set(re.findall(r"^(?:kvq_status|const char\*)\s+(kvq_\w+)\(", header, re.M))
    assert declared, "no declarations parsed"
    from quantized_kv_cache_append_amd import binding as B
    assert declared == set(B.EXPORTED)
    for name in declared:
        assert hasattr(kvq_lib, name), name


@pytest.mark.parametrize("kb,vb,G,GV,d,per_tok", [(2, 2, 32, 32, 128, 96), (4, 4, 32, 32, 128, 160),
                                                   (2, 2, 64, 64, 128, 80), (4, 2, 16, 32, 128, 144),
                                                   (2, 2, 32, 32, 64, 48)])
def test_layout_matches_oracle_record(kvq_lib, kb, vb, G, GV, d, per_tok):
    from quantized_kv_cache_append_amd import binding as B
    cfg = _cfg(B, k_bits=kb, v_bits=vb, k_group=G, v_group=GV, head_dim=d, res_capacity=128 + G)
    lay = B.kvq_layout_bytes(cfg)
    spec = kivi.CacheSpec(8, 32, 32, d, kb, vb, G, GV, 128, 128 + G, "f16")
    assert lay.record == kivi.record_bytes(spec) == per_tok * G
    assert lay.blocks == 8 * 32 * 128 * lay.record
    assert lay.ring == 8 * 32 * (128 + G) * d * 2
    assert lay.block_table == 0
    assert lay.state == (4 * 8 + 32 * 9) * 4   # per-sequence words, error word, decode queue counters


def test_paged_layout(kvq_lib):
    from quantized_kv_cache_append_amd import binding as B
    cfg = _cfg(B, batch=64, num_q_heads=48, num_kv_heads=8, k_bits=4, v_bits=2, k_group=16, v_group=32,
               residual=64, res_capacity=80, max_blocks=4096, num_pages=60000, dtype=1)
    lay = B.kvq_layout_bytes(cfg)
    assert lay.record == 2304
    assert lay.blocks == 60000 * 8 * 2304
    assert lay.block_table == 64 * 4096 * 4


def test_quantized_bytes_shrink_the_closed_form(kvq_lib):
    # 70B-shaped layer at INT2, G=G_V=64: 80 B per token per kv head against 512 B in bf16
    from quantized_kv_cache_append_amd import binding as B
    cfg = _cfg(B, batch=4, num_q_heads=64, num_kv_heads=8, k_group=64, v_group=64, res_capacity=192,
               max_blocks=2048, dtype=1)
    lay = B.kvq_layout_bytes(cfg)
    dense = kivi.kv_cache_bytes(1, 8, 128, 2048 * 64, 2) * 4
    assert dense / lay.blocks == pytest.approx(512 / 80)


@pytest.mark.parametrize("field,value,status", [
    ("num_kv_heads", 5, 1), ("k_bits", 3, 2), ("v_bits", 8, 2), ("head_dim", 96, 2), ("head_dim", 100, 1), ("head_dim", 256, 2),
    ("res_capacity", 159, 1), ("k_group", 24, 2), ("k_group", 128, 2), ("v_group", 24, 1), ("num_q_heads", 48, 1),
    ("dtype", 7, 1), ("batch", 0, 1), ("residual", -1, 1),
])
def test_invalid_configs_are_rejected(kvq_lib, field, value, status):
    from quantized_kv_cache_append_amd import binding as B
    cfg = _cfg(B, **{field: value})
    if field == "k_group":
        cfg.res_capacity = 128 + value
    lay = B.kvq_layout()
    assert kvq_lib.kvq_layout_bytes(ctypes.byref(cfg), ctypes.byref(lay)) == status


def test_group_query_ratio_above_eight_is_unsupported(kvq_lib):
    from quantized_kv_cache_append_amd import binding as B
    cfg = _cfg(B, num_q_heads=64, num_kv_heads=4)
    lay = B.kvq_layout()
    assert kvq_lib.kvq_layout_bytes(ctypes.byref(cfg), ctypes.byref(lay)) == B.KVQ_ERR_UNSUPPORTED


def test_calls_reject_null_and_misaligned_pointers(kvq_lib):
    from quantized_kv_cache_append_amd import binding as B
    cfg = _cfg(B)
    empty = B.kvq_cache()
    assert kvq_lib.kvq_append(ctypes.byref(cfg), ctypes.byref(empty), None, None, None, 1, None) == 1
    assert kvq_lib.kvq_flush_residual(ctypes.byref(cfg), None, None) == 1
    fake = B.kvq_cache(blocks=0x1000, block_table=None, k_ring=0x2008, v_ring=0x3000, state=0x4000)
    assert kvq_lib.kvq_flush_residual(ctypes.byref(cfg), ctypes.byref(fake), None) == 1
    ok = B.kvq_cache(blocks=0x1000, block_table=None, k_ring=0x2000, v_ring=0x3000, state=0x4000)
    # paged config without a table is inconsistent
    paged = _cfg(B, num_pages=10)
    assert kvq_lib.kvq_flush_residual(ctypes.byref(paged), ctypes.byref(ok), None) == 1
    # decode: too small a workspace is reported before any launch
    need = B.kvq_workspace_size(cfg, 4096)
    assert need > 0
    assert kvq_lib.kvq_decode_attention(ctypes.byref(cfg), ctypes.byref(ok), ctypes.c_void_p(0x5000),
                                        ctypes.c_void_p(0x6000), ctypes.c_float(0.0), 4096,
                                        ctypes.c_void_p(0x7000), need - 1, None) == B.KVQ_ERR_WORKSPACE
    assert kvq_lib.kvq_decode_attention(ctypes.byref(cfg), ctypes.byref(ok), None, ctypes.c_void_p(0x6000),
                                        ctypes.c_float(0.0), 4096, ctypes.c_void_p(0x7000), need, None) == 1
    assert kvq_lib.kvq_decode_attention(ctypes.byref(cfg), ctypes.byref(ok), ctypes.c_void_p(0x5000),
                                        ctypes.c_void_p(0x6000), ctypes.c_float(float("nan")), 4096,
                                        ctypes.c_void_p(0x7000), need, None) == 1


def test_workspace_grows_with_sequence_bound(kvq_lib):
    from quantized_kv_cache_append_amd import binding as B
    cfg = _cfg(B)
    a, b, c = (B.kvq_workspace_size(cfg, n) for n in (1000, 100000, 10_000_000))
    assert 0 < a <= b < c   # the unit count is capped by a fixed target until units hit their size cap
    assert B.kvq_workspace_size(cfg, 0) > 0   # every pair has its ring unit


def test_ctypes_structs_follow_the_header(kvq_lib):
    # the binding's field lists are the header's, in order
    from quantized_kv_cache_append_amd import binding as B
    header = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "kvq.h")).read(), flags=re.S)
    for struct in (B.kvq_config, B.kvq_layout, B.kvq_cache):
        body = re.search(r"typedef struct \{([^{}]*)\}\s*" + struct.__name__ + ";", header)
        assert body, struct.__name__
        fields = re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+);", body.group(1), re.M)
        assert fields == [f[0] for f in struct._fields_], struct.__name__


def test_sink_layout_and_checks(kvq_lib):
    from quantized_kv_cache_append_amd import binding as B
    cfg = _cfg(B, sink=4)
    lay = B.kvq_layout_bytes(cfg)
    assert lay.sink == 8 * 32 * 4 * 128 * 2
    assert B.kvq_layout_bytes(_cfg(B)).sink == 0
    # one sink partial state per output row on top of the split states, 16-byte aligned
    plain, with_sink = B.kvq_workspace_size(_cfg(B), 4096), B.kvq_workspace_size(cfg, 4096)
    assert with_sink == ((plain + 15) // 16) * 16 + 8 * 32 * (128 + 2) * 4
    bad = _cfg(B, sink=-1)
    assert kvq_lib.kvq_layout_bytes(ctypes.byref(bad), ctypes.byref(B.kvq_layout())) == B.KVQ_ERR_INVALID_ARG
    # a sink config needs both sink buffers, 16-byte aligned
    no_sink = B.kvq_cache(blocks=0x1000, block_table=None, k_ring=0x2000, v_ring=0x3000, state=0x4000)
    assert kvq_lib.kvq_flush_residual(ctypes.byref(cfg), ctypes.byref(no_sink), None) == 1
    odd = B.kvq_cache(blocks=0x1000, block_table=None, k_ring=0x2000, v_ring=0x3000, state=0x4000,
                      k_sink=0x8000, v_sink=0x9004)
    assert kvq_lib.kvq_flush_residual(ctypes.byref(cfg), ctypes.byref(odd), None) == 1


def test_multi_token_query_checks(kvq_lib):
    from quantized_kv_cache_append_amd import binding as B
    cfg = _cfg(B)   # MHA, R = 128
    assert B.kvq_workspace_size_multi(cfg, 4096, 1) == B.kvq_workspace_size(cfg, 4096)
    assert B.kvq_workspace_size_multi(cfg, 4096, 8) > B.kvq_workspace_size(cfg, 4096)   # 8 query rows per kv head
    n = ctypes.c_size_t(0)
    assert kvq_lib.kvq_workspace_size_multi(ctypes.byref(cfg), 4096, 0, ctypes.byref(n)) == B.KVQ_ERR_INVALID_ARG
    assert kvq_lib.kvq_workspace_size_multi(ctypes.byref(cfg), 4096, 9, ctypes.byref(n)) == B.KVQ_ERR_UNSUPPORTED
    gqa = _cfg(B, num_q_heads=32, num_kv_heads=8)   # n_g = 4: at most 2 tokens
    assert kvq_lib.kvq_workspace_size_multi(ctypes.byref(gqa), 4096, 2, ctypes.byref(n)) == B.KVQ_OK
    assert kvq_lib.kvq_workspace_size_multi(ctypes.byref(gqa), 4096, 3, ctypes.byref(n)) == B.KVQ_ERR_UNSUPPORTED
    short = _cfg(B, residual=2, res_capacity=34)   # T > R: the block would reach the quantized part
    assert kvq_lib.kvq_workspace_size_multi(ctypes.byref(short), 4096, 3, ctypes.byref(n)) == B.KVQ_ERR_INVALID_ARG
    ok = B.kvq_cache(blocks=0x1000, block_table=None, k_ring=0x2000, v_ring=0x3000, state=0x4000)
    need = B.kvq_workspace_size_multi(cfg, 4096, 4)
    assert kvq_lib.kvq_decode_attention_multi(ctypes.byref(cfg), ctypes.byref(ok), ctypes.c_void_p(0x5000), 4,
                                              ctypes.c_void_p(0x6000), ctypes.c_float(0.0), 4096,
                                              ctypes.c_void_p(0x7000), need - 1, None) == B.KVQ_ERR_WORKSPACE
    assert kvq_lib.kvq_decode_attention_multi(ctypes.byref(cfg), ctypes.byref(ok), None, 4, ctypes.c_void_p(0x6000),
                                              ctypes.c_float(0.0), 4096, ctypes.c_void_p(0x7000), need, None) == 1


def test_fp8_tier_layout_and_checks(kvq_lib):
    from quantized_kv_cache_append_amd import binding as B
    cfg = _cfg(B, fp8_blocks=4)
    lay = B.kvq_layout_bytes(cfg)
    assert lay.fp8_record == 2 * 32 * 128 + 4 * 32
    assert lay.fp8 == 8 * 32 * 4 * lay.fp8_record
    assert B.kvq_layout_bytes(_cfg(B)).fp8 == 0
    # side partial states per output row: one per 64 tokens of the tier (4 blocks of 32: 2), one for a sink
    plain, tier = B.kvq_workspace_size(_cfg(B), 4096), B.kvq_workspace_size(cfg, 4096)
    assert tier == ((plain + 15) // 16) * 16 + 2 * 8 * 32 * (128 + 2) * 4
    both = B.kvq_workspace_size(_cfg(B, fp8_blocks=4, sink=2), 4096)
    assert both == ((plain + 15) // 16) * 16 + 3 * 8 * 32 * (128 + 2) * 4
    bad = _cfg(B, fp8_blocks=-1)
    assert kvq_lib.kvq_layout_bytes(ctypes.byref(bad), ctypes.byref(B.kvq_layout())) == B.KVQ_ERR_INVALID_ARG
    no_store = B.kvq_cache(blocks=0x1000, block_table=None, k_ring=0x2000, v_ring=0x3000, state=0x4000)
    assert kvq_lib.kvq_flush_residual(ctypes.byref(cfg), ctypes.byref(no_store), None) == 1


def test_status_strings(kvq_lib):
    from quantized_kv_cache_append_amd import binding as B
    assert B.status_string(0) == "ok"
    assert "workspace" in B.status_string(B.KVQ_ERR_WORKSPACE)
    assert "capacity" in B.status_string(B.KVQ_ERR_CAPACITY)
    assert B.status_string(99) == "unknown status"


def test_status_codes_follow_the_header(kvq_lib):
    from quantized_kv_cache_append_amd import binding as B
    header = open(os.path.join(ROOT, "include", "kvq.h")).read()
    codes = dict((n, int(v)) for n, v in re.findall(r"^\s*(KVQ_(?:OK|ERR_\w+))\s*=\s*(\d+),", header, re.M))
    assert codes == {"KVQ_OK": 0, "KVQ_ERR_INVALID_ARG": 1, "KVQ_ERR_UNSUPPORTED": 2, "KVQ_ERR_CAPACITY": 3,
                     "KVQ_ERR_WORKSPACE": 4, "KVQ_ERR_LAUNCH": 5}
    for name, v in codes.items():
        assert getattr(B, name) == v
        kvq_lib.kvq_status_string.restype = ctypes.c_char_p
        assert kvq_lib.kvq_status_string(v) != b"unknown status"


def test_capacity_errors_are_reported_on_the_host(kvq_lib):
    from quantized_kv_cache_append_amd import binding as B
    cfg = _cfg(B, sink=8)   # holds 8 + 128 * 32 + 160 tokens per sequence
    ok = B.kvq_cache(blocks=0x1000, block_table=None, k_ring=0x2000, v_ring=0x3000, state=0x4000,
                     k_sink=0x5000, v_sink=0x6000)
    kv = ctypes.c_void_p(0x8000)
    # an append of more rows than the sink and the ring can take, fused or not
    for fn in (kvq_lib.kvq_append, kvq_lib.kvq_append_flush):
        assert fn(ctypes.byref(cfg), ctypes.byref(ok), kv, kv, None, 8 + 160 + 1, None) == B.KVQ_ERR_CAPACITY
    # decode with a length bound no sequence of this cache can reach
    cap = 8 + 128 * 32 + 160
    need = B.kvq_workspace_size(cfg, cap + 1)
    args = (ctypes.c_void_p(0x9000), ctypes.c_void_p(0xa000), ctypes.c_float(0.0))
    assert kvq_lib.kvq_decode_attention(ctypes.byref(cfg), ctypes.byref(ok), *args, cap + 1,
                                        ctypes.c_void_p(0xb000), need, None) == B.KVQ_ERR_CAPACITY
    assert kvq_lib.kvq_decode_partials(ctypes.byref(cfg), ctypes.byref(ok), args[0], args[2], cap + 1,
                                       ctypes.c_void_p(0xb000), need, None) == B.KVQ_ERR_CAPACITY
    # at the bound the arguments pass the host checks (a short workspace is the next error)
    assert kvq_lib.kvq_decode_attention(ctypes.byref(cfg), ctypes.byref(ok), *args, cap,
                                        ctypes.c_void_p(0xb000), 1, None) == B.KVQ_ERR_WORKSPACE


def test_batch_bound_keeps_the_plan_inside_lds(kvq_lib):
    # every decode workgroup copies the unit plan (16 + 7B ints) into LDS beside
    # its waves' buffers; B is capped so that the sum stays inside 160 KB
    from quantized_kv_cache_append_amd import binding as B
    lay = B.kvq_layout()
    for batch, status in ((1024, B.KVQ_OK), (1025, B.KVQ_ERR_UNSUPPORTED)):
        cfg = _cfg(B, batch=batch, num_q_heads=64, num_kv_heads=8, k_group=64, v_group=64, res_capacity=192,
                   dtype=1)
        assert kvq_lib.kvq_layout_bytes(ctypes.byref(cfg), ctypes.byref(lay)) == status
    assert (16 + 7 * 1024) * 4 + 4 * 15 * 1024 < 160 * 1024


def test_noalloc_decode_rejects_a_workspace_beyond_its_array_before_any_device_call(kvq_lib):
    # the no-allocation decode holds a fixed array per GPU; a configuration whose
    # workspace is larger gets KVQ_ERR_WORKSPACE from the host checks alone
    from quantized_kv_cache_append_amd import binding as B
    cfg = _cfg(B, batch=1024, num_q_heads=64, num_kv_heads=8, k_group=64, v_group=64, res_capacity=2048 + 191,
               max_blocks=64, dtype=1)
    need = B.kvq_workspace_size(cfg, 4096)
    assert need > B.KVQ_NOALLOC_WORKSPACE_BYTES
    fake = B.kvq_cache(blocks=0x1000, block_table=None, k_ring=0x2000, v_ring=0x3000, state=0x4000)
    assert kvq_lib.kvq_decode_attention_noalloc(ctypes.byref(cfg), ctypes.byref(fake), ctypes.c_void_p(0x5000),
                                                ctypes.c_void_p(0x6000), ctypes.c_float(0.0), 4096,
                                                None) == B.KVQ_ERR_WORKSPACE
    # and its other argument errors are the ones of kvq_decode_attention
    small = _cfg(B)
    assert kvq_lib.kvq_decode_attention_noalloc(ctypes.byref(small), ctypes.byref(fake), None,
                                                ctypes.c_void_p(0x6000), ctypes.c_float(0.0), 4096,
                                                None) == B.KVQ_ERR_INVALID_ARG
    assert kvq_lib.kvq_decode_attention_noalloc(ctypes.byref(small), ctypes.byref(fake), ctypes.c_void_p(0x5000),
                                                ctypes.c_void_p(0x6000), ctypes.c_float(0.0), 10 ** 8,
                                                None) == B.KVQ_ERR_CAPACITY
    assert B.KVQ_NOALLOC_WORKSPACE_BYTES == 64 << 20


def test_rotation_field_is_validated(kvq_lib):
    from quantized_kv_cache_append_amd import binding as B
    lay = B.kvq_layout()
    for rot, status in ((0, B.KVQ_OK), (1, B.KVQ_OK), (2, B.KVQ_OK), (3, B.KVQ_OK), (4, B.KVQ_ERR_INVALID_ARG),
                        (-1, B.KVQ_ERR_INVALID_ARG)):
        assert kvq_lib.kvq_layout_bytes(ctypes.byref(_cfg(B, rotate=rot)), ctypes.byref(lay)) == status, rot
    # the FP8 tier keeps unrotated rows: not together with a rotation
    assert kvq_lib.kvq_layout_bytes(ctypes.byref(_cfg(B, rotate=1, fp8_blocks=2)),
                                    ctypes.byref(lay)) == B.KVQ_ERR_UNSUPPORTED
    # the stored layout does not change with the rotation
    a, b = B.kvq_layout(), B.kvq_layout()
    kvq_lib.kvq_layout_bytes(ctypes.byref(_cfg(B)), ctypes.byref(a))
    kvq_lib.kvq_layout_bytes(ctypes.byref(_cfg(B, rotate=3)), ctypes.byref(b))
    assert (a.record, a.blocks, a.ring) == (b.record, b.blocks, b.ring)


def test_missing_library_fails_loudly(tmp_path):
    # no fallback: without the HIP library the binding raises instead of computing anything
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from quantized_kv_cache_append_amd import binding as B\n"
            "B.LIBRARY_PATH = %r\n"
            "try:\n"
            "    B.load()\n"
            "except Exception as e:\n"
            "    print('raised', type(e).__name__)\n"
            "else:\n"
            "    print('loaded')\n") % (ROOT, str(tmp_path / "libkvq_absent.so"))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.stdout.startswith("raised"), r.stdout + r.stderr
