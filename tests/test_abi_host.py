"""Host-only checks of the C ABI: the library loads, exports every function
include/moe.h declares, and validates arguments (no kernel is launched: every
call here fails validation before any device work, or is a size query)."""
import ctypes
import os
import re

import pytest

import quantized_moe_routed_router_amd as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(moe_[a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_header_function():
    L = m.lib()
    names = header_functions()
    assert len(names) >= 17
    for n in names:
        assert hasattr(L, n), n
    assert sorted(names) == m.exported_symbols()
    assert m.moe_abi_version() == 7


def test_sizes():
    d = m.dims(512, 2560, 640, 10)
    assert m.moe_packed_bytes(d, 0) == 512 * 1_843_200
    assert m.moe_packed_bytes(d, 1) == 512 * 921_600
    # 48 layers of experts: the "about 68 GB" of the stacked workload
    assert 48 * (m.moe_packed_bytes(d, 0) + m.moe_packed_bytes(d, 1)) == 67_947_724_800
    dc = m.dims(512, 2560, 640, 10, m.MOE_FMT_CB3G128)
    assert m.moe_packed_bytes(dc, 0) == 512 * 1_638_400
    assert m.moe_ffn_workspace_bytes(d, 1, False) >= 10 * 640 * 4
    assert m.moe_packed_bytes(m.dims(512, 2500, 640, 10), 0) == 0       # H not a multiple of 128
    assert m.moe_permute_workspace_bytes(4, 2, 16) > 0


def test_prefill_tile_rows_rule():
    fn = m.dims(512, 2560, 640, 10)
    assert m.moe_ffn_prefill_tile_rows(fn, 1) == 32
    assert m.moe_ffn_prefill_tile_rows(fn, 4915) == 32         # 49150 pairs <= 96 * 512
    assert m.moe_ffn_prefill_tile_rows(fn, 4916) == 256
    assert m.moe_ffn_prefill_tile_rows(fn, 65536) == 256
    cb = m.dims(512, 2560, 640, 10, m.MOE_FMT_CB3G128)
    assert m.moe_ffn_prefill_tile_rows(cb, 1) == 32
    assert m.moe_ffn_prefill_tile_rows(cb, 3276) == 32         # 32760 pairs <= 64 * 512
    assert m.moe_ffn_prefill_tile_rows(cb, 3277) == 256
    tiny = m.dims(16, 256, 128, 2)
    assert m.moe_ffn_prefill_tile_rows(tiny, 768) == 32
    assert m.moe_ffn_prefill_tile_rows(tiny, 769) == 128       # I = 128 < 256: 128-row tiles
    assert m.moe_ffn_prefill_tile_rows(m.dims(16, 256, 128, 2, m.MOE_FMT_CB3G128), 4) == 32
    assert m.moe_ffn_prefill_tile_rows(m.dims(16, 256, 128, 2, m.MOE_FMT_CB3G128), 800) == 128
    with pytest.raises(m.MoeError):
        m.moe_ffn_prefill_tile_rows(tiny, 0)
    with pytest.raises(m.MoeError):
        m.moe_ffn_prefill_tile_rows(m.dims(16, 200, 128, 2), 4)


def _err(fn, *args):
    with pytest.raises(m.MoeError) as ei:
        fn(*args)
    return ei.value.code, str(ei.value)


def test_validation_null_and_shape():
    d = m.dims(16, 256, 128, 2)
    code, msg = _err(m.moe_quantize_act, None, 4, 256, 1024, 1024, 1024, 0)
    assert code == m.MOE_ERR_INVALID and "x is NULL" in msg
    code, msg = _err(m.moe_quantize_act, 1024, 4, 250, 1024, 1024, 1024, 0)
    assert code == m.MOE_ERR_SHAPE and "250" in msg
    code, msg = _err(m.moe_quantize_act, 1028, 4, 256, 1024, 1024, 1024, 0)
    assert code == m.MOE_ERR_INVALID and "aligned" in msg
    code, msg = _err(m.moe_stream_read, 1024, 100, 1024, 0)
    assert code == m.MOE_ERR_SHAPE and "bytes = 100" in msg
    code, msg = _err(m.moe_stream_read, None, 4096, 1024, 0)
    assert code == m.MOE_ERR_INVALID and "src is NULL" in msg
    code, msg = _err(m.moe_router_topk, 1024, 1024, None, 4, m.dims(16, 256, 128, 17), 1024, 1024, 1024, 0)
    assert code == m.MOE_ERR_SHAPE and "k = 17" in msg
    code, msg = _err(m.moe_router_topk, 1024, 1024, None, 4, m.dims(2000, 256, 128, 2), 1024, 1024, 1024, 0)
    assert code == m.MOE_ERR_SHAPE and "E = 2000" in msg
    ex = dict(gate_up=1024, down=1024, ts_gate=1024, ts_up=1024, ts_down=1024)
    code, msg = _err(m.moe_expert_ffn_decode, d, ex, (1024, 1024, 1024), 1024, 65, 1024, 1024, 1 << 20, None, 0)
    assert code == m.MOE_ERR_SHAPE and "T = 65" in msg
    code, msg = _err(m.moe_layer_decode, d, ex, 1024, 1024, None, 17, False, 1024, None, None, 1024, 1 << 20, 0)
    assert code == m.MOE_ERR_SHAPE and "T = 17" in msg
    code, msg = _err(m.moe_expert_ffn_decode, d, ex, (1024, 1024, 1024), 1024, 4, 1024, 1024, 16, None, 0)
    assert code == m.MOE_ERR_WORKSPACE and "16 bytes" in msg
    ex2 = dict(ex, ts_gate=None)
    code, msg = _err(m.moe_expert_ffn_decode, d, ex2, (1024, 1024, 1024), 1024, 4, 1024, 1024, 1 << 20, None, 0)
    assert code == m.MOE_ERR_INVALID and "ts_gate" in msg
    # codebook gate/up: refused where a K split would cut a 128-element group
    # (H = 2688 is 21 groups; at 4 tokens the GEMVs split K in two)
    dcb = m.dims(16, 2688, 128, 2, m.MOE_FMT_CB3G128)
    code, msg = _err(m.moe_expert_ffn_decode, dcb, ex, (1024, 1024, 1024), 1024, 4, 1024, 1024, 1 << 30, None, 0)
    assert code == m.MOE_ERR_UNSUPPORTED and "H = 2688" in msg
    code, msg = _err(m.moe_combine, 1024, 1024, None, 3, 0, 256, 1024, 0)
    assert code == m.MOE_ERR_SHAPE
    code, msg = _err(m.moe_pack_nvfp4, d, 10, 7, 1024, 1024, 1024, 1024, None, None, 1024, None, 0)
    assert code == m.MOE_ERR_SHAPE and "[10, 17)" in msg
    code, msg = _err(m.moe_permute, 1024, 4, 2, 16, 1024, 1024, 1024, 1024, 1024, 8, 0)
    assert code == m.MOE_ERR_WORKSPACE
    code, msg = _err(m.moe_pack_codebook, d, 0, 1, 1024, 1024, 1024, 1024, 1024, 0)
    assert code == m.MOE_ERR_INVALID and "MOE_FMT_CB3G128" in msg
    code, msg = _err(m.moe_rms_norm, 1024, 2, 100, 1.0, 1024, 0)
    assert code == m.MOE_ERR_SHAPE and "H = 100" in msg
    code, msg = _err(m.moe_rms_norm, 1024, 2, 256, 0.0, 1024, 0)
    assert code == m.MOE_ERR_INVALID and "target_rms" in msg
    code, msg = _err(m.moe_rms_norm, 1024, 2, 256, float("nan"), 1024, 0)
    assert code == m.MOE_ERR_INVALID and "target_rms" in msg
    code, msg = _err(m.moe_rms_norm, None, 2, 256, 1.0, 1024, 0)
    assert code == m.MOE_ERR_INVALID and "x is NULL" in msg


def test_capacity_verdict_with_numbers():
    assert m.moe_capacity_verdict(100, 100) == 0
    assert m.moe_capacity_verdict(99, 100) == m.MOE_ERR_CAPACITY
    msg = m.last_error()
    assert "need 100 bytes" in msg and "99 bytes" in msg and "MOE_HBM_GUARD=0" in msg
    big = 67_947_724_800
    assert m.moe_capacity_verdict(10 << 30, big) == m.MOE_ERR_CAPACITY
    assert "63.28 GiB" in m.last_error()


def test_zero_sized_calls_enqueue_nothing():
    d = m.dims(16, 256, 128, 2)
    m.moe_quantize_act(None, 0, 256, None, None, None, 0)
    m.moe_router_topk(None, None, None, 0, d, None, None, None, 0)
    m.moe_combine(None, None, None, 0, 2, 256, None, 0)
    m.moe_rms_norm(None, 0, 256, 1.0, None, 0)
    m.moe_quantize_weights(None, 0, 4, 16, None, None, None, 0)
    m.moe_stream_read(None, 0, None, 0)


def test_noalloc_layer_refusals():
    """The no-allocation decode layer refuses shapes whose workspace exceeds
    its scratch array, with the numbers, before any device call."""
    big = m.dims(1024, 4096, 2560, 32)
    assert m.moe_layer_decode_workspace_bytes(big, 16) > m.MOE_NOALLOC_SCRATCH_BYTES
    L = m.lib()
    rc = L.moe_layer_decode_noalloc(ctypes.byref(big), None, None, None, None, 16, 1, None, None, None, None)
    assert rc == m.MOE_ERR_WORKSPACE
    msg = m.last_error()
    assert "8388608" in msg and str(m.moe_layer_decode_workspace_bytes(big, 16)) in msg
    fn = m.dims(512, 2560, 640, 10)
    assert m.moe_layer_decode_workspace_bytes(fn, 16) <= m.MOE_NOALLOC_SCRATCH_BYTES
    assert L.moe_layer_decode_noalloc(ctypes.byref(fn), None, None, None, None, 0, 1, None, None, None,
                                      None) == m.MOE_ERR_SHAPE
