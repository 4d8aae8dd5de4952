"""The C-ABI library loads, exports every function include/hc.h declares, and
rejects invalid configurations — all without touching a GPU."""
import ctypes

import pytest

from cache_gather_amd import hc


def test_library_exports_every_declared_function():
    names = hc.declared_functions()
    assert set(names) >= {"hc_workspace_bytes", "hc_create", "hc_host_rows", "hc_step",
                          "hc_append", "hc_flush", "hc_attend_workspace_bytes", "hc_attend",
                          "hc_attend_cached", "hc_export_state", "hc_profile_enable", "hc_profile_read",
                          "hc_steps_done", "hc_destroy", "hc_status_str"}
    L = hc.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5):
        assert hc.hc_status_str(code)
    assert hc.hc_status_str(-99) == "unknown status"


def test_workspace_grows_with_the_configuration_and_holds_the_hot_rows():
    base = hc.hc_workspace_bytes(hc.make_config(1, 1, 1, 32768, 2048, 51047))
    assert base >= 32768 * 656 + 51047 * 12 + 2 * 32768 * 4
    assert base % 256 == 0
    more_layers = hc.hc_workspace_bytes(hc.make_config(1, 78, 4, 32768, 2048, 51047))
    assert more_layers >= 78 * 32768 * 656
    more_pos = hc.hc_workspace_bytes(hc.make_config(1, 1, 1, 32768, 2048, 1048832))
    assert more_pos >= base + (1048832 - 51047) * 12 - 1024   # alignment slack


@pytest.mark.parametrize("bad", [
    dict(top_k=0), dict(top_k=4097, cache_slots=5000), dict(cache_slots=100, top_k=200),
    dict(n_sessions=0), dict(n_sessions=257), dict(n_layers=0), dict(layers_per_select=0),
    dict(max_positions=100, top_k=200, cache_slots=300), dict(max_positions=1 << 31),
    dict(flags=1), dict(cache_slots=262145),
    dict(ring_rows=64, copyback_rows=0), dict(ring_rows=64, copyback_rows=65),
    dict(ring_rows=0, copyback_rows=8), dict(ring_rows=65537, copyback_rows=64),
    dict(queries=17), dict(queries=4, cache_slots=1000), dict(queries=8, top_k=2048,
                                                              cache_slots=32768),
    dict(max_positions=(1 << 31) - (1 << 19) + 1),
])
def test_invalid_configurations_are_rejected(bad):
    kw = dict(n_sessions=1, n_layers=2, layers_per_select=1, cache_slots=1024, top_k=256,
              max_positions=5000)
    kw.update(bad)
    cfg = hc.make_config(**kw)
    with pytest.raises(hc.HcError) as e:
        hc.hc_workspace_bytes(cfg)
    assert e.value.status == -1


def test_ring_adds_its_rows_to_the_workspace():
    base = hc.hc_workspace_bytes(hc.make_config(2, 78, 4, 32768, 2048, 51047))
    ring = hc.hc_workspace_bytes(hc.make_config(2, 78, 4, 32768, 2048, 51047,
                                                ring_rows=128, copyback_rows=64))
    assert ring - base == 2 * 78 * 128 * 656


def test_config_without_the_ring_fields_is_accepted():
    cfg = hc.make_config(1, 3, 2, 1024, 256, 5000)
    full = hc.hc_workspace_bytes(cfg)
    assert hc.CONFIG_SIZE_NO_RING == 40
    cfg.struct_size = hc.CONFIG_SIZE_NO_RING
    cfg.ring_rows, cfg.copyback_rows = 99, 7   # ignored: beyond the short struct
    assert hc.hc_workspace_bytes(cfg) == full


def test_config_without_queries_means_one_query():
    cfg = hc.make_config(1, 3, 2, 1024, 256, 5000, ring_rows=16, copyback_rows=8)
    full = hc.hc_workspace_bytes(cfg)
    assert hc.CONFIG_SIZE_ONE_QUERY == 48 and ctypes.sizeof(hc.hc_config) == 56
    cfg.struct_size = hc.CONFIG_SIZE_ONE_QUERY
    cfg.queries = 9                         # ignored: beyond the short struct
    assert hc.hc_workspace_bytes(cfg) == full
    zero = hc.make_config(1, 3, 2, 1024, 256, 5000, ring_rows=16, copyback_rows=8, queries=0)
    assert hc.hc_workspace_bytes(zero) == full


def test_queries_grow_the_selection_arrays():
    one = hc.hc_workspace_bytes(hc.make_config(1, 78, 4, 32768, 2048, 51047))
    four = hc.hc_workspace_bytes(hc.make_config(1, 78, 4, 32768, 2048, 51047, queries=4))
    # per extra query and unit: cand (8 B per position) + 5 arrays of K ints + counters
    assert four - one >= 20 * 3 * (51047 * 8 + 5 * 2048 * 4)


def test_bad_struct_size_is_rejected():
    cfg = hc.make_config(1, 1, 1, 1024, 256, 5000)
    cfg.struct_size = 12
    with pytest.raises(hc.HcError):
        hc.hc_workspace_bytes(cfg)


def test_null_handles():
    L = hc.lib()
    assert L.hc_destroy(None) == 0
    assert L.hc_host_rows(None, 0, 0) is None
    assert L.hc_step(None, None, None, 0, None, None, None, None) == -1
    assert L.hc_append(None, None, None, None) == -1
    assert L.hc_flush(None, None, None) == -1
    n = ctypes.c_uint64()
    assert L.hc_steps_done(None, ctypes.byref(n)) == -1
    cfg = hc.make_config(1, 1, 1, 1024, 256, 5000)
    out = ctypes.c_void_p(1)
    assert L.hc_create(ctypes.byref(cfg), None, 0, ctypes.byref(out)) == -1
    assert out.value is None


@pytest.mark.parametrize("kw", [
    dict(n_sessions=1, n_layers=1, layers_per_select=1, cache_slots=262144, top_k=4096,
         max_positions=300004),
    dict(n_sessions=1, n_layers=2, layers_per_select=1, cache_slots=8192, top_k=512,
         max_positions=9005, queries=16),
    dict(n_sessions=256, n_layers=1, layers_per_select=1, cache_slots=96, top_k=64,
         max_positions=604),
    dict(n_sessions=1, n_layers=1, layers_per_select=1, cache_slots=1024, top_k=256,
         max_positions=4112, ring_rows=65536, copyback_rows=8),
    dict(n_sessions=16, n_layers=256, layers_per_select=1, cache_slots=80, top_k=48,
         max_positions=204),
    dict(n_sessions=1, n_layers=12000, layers_per_select=4, cache_slots=16, top_k=8,
         max_positions=44),
])
def test_limit_configurations_are_accepted(kw):
    """Each of HC_MAX_SLOTS, HC_MAX_TOPK, HC_MAX_QUERIES (with Q * K =
    HC_MAX_ROUND_ROWS = C), HC_MAX_SESSIONS, HC_MAX_RING_ROWS and HC_MAX_UNITS
    is accepted, and so are 12,000 layers of one session (the GPU parity tests
    run these configurations)."""
    assert hc.hc_workspace_bytes(hc.make_config(**kw)) > 0


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without libhc.so every call raises: there is no fallback path."""
    monkeypatch.setattr(hc, "_LIB", None)
    monkeypatch.setattr(hc, "LIB_PATH", str(tmp_path / "libhc.so"))
    with pytest.raises(RuntimeError, match="not built"):
        hc.lib()
    with pytest.raises(RuntimeError, match="not built"):
        hc.hc_workspace_bytes(hc.make_config(1, 1, 1, 64, 8, 64))


def test_no_gpu_means_no_context():
    """Creating a context needs a GPU: on a machine without one it raises
    instead of computing anything on the CPU."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(Exception):
        hc.HotCache(1, 1, 1, 64, 8, 64, 0)
