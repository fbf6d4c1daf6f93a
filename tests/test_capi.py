"""The C-ABI library loads and exports every entry point include/uno.h declares;
host-side validation works without a GPU (no compute call is made here)."""
import ctypes as C
import os
import re

import pytest

from diffusion_drafted_lora_amd import configs, uno

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "uno.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(uno_[a-z_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = _declared()
    for must in ("uno_init", "uno_draft", "uno_verify", "uno_step", "uno_prefill",
                 "uno_accept", "uno_forward", "uno_sync", "uno_destroy"):
        assert must in names
    assert set(names) == set(uno.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = uno.lib()
    for name in _declared():
        assert hasattr(lib, name), name
    # exported C symbols only (no C++ mangling on the boundary)
    out = os.popen(f"nm -D --defined-only {uno.LIB_PATH}").read()
    exported = set(re.findall(r" T (uno_\w+)", out))
    assert set(_declared()) <= exported


@pytest.mark.parametrize("cfg", list(configs.ALL.values()), ids=list(configs.ALL))
def test_query_sizes_host_only(cfg):
    ccfg = uno.make_config(cfg, max_seqs=max(1, cfg.batch), max_seq_len=cfg.max_len)
    kv, ws = uno.query_sizes(ccfg)
    pages = -(-cfg.max_len // cfg.page_size) * max(1, cfg.batch)
    ts = 2 if cfg.dtype == "bf16" else 4
    assert kv == cfg.n_layers * 2 * pages * cfg.kv_dim * cfg.page_size * ts
    assert ws > 0


def test_invalid_configs_rejected():
    bad = uno.make_config(configs.TINY)
    bad.mask_id = 3
    with pytest.raises(uno.UnoError) as e:
        uno.query_sizes(bad)
    assert e.value.status == 1
    bad = uno.make_config(configs.TINY.with_(block_size=65))
    with pytest.raises(uno.UnoError) as e:
        uno.query_sizes(bad)
    assert e.value.status == 6
    bad = uno.make_config(configs.TINY, max_rows=1)
    with pytest.raises(uno.UnoError):
        uno.query_sizes(bad)
    for tp in (-0.1, float("nan")):
        bad = uno.make_config(configs.TINY, top_p=tp)
        with pytest.raises(uno.UnoError) as e:
            uno.query_sizes(bad)
        assert e.value.status == 1
    for tp in (0.0, 0.95, 1.0, 2.0):              # off, on, off, off
        uno.query_sizes(uno.make_config(configs.TINY, top_p=tp))
    bad = uno.make_config(configs.TINY)
    bad.qk_norm = 2
    with pytest.raises(uno.UnoError) as e:
        uno.query_sizes(bad)
    assert e.value.status == 1
    for bad_k in (-1, 17):
        bad = uno.make_config(configs.TINY, tree_chains=bad_k)
        with pytest.raises(uno.UnoError) as e:
            uno.query_sizes(bad)
        assert e.value.status == 1
    # tree chains size the verify laws, the chain table and one residual row per sequence
    T = configs.TINY
    t0 = uno.query_sizes(uno.make_config(T, max_seqs=2))[1]
    t4 = uno.query_sizes(uno.make_config(T, max_seqs=2, tree_chains=4))[1]
    extra = 2 * (1 + 4 * (T.block_size - 1) - T.block_size) * T.vocab * 4 + 2 * T.vocab * 8
    assert extra <= t4 - t0 <= extra + 8192
    # QK-norm adds one float32 q|k|v staging buffer of max_rows rows to the workspace
    c0, c1 = uno.make_config(configs.TINY), uno.make_config(configs.TINY.with_(qk_norm=True))
    assert c1.qk_norm == 1
    T = configs.TINY
    grow = uno.query_sizes(c1)[1] - uno.query_sizes(c0)[1]
    need = c0.max_rows * (T.n_q_heads + 2 * T.n_kv_heads) * T.head_dim * 4
    assert need <= grow <= need + 256


def test_init_rejects_null_buffers_before_touching_the_device():
    ccfg = uno.make_config(configs.TINY)
    h = C.c_void_p()
    st = uno.lib().uno_init(C.byref(ccfg), C.byref(uno.UnoWeightsC()), None, 0, None, 0, None,
                            C.byref(h))
    assert st == 1 and not h.value
    assert b"null" in uno.lib().uno_last_error(None)


def test_accept_noalloc_rejects_sizes_beyond_its_scratch():
    """Host-side checks of uno_accept_noalloc run before any device call."""
    lib = uno.lib()
    nz = C.c_void_p(16)          # never dereferenced: validation fails first
    for n, B, V in ((1025, 16, 151936), (0, 16, 32), (4, 65, 32), (4, 16, 262145), (4, 16, 1)):
        st = lib.uno_accept_noalloc(C.c_uint64(1), n, B, V, nz, nz, nz, nz, nz, nz, nz, nz,
                                    None, None)
        assert st == 1, (n, B, V)
        assert b"accept_noalloc" in lib.uno_last_error(None)
    st = lib.uno_accept_noalloc(C.c_uint64(1), 4, 16, 32, nz, None, nz, nz, nz, nz, nz, nz,
                                None, None)
    assert st == 1 and b"null" in lib.uno_last_error(None)
