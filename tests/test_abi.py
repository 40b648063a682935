"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, the binding's structs match the C layout, and host-side
argument validation returns the documented status before anything launches."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hstu.h")

hs = pytest.importorskip("hstu_jagged_silu_amd")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hstu_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("hstu_attn_fwd", "hstu_attn_fwd_cached", "hstu_mfalcon_fwd", "hstu_kv_append",
              "hstu_workspace_size", "hstu_status_string"):
        assert n in names


def test_library_exports_every_declared_function():
    lib = hs.lib()
    for n in declared_functions():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", hs.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (hstu_\w+)", out))
    assert set(declared_functions()) <= exported
    assert set(hs.EXPORTED_SYMBOLS) == set(declared_functions())


def test_struct_layout_matches_c(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(r'''
#include <stdio.h>
#include <stddef.h>
#include "hstu.h"
#define P(s, f) printf(#s "." #f " %zu\n", offsetof(s, f))
int main(void) {
  printf("hstu_params_t %zu\n", sizeof(hstu_params_t));
  P(hstu_params_t, num_heads); P(hstu_params_t, head_dim); P(hstu_params_t, dtype); P(hstu_params_t, alpha);
  P(hstu_params_t, norm_n); P(hstu_params_t, pos_tab); P(hstu_params_t, n_pos); P(hstu_params_t, pos_head_stride);
  P(hstu_params_t, time_tab); P(hstu_params_t, n_time); P(hstu_params_t, time_head_stride);
  P(hstu_params_t, ln_w); P(hstu_params_t, ln_b); P(hstu_params_t, ln_eps); P(hstu_params_t, timing_events);
  P(hstu_params_t, flags);
  printf("hstu_kv_cache_t %zu\n", sizeof(hstu_kv_cache_t));
  P(hstu_kv_cache_t, k_pages); P(hstu_kv_cache_t, v_pages); P(hstu_kv_cache_t, ts_pages);
  P(hstu_kv_cache_t, page_table); P(hstu_kv_cache_t, num_pages); P(hstu_kv_cache_t, page_size);
  P(hstu_kv_cache_t, max_pages_per_seq);
  printf("hstu_grads_t %zu\n", sizeof(hstu_grads_t));
  P(hstu_grads_t, dq); P(hstu_grads_t, dk); P(hstu_grads_t, dv); P(hstu_grads_t, du);
  P(hstu_grads_t, d_pos_tab); P(hstu_grads_t, d_time_tab); P(hstu_grads_t, d_ln_w); P(hstu_grads_t, d_ln_b);
  printf("hstu_layer_weights_t %zu\n", sizeof(hstu_layer_weights_t));
  P(hstu_layer_weights_t, embed_dim); P(hstu_layer_weights_t, w1); P(hstu_layer_weights_t, w2);
  P(hstu_layer_weights_t, products);
  return 0;
}
''')
    exe = tmp_path / "layout"
    r = subprocess.run(["gcc", "-std=c11", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                        "-I", "/opt/rocm/include", str(src), "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    lines = subprocess.run([str(exe)], capture_output=True, text=True).stdout.split("\n")
    got = dict(l.rsplit(" ", 1) for l in lines if l)
    assert int(got["hstu_params_t"]) == ctypes.sizeof(hs._Params)
    assert int(got["hstu_kv_cache_t"]) == ctypes.sizeof(hs._KVCache)
    for name, _ in hs._Params._fields_:
        assert int(got[f"hstu_params_t.{name}"]) == getattr(hs._Params, name).offset, name
    for name, _ in hs._KVCache._fields_:
        assert int(got[f"hstu_kv_cache_t.{name}"]) == getattr(hs._KVCache, name).offset, name
    assert int(got["hstu_grads_t"]) == ctypes.sizeof(hs._Grads)
    for name, _ in hs._Grads._fields_:
        assert int(got[f"hstu_grads_t.{name}"]) == getattr(hs._Grads, name).offset, name
    assert int(got["hstu_layer_weights_t"]) == ctypes.sizeof(hs._LayerWeights)
    for name, _ in hs._LayerWeights._fields_:
        assert int(got[f"hstu_layer_weights_t.{name}"]) == getattr(hs._LayerWeights, name).offset, name


def test_version_and_status_strings():
    assert hs.version() == 10000
    for code in range(5):
        assert hs.status_string(code).startswith("HSTU")
    assert "unknown" in hs.status_string(99)


def _params(**kw):
    p = hs._Params()
    p.num_heads, p.head_dim, p.dtype, p.alpha, p.norm_n, p.ln_eps = 4, 128, 1, 1.0, 0, 1e-5
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def _ws(fn, p, B, T, L):
    return int(hs.lib().hstu_workspace_size(fn, ctypes.byref(p), B, T, L))


def test_workspace_size_valid_and_invalid():
    p = _params()
    full = _ws(0, p, 8, 65536, 8192)
    # header + items + per-user scratch + fp32 O of T x H*d
    assert full >= 65536 * 512 * 4
    assert full % 256 == 0
    assert _ws(0, p, 8, 65536, 8192) == full              # deterministic
    assert _ws(0, p, 16, 65536, 8192) >= full              # more users, more items
    assert _ws(0, p, 8, 131072, 8192) > full               # more tokens
    cached = _ws(1, p, 8, 1024, 8320)
    assert cached >= 1024 * 512 * 4 * 2                    # at least two key splits of O
    assert _ws(2, p, 4, 20480, 5120) >= 20480 * 512 * 4
    assert _ws(3, p, 4, 4096, 4096) >= 4096 * 512 * 4 * 8  # paged M-FALCON: eight key splits of O
    assert _ws(3, p, 4, 4096, 4097) >= _ws(3, p, 4, 4096, 4096)
    assert _ws(7, p, 8, 1024, 1024) == 0                   # unknown entry point
    assert _ws(0, _params(dtype=5), 8, 1024, 128) == 0      # unknown dtype
    assert _ws(0, _params(head_dim=48), 8, 1024, 128) == 0  # unsupported head dim
    assert _ws(0, _params(num_heads=32), 8, 1024, 128) == 0  # H*d > 2048
    assert _ws(0, _params(num_heads=0), 8, 1024, 128) == 0
    assert _ws(0, p, -1, 1024, 128) == 0
    assert _ws(0, _params(ln_eps=0.0), 8, 1024, 128) == 0
    assert _ws(0, _params(flags=hs.HSTU_FLAG_FP32_NORM_INPUT), 8, 65536, 8192) == full  # same workspace
    assert _ws(0, _params(flags=hs.HSTU_FLAG_SAVED_FORWARD), 8, 65536, 8192) == full  # same workspace
    assert _ws(0, _params(flags=4), 8, 1024, 128) == 0          # unknown flag bit


FAKE = 0x10000  # aligned, never dereferenced: validation fails before any launch


def test_attn_fwd_rejects_bad_arguments_before_launch():
    lib = hs.lib()
    f = lib.hstu_attn_fwd

    def call(p, B=2, off=FAKE, L=16, T=32, q=FAKE, y=FAKE, ws=FAKE, wsb=0):
        return f(ctypes.byref(p), B, off, L, T, q, FAKE, FAKE, FAKE, FAKE, y, ws, wsb, None)

    assert call(_params(dtype=3)) == UNSUPPORTED
    assert call(_params(head_dim=16)) == UNSUPPORTED
    assert call(_params(num_heads=0)) == INVALID
    assert call(_params(norm_n=-1)) == INVALID
    assert call(_params(), B=-1) == INVALID
    assert call(_params(), q=None) == INVALID
    assert call(_params(), off=None) == INVALID
    assert call(_params(), q=FAKE + 4) == INVALID         # misaligned
    assert call(_params(), ws=None, wsb=1 << 30) == WORKSPACE
    assert call(_params(), wsb=16) == WORKSPACE           # too small
    pt = _params(pos_tab=FAKE, n_pos=0)
    assert call(pt) == INVALID
    assert call(_params(pos_tab=FAKE, n_pos=4096)) == UNSUPPORTED
    assert call(_params(time_tab=FAKE, n_time=0)) == INVALID
    assert call(_params(pos_tab=FAKE, n_pos=128, pos_head_stride=64)) == INVALID
    # empty work is a no-op that never touches the device
    assert call(_params(), B=0) == OK
    assert call(_params(), T=0) == OK


def test_cached_and_mfalcon_and_append_reject_bad_arguments():
    lib = hs.lib()
    c = hs._KVCache()
    c.k_pages = c.v_pages = c.ts_pages = c.page_table = FAKE
    c.num_pages, c.page_size, c.max_pages_per_seq = 10, 64, 4
    p = _params()
    r = lib.hstu_attn_fwd_cached(ctypes.byref(p), 2, FAKE, FAKE, 16, 200, 32, FAKE, FAKE, FAKE, ctypes.byref(c),
                                 FAKE, FAKE, 0, None)
    assert r == WORKSPACE
    # max_total beyond what the page table can address
    r = lib.hstu_attn_fwd_cached(ctypes.byref(p), 2, FAKE, FAKE, 16, 4 * 64 + 1, 32, FAKE, FAKE, FAKE,
                                 ctypes.byref(c), FAKE, FAKE, 1 << 40, None)
    assert r == INVALID
    c.page_size = 32
    r = lib.hstu_attn_fwd_cached(ctypes.byref(p), 2, FAKE, FAKE, 16, 200, 32, FAKE, FAKE, FAKE, ctypes.byref(c),
                                 FAKE, FAKE, 1 << 40, None)
    assert r == UNSUPPORTED
    assert lib.hstu_kv_append(ctypes.byref(c), ctypes.byref(p), 2, FAKE, FAKE, 32, FAKE, FAKE, FAKE, None) == UNSUPPORTED
    c.page_size = 64
    assert lib.hstu_kv_append(ctypes.byref(c), ctypes.byref(p), 2, None, FAKE, 32, FAKE, FAKE, FAKE, None) == INVALID
    assert lib.hstu_kv_append(ctypes.byref(c), ctypes.byref(p), 0, FAKE, FAKE, 32, FAKE, FAKE, FAKE, None) == OK
    r = lib.hstu_mfalcon_fwd(ctypes.byref(p), 2, FAKE, None, 16, 32, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                             1 << 40, None)
    assert r == INVALID
    r = lib.hstu_mfalcon_fwd(ctypes.byref(p), 2, FAKE, FAKE, 16, 32, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, None)
    assert r == WORKSPACE


def test_noalloc_cached_rejects_before_touching_the_gpu():
    # every case here returns before the scratch lookup (the first HIP call),
    # so it is safe with fake pointers on any machine
    lib = hs.lib()
    c = hs._KVCache()
    c.k_pages = c.v_pages = c.ts_pages = c.page_table = FAKE
    c.num_pages, c.page_size, c.max_pages_per_seq = 1000, 64, 200
    p = _params()
    f = lib.hstu_attn_fwd_cached_noalloc
    assert hs.HSTU_NOALLOC_SCRATCH_BYTES == 64 << 20
    # the KV-delta serving shape fits: 8 users x 128 new, 8,320 keys, 4 x 128
    need = lib.hstu_workspace_size(hs.HSTU_FN_CACHED, ctypes.byref(p), 8, 1024, 8320)
    assert 0 < need <= hs.HSTU_NOALLOC_SCRATCH_BYTES
    # 32,768 new tokens over 12,800 keys need more than the scratch holds
    big = lib.hstu_workspace_size(hs.HSTU_FN_CACHED, ctypes.byref(p), 8, 32768, 12800)
    assert big > hs.HSTU_NOALLOC_SCRATCH_BYTES
    assert f(ctypes.byref(p), 8, FAKE, FAKE, 4096, 12800, 32768, FAKE, FAKE, FAKE, ctypes.byref(c), FAKE,
             None) == WORKSPACE
    # argument checks as in hstu_attn_fwd_cached
    assert f(ctypes.byref(p), 8, FAKE, None, 128, 8320, 1024, FAKE, FAKE, FAKE, ctypes.byref(c), FAKE,
             None) == INVALID
    assert f(ctypes.byref(p), 8, FAKE, FAKE, 128, 200 * 64 + 1, 1024, FAKE, FAKE, FAKE, ctypes.byref(c), FAKE,
             None) == INVALID
    c.page_size = 32
    assert f(ctypes.byref(p), 8, FAKE, FAKE, 128, 8320, 1024, FAKE, FAKE, FAKE, ctypes.byref(c), FAKE,
             None) == UNSUPPORTED
    c.page_size = 64
    assert f(ctypes.byref(p), 0, FAKE, FAKE, 128, 8320, 0, FAKE, FAKE, FAKE, ctypes.byref(c), FAKE, None) == OK


def test_layer_workspace_and_bad_arguments_before_launch():
    lib = hs.lib()
    p = _params(num_heads=8)
    size = lambda p, E, B, T, L: int(lib.hstu_layer_workspace_size(ctypes.byref(p), E, B, T, L))
    n = size(p, 1024, 16, 45800, 8192)
    # U, V, Q, K and the attention output in bf16, plus the attention workspace
    assert n >= 5 * 45800 * 1024 * 2 + _ws(0, p, 16, 45800, 8192)
    assert size(p, 1024, 16, 45801, 8192) >= n and size(p, 1024, 17, 45800, 8192) >= n
    assert size(p, 1024, 16, 45800, 8193) >= n
    assert size(p, 1020, 16, 45800, 8192) == 0          # E not a multiple of 8
    assert size(_params(num_heads=8, dtype=0), 1024, 16, 45800, 8192) == 0  # fp32 layer unsupported
    f = lib.hstu_layer_fwd
    w = hs._LayerWeights(1024, FAKE, FAKE)

    def call(p, w=w, B=2, T=32, x=FAKE, wsb=0):
        return f(ctypes.byref(p), ctypes.byref(w), B, FAKE, 16, T, x, FAKE, FAKE, FAKE, wsb, None)

    assert call(_params(dtype=0)) == UNSUPPORTED
    assert call(p, w=hs._LayerWeights(1020, FAKE, FAKE)) == INVALID
    assert call(p, w=hs._LayerWeights(1024, None, FAKE)) == INVALID
    assert call(p, w=hs._LayerWeights(1024, FAKE, FAKE, 3)) == INVALID       # unknown product backend
    assert call(p, w=hs._LayerWeights(1000, FAKE, FAKE, 1)) == UNSUPPORTED   # own products need E % 256 == 0
    # AUTO falls back to hipBLASLt where the own kernel does not fit: the
    # call gets as far as the workspace check
    assert call(p, w=hs._LayerWeights(1000, FAKE, FAKE, 2)) == WORKSPACE
    assert call(p, x=None) == INVALID
    assert call(p, x=FAKE + 2) == INVALID
    assert call(_params(head_dim=48)) == INVALID
    assert call(p) == WORKSPACE
    assert call(p, B=0) == OK


def test_paged_mfalcon_rejects_bad_arguments_before_launch():
    lib = hs.lib()
    c = hs._KVCache()
    c.k_pages = c.v_pages = c.ts_pages = c.page_table = FAKE
    c.num_pages, c.page_size, c.max_pages_per_seq = 10, 64, 4
    p = _params()
    f = lib.hstu_mfalcon_fwd_cached

    def call(p=p, c=c, B=2, T=32, max_hist=200, q=FAKE, wsb=0):
        return f(ctypes.byref(p), B, FAKE, FAKE, 16, max_hist, T, q, FAKE, FAKE, FAKE, FAKE, ctypes.byref(c), FAKE,
                 FAKE, wsb, None)

    assert call() == WORKSPACE
    assert call(max_hist=4 * 64 + 1, wsb=1 << 40) == INVALID   # history beyond the page table
    assert call(q=None, wsb=1 << 40) == INVALID
    assert call(q=FAKE + 8, wsb=1 << 40) == INVALID
    assert call(p=_params(head_dim=48)) == UNSUPPORTED
    assert call(B=0) == OK
    assert call(T=0) == OK
    c.page_size = 32
    assert call(wsb=1 << 40) == UNSUPPORTED


def test_backward_workspace_and_bad_arguments_before_launch():
    lib = hs.lib()
    p = _params()
    fwd, bwd = _ws(0, p, 8, 8192, 1024), _ws(4, p, 8, 8192, 1024)
    assert bwd >= fwd + 8192 * 512 * 2                   # plus the bf16 gradient reaching O
    tab = _params(pos_tab=FAKE, n_pos=128, ln_w=FAKE)
    assert _ws(4, tab, 8, 8192, 1024) > bwd               # table and affine partials
    f = lib.hstu_attn_bwd

    def call(p=p, g=None, B=2, T=32, q=FAKE, wsb=0, grads=True):
        if g is None:
            g = hs._Grads(FAKE, FAKE, FAKE, FAKE, None, None, None, None)
        return f(ctypes.byref(p), B, FAKE, 16, T, q, FAKE, FAKE, FAKE, FAKE, FAKE,
                 ctypes.byref(g) if grads else None, FAKE, wsb, None)

    assert call() == WORKSPACE
    assert call(p=_params(dtype=0)) == UNSUPPORTED                            # fp32
    assert call(p=_params(pos_tab=FAKE, n_pos=513)) == UNSUPPORTED            # position table too long
    assert call(grads=False, wsb=1 << 40) == INVALID
    assert call(g=hs._Grads(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None), wsb=1 << 40) == INVALID  # no table
    assert call(g=hs._Grads(FAKE, FAKE, FAKE, None, None, None, None, None), wsb=1 << 40) == INVALID  # no du
    assert call(q=None, wsb=1 << 40) == INVALID
    assert call(q=FAKE + 4, wsb=1 << 40) == INVALID
    assert call(p=_params(head_dim=48)) == UNSUPPORTED
    both = hs.HSTU_FLAG_SAVED_FORWARD | hs.HSTU_FLAG_FP32_NORM_INPUT
    assert call(p=_params(flags=both), wsb=1 << 40) == INVALID  # a saved forward has no fp32 store
    assert call(B=0, wsb=1 << 40) == OK      # nothing to compute and no table or affine gradient requested
    assert call(p=_params(flags=hs.HSTU_FLAG_SAVED_FORWARD), B=0, wsb=1 << 40) == OK


def test_matmul_rejects_bad_arguments_before_launch():
    f = hs.lib().hstu_matmul_bf16
    call = lambda M=512, N=256, K=64, a=FAKE, epi=0, w=0: f(M, N, K, a, FAKE, FAKE, epi, w, None)
    assert call(N=100) == UNSUPPORTED
    assert call(K=96) == UNSUPPORTED
    assert call(M=-1) == INVALID
    assert call(epi=7) == INVALID
    assert call(epi=1, w=48) == UNSUPPORTED
    assert call(epi=1, w=96) == UNSUPPORTED      # does not divide N
    assert call(a=None) == INVALID
    assert call(a=FAKE + 2) == INVALID
    assert call(M=0) == OK


def test_pair_count_matches_closed_forms():
    assert hs.pair_count("full", [8192] * 8) == 8 * 8192 * 8193 // 2
    assert hs.pair_count("cached", [128] * 8, [8192] * 8) == 8 * (128 * 8192 + 128 * 129 // 2)
    assert hs.pair_count("mfalcon", [4096] * 4, [1024] * 4) == 4 * (4096 * 4097 // 2 + 1024 * 4097)


def test_debug_mode_constants_match_header():
    import re
    hdr = open(os.path.join(os.path.dirname(__file__), "..", "include", "hstu.h")).read()
    assert int(re.search(r"#define HSTU_WS_DEBUG_FLAG_OFFSET (\d+)", hdr).group(1)) == hs.HSTU_WS_DEBUG_FLAG_OFFSET
    for name in ("OFFSETS", "LENGTH", "CANDIDATES", "CACHE_LEN", "PAGE"):
        val = int(re.search(rf"HSTU_DEBUG_BAD_{name} = (\d+)", hdr).group(1))
        assert val == getattr(hs, f"HSTU_DEBUG_BAD_{name}"), name
    assert hs.HSTU_WS_DEBUG_FLAG_OFFSET + 4 <= 256   # inside the 256-byte header, after the item count
