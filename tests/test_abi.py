"""CPU tests of the C ABI: the library loads, exports every function include/invattn.h declares,
and rejects bad configurations and arguments on the host before anything is launched (no GPU
call is made by any test here)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from invariant_attention_amd import binding as ia

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "invattn.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = set(re.findall(r"\b(ia_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def test_library_exports_every_declared_function():
    ia.load()
    out = subprocess.run(["nm", "-D", "--defined-only", ia.LIB_PATH], capture_output=True, text=True, check=True)
    exported = set(re.findall(r"\sT\s+(ia_\w+)", out.stdout))
    declared = _declared_functions()
    assert len(declared) >= 20
    missing = [n for n in declared if n not in exported]
    assert not missing, missing
    assert set(declared) == set(ia.EXPORTS)


def test_version_and_clean_error_state():
    assert "gfx950" in ia.ia_version()


@pytest.mark.parametrize("kw,msg", [
    (dict(Hq=32, Hkv=8, d=96), "head_dim"),
    (dict(Hq=30, Hkv=8, d=128), "multiple"),
    (dict(Hq=64, Hkv=2, d=128), "<= 16"),
    (dict(Hq=32, Hkv=8, d=128, page_size=32), "page_size"),
    (dict(Hq=32, Hkv=8, d=128, split_tokens=100), "split_tokens"),
    (dict(Hq=32, Hkv=8, d=128, split_tokens=0), "split_tokens"),
    (dict(Hq=32, Hkv=8, d=128, kv_dtype=7), "kv_dtype"),
    (dict(Hq=32, Hkv=8, d=128, split_policy=3), "split_policy"),
    (dict(Hq=32, Hkv=8, d=128, sm_scale=-1.0), "sm_scale"),
    (dict(Hq=32, Hkv=8, d=128, sliding_window=-1), "sliding_window"),
    (dict(Hq=32, Hkv=8, d=128, decode_kernel=4), "decode_kernel"),
    (dict(Hq=32, Hkv=8, d=128, kv_cache_hint=3), "kv_cache_hint"),
    (dict(Hq=32, Hkv=8, d=128, prefill_grid=3), "prefill_grid"),
])
def test_unsupported_configs_are_rejected(kw, msg):
    Hq, Hkv, d = kw.pop("Hq"), kw.pop("Hkv"), kw.pop("d")
    with pytest.raises(ia.IAError) as e:
        ia.Context(ia.make_config(Hq, Hkv, d, **kw))
    assert e.value.status == ia.IA_ERR_UNSUPPORTED_CONFIG and msg in str(e.value)


def test_workspace_size_formula():
    ctx = ia.Context(ia.make_config(32, 8, 128, split_tokens=2048))
    # B * ceil(max_len / S) * Hq rows of (d + 2) floats, plus one int32 per (sequence, split) for
    # the dispatch order, each array rounded up to 256 bytes
    got = ia.ia_decode_workspace_bytes(ctx, 256, 8192)
    rows = 256 * 4 * 32
    up = lambda x: (x + 255) // 256 * 256
    assert got == up(rows * 128 * 4) + up(rows * 2 * 4) + up(256 * 4 * 4)
    assert ia.ia_decode_workspace_bytes(ctx, 0, 8192) == 0
    bc = ia.Context(ia.make_config(32, 8, 128, split_policy=ia.IA_SPLIT_BY_COUNT))
    # a launch of at most 32 split units runs the spread kernels, which add one slot per
    # (sequence, split, kv head, tile): group x 64 fp32 scores, 16 fp32 row maxima, 16 (alpha, sum, max, 0)
    slots = 1 * 4 * 8 * 32
    assert ia.ia_decode_workspace_bytes(ctx, 1, 8192) == (up(4 * 32 * 128 * 4) + up(4 * 32 * 2 * 4) + up(4 * 4)
                                                         + up(slots * 4 * 64 * 4) + up(slots * 16 * 4)
                                                         + up(slots * 16 * 4 * 4))
    split_only = ia.Context(ia.make_config(32, 8, 128, split_tokens=2048, decode_kernel=ia.IA_DECODE_SPLIT))
    assert ia.ia_decode_workspace_bytes(split_only, 1, 8192) == up(4 * 32 * 128 * 4) + up(4 * 32 * 2 * 4) + up(16)
    # split-by-count: at most min(64, 256 // B) pieces, and no more than one per 64-key tile
    assert ia.ia_decode_workspace_bytes(bc, 1, 64) == (up(1 * 1 * 32 * 128 * 4) + up(32 * 2 * 4) + up(4)
                                                       + up(8 * 4 * 64 * 4) + up(8 * 16 * 4) + up(8 * 16 * 4 * 4))
    assert ia.ia_decode_workspace_bytes(bc, 4, 100000) == (up(4 * 64 * 32 * 128 * 4) + up(4 * 64 * 32 * 2 * 4)
                                                          + up(4 * 64 * 4))
    # prefill: none while no row can see keys of two splits; else per (query row, head) a state of
    # d + 2 floats (two arrays rounded up to 256 bytes), and for the split grid B x r row blocks of
    # 32 positions (group 4, bf16) x the splits past the first x Hq more, r = min(4, row blocks)
    def states(e):
        return up(e * 128 * 4) + up(e * 2 * 4)
    assert ia.ia_prefill_workspace_bytes(ctx, 8, 1000, 125, 2048) == 0
    assert ia.ia_prefill_workspace_bytes(ctx, 0, 0, 0, 4096) == 0
    # 8 sequences, 125 rows each (4 row blocks), keys up to 2049 (2 splits)
    assert ia.ia_prefill_workspace_bytes(ctx, 8, 1000, 125, 2049) == states(1000 * 32) + states(8 * 4 * 32 * 1 * 32)
    # up to 8192 keys: 3 splits past the first; at most 300 rows: 10 row blocks, 4 of them split
    assert ia.ia_prefill_workspace_bytes(ctx, 4, 1000, 300, 8192) == states(1000 * 32) + states(4 * 4 * 32 * 3 * 32)
    # ... unless total_q leaves no room for a sequence of at most 4 row blocks (128 positions)
    assert ia.ia_prefill_workspace_bytes(ctx, 4, 1029, 300, 8192) == states(1029 * 32)
    assert ia.ia_prefill_workspace_bytes(ctx, 4, 1028, 300, 8192) == states(1028 * 32) + states(4 * 4 * 32 * 3 * 32)
    # 1 sequence of 64 rows: 8 workgroups with 2 row blocks per wave, fewer than the 256 compute
    # units, so 1 row block per wave (16 positions per workgroup): 4 row blocks, all split
    assert ia.ia_prefill_workspace_bytes(ctx, 1, 64, 64, 4096) == states(64 * 32) + states(1 * 4 * 16 * 1 * 32)
    # 8 sequences of 64 rows (the Qwen3-8B chunks of 64): 128 workgroups, 1 row block per wave
    assert ia.ia_prefill_workspace_bytes(ctx, 8, 512, 64, 4096) == states(512 * 32) + states(8 * 4 * 16 * 1 * 32)
    # 8192 or more (sequence, row block, kv head) workgroups: folds only
    assert ia.ia_prefill_workspace_bytes(ctx, 8, 8 * 4096, 4096, 4096) == states(8 * 4096 * 32)
    # split states over 128 MiB: the row blocks split per sequence halve until they fit (here to 1)
    big = ia.ia_prefill_workspace_bytes(ctx, 8, 800, 100, 65536)
    assert big == states(800 * 32) + states(8 * 1 * 32 * 31 * 32)
    # a launch of 8192 or more workgroups with few row blocks: folds only
    assert ia.ia_prefill_workspace_bytes(ctx, 1024, 1024, 1, 65536) == states(1024 * 32)
    fold = ia.Context(ia.make_config(32, 8, 128, split_tokens=2048, prefill_grid=ia.IA_PREFILL_FOLD))
    assert ia.ia_prefill_workspace_bytes(fold, 8, 1000, 125, 2049) == states(1000 * 32)
    split = ia.Context(ia.make_config(32, 8, 128, split_tokens=2048, prefill_grid=ia.IA_PREFILL_SPLIT))
    assert ia.ia_prefill_workspace_bytes(split, 4, 1200, 300, 8192) == states(1200 * 32) + states(4 * 10 * 32 * 3 * 32)
    # the Qwen3-8B chunks of 256 (8 x 256 rows, 8 row blocks each) split nothing under AUTO
    assert ia.ia_prefill_workspace_bytes(ctx, 8, 2048, 256, 4096) == states(2048 * 32)


FAKE = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails validation first


def _decode(ctx, **over):
    args = dict(q=FAKE, kc=FAKE, vc=FAKE, num_pages=10, ks=None, vs=None, bt=FAKE, bt_stride=512, sl=FAKE,
                B=4, max_seq_len=8192, out=FAKE, ws=FAKE, ws_bytes=1 << 30)
    args.update(over)
    lib = ia.load()
    return lib.ia_paged_attn_decode(ctx.handle, args["q"], args["kc"], args["vc"], args["num_pages"], args["ks"],
                                    args["vs"], args["bt"], args["bt_stride"], args["sl"], args["B"],
                                    args["max_seq_len"], args["out"], args["ws"], args["ws_bytes"], None)


def test_decode_argument_errors_launch_nothing():
    ctx = ia.Context(ia.make_config(32, 8, 128))
    assert _decode(ctx, B=0) == ia.IA_OK  # empty batch: nothing to do
    assert _decode(ctx, B=-1) == ia.IA_ERR_INVALID_ARG
    assert _decode(ctx, ws_bytes=100) == ia.IA_ERR_WORKSPACE_TOO_SMALL
    assert "workspace" in ia.ia_last_error()
    assert _decode(ctx, bt_stride=10) == ia.IA_ERR_INVALID_ARG  # 10 pages cannot hold 8192 keys
    assert _decode(ctx, num_pages=0) == ia.IA_ERR_INVALID_ARG
    assert _decode(ctx, q=None) == ia.IA_ERR_INVALID_ARG
    assert _decode(ctx, max_seq_len=0) == ia.IA_ERR_INVALID_ARG
    assert _decode(ctx, ks=FAKE) == ia.IA_ERR_INVALID_ARG  # scales only for fp8 pages
    assert _decode(ctx, q=ctypes.c_void_p((1 << 20) + 2)) == ia.IA_ERR_INVALID_ARG  # misaligned
    fp8 = ia.Context(ia.make_config(32, 8, 128, kv_dtype=ia.IA_KV_FP8_E4M3))
    assert _decode(fp8) == ia.IA_ERR_INVALID_ARG  # fp8 pages need scales


def test_append_and_prefill_argument_errors():
    ctx = ia.Context(ia.make_config(8, 2, 64, split_tokens=128))
    lib = ia.load()
    assert lib.ia_kv_append(ctx.handle, FAKE, FAKE, FAKE, 0, FAKE, FAKE, 4, None, None, None) == ia.IA_OK
    assert lib.ia_kv_append(ctx.handle, FAKE, FAKE, FAKE, -1, FAKE, FAKE, 4, None, None, None) == ia.IA_ERR_INVALID_ARG
    assert lib.ia_kv_append(ctx.handle, None, FAKE, FAKE, 3, FAKE, FAKE, 4, None, None, None) == ia.IA_ERR_INVALID_ARG
    assert lib.ia_kv_append(ctx.handle, FAKE, FAKE, FAKE, 3, None, FAKE, 4, None, None, None) == ia.IA_ERR_INVALID_ARG
    pre = lib.ia_paged_attn_prefill
    assert pre(ctx.handle, FAKE, FAKE, FAKE, FAKE, FAKE, 4, None, None, FAKE, 64, 0, 0, 0, 0, FAKE, None, 0,
               None) == ia.IA_OK
    assert pre(ctx.handle, FAKE, FAKE, FAKE, FAKE, FAKE, 4, None, None, FAKE, 1, 2, 10, 5, 100, FAKE, None, 0,
               None) == ia.IA_ERR_INVALID_ARG  # bt_stride too small for max_seq_len
    assert pre(ctx.handle, FAKE, None, FAKE, FAKE, FAKE, 4, None, None, FAKE, 64, 2, 10, 5, 100, FAKE, None, 0,
               None) == ia.IA_ERR_INVALID_ARG
    assert pre(ctx.handle, FAKE, FAKE, FAKE, FAKE, FAKE, 4, None, None, FAKE, 64, 2, 10, 0, 100, FAKE, None, 0,
               None) == ia.IA_ERR_INVALID_ARG  # rows but max_q_len 0
    # keys past one split (128) need the workspace
    assert pre(ctx.handle, FAKE, FAKE, FAKE, FAKE, FAKE, 4, None, None, FAKE, 64, 2, 10, 5, 200, FAKE, None, 0,
               None) == ia.IA_ERR_WORKSPACE_TOO_SMALL
    assert "workspace" in ia.ia_last_error()
    # the launch needs at least the row states (10 rows x 8 heads); the size returned also holds
    # the split states: 2 sequences x 1 row block x 1 more split x 8 heads, the row block of 16
    # positions (a launch this small runs one 16-row block per wave: 4 positions x 4 waves)
    up = lambda x: (x + 255) // 256 * 256
    need = up(10 * 8 * 64 * 4) + up(10 * 8 * 2 * 4)
    assert ia.ia_prefill_workspace_bytes(ctx, 2, 10, 5, 200) == need + up(2 * 16 * 8 * 64 * 4) + up(2 * 16 * 8 * 2 * 4)
    assert pre(ctx.handle, FAKE, FAKE, FAKE, FAKE, FAKE, 4, None, None, FAKE, 64, 2, 10, 5, 200, FAKE, FAKE, need - 1,
               None) == ia.IA_ERR_WORKSPACE_TOO_SMALL


def test_binding_constants_match_header():
    import re
    hdr = open(os.path.join(os.path.dirname(__file__), "..", "include", "invattn.h")).read()
    for name in ("IA_DECODE_AUTO", "IA_DECODE_SPLIT", "IA_DECODE_WIDE", "IA_DECODE_SPREAD", "IA_SPLIT_FIXED", "IA_SPLIT_BY_COUNT",
                 "IA_KV_HINT_AUTO", "IA_KV_HINT_STREAM", "IA_KV_HINT_CACHED", "IA_PREFILL_AUTO", "IA_PREFILL_FOLD",
                 "IA_PREFILL_SPLIT"):
        m = re.search(name + r" = (\d+)", hdr)
        assert m and int(m.group(1)) == getattr(ia, name), name


@pytest.mark.parametrize("M,H,eps,msg", [(4, 12, 1e-5, "multiple of 8"), (4, 0, 1e-5, "multiple of 8"),
                                         (4, 16392, 1e-5, "multiple of 8"), (4, 64, -1.0, "eps"),
                                         (4, 64, float("inf"), "eps"), (-1, 64, 1e-5, "M must"),
                                         (4, 64, 1e-5, "NULL")])
def test_rmsnorm_argument_errors_launch_nothing(M, H, eps, msg):
    lib = ia.load()
    st = lib.ia_rmsnorm(None, None, M, H, eps, None, None)
    assert st == ia.IA_ERR_INVALID_ARG and msg in lib.ia_last_error().decode()


@pytest.mark.parametrize("M,N,K,msg", [(4, 100, 64, "N must"), (4, 0, 64, "N must"), (4, 128, 64, "N must"),
                                       (4, 256, 48, "K must"), (4, 256, 0, "K must"), (-2, 256, 64, "M must"),
                                       (4, 256, 64, "NULL")])
def test_gemm_argument_errors_launch_nothing(M, N, K, msg):
    lib = ia.load()
    st = lib.ia_gemm_bf16(None, None, M, N, K, None, None)
    assert st == ia.IA_ERR_INVALID_ARG and msg in lib.ia_last_error().decode()


def test_layer_ops_empty_batch_is_a_noop_without_pointers():
    lib = ia.load()
    assert lib.ia_rmsnorm(None, None, 0, 64, 1e-5, None, None) == ia.IA_OK
    assert lib.ia_gemm_bf16(None, None, 0, 256, 64, None, None) == ia.IA_OK


def test_header_is_plain_c_and_config_layout_matches_binding(tmp_path):
    """include/invattn.h compiles as C99 (-pedantic, no warnings), and a C caller's ia_config has
    the size and field offsets the ctypes binding passes."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    fields = [f for f, _ in ia.ia_config._fields_]
    src = tmp_path / "hdr.c"
    src.write_text("#include <stddef.h>\n#include <stdio.h>\n#include \"invattn.h\"\nint main(void) {\n"
                   "  printf(\"%zu\", sizeof(ia_config));\n"
                   + "".join(f"  printf(\" %zu\", offsetof(ia_config, {f}));\n" for f in fields)
                   + "  return 0;\n}\n")
    exe = tmp_path / "hdr"
    proc = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I",
                           os.path.dirname(HEADER), "-o", str(exe), str(src)], capture_output=True, text=True)
    assert proc.returncode == 0, proc.stderr
    out = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert out[0] == ctypes.sizeof(ia.ia_config)
    assert out[1:] == [getattr(ia.ia_config, f).offset for f in fields]


def test_prefill_workspace_bounds_over_random_launch_shapes():
    """Over random launch bounds: no workspace while no row can see two splits; otherwise at
    least the per-row states (what the launch requires), at most 128 MiB more for the split grid
    (plus alignment), and exactly the per-row states under IA_PREFILL_FOLD."""
    rng = np.random.default_rng(5)
    up = lambda x: (x + 255) // 256 * 256
    for Hq, Hkv, d, S in ((32, 8, 128, 2048), (64, 4, 128, 2048), (8, 2, 64, 128)):
        auto = ia.Context(ia.make_config(Hq, Hkv, d, split_tokens=S))
        fold = ia.Context(ia.make_config(Hq, Hkv, d, split_tokens=S, prefill_grid=ia.IA_PREFILL_FOLD))
        split = ia.Context(ia.make_config(Hq, Hkv, d, split_tokens=S, prefill_grid=ia.IA_PREFILL_SPLIT))
        for _ in range(300):
            B = int(rng.integers(1, 300))
            mql = int(rng.integers(1, 5000))
            total_q = int(rng.integers(1, B * mql + 1))
            msl = int(rng.integers(mql, 140000))
            rows = total_q * Hq
            need = up(rows * d * 4) + up(rows * 2 * 4) if msl > S else 0
            assert ia.ia_prefill_workspace_bytes(fold, B, total_q, mql, msl) == need
            for c in (auto, split):
                got = ia.ia_prefill_workspace_bytes(c, B, total_q, mql, msl)
                assert need <= got <= need + (128 << 20) + 512, (B, total_q, mql, msl, got, need)
                assert (got == 0) == (msl <= S)
