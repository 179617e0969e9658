"""C-ABI checks that need no GPU: the library loads, exports every function
include/pkv.h declares, and rejects bad arguments on the host (these paths
return before any HIP call)."""
import ctypes
import os
import re

import pytest

from paged_kv_gqa_pkv_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bd.LIB_PATH):
        pytest.fail("libpkv.so is not built (run python -m paged_kv_gqa_pkv_amd.build)")
    return bd.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"pkv_append", "pkv_attn_decode", "pkv_attn_prefill_chunk", "pkv_slot_mapping",
            "pkv_decode_workspace_bytes", "pkv_prefill_workspace_bytes",
            "pkv_last_error"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
        assert n in bd.SIGNATURES, f"binding lacks {n}"


def test_version(lib):
    assert b"gfx950" in lib.pkv_version()


NULL = None


def test_append_rejects_bad_arguments(lib):
    # block size other than 16
    assert lib.pkv_append(1, 1, 1, 1, 2, 4, 8, 8, 128, 8, NULL) == bd.PKV_EUNSUPPORTED
    # head_dim other than 128
    assert lib.pkv_append(1, 1, 1, 1, 2, 4, 8, 8, 64, 16, NULL) == bd.PKV_EUNSUPPORTED
    assert b"head_dim" in lib.pkv_last_error()
    # null pointers with tokens to write
    assert lib.pkv_append(NULL, 1, 1, 1, 2, 4, 8, 8, 128, 16, NULL) == bd.PKV_EINVAL
    # same pool for K and V
    assert lib.pkv_append(1, 1, 1, 5, 5, 4, 8, 8, 128, 16, NULL) == bd.PKV_EINVAL
    # negative sizes
    assert lib.pkv_append(1, 1, 1, 1, 2, -1, 8, 8, 128, 16, NULL) == bd.PKV_EINVAL
    # nothing to do is fine and launches nothing
    assert lib.pkv_append(NULL, NULL, NULL, NULL, NULL, 0, 8, 8, 128, 16, NULL) == bd.PKV_OK


def test_slot_mapping_rejects_bad_arguments(lib):
    assert lib.pkv_slot_mapping(1, 1, 1, 1, 2, 4, 3, 8, NULL) == bd.PKV_EUNSUPPORTED
    assert lib.pkv_slot_mapping(NULL, 1, 1, 1, 2, 4, 3, 16, NULL) == bd.PKV_EINVAL
    assert lib.pkv_slot_mapping(1, 1, 1, 1, 0, 4, 3, 16, NULL) == bd.PKV_EINVAL
    assert lib.pkv_slot_mapping(1, 1, 1, 1, -2, 4, 3, 16, NULL) == bd.PKV_EINVAL
    assert lib.pkv_slot_mapping(1, 1, 1, 1, 2, 1 << 27, 3, 16, NULL) == bd.PKV_EINVAL  # int32 positions
    assert lib.pkv_slot_mapping(NULL, NULL, NULL, NULL, 2, 4, 0, 16, NULL) == bd.PKV_OK


def _decode(lib, out=1, q=2, B=2, Hq=16, Hkv=8, D=128, bs=16, nb=32, mb=4, mcl=64, scale=0.088):
    return lib.pkv_attn_decode(out, q, 3, 4, 5, 6, B, Hq, Hkv, D, bs, nb, mb, mcl, scale,
                               NULL, 0, NULL)


def test_decode_rejects_bad_arguments(lib):
    assert _decode(lib, Hq=12, Hkv=8) == bd.PKV_EUNSUPPORTED       # Hq % Hkv
    assert _decode(lib, Hq=48, Hkv=16) == bd.PKV_EUNSUPPORTED      # group 3
    assert _decode(lib, Hq=32, Hkv=2) == bd.PKV_EUNSUPPORTED       # group 16
    assert _decode(lib, D=64) == bd.PKV_EUNSUPPORTED
    assert _decode(lib, bs=32) == bd.PKV_EUNSUPPORTED
    assert _decode(lib, out=NULL) == bd.PKV_EINVAL
    assert _decode(lib, out=7, q=7) == bd.PKV_EINVAL                # aliasing
    assert _decode(lib, mcl=65, mb=4) == bd.PKV_EINVAL              # beyond the table
    assert _decode(lib, mb=1 << 27) == bd.PKV_EINVAL                # wider than int32 positions
    assert _decode(lib, B=-1) == bd.PKV_EINVAL
    assert _decode(lib, Hkv=0) == bd.PKV_EINVAL
    assert _decode(lib, scale=float("nan")) == bd.PKV_EINVAL
    assert _decode(lib, B=0, out=NULL) == bd.PKV_OK


def test_prefill_rejects_bad_arguments(lib):
    def call(out=1, q=2, B=1, total_q=8, mq=8, Hq=16, Hkv=8, D=128, bs=16, mb=4, mcl=64):
        return lib.pkv_attn_prefill_chunk(out, q, 3, 4, 5, 6, 7, B, total_q, mq, Hq, Hkv, D, bs,
                                          32, mb, mcl, 0.088, NULL, 0, NULL)
    assert call(D=256) == bd.PKV_EUNSUPPORTED
    assert call(Hq=10, Hkv=4) == bd.PKV_EUNSUPPORTED
    assert call(q=NULL) == bd.PKV_EINVAL
    assert call(mq=9) == bd.PKV_EINVAL                               # max_q_len > total_q
    assert call(mcl=100, mb=4) == bd.PKV_EINVAL
    assert call(mb=1 << 27) == bd.PKV_EINVAL
    assert call(mcl=131073, mb=8193) == bd.PKV_EUNSUPPORTED           # past 32 x 64 x 64 keys
    assert call(total_q=0, out=NULL) == bd.PKV_OK


def test_header_documents_each_entry_point():
    """Each declaration carries a comment citing the passage it implements (or
    stating what it is for)."""
    src = open(HEADER).read()
    for name in declared_functions():
        m = re.search(r"^(?:const\s+)?\w+\s*\*?\s*" + name + r"\s*\(", src, flags=re.M)
        assert m, name
        before = src[:m.start()].rstrip()
        assert before.endswith("*/"), f"{name} has no comment right above its declaration"


def test_int8_entry_points_reject_bad_arguments(lib):
    # append: D other than 128, null scales, same code pool for K and V, same
    # scale array for K and V, nothing to do
    assert lib.pkv_append_int8(1, 1, 1, 16, 32, 48, 64, 4, 8, 8, 64, 16,
                               NULL) == bd.PKV_EUNSUPPORTED
    assert lib.pkv_append_int8(1, 1, 1, 16, 32, NULL, 64, 4, 8, 8, 128, 16, NULL) == bd.PKV_EINVAL
    assert lib.pkv_append_int8(1, 1, 1, 16, 32, 48, NULL, 4, 8, 8, 128, 16, NULL) == bd.PKV_EINVAL
    assert lib.pkv_append_int8(1, 1, 1, 16, 16, 48, 64, 4, 8, 8, 128, 16, NULL) == bd.PKV_EINVAL
    assert lib.pkv_append_int8(1, 1, 1, 16, 32, 48, 48, 4, 8, 8, 128, 16, NULL) == bd.PKV_EINVAL
    assert lib.pkv_append_int8(NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, 8, 8, 128, 16,
                               NULL) == bd.PKV_OK
    # decode: missing scales, group size 3
    assert lib.pkv_attn_decode_int8(1, 2, 3, 4, NULL, 9, 5, 6, 2, 16, 8, 128, 16, 32, 4, 64,
                                    0.088, NULL, 0, NULL) == bd.PKV_EINVAL
    assert lib.pkv_attn_decode_int8(1, 2, 3, 4, 8, NULL, 5, 6, 2, 16, 8, 128, 16, 32, 4, 64,
                                    0.088, NULL, 0, NULL) == bd.PKV_EINVAL
    assert lib.pkv_attn_decode_int8(1, 2, 3, 4, 8, 9, 5, 6, 2, 24, 8, 128, 16, 32, 4, 64, 0.088,
                                    NULL, 0, NULL) == bd.PKV_EUNSUPPORTED
    # prefill: missing scales, D other than 128, context past the table, nothing to do
    def pre(ks=5, vs=9, D=128, mcl=64, total_q=8, out=1):
        return lib.pkv_attn_prefill_chunk_int8(out, 2, 3, 4, 6, ks, vs, 7, 8, 1, total_q, 8, 16,
                                               8, D, 16, 32, 4, mcl, 0.088, NULL, 0, NULL)
    assert pre(ks=NULL) == bd.PKV_EINVAL
    assert pre(vs=NULL) == bd.PKV_EINVAL
    assert pre(D=64) == bd.PKV_EUNSUPPORTED
    assert pre(mcl=100) == bd.PKV_EINVAL
    assert pre(total_q=0, out=NULL, ks=NULL, vs=NULL) == bd.PKV_OK


def test_copy_blocks_rejects_bad_arguments(lib):
    call = lambda **k: lib.pkv_copy_blocks(
        k.get("kp", 16), k.get("vp", 32), 48, 64, k.get("n", 2), k.get("nb", 8),
        k.get("bb", 1024), k.get("layers", 1), k.get("stride", 0), NULL)
    assert call(n=-1) == bd.PKV_EINVAL
    assert call(bb=1000) == bd.PKV_EINVAL                      # not a multiple of 16
    assert call(kp=8) == bd.PKV_EINVAL                         # misaligned pool
    assert call(kp=16, vp=16) == bd.PKV_EINVAL                 # same pool twice
    assert call(layers=2, stride=4096) == bd.PKV_EINVAL         # layers overlap (8 x 1024 B)
    assert b"layer_stride" in lib.pkv_last_error()
    assert call(n=0) == bd.PKV_OK and call(layers=0) == bd.PKV_OK


def test_fused_norm_rope_append_rejects_bad_arguments(lib):
    p8 = [16, 32, 48, 64, 80, 96, 112, 128]
    tail = [144, 160, 176, 192, 208, 224]
    # block size 8, negative T, G = 3, null pool, NaN eps, nothing to do
    assert lib.pkv_qk_norm_rope_append(*p8, 4096, *tail, 2, 4, 3, 32, 16, 8, 128, 8, 1e-6,
                                       NULL) == bd.PKV_EUNSUPPORTED
    assert lib.pkv_qk_norm_rope_append(*p8, 4096, *tail, 2, 4, -3, 32, 16, 8, 128, 16, 1e-6,
                                       NULL) == bd.PKV_EINVAL
    assert lib.pkv_qk_norm_rope_append(*p8, 4096, *tail, 2, 4, 3, 32, 24, 8, 128, 16, 1e-6,
                                       NULL) == bd.PKV_EUNSUPPORTED
    assert lib.pkv_qk_norm_rope_append(*p8, 4096, *tail[:5], NULL, 2, 4, 3, 32, 16, 8, 128, 16,
                                       1e-6, NULL) == bd.PKV_EINVAL
    assert lib.pkv_qk_norm_rope_append(*p8, 4096, *tail, 2, 4, 3, 32, 16, 8, 128, 16,
                                       float("nan"), NULL) == bd.PKV_EINVAL
    assert lib.pkv_qk_norm_rope_append(*([NULL] * 8), 0, *([NULL] * 6), 0, 0, 0, 0, 16, 8, 128,
                                       16, 1e-6, NULL) == bd.PKV_OK


def test_ring_entry_points_reject_bad_windows(lib):
    # window not a multiple of 16, window beyond the table, chunk longer than the ring
    assert lib.pkv_slot_mapping_ring(1, 2, 3, 4, 2, 4, 3, 16, 40, NULL) == bd.PKV_EINVAL
    assert lib.pkv_slot_mapping_ring(1, 2, 3, 4, 2, 4, 3, 16, 128, NULL) == bd.PKV_EINVAL
    assert lib.pkv_attn_decode_ring(1, 2, 3, 4, 5, 6, 2, 16, 8, 128, 16, 32, 4, 500, 0, 0.088,
                                    NULL, 0, NULL) == bd.PKV_EINVAL
    assert lib.pkv_attn_prefill_chunk_ring(1, 2, 3, 4, 5, 6, 7, 1, 100, 100, 16, 8, 128, 16, 64,
                                           8, 1000, 64, 0.088, NULL, 0, NULL) == bd.PKV_EINVAL
    assert b"ring" in lib.pkv_last_error()


def test_noalloc_decode_rejects_shapes_beyond_its_array(lib):
    """pkv_attn_decode_noalloc refuses, on the host, a split plan whose
    partials do not fit the library's array (here 64 sequences x 64 heads at
    131072 tokens: about 65 MiB of partials), and checks arguments like
    pkv_attn_decode."""
    def call(B=64, Hq=64, Hkv=8, mb=8192, mcl=131072, out=1, q=2):
        return lib.pkv_attn_decode_noalloc(out, q, 3, 4, 5, 6, B, Hq, Hkv, 128, 16, 1 << 20, mb,
                                           mcl, 0.088, NULL)
    assert bd.pkv_decode_workspace_bytes(64, 64, 8, 128, 131072) > 16 << 20
    assert call() == bd.PKV_EWORKSPACE
    assert b"pkv_attn_decode with a workspace" in lib.pkv_last_error()
    assert call(Hq=24) == bd.PKV_EUNSUPPORTED
    assert call(out=7, q=7) == bd.PKV_EINVAL
    assert call(mcl=131073) == bd.PKV_EINVAL                        # beyond the table
    assert call(B=0, out=NULL) == bd.PKV_OK


def test_fused_decode_append_rejects_bad_arguments(lib):
    """pkv_attn_decode_append checks what pkv_attn_decode checks, plus its new
    rows and two distinct pools."""
    def call(out=1, q=2, kn=3, vn=4, kc=5, vc=6, B=2, Hq=16, Hkv=8, D=128, bs=16, mb=4, mcl=64):
        return lib.pkv_attn_decode_append(out, q, kn, vn, kc, vc, 7, 8, B, Hq, Hkv, D, bs, 32,
                                          mb, mcl, 0.088, NULL, 0, NULL)
    assert call(kn=NULL) == bd.PKV_EINVAL
    assert call(vn=NULL) == bd.PKV_EINVAL
    assert call(kc=9, vc=9) == bd.PKV_EINVAL                       # one pool for K and V
    assert call(Hq=24) == bd.PKV_EUNSUPPORTED
    assert call(D=64) == bd.PKV_EUNSUPPORTED
    assert call(mcl=65) == bd.PKV_EINVAL                            # beyond the table
    assert call(out=7, q=7) == bd.PKV_EINVAL
    assert call(B=0, out=NULL, kn=NULL) == bd.PKV_OK


def test_fused_int8_decode_append_rejects_bad_arguments(lib):
    """pkv_attn_decode_append_int8 checks what pkv_attn_decode_int8 checks,
    plus its new rows, two distinct code pools and two distinct scale arrays."""
    def call(out=1, q=2, kn=3, vn=4, kc=5, vc=6, ks=10, vs=11, B=2, Hq=16, Hkv=8, D=128, mb=4,
             mcl=64):
        return lib.pkv_attn_decode_append_int8(out, q, kn, vn, kc, vc, ks, vs, 7, 8, B, Hq, Hkv,
                                               D, 16, 32, mb, mcl, 0.088, NULL, 0, NULL)
    assert call(ks=NULL) == bd.PKV_EINVAL
    assert call(vs=NULL) == bd.PKV_EINVAL
    assert call(kn=NULL) == bd.PKV_EINVAL
    assert call(vn=NULL) == bd.PKV_EINVAL
    assert call(kc=9, vc=9) == bd.PKV_EINVAL                       # one code pool for K and V
    assert call(ks=12, vs=12) == bd.PKV_EINVAL                     # one scale array for both
    assert b"scales" in lib.pkv_last_error()
    assert call(Hq=24) == bd.PKV_EUNSUPPORTED
    assert call(D=64) == bd.PKV_EUNSUPPORTED
    assert call(mcl=65) == bd.PKV_EINVAL                            # beyond the table
    assert call(B=0, out=NULL, kn=NULL, ks=NULL) == bd.PKV_OK


def _mixed(lib, out_p=1, out_d=2, Bp=1, T=64, mql=64, mclp=64, Bd=2, mcld=64, Hq=16, Hkv=8,
           D=128, mb=4, pws=NULL, pwb=0, dws=NULL, dwb=0):
    return lib.pkv_attn_prefill_decode(out_p, 3, 4, 5, 6, Bp, T, mql, mclp,
                                       out_d, 7, 8, 9, Bd, mcld, 10, 11, Hq, Hkv, D, 16, 32, mb,
                                       0.088, pws, pwb, dws, dwb, NULL)


def _mixed_int8(lib, out_p=1, out_d=2, Bp=1, T=64, mql=64, mclp=64, Bd=2, mcld=64, Hq=16,
                Hkv=8, D=128, mb=4, ks=12, vs=13):
    return lib.pkv_attn_prefill_decode_int8(out_p, 3, 4, 5, 6, Bp, T, mql, mclp,
                                            out_d, 7, 8, 9, Bd, mcld, 10, 11, ks, vs, Hq, Hkv, D,
                                            16, 32, mb, 0.088, NULL, 0, NULL, 0, NULL)


def test_prefill_decode_int8_rejects_bad_arguments(lib):
    assert _mixed_int8(lib, ks=NULL) == bd.PKV_EINVAL               # scales required
    assert _mixed_int8(lib, vs=NULL) == bd.PKV_EINVAL
    assert _mixed_int8(lib, Hq=12) == bd.PKV_EUNSUPPORTED           # Hq % Hkv
    assert _mixed_int8(lib, out_p=NULL) == bd.PKV_EINVAL
    assert _mixed_int8(lib, out_d=1) == bd.PKV_EINVAL               # one output for both halves
    assert b"outputs" in lib.pkv_last_error()
    assert _mixed_int8(lib, mql=65) == bd.PKV_EINVAL                # max_q_len > total_q
    assert _mixed_int8(lib, Bp=0, T=0, mql=0, Bd=0, ks=NULL, vs=NULL) == bd.PKV_OK


def test_prefill_decode_rejects_bad_arguments(lib):
    assert _mixed(lib, Hq=12) == bd.PKV_EUNSUPPORTED                # Hq % Hkv
    assert _mixed(lib, D=64) == bd.PKV_EUNSUPPORTED
    assert _mixed(lib, out_p=NULL) == bd.PKV_EINVAL                 # a half's null pointer
    assert _mixed(lib, out_d=NULL) == bd.PKV_EINVAL
    assert _mixed(lib, out_d=1) == bd.PKV_EINVAL                    # one output for both halves
    assert b"outputs" in lib.pkv_last_error()
    assert _mixed(lib, mql=65) == bd.PKV_EINVAL                     # max_q_len > total_q
    # a decode half that needs split buffers, given none
    need = bd.pkv_decode_workspace_bytes(2, 16, 8, 128, 64 * 16)
    assert need > 0
    assert _mixed(lib, mb=64, mcld=64 * 16) == bd.PKV_EWORKSPACE
    # the same buffer as both workspaces
    pneed = bd.pkv_prefill_workspace_bytes(1, 64, 16, 8, 128, 64 * 16)
    assert pneed > 0
    size = max(need, pneed)
    assert _mixed(lib, mb=64, mcld=64 * 16, mclp=64 * 16, pws=99, pwb=size, dws=99,
                  dwb=size) == bd.PKV_EINVAL
    assert b"workspaces" in lib.pkv_last_error()
    # nothing to do in either half
    assert _mixed(lib, Bp=0, T=0, mql=0, Bd=0) == bd.PKV_OK
