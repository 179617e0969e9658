"""Host-side split planners, through the C ABI on the CPU (no device: the
planners then assume 256 compute units, an MI355X).  The workspace queries
must cover every partial the kernels write, and the plans the measurements
and design notes quote are pinned."""
import itertools

import pytest

from paged_kv_gqa_pkv_amd import binding as bd

D = 128


@pytest.fixture(scope="module")
def lib():
    return bd.load()


def test_decode_workspace_covers_the_partials(lib):
    for B, (Hq, Hkv), ctx in itertools.product(
            [1, 2, 7, 13, 64, 160], [(16, 8), (32, 8), (8, 1), (64, 8)],
            [1, 16, 17, 255, 256, 4096, 5000, 32768, 131072]):
        S = bd.pkv_decode_num_splits(B, Hq, Hkv, D, ctx)
        ws = bd.pkv_decode_workspace_bytes(B, Hq, Hkv, D, ctx)
        assert S >= 1
        if S == 1:
            assert ws == 0, (B, Hq, Hkv, ctx)
        else:
            # (m, l) and acc per (sequence, query head, split), and at least
            # one arrival counter per sequence (one per (sequence, head group))
            assert ws >= B * Hq * S * (D + 2) * 4 + B * 4, (B, Hq, Hkv, ctx, S, ws)
            pages = -(-ctx // 16)
            assert S <= pages, (B, ctx, S)


def test_decode_plans_quoted_in_the_measurements(lib):
    assert bd.pkv_decode_num_splits(64, 32, 8, D, 4096) == 1      # c4a: one pass
    assert bd.pkv_decode_num_splits(13, 32, 8, D, 32768) == 9     # c4b: 9 x 228 pages
    assert bd.pkv_decode_num_splits(8, 16, 8, D, 1024) == 4       # c3: 4 x 16 pages
    assert bd.pkv_decode_num_splits(8, 16, 8, D, 959) == 4        # c2
    assert bd.pkv_decode_num_splits(7, 16, 8, D, 1977) == 4       # c5's decode batch
    assert bd.pkv_decode_num_splits(1, 16, 8, D, 64) == 1         # c1: one pass


def test_prefill_workspace_covers_the_partials(lib):
    for B, T, (Hq, Hkv), ctx in itertools.product(
            [1, 3, 8], [1, 64, 512], [(16, 8), (32, 8), (8, 1)],
            [64, 256, 3000, 8192, 131072]):
        if ctx < T:
            continue
        ws = bd.pkv_prefill_workspace_bytes(B, T, Hq, Hkv, D, ctx)
        assert ws >= 0
        if ws:
            # at least two splits of every (128-row tile, KV head) group: partial
            # outputs [D][128] and (m, l) [128][2] in fp32, and a counter each
            groups = B * -(-T * (Hq // Hkv) // 128) * Hkv
            assert ws >= groups * (2 * 128 * (D + 2) * 4 + 4), (B, T, Hq, Hkv, ctx, ws)


def test_prefill_plans_quoted_in_the_measurements(lib):
    # short contexts (at most 4 key tiles) run without splits
    assert bd.pkv_prefill_workspace_bytes(2, 106, 16, 8, D, 256) == 0
    # a c5 chunk (Qwen3-0.6B heads, 512 queries, up to 3000 keys): 8 row tiles
    # x 8 KV heads x 4 key splits of partials [D][128] and (m, l) [128][2],
    # then one arrival counter per (row tile, KV head), padded to 256 bytes
    assert bd.pkv_prefill_workspace_bytes(1, 512, 16, 8, D, 3000) == \
        64 * 4 * 128 * (D + 2) * 4 + 256
    # the longest supported context, and one key more (unsupported: 0)
    assert bd.pkv_prefill_workspace_bytes(1, 64, 32, 8, D, 131072) > 0
    assert bd.pkv_prefill_workspace_bytes(1, 64, 32, 8, D, 131073) == 0
