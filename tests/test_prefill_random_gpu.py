"""Seeded random prefill batches against the fp64 oracle, bf16 and int8
pages: ragged chunk lengths and prefixes (key-tile counts odd and even, 1 ..
14, and contexts that cross the 64-tile split bound), group sizes 1 .. 8,
decode sequences mixed in.  They exercise the pipelined key loop's entry
and exit paths (one tile, the last step alone, the two-step unroll), the
diagonal and past-context masks on first and last tiles, and the split
merge with differing split counts per sequence."""
import numpy as np
import pytest

from paged_kv_gqa_pkv_amd import synth as S

from test_parity_gpu import check_workload
from test_parity_int8_gpu import run_int8_step

pytestmark = pytest.mark.gpu


def random_batch(seed):
    rng = np.random.default_rng(2000 + seed)
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 4, 8])) if G < 8 else int(rng.choice([1, 2]))
    n_pre = int(rng.integers(1, 7))
    seqs = []
    for _ in range(n_pre):
        new = int(rng.integers(1, 161))
        pre = int(rng.choice([0, int(rng.integers(0, 900))]))
        seqs.append(S.SeqSpec(pre, new, True))
    if seed % 3 == 0:
        seqs.append(S.SeqSpec(4200 - 40, 40, True))   # past 64 tiles: key splits
    for _ in range(int(rng.integers(0, 4))):
        seqs.append(S.SeqSpec(int(rng.integers(0, 500)), 1, False))
    pages = sum((s.pre_len + s.new_len + 15) // 16 for s in seqs)
    return S.custom_workload(f"random_prefill_{seed}", seqs, Hq=Hkv * G, Hkv=Hkv, D=128,
                             num_blocks=pages + 16, base_seed=2000 + seed)


@pytest.mark.parametrize("seed", range(6))
def test_random_prefill_batches_bf16(seed):
    check_workload(random_batch(seed))


@pytest.mark.parametrize("seed", range(6))
def test_random_prefill_batches_int8(seed):
    run_int8_step(random_batch(seed))
