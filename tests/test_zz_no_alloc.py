"""moe_permute_noalloc, the variant of moe_permute for callers that cannot
allocate device memory, against moe_permute through the C ABI (needs an
MI355X).  Integer results, so bit-exact: counts, offsets, both permutations
and the gathered rows.  Calls follow one another on one device and share its
static scratch, so each case makes two calls in a row, the second smaller,
and the largest case fills the scratch's limit of 2^20 pairs."""

import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _selection(T, k, E, seed):
    """Top-k expert ids of random logits (distinct per token, any order)."""
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx = np.argsort(-logits, axis=1, kind="stable")[:, :k].astype(np.int32)
    return torch.from_numpy(np.ascontiguousarray(idx)).cuda()


def _compare(L, T, k, E, cap, d, seed):
    idx = _selection(T, k, E, seed)
    x = None
    if d:
        x = torch.from_numpy(np.random.default_rng(seed + 1).standard_normal((T, d))
                             .astype(np.float32)).cuda().to(torch.bfloat16)
    want = L.moe_permute(idx, E, cap, x)
    got = L.moe_permute_noalloc(idx, E, cap, x)
    torch.cuda.synchronize()
    names = ("expert_count", "expert_offset", "pair_row", "row_pair", "x_perm")
    for name, a, b in zip(names, want, got):
        if a is None:
            assert b is None, name
            continue
        if name == "x_perm":  # rows past the kept count are not written by either call
            n = int(want[1][-1])
            a, b = a[:n], b[:n]
        assert torch.equal(a, b), (name, T, k, E, cap)
    return int(want[1][-1])


@pytest.mark.parametrize("first,second", [
    ((131072, 8, 256, -1, 0), (4096, 2, 8, -1, 64)),          # the scratch's limit, then small
    ((16384, 2, 64, 640, 128), (2048, 2, 64, 40, 128)),       # capacity drops, with the gather
    ((65536, 8, 128, -1, 0), (1, 1, 1, -1, 0)),               # fine-grained, then one pair
    ((3000, 5, 200, 7, 96), (999, 3, 17, 0, 0)),              # ragged sizes; C = 0 drops all
])
def test_permute_noalloc_matches_permute(first, second):
    from sparse_mixture_experts_moe_amd import _lib as L
    for n, (T, k, E, cap, d) in enumerate((first, second)):
        _say(f"[case] noalloc call {n}: T={T} k={k} E={E} cap={cap} d={d}")
        kept = _compare(L, T, k, E, cap, d, seed=T + k + E)
        _say(f"[ok] noalloc call {n}: {kept} kept rows")


def test_permute_noalloc_limits():
    """Past the scratch's 2^20 pairs (or E > 256) the call is rejected on the
    host, before anything is enqueued; T = 0 writes zero counts."""
    from sparse_mixture_experts_moe_amd import _lib as L
    idx = torch.zeros((131072 + 1, 8), dtype=torch.int32, device="cuda")
    with pytest.raises(L.MoEError) as e:
        L.moe_permute_noalloc(idx, 8)
    assert e.value.status == L.MOE_EUNSUPPORTED and "scratch" in str(e.value)
    empty = torch.zeros((0, 2), dtype=torch.int32, device="cuda")
    cnt = torch.full((8,), 7, dtype=torch.int32, device="cuda")
    off = torch.full((9,), 7, dtype=torch.int32, device="cuda")
    L.moe_permute_noalloc(empty, 8, expert_count=cnt, expert_offset=off)
    torch.cuda.synchronize()
    assert int(cnt.abs().sum()) == 0 and int(off.abs().sum()) == 0
