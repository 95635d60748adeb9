"""The measurement probes behind the bench's measured ceilings compute what
they claim (needs an MI355X).

The MFMA probe gets small-integer bf16 operands, so every product and sum is
exact in fp32 and each wave's total follows from the operand layout of
v_mfma_f32_32x32x16_bf16: lane l supplies row (first operand) or column
(second operand) l mod 32 and the eight k values 8 (l div 32) .. +7.  The sum
of all elements of D = X Y is sum_k (sum_i X[i,k]) (sum_j Y[k,j]).
"""

import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def L():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import sparse_mixture_experts_moe_amd._lib as lib
    return lib


def _column_sums(frag):
    """frag [64, 8] (lane, element) -> length-16 vector over k of the sum of
    the 32 lanes that carry k."""
    return np.concatenate([frag[:32].sum(0), frag[32:].sum(0)])


@pytest.mark.parametrize("blocks,iters", [(1, 1), (3, 5), (256, 2)])
def test_mfma_probe_exact(L, blocks, iters):
    _say(f"mfma probe blocks={blocks} iters={iters}")
    rng = np.random.default_rng(blocks * 100 + iters)
    vals = rng.integers(-3, 4, size=(blocks * 256, 8, 8)).astype(np.float32)
    src = torch.from_numpy(vals.reshape(-1)).to(torch.bfloat16).cuda()
    out = L.moe_probe_mfma_bf16(src, blocks, iters)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64).reshape(blocks * 4, 64).sum(1)
    want = np.zeros(blocks * 4)
    for w in range(blocks * 4):
        lanes = vals[w * 64:(w + 1) * 64].astype(np.float64)  # [64 lanes, 8 fragments, 8]
        sa = [_column_sums(lanes[:, i, :]) for i in range(4)]       # second operand a[i]
        sb = [_column_sums(lanes[:, 4 + j, :]) for j in range(4)]   # first operand b[j]
        want[w] = iters * sum(float(np.dot(sb[j], sa[i])) for i in range(4) for j in range(4))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("nbytes,blocks", [(16, 1), (16 * 1000 + 16 * 7, 3), (64 << 20, 2048)])
def test_read_probe_xor(L, nbytes, blocks):
    _say(f"read probe bytes={nbytes} blocks={blocks}")
    rng = np.random.default_rng(nbytes % 9973)
    words = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    out = L.moe_probe_read(buf, blocks)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)
