"""CPU checks of the inference-layout definition the GPU tests read weights with."""
import numpy as np
import pytest

from layout import block_width, from_inference, to_inference


@pytest.mark.parametrize("N,K", [(16, 32), (32, 768), (48, 1024), (16, 2560), (64, 96)])
def test_round_trip_is_a_permutation(N, K):
    W = np.arange(N * K, dtype=np.int64).reshape(N, K)
    S = to_inference(W)
    assert sorted(S.ravel().tolist()) == list(range(N * K))
    assert np.array_equal(from_inference(S), W)


@pytest.mark.parametrize("K", [512, 1024, 4096])
def test_mfma_fragments_are_contiguous(K):
    """With BW = 512 the operand of k-step s for rows 16 rb .. + 16 is the 1 KB at
    row 16 rb + s % 16, columns 512 (s // 16) .. + 512, lane l holding row l % 16 and
    k 32 s + 8 (l // 16) .. + 8."""
    N = 32
    W = np.arange(N * K, dtype=np.int64).reshape(N, K)
    S = to_inference(W)
    assert block_width(K) == 512
    for rb in range(N // 16):
        for s in range(K // 32):
            frag = S[rb * 16 + s % 16, 512 * (s // 16):512 * (s // 16) + 512].reshape(64, 8)
            for l in range(64):
                want = W[rb * 16 + l % 16, 32 * s + 8 * (l // 16):32 * s + 8 * (l // 16) + 8]
                assert np.array_equal(frag[l], want)


def test_block_width():
    assert [block_width(k) for k in (32, 96, 768, 3072, 5120, 20480)] == [32, 32, 256, 512, 512, 512]
