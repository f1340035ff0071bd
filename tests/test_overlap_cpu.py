"""Host logic of the overlap module that needs no GPU: CU-mask bit packing."""

import pytest

from reduce_rmsnorm_amd.overlap import NUM_MASK_BITS, mask_words


def test_mask_words_packs_bits_little_endian_per_word():
    w = mask_words([0, 1, 31, 32, 255])
    assert len(w) == NUM_MASK_BITS // 32
    assert w == [0x80000003, 0x1, 0, 0, 0, 0, 0, 0x80000000]


def test_mask_words_first_k_bits_and_duplicates():
    assert mask_words(range(8)) == [0xFF] + [0] * 7
    assert mask_words(range(256)) == [0xFFFFFFFF] * 8
    assert mask_words([5, 5, 5]) == [1 << 5] + [0] * 7
    assert mask_words([]) == [0] * 8


@pytest.mark.parametrize("bad", [-1, 256, 1000])
def test_mask_words_rejects_bits_outside_the_mask(bad):
    with pytest.raises(ValueError):
        mask_words([bad])
