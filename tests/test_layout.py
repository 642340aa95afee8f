"""The packed weight layout (MOE_LAYOUT_FRAG16, include/moe.h) as the
tests write it down, pinned on the CPU to what it is for: a 1 KiB block is
the B operand of one v_mfma_f32_16x16x32_bf16 in lane order (lane l holds
row l % 16, columns 8 (l / 16) .. + 7; the gfx950 ISA's operand layout for
the 16x16x32 bf16 MFMA), and the layout is a permutation."""
import torch

from parity import frag16_fp8_reference, frag16_reference


def test_reference_layout_matches_the_mfma_operand_order():
    # Lane l of a 16x16x32 MFMA B operand holds row l % 16, columns
    # 8 (l / 16) .. + 7: the 16 bytes at 16 l of a block are those elements.
    R, C = 32, 64
    w = torch.arange(R * C, dtype=torch.int32).reshape(R, C)
    p = frag16_reference(w).reshape(-1)
    for i in range(R // 16):
        for j in range(C // 32):
            blk = p[(i * (C // 32) + j) * 512:(i * (C // 32) + j + 1) * 512].reshape(64, 8)
            for lane in range(64):
                r, c0 = i * 16 + lane % 16, j * 32 + 8 * (lane // 16)
                assert blk[lane].tolist() == w[r, c0:c0 + 8].tolist()


def test_reference_layout_is_a_permutation():
    w = torch.arange(3 * 48 * 96, dtype=torch.int32).reshape(3, 48, 96)
    p = frag16_reference(w)
    assert p.shape == w.shape
    assert torch.equal(torch.sort(p.reshape(-1)).values, w.reshape(-1))
    # stacked matrices keep their own stride: matrix m stays in its slice
    for m in range(3):
        assert p[m].min() == m * 48 * 96 and p[m].max() == (m + 1) * 48 * 96 - 1


def test_fp8_reference_layout_feeds_both_slabs_of_a_lane():
    # FP8 blocks of 16 rows x 64 columns: lane l's 16 bytes are the 8 codes
    # lane l supplies to the MFMA of columns 0-31 (row l % 16, columns
    # 8 (l / 16) .. + 7), then the 8 it supplies to columns 32-63.
    R, C = 32, 128
    w = torch.arange(R * C, dtype=torch.int32).reshape(R, C)
    p = frag16_fp8_reference(w).reshape(-1)
    for i in range(R // 16):
        for j in range(C // 64):
            blk = p[(i * (C // 64) + j) * 1024:(i * (C // 64) + j + 1) * 1024].reshape(64, 16)
            for lane in range(64):
                r, c0 = i * 16 + lane % 16, j * 64 + 8 * (lane // 16)
                assert blk[lane, :8].tolist() == w[r, c0:c0 + 8].tolist()
                assert blk[lane, 8:].tolist() == w[r, c0 + 32:c0 + 40].tolist()
    q = frag16_fp8_reference(torch.arange(2 * 48 * 192, dtype=torch.int32).reshape(2, 48, 192))
    assert torch.equal(torch.sort(q.reshape(-1)).values, torch.arange(2 * 48 * 192, dtype=torch.int32))
