"""Bank-conflict model of the varlen kernel's transposed V tile in LDS
(csrc/varlen_attention.hip, VarlenTile): 64 banks of 4 bytes, 8-byte
accesses served 32 lanes per cycle.  Both the transposing stores of a
staged tile and the matrix-core operand reads must touch every bank at most
once per 32-lane phase with the kernel's stride (KT/2 + 2 words) and word
swizzle (column XOR V_XOR * (row / 32)); without the swizzle or the padding
they conflict, so the model is not vacuous.  The addressing is restated
from the kernel source, and the test first checks that the source still
holds those expressions."""
import os

import pytest

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "paged_kv_decode_store_amd", "csrc", "varlen_attention.hip")
GROUP_THREADS = 256   # threads of one wave group, which stages one tile
BANKS = 64
PHASE = 32            # lanes served per cycle for 8-byte accesses


def kernel_source():
    with open(SRC) as f:
        return f.read()


def test_source_still_holds_the_modelled_addressing():
    s = kernel_source()
    for line in ("static constexpr int V_RS = KT / 2 + 2;",
                 "static constexpr int V_XOR = D == 128 ? 4 : 8;",
                 "const int col = (2 * kq) ^ (T::V_XOR * (row >> 5));",
                 "*reinterpret_cast<u2_t *>(vs + row * T::V_RS + col) = u2_t{w0, w1};",
                 "const int v_lane = T::K_BYTES + (c * T::V_RS + 2 * h) * 4;",
                 "return v_lane + (32 * j * T::V_RS + ((8 * u + 4 * e) ^ (T::V_XOR * j))) * 4;",
                 "constexpr int kVGroupThreads = kVRowWaves * 64;",
                 "constexpr int kVRowWaves = 4;"):
        assert line in s, line


def worst_bank_use(D, v_rs, v_xor):
    """Largest number of 4-byte words any bank serves in one 32-lane phase,
    over every store and every operand read of a tile."""
    KT = 8192 // D
    pieces = D // 8
    worst = 0

    def count(word_addrs):
        use = {}
        for a in word_addrs:
            for w in (a, a + 1):   # 8-byte access: two consecutive words
                use[w % BANKS] = use.get(w % BANKS, 0) + 1
        return max(use.values())

    # stores: thread t writes dims piece*8 + d, position pair column 2*kq
    for d in range(8):
        for p0 in range(0, GROUP_THREADS, PHASE):
            addrs = []
            for t in range(p0, p0 + PHASE):
                piece, kq = t % pieces, t // pieces
                row = piece * 8 + d
                col = (2 * kq) ^ (v_xor * (row >> 5))
                addrs.append(row * v_rs + col)
            worst = max(worst, count(addrs))
    # operand reads: lane l reads dim row 32j + l%32, columns
    # ((8u + 4e) ^ (V_XOR j)) + 2 (l / 32)
    for j in range(D // 32):
        for u in range(KT // 16):
            for e in range(2):
                for half in range(2):
                    addrs = []
                    for l in range(half * PHASE, (half + 1) * PHASE):
                        c, h = l % 32, l // 32
                        addrs.append(32 * j * v_rs + c * v_rs + 2 * h + ((8 * u + 4 * e) ^ (v_xor * j)))
                    worst = max(worst, count(addrs))
    return worst


@pytest.mark.parametrize("D", [128, 64])
def test_transposed_v_tile_is_bank_conflict_free(D):
    KT = 8192 // D
    v_xor = 4 if D == 128 else 8
    assert v_xor * (D // 32 - 1) < KT // 2   # the swizzle stays inside a row
    assert worst_bank_use(D, KT // 2 + 2, v_xor) == 1


@pytest.mark.parametrize("D", [128, 64])
def test_without_swizzle_or_padding_the_tile_conflicts(D):
    KT = 8192 // D
    v_xor = 4 if D == 128 else 8
    assert worst_bank_use(D, KT // 2 + 2, 0) > 1    # no swizzle
    assert worst_bank_use(D, KT // 2, v_xor) > 1    # no padding
