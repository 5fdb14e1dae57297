"""The attention kernels' LDS key-tile layout is free of bank conflicts.

A 512-wide bf16 key row is 1 KiB with its 16-byte chunks permuted per key:
chunk c of key r sits at chunk c ^ swz(r), swz(r) = A[r % 4] ^ ((r // 4) % 4) with
A = (0, 4, 10, 14).  The score product reads one 16-byte chunk per lane (lane l:
key l % 32, chunk half l // 32) and the value product reads 8 bytes per lane with
transposing reads (keys 4g + j // 4 and 8 more, a column chunk per lane).  The
address formulas below are the ones csrc/verify_attn.hip uses; the check is that,
under a 64-bank x 4-byte model, every group of lanes the LDS serves together
(16 lanes of a 16-byte read, 32 lanes of an 8-byte read) touches distinct banks.
Host logic only."""
import itertools


def swz_a(r):
    return (0xEA40 >> (4 * (r & 3))) & 15


def swz(r):
    return swz_a(r) ^ ((r >> 2) & 3)


def qk_read_addr(lane, step):
    n, g = lane & 31, lane >> 5
    base = n * 1024 + 16 * (g ^ swz(n))
    return (base ^ ((step & 7) << 5)) + 256 * (step >> 3)


def vt_read_addrs(lane, cb, k1):
    """The two 8-byte transposing reads of lane `lane` for output block cb and key half k1."""
    j, q, g = lane & 15, lane >> 4, lane >> 5
    x = 2 * (q & 1) + ((j & 3) >> 1)
    f0 = swz_a(j >> 2) ^ g
    f1 = f0 ^ 2
    rb = (4 * g + (j >> 2)) * 1024 + 8 * (j & 1)
    p0 = rb + 16 * ((x ^ f0) & 3) + 64 * (f0 >> 2)
    p1 = rb + 16 * ((x ^ f1) & 3) + 64 * (f1 >> 2)
    c, h = 64 * (cb & 3), 256 * (cb >> 2) + 16384 * k1
    return (p0 ^ c) + h, (p1 ^ c) + h + 8192


def banks(addr, nbytes):
    return [((addr + b) // 4) % 64 for b in range(0, nbytes, 4)]


def test_swz_is_a_permutation_per_16_keys():
    for base in range(0, 64, 16):
        assert sorted(swz(base + r) for r in range(16)) == list(range(16))


def test_score_reads_conflict_free():
    for step in range(32):
        for g0 in range(0, 64, 16):  # 16 lanes x 16 bytes = all 64 banks
            used = list(itertools.chain.from_iterable(
                banks(qk_read_addr(l, step), 16) for l in range(g0, g0 + 16)))
            assert len(set(used)) == 64, (step, g0)


def test_score_reads_stay_in_their_key_row():
    for lane in range(64):
        for step in range(32):
            a = qk_read_addr(lane, step)
            assert a // 1024 == lane & 31 and a % 16 == 0


def test_value_reads_conflict_free():
    for cb in range(16):
        for k1 in range(2):
            for which in range(2):
                for g0 in (0, 32):  # 32 lanes x 8 bytes = all 64 banks
                    used = list(itertools.chain.from_iterable(
                        banks(vt_read_addrs(l, cb, k1)[which], 8) for l in range(g0, g0 + 32)))
                    assert len(set(used)) == 64, (cb, k1, which, g0)


def test_value_reads_hit_the_right_logical_chunk():
    """Each transposing read lands on the key row and logical 16-byte column chunk
    the value operand needs (keys 4g + j//4 + 8*which + 16*k1, columns of block cb)."""
    for lane in range(64):
        j, q, g = lane & 15, lane >> 4, lane >> 5
        for cb in range(16):
            for k1 in range(2):
                for which in range(2):
                    a = vt_read_addrs(lane, cb, k1)[which]
                    key = a // 1024
                    assert key == 4 * g + (j >> 2) + 8 * which + 16 * k1
                    phys = (a % 1024) // 16
                    logical = phys ^ swz(key)
                    col = 8 * logical + (4 if (a % 16) >= 8 else 0)
                    assert col // 32 == cb
                    assert col % 32 == 16 * (q & 1) + 4 * (j & 3)
