"""A model, on the CPU, of how the VQ3R dequant-GEMV forms its LDS lookup
addresses from the packed record words (v_perm_b32 byte selection, as in
residual_vector_quantization_amd/csrc/vq_gemv.hip, direct form): for random
records, every lookup must read the intended stage's index, the lane's slice
and the right table buffer, each record must read its three stages once, and
the 32 lanes of every half-wave lookup instruction must fall in 32 distinct
LDS banks (32 banks of 4 bytes). The constants mirror the kernel's set-up."""
import random

GJ = 16                      # slices per block
SLOT_STAGE = [0, 1, 2, 0]    # table row slots: stages 0, 1, 2 and stage 0 again


def perm(src0, src1, sel):
    """v_perm_b32: byte i of the result is byte sel_i of {src0 : src1}
    (0-3 from src1, 4-7 from src0), 0x0c gives 0x00."""
    b = [(src1 >> (8 * i)) & 255 for i in range(4)] + [(src0 >> (8 * i)) & 255 for i in range(4)]
    out = 0
    for i in range(4):
        s = (sel >> (8 * i)) & 255
        assert s < 8 or s == 0x0C, hex(sel)
        out |= (b[s] if s < 8 else 0) << (8 * i)
    return out


def lane_setup(lane):
    hb = (lane >> 4) & 1

    def off(slot, m):
        return slot * 64 + ((m + lane) & (GJ - 1)) * 4

    soff_d = [[[0] * 4 for _ in range(3)] for _ in range(2)]
    soff2 = [0] * 3
    sel_a, sel_b, sel_c = [0] * 3, [0] * 3, [0] * 2
    for k in range(3):
        sl = k + hb
        s1 = (3 if hb else 0) if k == 0 else ((1 + hb) if k == 1 else (2 - hb))
        for c in range(4):
            v = off(sl, 4 * c) | (off(s1, 4 * c + 1) << 8) | (off(sl, 4 * c + 3) << 24)
            soff_d[0][k][c] = v
            soff_d[1][k][c] = v | 0x10000
            soff2[k] |= off(sl, 4 * c + 2) << (8 * c)
        st = (k + hb) % 3
        sel_a[k] = 0x0C060004 | (st << 8)
        sel_b[k] = 0x0C060007 | ((1 + st) << 8)
        if k > 0:
            sel_c[k - 1] = 0x0C060005 | ((0 if (k == 1) == (hb == 0) else 1) << 8)
    sel2 = (3 | (4 << 8) | (2 << 16) | 0x0C000000) if hb else (2 | (3 << 8) | (4 << 16) | 0x0C000000)
    return soff_d, soff2, sel_a, sel_b, sel_c, sel2


def chunk_addresses(lane, chunk_bytes, c, lb):
    """The 12 lookup addresses (record qq, lookup k) of chunk c of a lane."""
    soff_d, soff2, sel_a, sel_b, sel_c, sel2 = lane_setup(lane)
    w0, w1, w2 = (int.from_bytes(bytes(chunk_bytes[4 * i:4 * i + 4]), "little") for i in range(3))
    sd = soff_d[lb]
    a = {}
    for k in range(3):
        a[(0, k)] = perm(sd[k][c], w0, sel_a[k])
        a[(3, k)] = perm(sd[k][c], w2, sel_b[k])
    a[(1, 0)] = perm(sd[0][c], w0, 0x0C060305)
    a[(1, 1)] = perm(sd[1][c], w1, sel_c[0])
    a[(1, 2)] = perm(sd[2][c], w1, sel_c[1])
    w = perm(w2, w1, sel2) | ((1 << 24) if lb else 0)
    for k in range(3):
        a[(2, k)] = perm(soff2[k], w, 0x0C030004 | (k << 8) | c)
    return a


def test_direct_addressing_reads_the_right_entries_without_bank_conflicts():
    rng = random.Random(7)
    for trial in range(40):
        lb = trial & 1
        recs = [[[rng.randrange(256) for _ in range(3)] for _ in range(16)] for _ in range(64)]
        per_instr = {}
        for lane in range(64):
            for c in range(4):
                chunk = sum((recs[lane][4 * c + qq] for qq in range(4)), [])
                a = chunk_addresses(lane, chunk, c, lb)
                for qq in range(4):
                    stages = set()
                    for k in range(3):
                        ad = a[(qq, k)]
                        assert ad >> 16 == lb                           # the table buffer
                        slot, e = (ad & 255) >> 6, (ad >> 8) & 255
                        assert ((ad & 255) >> 2) & 15 == (4 * c + qq + lane) & 15   # the lane's slice
                        assert e == recs[lane][4 * c + qq][SLOT_STAGE[slot]]         # that stage's index
                        stages.add(SLOT_STAGE[slot])
                        per_instr.setdefault((c, qq, k), []).append(ad)
                    assert stages == {0, 1, 2}
        for key, addrs in per_instr.items():
            for half in range(2):
                banks = {(x >> 2) & 31 for x in addrs[32 * half:32 * half + 32]}
                assert len(banks) == 32, (key, half)


def test_one_copy_of_stage_0_would_conflict():
    """Counter-check of the layout argument: with the rotated stage orders but
    slots equal to stages (no second copy of stage 0), the third lookup of a
    record pairs slots 2 and 0 in the two halves: same banks, a two-way conflict."""
    lane_slots = {}
    for lane in range(32):
        hb = (lane >> 4) & 1
        slot = (2 + hb) % 3
        lane_slots[lane] = slot * 16 + (lane & 15)
    assert len({b % 32 for b in lane_slots.values()}) == 16
