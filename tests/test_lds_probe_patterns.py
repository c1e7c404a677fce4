"""The LDS probe's attention patterns (hybrid_mamba_attention_amd.lds_probe)
restate the stage layout: the stage writes cover every 16-byte chunk of the
two pages exactly once, and every K / V operand read lands on the chunk that
holds the token row and elements the matrix-core operand needs.  The pass
model of 16-byte reads reproduces the probe's measured cost of each
calibration pattern (cycles per wave instruction, in the profile of the LDS
patterns), and predicts conflict-free K and V operand reads."""
import pytest

from hybrid_mamba_attention_amd.lds_probe import (LANES, Stage, all_patterns, calibration_patterns,
                                                  read128_cycles, vchunk)

FORMS = [Stage(2, 128, 2, 8), Stage(2, 128, 1, 4), Stage(2, 64, 1, 4), Stage(4, 128, 1, 4)]


def written(st):
    """LDS chunk position -> (stage row, chunk of the row) from the writes."""
    where = {}
    for wave in range(st.NW):
        for tt in range(2):
            for qq in range(st.RND):
                for lane, off in enumerate(st.write_offsets(wave, tt, qq)):
                    if off is None:
                        continue
                    t = wave * 64 + lane
                    key = off // 16
                    assert key not in where, "chunk written twice"
                    where[key] = (tt * 16 + t // st.CPR + qq * st.RPP, t % st.CPR)
    return where


@pytest.mark.parametrize("st", FORMS, ids=lambda s: f"e{s.esize}-D{s.D}-HP{s.HP}-NW{s.NW}")
def test_stage_layout(st):
    where = written(st)
    assert sorted(where.values()) == [(r, c) for r in range(32) for c in range(st.CPR)]
    for wave in range(st.NW):
        hl = wave // st.WPH
        for tt in range(2):
            for ds in range(st.D // 32):
                for h in range(8 // st.EPC):
                    for lane, off in enumerate(st.k_offsets(wave, tt, ds, h)):
                        li, lg = lane & 15, lane >> 4
                        elem = hl * st.D + 8 * (lg + 4 * ds) + h * st.EPC
                        assert off % 16 == 0 and where[off // 16] == (16 * tt + li, elem // st.EPC)
        for e in range(8):
            for h in range(max(1, st.D // 16 * st.esize // 16)):
                for lane, off in enumerate(st.v_offsets(wave, e, h)):
                    li, lg = lane & 15, lane >> 4
                    elem = hl * st.D + st.dchunk(li) * (st.D // 16) + h * st.EPC
                    assert where[off // 16] == (16 * (e >> 2) + 4 * lg + (e & 3), elem // st.EPC)
                    assert off % 16 == (elem % st.EPC) * st.esize


def test_patterns_fit_the_probe():
    for name, kind, offs in all_patterns():
        size = 8 if kind == "read64" else 16
        assert len(offs) == LANES and all(o % size == 0 and 0 <= o <= 16384 - size for o in offs), name


# SQ_LDS_IDX_ACTIVE per wave instruction measured for the 16-byte read
# calibration patterns (one MI355X, the LDS patterns profile)
MEASURED_READ128 = {
    "cal linear 16B": 4, "cal broadcast 16B": 4, "cal one bank group 16B": 64, "cal f=l%16": 4,
    "cal f=l%8": 8, "cal f=l%4": 16, "cal f=(l/4)%16": 16, "cal f=(l/8)%8": 16, "cal f=(l/16)+4*(l%4)": 8,
    "cal f=l%8+8*((l/32)%2)": 8, "cal f=l%8+8*((l/16)%2)": 4, "cal f=l%8+8*((l/8)%2)": 4,
}


def test_pass_model_reproduces_the_calibration():
    got = {n: read128_cycles(o) for n, k, o in calibration_patterns() if k == "read128"}
    assert got == MEASURED_READ128


@pytest.mark.parametrize("st", FORMS[:2], ids=["hp2", "hp1"])
def test_operand_reads_are_conflict_free(st):
    assert sorted(vchunk(i) for i in range(16)) == list(range(16))
    for wave in range(st.NW):
        for tt in range(2):
            for ds in range(st.D // 32):
                assert read128_cycles(st.k_offsets(wave, tt, ds)) == 4
        for e in range(8):
            assert read128_cycles(st.v_offsets(wave, e)) == 4
            assert read128_cycles(st.v_offsets(wave, e, permuted=False)) == 8   # the 2-way conflict it removes
