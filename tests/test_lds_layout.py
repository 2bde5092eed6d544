"""CPU model of the matrix engine's LDS staging (engine_mfma.hip).

The engine moves each 256 x 64 operand stage from global memory into LDS with
16-byte direct loads and feeds the MFMA fragments from there.  Two layouts:

* k-major operands (reduction index contiguous in memory: W and H of the
  logits, G of dH) sit as [256 rows][64 k]; 16-byte chunk p of row R holds
  k-chunk p ^ ((R >> 1) & 7); fragments are read with ds_read_b128;
* mn-major operands (reduction index strided: W of dH, G^T and H of dW) sit
  as [64 k][256 mn]; chunk p of row k holds mn-chunk p ^ (4 (k & 3)); the
  fragments come through the gfx950 transpose read ds_read_b64_tr_b16.

This test restates the kernel's per-lane offset formulas (lane_load_offsets,
the load placement of load_stage_fast / load_stage_edge, lane_frag_offsets,
read_frag) in Python, fills a simulated LDS from a random operand exactly as
the loads place it, reads every fragment of every k-step back and checks each
element against the operand element that the MFMA operand layout asks for:
for v_mfma_f32_32x32x16_bf16, lane l of a fragment holds operand row
(A: m, B: n) l % 32 and reduction indices 8 (l // 32) .. 8 (l // 32) + 7.

Transpose read model (the semantics the kernel's comments state): within each
group of 16 lanes, lane j supplies the address of 4 consecutive 16-bit values;
lane s of the group receives value s % 4 of lane 4 t + s // 4, for t = 0..3.

Bank model: 64 banks of 4 bytes; a 16-byte read is served 16 lanes at a time
and an 8-byte read 32 lanes at a time (256 bytes per pass).  A pass without
two lanes on one bank with different addresses is conflict-free.
"""
import numpy as np
import pytest

TM = 256          # stage rows (mn)
TK = 64           # stage depth (k)
ROW_K = TK * 2    # bytes of a k-major stage row
ROW_MN = TM * 2   # bytes of an mn-major stage row
STAGE = TM * TK * 2


# ---- the kernel's formulas, restated -------------------------------------------------

def lane_load_offsets(kmaj, ld, lane):
    """Byte offsets (even load i, odd load i) of a lane's 16-byte load, relative to
    the first row of the load."""
    out = []
    for par in range(2):
        if kmaj:
            kc = (lane & 7) ^ ((4 * par + (lane >> 4)) & 7)
            out.append((lane >> 3) * ld * 2 + 16 * kc)
        else:
            c = (lane & 31) ^ (4 * ((2 * par + (lane >> 5)) & 3))
            out.append((lane >> 5) * ld * 2 + 16 * c)
    return out


def load_rows(kmaj, w, i):
    """First operand row (relative to the stage) of load i of wave w: 8 rows
    (k-major) or 2 rows (mn-major) per load; the load fills LDS bytes
    [1024 (8 w + i), + 1024), lane L at + 16 L."""
    return 64 * w + 8 * i if kmaj else 16 * w + 2 * i


def lane_frag_offsets(kmaj, wbase, lane):
    if kmaj:
        r, h = lane & 31, lane >> 5
        sw = (r >> 1) & 7
        return [(wbase + r) * 128 + 16 * ((2 * ks + h) ^ sw) for ks in range(4)]
    g, s = lane >> 4, lane & 15
    q = s >> 2
    low = 2 * (g & 1) + ((s & 3) >> 1)
    base = (8 * (g >> 1) + q) * 512 + 2 * wbase + 16 * low + 8 * (s & 1)
    return [base + 64 * (i ^ q) for i in range(4)]


# ---- simulation -----------------------------------------------------------------------

def fill_stage(kmaj, op, mn0, k0):
    """LDS bytes of one stage of operand `op` (uint16 array, rows = mn for k-major,
    rows = k for mn-major), as the 4 waves' 8 loads each place it."""
    lds = np.zeros(STAGE, dtype=np.uint8)
    ld = op.shape[1]
    flat = op.reshape(-1).view(np.uint8)
    for w in range(4):
        for i in range(8):
            r0 = load_rows(kmaj, w, i)
            first = ((mn0 + r0) * ld + k0) * 2 if kmaj else ((k0 + r0) * ld + mn0) * 2
            for lane in range(64):
                src = first + lane_load_offsets(kmaj, ld, lane)[i & 1]
                dst = 1024 * (8 * w + i) + 16 * lane
                lds[dst:dst + 16] = flat[src:src + 16]
    return lds


def read16(lds, addr, nbytes):
    return lds[addr:addr + nbytes].view(np.uint16)


def tr_b16(lds, addrs):
    """ds_read_b64_tr_b16 over 64 lanes: returns [64][4] uint16."""
    out = np.zeros((64, 4), dtype=np.uint16)
    for g in range(4):
        m = np.stack([read16(lds, addrs[16 * g + j], 8) for j in range(16)])  # [16 lanes][4 values]
        for s in range(16):
            for t in range(4):
                out[16 * g + s, t] = m[4 * t + s // 4, s % 4]
    return out


def fragment(kmaj, lds, wbase, i, ks):
    """[64 lanes][8] uint16 of fragment (subtile i, k-step ks)."""
    fo = [lane_frag_offsets(kmaj, wbase, lane) for lane in range(64)]
    if kmaj:
        return np.stack([read16(lds, fo[lane][ks] + 4096 * i, 16) for lane in range(64)])
    lo = tr_b16(lds, [fo[lane][i] + 8192 * ks for lane in range(64)])
    hi = tr_b16(lds, [fo[lane][i] + 8192 * ks + 2048 for lane in range(64)])
    return np.concatenate([lo, hi], axis=1)


def expected(kmaj, op, mn0, k0, wbase, i, ks):
    out = np.zeros((64, 8), dtype=np.uint16)
    for lane in range(64):
        mn = mn0 + wbase + 32 * i + lane % 32
        k = k0 + 16 * ks + 8 * (lane // 32)
        out[lane] = op[mn, k:k + 8] if kmaj else op[k:k + 8, mn]
    return out


@pytest.mark.parametrize("kmaj", [True, False], ids=["k-major", "mn-major"])
def test_every_fragment_element(kmaj):
    # an operand larger than one stage, read at a nonzero stage origin; every value is
    # distinct (its own index), so any misplaced element shows
    shape = (320, 128) if kmaj else (128, 320)
    rng = np.random.default_rng(5)
    op = rng.permutation(shape[0] * shape[1]).astype(np.uint16).reshape(shape)
    mn0, k0 = 64, 64
    lds = fill_stage(kmaj, op, mn0, k0)
    for wbase in (0, 128):
        for i in range(4):
            for ks in range(4):
                got = fragment(kmaj, lds, wbase, i, ks)
                np.testing.assert_array_equal(got, expected(kmaj, op, mn0, k0, wbase, i, ks),
                                              err_msg=f"wbase {wbase} subtile {i} k-step {ks}")


@pytest.mark.parametrize("kmaj", [True, False], ids=["k-major", "mn-major"])
def test_stage_is_a_permutation(kmaj):
    """Every byte of the stage is written exactly once and every operand element of
    the stage lands somewhere: the swizzle loses nothing."""
    shape = (256, 64) if kmaj else (64, 256)
    op = np.arange(256 * 64, dtype=np.uint16).reshape(shape)
    lds = fill_stage(kmaj, op, 0, 0).view(np.uint16)
    assert sorted(lds.tolist()) == list(range(256 * 64))


def _conflicts(addrs, nbytes, lanes_per_pass):
    """Number of passes in which two lanes hit one bank at different addresses."""
    bad = 0
    for p0 in range(0, 64, lanes_per_pass):
        owner = {}
        for lane in range(p0, p0 + lanes_per_pass):
            for b in range(nbytes // 4):
                dword = addrs[lane] // 4 + b
                bank = dword % 64
                if owner.setdefault(bank, dword) != dword:
                    bad += 1
                    break
    return bad


@pytest.mark.parametrize("kmaj", [True, False], ids=["k-major", "mn-major"])
def test_fragment_reads_are_bank_conflict_free(kmaj):
    for wbase in (0, 128):
        fo = [lane_frag_offsets(kmaj, wbase, lane) for lane in range(64)]
        for i in range(4):
            for ks in range(4):
                if kmaj:
                    assert _conflicts([fo[l][ks] + 4096 * i for l in range(64)], 16, 16) == 0
                else:
                    for extra in (0, 2048):
                        assert _conflicts([fo[l][i] + 8192 * ks + extra for l in range(64)], 8, 32) == 0


def test_direct_loads_write_whole_kilobytes():
    """Each direct load of a wave writes one contiguous 1 KB block (lane L at +16 L), so
    the loads of a stage tile it without overlap and without bank conflicts."""
    blocks = sorted(1024 * (8 * w + i) for w in range(4) for i in range(8))
    assert blocks == list(range(0, STAGE, 1024))
    assert _conflicts([16 * lane for lane in range(64)], 16, 16) == 0
